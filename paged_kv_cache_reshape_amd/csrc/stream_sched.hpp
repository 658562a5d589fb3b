// The balanced ("stream") decode schedule: the batch's K/V blocks, sequence
// after sequence, form one list per kv head, and each kv head's list is cut
// into R equal ranges of consecutive blocks, one per worker wave.  A worker
// streams its range, finishing a sequence's state whenever the sequence ends
// inside it; a sequence whose blocks fall in several ranges leaves one
// partial state per range, and the worker holding its last block merges
// them in the same launch (log-sum-exp merge; a multi-block reduction
// finished inside the launch, as in the LLAISYS README, CUDA argmax item,
// with the finishing block chosen statically: see stream_merge_last).
//
// Why: with fixed partitions per sequence the busiest compute unit streams a
// whole 1024-token partition while others idle; equal ranges give every
// worker the same bytes whatever the context lengths, and a pure-read probe
// of the Qwen3-shaped batch streamed its 152 MB in 24.5-25.6 us this way
// against 28-41 us for fixed partitions (measured on MI355X).
//
// Ranges come from the context lengths on the device: every workgroup scans
// the lengths (an exclusive prefix sum of blocks per sequence, T blocks in
// all) and worker r of a kv head takes blocks [r T / R, (r+1) T / R).
#pragma once

#include "attn_common.hpp"

namespace pa {

// Sequences a stream launch can take (the prefix sum lives in LDS).
constexpr int kStreamMaxSeqs = 2048;
// Blocks in one worker's range, at most: two table entries per lane.
constexpr int kStreamMaxRange = 128;
// Loads of a chunk repeated while a word of an arrived piece is still zero,
// at most (each is one memory round trip; in practice one or two suffice).
constexpr int kStreamMergeRetries = 4096;

// Blocks of a sequence of context length c; 0 when empty or longer than the
// table (those rows are written as zeros or NaN, nothing is streamed).
__device__ __forceinline__ int seq_blocks(int c, int bs, int max_blocks) {
  return (c > 0 && c <= max_blocks * bs) ? (c + bs - 1) / bs : 0;
}

// First block of worker r's range: floor(r T / R).
__device__ __forceinline__ int range_start(int r, int T, int R) {
  return (int)(((long long)r * T) / R);
}

// The worker whose range holds block x (x < T): the largest r with
// range_start(r) <= x, i.e. ceil((x + 1) R / T) - 1.
__device__ __forceinline__ int range_of(int x, int T, int R) {
  return (int)((((long long)x + 1) * R + T - 1) / T) - 1;
}

// Exclusive prefix sum of blocks per sequence into s_cum[0..B] (s_cum[B] =
// T), by the whole workgroup; returns T.  Sequences that are empty or longer
// than the table take no blocks; `empty(b, c)` is called once for each of
// them (by one thread) so that their output rows can be written.
template <int NT, class Empty>
__device__ __forceinline__ int stream_prefix(const DecodeArgs& a, int bs, int* s_cum,
                                             int* s_part, Empty&& empty) {
  constexpr int NWV = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.num_seqs;
  int carry = 0;
  for (int c0 = 0; c0 < B; c0 += NT) {
    const int b = c0 + tid;
    int nb = 0;
    if (b < B) {
      const int c = a.context_lens[b];
      nb = seq_blocks(c, bs, a.max_blocks);
      if (nb == 0) empty(b, c);
    }
    int x = nb;  // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(x, o, 64);
      if (lane >= o) x += t;
    }
    if (lane == 63) s_part[wave] = x;
    __syncthreads();
    int off = carry, tot = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const int v = s_part[w];
      off += w < wave ? v : 0;
      tot += v;
    }
    if (b < B) s_cum[b] = off + x - nb;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) s_cum[B] = carry;
  __syncthreads();
  return carry;
}

// One worker's range and, per lane, what it needs of the range's blocks i =
// lane and i = 64 + lane: the physical block (0 in place of an id outside
// the pool), the sequence, the block's index in it and the sequence's
// length.  Read back for block i (wave-uniform) with readlane.
struct StreamRange {
  int s, n;        // first block (in the kv head's list) and number of blocks
  int ent[2];      // physical block id
  int bj[2];       // (b << 16) | j, bit 31 set when the table entry is outside the pool
  int cx[2];       // context length of the block's sequence

  __device__ __forceinline__ int entry(int i) const {
    return __builtin_amdgcn_readlane(i < 64 ? ent[0] : ent[1], i & 63);
  }
  __device__ __forceinline__ int seqblk(int i) const {
    return __builtin_amdgcn_readlane(i < 64 ? bj[0] : bj[1], i & 63);
  }
  __device__ __forceinline__ int ctx(int i) const {
    return __builtin_amdgcn_readlane(i < 64 ? cx[0] : cx[1], i & 63);
  }
};

// Fill a worker's range (worker r of R, T blocks in all, R <= T so that
// every range holds at least one block).  The sequence of
// block g is the last b with s_cum[b] <= g; found for the range's first
// block with two ballots over LDS, then for each lane's blocks by counting
// the sequence starts that follow it.  The table entries and lengths are
// requested together, and nothing waits on them here.
__device__ __forceinline__ void stream_range(const DecodeArgs& a, const int* s_cum, int T, int R,
                                             int r, int lane, StreamRange& w) {
  const int B = a.num_seqs;
  w.s = range_start(r, T, R);
  w.n = range_start(r + 1, T, R) - w.s;
  w.ent[0] = w.ent[1] = 0;
  w.bj[0] = w.bj[1] = 0;
  w.cx[0] = w.cx[1] = 0;
  const int s = w.s, e = w.s + w.n;
  // Sequence of block s: chunk of 64 sequences, then the sequence in it.
  const int c1 = __popcll(__ballot(s_cum[min(64 * lane, B)] <= s)) - 1;
  const int b0 = 64 * c1 + __popcll(__ballot(s_cum[min(64 * c1 + lane, B)] <= s)) - 1;
  const int g0 = s + lane, g1 = s + 64 + lane;
  int b_0 = b0, b_1 = b0;
  for (int base = b0;; base += 64) {
    const int cs = s_cum[min(base + 1 + lane, B)];
    const int nk = __popcll(__ballot(cs < e));  // starts inside the range (uniform)
    for (int k = 0; k < nk; ++k) {
      const int c = __builtin_amdgcn_readlane(cs, k);
      b_0 += c <= g0;
      b_1 += c <= g1;
    }
    if (nk < 64) break;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = 64 * h + lane;
    if (i < w.n) {
      const int b = h ? b_1 : b_0;
      const int j = (h ? g1 : g0) - s_cum[b];
      const int id = a.block_tables[(size_t)b * a.max_blocks + j];
      const bool bad = id < 0 || id >= a.num_blocks;
      w.ent[h] = bad ? 0 : id;
      w.bj[h] = (b << 16) | j | (bad ? (int)0x80000000u : 0);
      w.cx[h] = a.context_lens[b];
    }
  }
}

// The same set-up for batches of at most 64 sequences, held in registers:
// every wave reads the lengths (lane b: sequence b) and scans them itself,
// so there is no LDS and no workgroup barrier, and a range's sequences are
// found with one ballot and lane shuffles instead of dependent LDS reads.
// Measured on MI355X (Qwen3-shaped batch, per-wave clock stamps): the LDS
// set-up took 0.56 us between the prefix sum and the first table request.
constexpr int kStreamSmallSeqs = 64;

// Lane b < B gets the first block of sequence b in `start` (the exclusive
// prefix sum of blocks) and its length in `len`; returns T.  `empty(b, c)`
// is called for sequences that take no blocks, by the first wave only.
template <class Empty>
__device__ __forceinline__ int stream_prefix_small(const DecodeArgs& a, int bs, int lane,
                                                   bool first_wave, int& start, int& len,
                                                   Empty&& empty) {
  const int B = a.num_seqs;
  len = lane < B ? a.context_lens[lane] : 0;
  const int nb = lane < B ? seq_blocks(len, bs, a.max_blocks) : 0;
  if (first_wave && lane < B && nb == 0) empty(lane, len);
  int x = nb;  // inclusive scan over the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(x, o, 64);
    if (lane >= o) x += t;
  }
  start = x - nb;
  return __builtin_amdgcn_readlane(x, 63);
}

// First block of sequence b (b <= B, wave-uniform) from those registers.
__device__ __forceinline__ int small_seq_start(int start, int b, int B, int T) {
  return b < B ? __builtin_amdgcn_readlane(start, b) : T;
}

// stream_range from those registers (B <= 64).
__device__ __forceinline__ void stream_range_small(const DecodeArgs& a, int start, int len, int T,
                                                   int R, int r, int lane, StreamRange& w) {
  const int B = a.num_seqs;
  w.s = range_start(r, T, R);
  w.n = range_start(r + 1, T, R) - w.s;
  w.ent[0] = w.ent[1] = 0;
  w.bj[0] = w.bj[1] = 0;
  w.cx[0] = w.cx[1] = 0;
  const int s = w.s, e = w.s + w.n;
  // Sequence of block s: the last b with start(b) <= s (empty sequences share
  // the next one's start, so the last such b holds the block).
  const int b0 = __popcll(__ballot(lane < B && start <= s)) - 1;
  // Starts of the sequences after b0 that fall inside the range (T past the
  // last sequence, which is >= e, so fewer than 64 of them).
  const int idx = b0 + 1 + lane;
  const int nxt = __shfl(start, min(idx, 63), 64);
  const int cs = idx < B ? nxt : T;
  const int nk = __popcll(__ballot(cs < e));
  const int g0 = s + lane, g1 = s + 64 + lane;
  int b_0 = b0, b_1 = b0;
  for (int k = 0; k < nk; ++k) {
    const int c = __builtin_amdgcn_readlane(cs, k);
    b_0 += c <= g0;
    b_1 += c <= g1;
  }
  // Start and length of each lane's two sequences, shuffled with every lane
  // active (b_0, b_1 < B).
  const int st[2] = {__shfl(start, b_0, 64), __shfl(start, b_1, 64)};
  const int ln[2] = {__shfl(len, b_0, 64), __shfl(len, b_1, 64)};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = 64 * h + lane;
    if (i < w.n) {
      const int b = h ? b_1 : b_0;
      const int j = (h ? g1 : g0) - st[h];
      const int id = a.block_tables[(size_t)b * a.max_blocks + j];
      const bool bad = id < 0 || id >= a.num_blocks;
      w.ent[h] = bad ? 0 : id;
      w.bj[h] = (b << 16) | j | (bad ? (int)0x80000000u : 0);
      w.cx[h] = ln[h];
    }
  }
}

// Partial states of the balanced schedule are stored encoded, one 32-bit
// word per float: the bitwise complement of the float, with every NaN first
// made the one quiet NaN 0x7FC00000.  No float then encodes to 0, so a zero
// word means "not written yet": a merger that loads a piece's state can
// tell, word by word, whether the piece's stores have landed (a 4-byte word
// is read whole), without waiting for the writer to acknowledge them.  The
// workspace is all zero before a call, and every reader zeroes what it read
// (each lane what it loaded, after using it), so every call leaves it zero.
__device__ __forceinline__ float ws_canon(float x) {
  return x != x ? __uint_as_float(0x7FC00000u) : x;
}
__device__ __forceinline__ uint32_t ws_encode(float x) { return ~__float_as_uint(ws_canon(x)); }
__device__ __forceinline__ float ws_decode(uint32_t w) { return __uint_as_float(~w); }

// Zero a lane's EL consecutive words (EL in {1, 2, 4, 8, 16}) with ordinary
// stores of exactly that width.
template <int EL>
__device__ __forceinline__ void zero_words(uint32_t* p) {
  if constexpr (EL == 1) {
    *p = 0u;
  } else if constexpr (EL == 2) {
    *reinterpret_cast<uint2*>(p) = make_uint2(0u, 0u);
  } else {
    static_assert(EL % 4 == 0, "whole 16-byte pieces");
#pragma unroll
    for (int k = 0; k < EL; k += 4) *reinterpret_cast<uint4*>(p + k) = make_uint4(0, 0, 0, 0);
  }
}

// Where partial states live: worker r of kv head h keeps up to two, slot 0
// for the sequence its range starts in, slot 1 for the one it ends in (the
// sequences between lie wholly inside the range).  Row index of query row
// gq (of G) of that state; acc at ws_acc[row * D], (max, sum) at ws_ml[row * 2].
__device__ __forceinline__ size_t stream_piece_row(int h, int r, int slot, int gq, int R,
                                                   int G) {
  return (((size_t)h * R + r) * 2 + slot) * G + gq;
}

// Where the partial states of one sequence's blocks [cb, cb + nb) lie: the
// workers r0 .. r1 whose ranges hold them (every range holds a block, R <=
// T); worker r0's state is in slot 1 when its range starts before cb (the
// sequence is the last one it holds), every other worker's in slot 0.
struct SeqPieces {
  int r0, r1, slot0;
  __device__ __forceinline__ SeqPieces(int cb, int nb, int T, int R)
      : r0(range_of(cb, T, R)),
        r1(range_of(cb + nb - 1, T, R)),
        slot0(range_start(range_of(cb, T, R), T, R) < cb ? 1 : 0) {}
  __device__ __forceinline__ int count() const { return r1 - r0 + 1; }
};

// 2 * EL bytes of bfloat16 output (nearest even) or 4 * EL of float32.
template <int EL>
__device__ __forceinline__ void store_row_part(BF16, void* base, size_t i, const float* x) {
  uint16_t* p = static_cast<uint16_t*>(base) + i;
  if constexpr (EL % 4 == 0) {
#pragma unroll
    for (int k = 0; k < EL; k += 4) {
      const uint2 v = make_uint2(
          (uint32_t)f32_to_bf16_rne(x[k]) | ((uint32_t)f32_to_bf16_rne(x[k + 1]) << 16),
          (uint32_t)f32_to_bf16_rne(x[k + 2]) | ((uint32_t)f32_to_bf16_rne(x[k + 3]) << 16));
      *reinterpret_cast<uint2*>(p + k) = v;
    }
  } else {
#pragma unroll
    for (int k = 0; k < EL; ++k) p[k] = f32_to_bf16_rne(x[k]);
  }
}
template <int EL>
__device__ __forceinline__ void store_row_part(F32, void* base, size_t i, const float* x) {
  float* p = static_cast<float*>(base) + i;
  if constexpr (EL % 4 == 0) {
#pragma unroll
    for (int k = 0; k < EL; k += 4)
      *reinterpret_cast<float4*>(p + k) = make_float4(x[k], x[k + 1], x[k + 2], x[k + 3]);
  } else {
#pragma unroll
    for (int k = 0; k < EL; ++k) p[k] = x[k];
  }
}

// Merge of every partial state of (sequence b, kv head h) into the output
// rows of its G query heads, by one wave of the merge kernel that runs after
// the stream launch (every piece is stored by then).  Pieces are folded in worker order, so the result does not depend
// on the order in which they were written; up to kBatch pieces are requested
// in one round trip.  Each lane takes EL consecutive elements of one query
// row, and zeroes the words it read once it has used them.
template <class DT, int D, int G>
__device__ __forceinline__ void stream_merge(const DecodeArgs& a, int b, int h,
                                             const SeqPieces& sp, int R, int lane) {
  constexpr int EL = G * D / 64;  // elements per lane (1 .. 16)
  static_assert(EL >= 1 && D % EL == 0, "a lane's elements lie in one row");
  constexpr int kBatch = EL <= 4 ? 8 : 4;
  const int gq = lane * EL / D;
  const int d0 = lane * EL % D;
  float M = kNoMax, L = 0.0f, A[EL];
#pragma unroll
  for (int k = 0; k < EL; ++k) A[k] = 0.0f;
  for (int p0 = sp.r0; p0 <= sp.r1; p0 += kBatch) {
    float pm[kBatch], pl[kBatch], pa[kBatch][EL];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int r = min(p0 + u, sp.r1);
      const int slot = r == sp.r0 ? sp.slot0 : 0;
      const size_t row0 = stream_piece_row(h, r, slot, 0, R, G);
      const CoherentRegion racc(a.ws_acc + row0 * D, G * D * 4);
      const CoherentRegion rml(a.ws_ml + row0 * 2, G * 2 * 4);
      uint32_t ml[2], w[EL];
      rml.loadu<2>(gq * 8, ml);
      if constexpr (EL == 1) {
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(racc.r, (gq * D + d0) * 4, 0, kSystemCoherent);
      } else {
        racc.loadu<EL>((gq * D + d0) * 4, w);
      }
      pm[u] = ws_decode(ml[0]);
      pl[u] = ws_decode(ml[1]);
#pragma unroll
      for (int k = 0; k < EL; ++k) pa[u][k] = ws_decode(w[k]);
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (p0 + u <= sp.r1) Mn = fmaxf(Mn, pm[u]);
    const float f0 = fast_exp2(M - Mn);
    L *= f0;
#pragma unroll
    for (int k = 0; k < EL; ++k) A[k] *= f0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (p0 + u <= sp.r1) {
        const float f = fast_exp2(pm[u] - Mn);
        L += pl[u] * f;
#pragma unroll
        for (int k = 0; k < EL; ++k) A[k] += pa[u][k] * f;
      }
    }
    M = Mn;
    // The batch's words are used: zero them (the same lanes, the same
    // words), with ordinary stores, as stream_merge_last does.
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (p0 + u <= sp.r1) {
        const int r = p0 + u;
        const int slot = r == sp.r0 ? sp.slot0 : 0;
        const size_t row0 = stream_piece_row(h, r, slot, 0, R, G);
        uint32_t* wacc = reinterpret_cast<uint32_t*>(a.ws_acc + row0 * D) + gq * D + d0;
        uint32_t* wml = reinterpret_cast<uint32_t*>(a.ws_ml + row0 * 2) + gq * 2;
        zero_words<2>(wml);
        zero_words<EL>(wacc);
      }
    }
  }
  float x[EL];
#pragma unroll
  for (int k = 0; k < EL; ++k) x[k] = A[k] / L;
  store_row_part<EL>(DT{}, a.out, ((size_t)b * a.num_q_heads + (size_t)h * G + gq) * D + d0, x);
}


// In-launch merge of a split (sequence, kv head) by the wave holding its
// last piece (worker sp.r1), once that wave has stored its own piece: the
// pieces of workers sp.r0 .. sp.r1 - 1 are waited for by loading their
// words until none is zero (the encoding has no zero word, so a zero word
// is a store still on its way).  Those workers belong to this workgroup or
// to earlier ones (worker index grows with the workgroup index), which the
// hardware dispatches before this one and which never wait on later ones,
// so every piece waited for is being computed or done: the same forward-
// progress argument as a decoupled look-back scan.  The wait is bounded all
// the same (kStreamMergeRetries round trips), so a broken invariant shows
// as a wrong row, never as a hang.  There is no arrival counter.
//
// Pieces are folded in worker order, KB per round trip, each lane taking EL
// consecutive elements of one query row; the words are then zeroed with
// ordinary stores (nothing in this launch reads them again, and the end of
// the launch writes them back before any later launch reads them).  One
// rolled loop with a single load site: this code runs once per merge, cold,
// at the end of the launch, where every extra kilobyte of instructions
// costs instruction fetches on the critical path.
template <class DT, int D, int G>
__device__ __forceinline__ void stream_merge_last(const DecodeArgs& a, int b, int h,
                                                  const SeqPieces& sp, int R, int lane) {
  constexpr int EL = G * D / 64;  // elements per lane (1 .. 16)
  static_assert(EL >= 1 && D % EL == 0, "a lane's elements lie in one row");
  constexpr int KB = EL <= 4 ? 8 : 4;  // pieces per round trip
  const int gq = lane * EL / D;
  const int d0 = lane * EL % D;
  float M = kNoMax, L = 0.0f, A[EL];
#pragma unroll
  for (int k = 0; k < EL; ++k) A[k] = 0.0f;
  uint32_t wm[KB], wl[KB], wa[KB][EL];
  int p0 = sp.r0, tries = 0;
#pragma unroll 1
  while (p0 <= sp.r1) {
    // Pieces p0 .. p0 + KB - 1; slots past r1 get a resource of zero bytes
    // (their loads read nothing and return zeros).
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int r = min(p0 + u, sp.r1);
      const uint32_t live = p0 + u <= sp.r1 ? 1u : 0u;
      const size_t row0 = stream_piece_row(h, r, r == sp.r0 ? sp.slot0 : 0, 0, R, G);
      const CoherentRegion racc(a.ws_acc + row0 * D, live * (G * D * 4));
      const CoherentRegion rml(a.ws_ml + row0 * 2, live * (G * 2 * 4));
      uint32_t ml[2];
      rml.loadu<2>(gq * 8, ml);
      wm[u] = ml[0];
      wl[u] = ml[1];
      if constexpr (EL == 1) {
        wa[u][0] = __builtin_amdgcn_raw_buffer_load_b32(racc.r, (gq * D + d0) * 4, 0,
                                                        kSystemCoherent);
      } else {
        racc.loadu<EL>((gq * D + d0) * 4, wa[u]);
      }
    }
    bool miss = false;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (p0 + u > sp.r1) continue;
      miss = miss || wm[u] == 0u || wl[u] == 0u;
#pragma unroll
      for (int k = 0; k < EL; ++k) miss = miss || wa[u][k] == 0u;
    }
    if (__ballot(miss) != 0 && tries < kStreamMergeRetries) {
      ++tries;  // a piece is still being computed or stored: load again
      __builtin_amdgcn_s_sleep(2);
      continue;
    }
    tries = 0;
    float Mn = M;
#pragma unroll
    for (int u = 0; u < KB; ++u)
      if (p0 + u <= sp.r1) Mn = fmaxf(Mn, ws_decode(wm[u]));
    const float f0 = fast_exp2(M - Mn);
    L *= f0;
#pragma unroll
    for (int k = 0; k < EL; ++k) A[k] *= f0;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (p0 + u <= sp.r1) {
        const float f = fast_exp2(ws_decode(wm[u]) - Mn);
        L += ws_decode(wl[u]) * f;
#pragma unroll
        for (int k = 0; k < EL; ++k) A[k] += ws_decode(wa[u][k]) * f;
      }
    }
    M = Mn;
    const bool done = p0 + KB > sp.r1;
    if (done) {
      float x[EL];
#pragma unroll
      for (int k = 0; k < EL; ++k) x[k] = A[k] / L;
      store_row_part<EL>(DT{}, a.out, ((size_t)b * a.num_q_heads + (size_t)h * G + gq) * D + d0,
                         x);
    }
    // The batch's words are used: zero them (the lanes that read them).
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (p0 + u <= sp.r1) {
        const int r = p0 + u;
        const size_t row0 = stream_piece_row(h, r, r == sp.r0 ? sp.slot0 : 0, 0, R, G);
        uint32_t* wacc = reinterpret_cast<uint32_t*>(a.ws_acc + row0 * D) + gq * D + d0;
        uint32_t* wml = reinterpret_cast<uint32_t*>(a.ws_ml + row0 * 2) + gq * 2;
        zero_words<2>(wml);
        zero_words<EL>(wacc);
      }
    }
    p0 += KB;
  }
}

}  // namespace pa
