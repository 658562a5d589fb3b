// The balanced ("stream") decode schedule: the batch's K/V blocks, sequence
// after sequence, form one list per kv head, and each kv head's list is cut
// into R equal ranges of consecutive blocks, one per worker wave.  A worker
// streams its range, finishing a sequence's state whenever the sequence ends
// inside it; a sequence whose blocks fall in several ranges leaves one
// partial state per range, and the last of those workers to finish merges
// them (log-sum-exp merge, the last-block pattern of the LLAISYS README,
// CUDA argmax item).
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
// rows of its G query heads, by one wave.  Pieces are folded in worker
// order, so the result does not depend on the order in which they were
// written; up to kBatch pieces are requested in one round trip.  Each lane
// takes EL consecutive elements of one query row.
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
      float ml[2];
      rml.load<2>(gq * 8, ml);
      pm[u] = ml[0];
      pl[u] = ml[1];
      racc.load<EL>((gq * D + d0) * 4, pa[u]);
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
  }
  float x[EL];
#pragma unroll
  for (int k = 0; k < EL; ++k) x[k] = A[k] / L;
  store_row_part<EL>(DT{}, a.out, ((size_t)b * a.num_q_heads + (size_t)h * G + gq) * D + d0, x);
}

// Arrival of a worker's piece of (b, h), after its partial state has been
// published: returns true (in every lane) when this worker is the last of
// the sequence's `pieces` workers to arrive, and then leaves the counter at
// zero for the next call.  The caller has waited for its published stores.
__device__ __forceinline__ int stream_arrive_issue(int32_t* counter, int lane) {
  int prev = 0;
  if (lane == 0)
    prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  return prev;
}

}  // namespace pa
