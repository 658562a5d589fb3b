// Paged prefill (and chunked-prefill) attention, bfloat16, causal, on the
// matrix cores.
//
// The step before decode on the pages' data flow: a prompt, or a chunk of it
// after a cached prefix, is processed at once, each new token attending to
// every cached position up to its own (MinivLLM article, "Engine Layout":
// flash attention while prefilling, paged attention while decoding;
// nano-vllm overview, "Prefill vs. Decode").  Here both read the same paged
// cache: the new tokens' K/V rows are written first (pa_reshape_and_cache),
// then this kernel runs.
//
// Query rows are (token, head) pairs: row r of sequence b is new token r / G,
// query head g * G + r % G of kv head g.  A workgroup takes 8 waves x 32 rows
// (a row group) of one (sequence, kv head).  Row groups differ in cost -- the
// keys they fold, up to their last row's position -- so the workgroups take
// them longest first (pick_unit: the grid is ranked, not laid out by
// sequence; a hardware dispatcher that hands workgroups out in order would
// otherwise leave compute units idle behind long ones).  Per K/V block (the
// blocks up to the workgroup's last row position):
//   * the whole workgroup loads 64 keys' worth of blocks (K and V rows for kv
//     head g) with full-row coalesced 16-byte loads into one of two LDS stages
//     (the next stage's loads are in flight while the current one is used);
//   * every wave folds the block into its rows' online-softmax state
//     (mfma_attn.hpp), each score masked past its row's position; a wave
//     whose rows all end before the block skips it.
// There is no split over key ranges, so no workspace and no merge: each
// wave's state ends complete and is normalised and stored directly.
#include "mfma_tile32.hpp"
#include "options.hpp"

#include "decode_launch.hpp"

#include <stdlib.h>

#include <algorithm>

namespace pa {

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t row_groups;    // row groups of the longest sequence (grid: num_seqs x this)
  int32_t bucket_width;  // keys per cost bucket of the longest-first order
  int32_t num_buckets;   // cost buckets, at most kMaxCostBuckets
  float scale_log2;
};

constexpr int kMaxCostBuckets = 1024;

// The row group a workgroup takes.  Units are (sequence b, row group rg); a
// unit folds first_b + min(n_b, (rg + 1) T) keys (first_b = cached positions
// before the new tokens, n_b new tokens, T tokens per row group).  Units are
// ranked by that cost in buckets of bucket_width keys, highest first, then by
// b ascending and rg descending; workgroup `u` (of each kv head) takes the
// unit of rank u.  Every workgroup of the launch computes the same ranking
// from the lengths: a histogram of unit costs, its suffix sums, then the
// unit within the bucket by a scan over the sequences.  Returns false (in
// every thread) when u is past the last unit.
template <int G, int RPW, int NT>
__device__ __forceinline__ bool pick_unit(const PrefillArgs& a, int max_tokens, int u,
                                          int& b_out, int& rg_out) {
  constexpr int T = RPW / G;  // tokens per row group
  __shared__ int s_hist[kMaxCostBuckets];
  __shared__ int s_cum[kMaxCostBuckets];
  __shared__ int s_wsum[NT / 64];
  __shared__ int s_pick[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.num_seqs, W = a.bucket_width, NBK = a.num_buckets;
  auto seq = [&](int bb, int& first, int& n) {
    const int q0 = a.query_start[bb];
    n = a.query_start[bb + 1] - q0;
    const int c = a.context_lens[bb];
    const bool ok = n >= 0 && n <= c && c <= max_tokens;
    first = ok ? c - n : 0;
    n = n < 0 ? 0 : n;
  };
  auto groups = [&](int n) { return (int)(((int64_t)n * G + RPW - 1) / RPW); };
  auto bucket = [&](int first, int n, int rg) {
    const int cost = first + min(n, (rg + 1) * T);
    return min(max((cost - 1) / W, 0), NBK - 1);
  };
  // Wave-wide inclusive prefix sum.
  auto wave_scan = [&](int v) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(v, d);
      v += lane >= d ? o : 0;
    }
    return v;
  };

  for (int k = tid; k < NBK; k += NT) s_hist[k] = 0;
  __syncthreads();
  for (int bb = tid; bb < B; bb += NT) {
    int first, n;
    seq(bb, first, n);
    const int ng = groups(n);
    for (int rg = 0; rg < ng; ++rg) atomicAdd(&s_hist[bucket(first, n, rg)], 1);
  }
  __syncthreads();
  if (wave == 0) {  // s_cum[k] = units in buckets above k; lane 0 takes the top ones
    const int per = (NBK + 63) / 64;
    const int top = NBK - 1 - lane * per;
    int sum = 0;
    for (int i = 0; i < per; ++i)
      if (top - i >= 0) sum += s_hist[top - i];
    const int incl = wave_scan(sum);
    int run = incl - sum;
    for (int i = 0; i < per; ++i)
      if (top - i >= 0) {
        s_cum[top - i] = run;
        run += s_hist[top - i];
      }
    if (lane == 63) s_pick[2] = incl;  // all units
  }
  __syncthreads();
  if (u >= s_pick[2]) return false;
  for (int k = tid; k < NBK; k += NT)
    if (s_hist[k] > 0 && s_cum[k] <= u && u < s_cum[k] + s_hist[k]) {
      s_pick[0] = k;
      s_pick[1] = u - s_cum[k];
    }
  __syncthreads();
  const int kstar = s_pick[0], r = s_pick[1];
  // Units in bucket kstar, sequences in order: each thread takes a range of
  // sequences, counts theirs, and a scan over the threads finds the one.
  const int per_b = (B + NT - 1) / NT;
  const int b_lo = min(B, tid * per_b), b_hi = min(B, b_lo + per_b);
  auto count_in = [&](int bb) {
    int first, n;
    seq(bb, first, n);
    int c = 0;
    for (int rg = groups(n) - 1; rg >= 0; --rg) c += bucket(first, n, rg) == kstar;
    return c;
  };
  int cnt = 0;
  for (int bb = b_lo; bb < b_hi; ++bb) cnt += count_in(bb);
  const int incl = wave_scan(cnt);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int pre = incl - cnt;
  for (int w = 0; w < wave; ++w) pre += s_wsum[w];
  if (r >= pre && r < pre + cnt) {
    for (int bb = b_lo; bb < b_hi; ++bb) {
      int first, n;
      seq(bb, first, n);
      for (int rg = groups(n) - 1; rg >= 0; --rg)
        if (bucket(first, n, rg) == kstar) {
          if (pre == r) {
            s_pick[0] = bb;
            s_pick[1] = rg;
          }
          ++pre;
        }
    }
  }
  __syncthreads();
  b_out = s_pick[0];
  rg_out = s_pick[1];
  return true;
}

#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8
#endif
#ifndef PA_PREFILL_STAGE_KEYS
#define PA_PREFILL_STAGE_KEYS 64
#endif
#ifndef PA_PREFILL_FOLD_KEYS
#define PA_PREFILL_FOLD_KEYS 64
#endif
constexpr int kPrefillWaves = PA_PREFILL_WAVES;
constexpr int kPrefillRows = 32;  // query rows per wave
// Keys per LDS stage (several blocks): 64, or 32 at head_dim 64, where the
// workgroup is held to 128 VGPRs so that two fit on a compute unit.
template <int D>
constexpr int prefill_stage_keys() { return D == 64 ? 32 : PA_PREFILL_STAGE_KEYS; }

// KS = 1: each wave folds every key of the workgroup's range into its 32
// rows.  KS = 2: the waves form NW / 2 row sets x 2 key halves -- wave w and
// wave w + NW/2 hold the same rows and fold alternate 32-key folds (the two
// of a 64-key stage, or alternate 32-key stages) -- and combine their states
// through LDS at the end.  That halves a
// workgroup's serial key loop (and doubles the workgroups) for batches with
// few new rows against long contexts (chunks after a cached prefix).
template <int D, int BS, int G, int NW, int KS>
__global__ __launch_bounds__(NW * 64, D == 64 ? 4 : 2) void prefill_mfma_kernel(PrefillArgs a) {
  static_assert(KS == 1 || KS == 2, "one or two key halves");
  constexpr int NR = kPrefillRows;
  constexpr int RW = NW / KS;  // row sets (waves with distinct rows)
  // Keys folded per call: a whole stage (two or four 16-token tiles, so p.v
  // runs on v_mfma_f32_16x16x32_bf16 whatever the block size); one running
  // maximum update and one branch per call.
  constexpr int SKEYS = prefill_stage_keys<D>();
  constexpr int KC = KS == 2 ? 32
                     : PA_PREFILL_FOLD_KEYS < SKEYS ? PA_PREFILL_FOLD_KEYS : SKEYS;
  using T = RowTile32Attn<D>;
  static_assert(NR == 32 && KC % T::KC == 0, "a wave holds one 32-row tile");
  constexpr int RL = D * 2 / 16;  // lanes per token row in a 16-byte global load
  constexpr int KPITCH = T::Sh::KPITCH, VPITCH = T::Sh::VPITCH;
  constexpr int NT = NW * 64;
  constexpr int kChunks = BS * RL;  // 16-byte chunks of one block's rows, K or V
  static_assert(kChunks % 64 == 0, "a wave's chunks are all K or all V");
  constexpr int NCH = (2 * kChunks + NT - 1) / NT;  // chunks per thread per block, K and V
  constexpr int KB = SKEYS / BS;              // blocks per stage
  constexpr int SK = SKEYS * KPITCH;          // one stage's K rows
  constexpr int SV = SKEYS * VPITCH;          // one stage's V rows
  // [stage][K rows | V rows]: the stage's KB blocks are consecutive logical
  // blocks, so row t of a stage is key position (first block) * BS + t.
  // With key halves the same bytes afterwards hold the halves' exchange.
  constexpr int NV = 2 + T::DT * 16;  // floats per lane of a wave's state
  constexpr int kStages = 2 * (SK + SV);
  constexpr int kExchange = KS == 2 ? RW * NV * 64 * 4 : 0;
  __shared__ __attribute__((aligned(16))) char s_raw[kStages > kExchange ? kStages : kExchange];
  char (*s_kv)[SK + SV] = reinterpret_cast<char (*)[SK + SV]>(s_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = wave % RW;  // row set
  const int kh = wave / RW;  // key half (always 0 with KS = 1)
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  // Workgroup L takes kv head L % Hkv (so, with Hkv a multiple of the eight
  // XCDs that workgroups are dealt to in turn, a head's K/V stays in one
  // XCD's L2) of the unit ranked L / Hkv.
  const int L = blockIdx.y * gridDim.x + blockIdx.x;
  const int g = L % Hkv;
  int b, rg;
  if (!pick_unit<G, RW * NR, NT>(a, a.max_blocks * BS, L / Hkv, b, rg)) return;
  const int qs = a.query_start[b];
  const int nq = a.query_start[b + 1] - qs;
  const int ctx = a.context_lens[b];
  const int nrows = nq * G;
  const int r0 = rg * RW * NR;
  if (r0 >= nrows) return;
  const int r_end = min(nrows, r0 + RW * NR);
  uint16_t* out = static_cast<uint16_t*>(a.out);
  auto out_at = [&](int r, int d) -> size_t {
    return ((size_t)(qs + r / G) * Hq + (size_t)g * G + r % G) * D + d;
  };
  if (nq > ctx || ctx > a.max_blocks * BS) {  // no such positions: NaN rows
    for (int e = tid; e < (r_end - r0) * D; e += NT)
      out[out_at(r0 + e / D, e % D)] = 0x7FC0;
    return;
  }
  const int first = ctx - nq;  // position of new token 0
  const int nblk = (first + (r_end - 1) / G + 1 + BS - 1) / BS;

  const int wr0 = r0 + rw * NR;  // this wave's first row
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  T st;
  const QScale qsc(a.scale_log2);
  st.reset();
  st.load_q(
      [&](int r) -> const uint16_t* {
        const int R = wr0 + r;
        return R < nrows ? q + ((size_t)(qs + R / G) * Hq + (size_t)g * G + R % G) * D
                         : nullptr;
      },
      qsc, lane);
  const int rowpos = wr0 + (lane & 31) < nrows ? first + (wr0 + (lane & 31)) / G : -1;
  // Keys this wave's rows reach (0 if it has no rows); chunks ending at or
  // before its first row's position need no causal mask.
  const int wave_kend = wr0 < nrows ? first + (min(nrows, wr0 + NR) - 1) / G + 1 : 0;
  const int wave_pos0 = first + wr0 / G;

  // Block loads: chunk c < 2 * kChunks is K chunk c or V chunk c - kChunks;
  // chunk cc of a block is token cc / RL, 16 bytes at d = 8 (cc % RL).  Every
  // thread takes chunks tid + i * NT wrapped into range (when a block has
  // fewer chunks than threads, some threads load and store a duplicate of
  // another's chunk -- same bytes, same LDS address), so the loads and stores
  // have no branch and the compiler keeps the loads in flight.
  const uint32_t tok_bytes = (uint32_t)Hkv * D * 2;
  const uint32_t blk_bytes = tok_bytes * BS;
  const uint32_t head_off = (uint32_t)g * D * 2;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  // The table row is read through the constant address space: scalar loads,
  // counted apart from the vector loads, so fetching a stage's entries never
  // waits for the K/V loads still in flight (vector loads complete in order).
  const __attribute__((address_space(4))) int32_t* trow =
      (const __attribute__((address_space(4))) int32_t*)(a.block_tables +
                                                          (size_t)b * a.max_blocks);
  bool bad = false;  // a block id outside the pool: rows become NaN
  uint4 r[2][KB][NCH];  // two stages of K/V rows in flight
  auto chunk = [&](int i) { return (tid + i * NT) % (2 * kChunks); };
  // Loads of blocks jb0 .. jb0 + KB - 1 into register set rs (ids past the
  // last block read the last one again: in range, never folded in).
  auto fetch = [&](uint4 (&rr)[KB][NCH], int jb0) {
    int ids[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) ids[kb] = trow[jb0 + kb < nblk ? jb0 + kb : nblk - 1];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int jb = jb0 + kb < nblk ? jb0 + kb : nblk - 1;
      int id = __builtin_amdgcn_readfirstlane(ids[kb]);
      const bool ok = id >= 0 && id < a.num_blocks;
      bad = bad || !ok;
      id = ok ? id : 0;
      const size_t boff = (size_t)id * blk_bytes;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(kbase + boff), 0, blk_bytes, kBufferRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(vbase + boff), 0, blk_bytes, kBufferRsrcWord3);
      const int pos0 = jb * BS;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = chunk(i);
        // A wave's 64 chunks are all K or all V (kChunks is a multiple of 64).
        const bool is_k = __builtin_amdgcn_readfirstlane(c) < kChunks;
        const int cc = is_k ? c : c - kChunks;
        const int tok = cc / RL;
        // Tokens at or past the context read the block's token 0 (finite).
        const uint32_t off = head_off + 16u * (cc % RL) +
                             (pos0 + tok < ctx ? (uint32_t)tok * tok_bytes : 0u);
        rr[kb][i] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(is_k ? rk : rv, off, 0, 0));
      }
    }
  };
  auto stage = [&](const uint4 (&rr)[KB][NCH], int s) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = chunk(i);
        const bool is_k = __builtin_amdgcn_readfirstlane(c) < kChunks;
        const int cc = is_k ? c : c - kChunks;
        *reinterpret_cast<uint4*>(s_kv[s] + (is_k ? (kb * BS + cc / RL) * KPITCH
                                                  : SK + (kb * BS + cc / RL) * VPITCH) +
                                  (cc % RL) * 16) = rr[kb][i];
      }
  };
  // Fold LDS stage s (blocks jb0 ..) into the rows: 32 keys at a time; keys
  // past the last block (stage rows loaded from the last block again) sit
  // past every row's position and are masked.
  auto fold = [&](int s, int jb0) {
#pragma unroll
    for (int kc = 0; kc < SKEYS / KC; ++kc) {
      const int p0 = jb0 * BS + kc * KC;
      if ((p0 / T::KC) % KS == kh && p0 < nblk * BS && p0 < wave_kend) {
#pragma unroll
        for (int t = 0; t < KC / T::KC; ++t) {
          const int pt = p0 + t * T::KC;
          st.consume(s_kv[s] + (kc * KC + t * T::KC) * KPITCH,
                     s_kv[s] + SK + (kc * KC + t * T::KC) * VPITCH, pt, rowpos,
                     pt + T::KC - 1 > wave_pos0, qsc.c, lane);
        }
      }
    }
  };
  auto clampb = [&](int jb) { return jb < nblk ? jb : nblk - 1; };

  fetch(r[0], 0);
  stage(r[0], 0);
  __builtin_amdgcn_s_waitcnt(0);  // q rows and the first blocks are in: nothing pending
  __syncthreads();
  {
    // Two stages of loads in flight: while LDS stage s is folded in, the
    // registers hold the next stage (staged to LDS after the fold) and the
    // one after it is being loaded.  Unrolled by two so that each register
    // set has fixed names.
    fetch(r[1], clampb(KB));
    for (int jb0 = 0; jb0 < nblk; jb0 += 2 * KB) {
      fetch(r[0], clampb(jb0 + 2 * KB));
      __builtin_amdgcn_sched_barrier(0);
      fold(0, jb0);
      stage(r[1], 1);
      __syncthreads();
      if (jb0 + KB >= nblk) break;
      fetch(r[1], clampb(jb0 + 3 * KB));
      __builtin_amdgcn_sched_barrier(0);
      fold(1, jb0 + KB);
      stage(r[0], 0);
      __syncthreads();
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load left in flight past the loop

  if (bad) {
    if (kh == 0)
      for (int e = lane; e < NR * D; e += 64) {
        const int R = wr0 + e / D;
        if (R < nrows) out[out_at(R, e % D)] = 0x7FC0;
      }
    return;
  }
  if constexpr (KS == 2) {
    // The key-half-1 wave of each row set hands its state (max, sum, output
    // registers) to the key-half-0 wave through LDS, lane for lane: both hold
    // the same rows in the same register layout.
    float* s_x = reinterpret_cast<float*>(s_raw) + rw * NV * 64;
    __syncthreads();  // every wave is done with the stages
    if (kh == 1) {
      s_x[lane] = st.m;
      s_x[64 + lane] = st.l;
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s_x[(2 + dt * 16 + r) * 64 + lane] = st.o[dt][r];
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = s_x[lane], l1 = s_x[64 + lane];
    const float M = fmaxf(st.m, m1);
    const float a0 = fast_exp2(st.m - M), a1 = fast_exp2(m1 - M);  // this lane's row
    st.l = st.l * a0 + l1 * a1;
    st.m = M;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float f0 = T::from_row(a0, lane, r), f1 = T::from_row(a1, lane, r);
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
        st.o[dt][r] = st.o[dt][r] * f0 + s_x[(2 + dt * 16 + r) * 64 + lane] * f1;
    }
  }
  st.store_rows(
      [&](int row, int d, float v) {
        const int R = wr0 + row;
        if (R < nrows) out[out_at(R, d)] = f32_to_bf16_rne(v);
      },
      lane);
}

namespace {

template <int D, int BS, int G>
hipError_t launch_prefill_t(const PrefillArgs& a, int num_seqs, int ks, hipStream_t stream) {
  dim3 grid(num_seqs * a.num_kv_heads, a.row_groups);
  if (ks == 2)
    prefill_mfma_kernel<D, BS, G, kPrefillWaves, 2><<<grid, kPrefillWaves * 64, 0, stream>>>(a);
  else
    prefill_mfma_kernel<D, BS, G, kPrefillWaves, 1><<<grid, kPrefillWaves * 64, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefill(int D, int BS, int G, const PrefillArgs& a, int num_seqs, int ks,
                          hipStream_t s) {
  auto by_g = [&](auto d, auto bs) -> hipError_t {
    constexpr int Dv = decltype(d)::value, BSv = decltype(bs)::value;
    switch (G) {
      case 1: return launch_prefill_t<Dv, BSv, 1>(a, num_seqs, ks, s);
      case 2: return launch_prefill_t<Dv, BSv, 2>(a, num_seqs, ks, s);
      case 4: return launch_prefill_t<Dv, BSv, 4>(a, num_seqs, ks, s);
      case 8: return launch_prefill_t<Dv, BSv, 8>(a, num_seqs, ks, s);
      case 16: return launch_prefill_t<Dv, BSv, 16>(a, num_seqs, ks, s);
      case 32: return launch_prefill_t<Dv, BSv, 32>(a, num_seqs, ks, s);
    }
    return hipErrorInvalidValue;
  };
  auto by_bs = [&](auto d) -> hipError_t {
    return BS == 16 ? by_g(d, IntC<16>{}) : by_g(d, IntC<32>{});
  };
  return D == 64 ? by_bs(IntC<64>{}) : by_bs(IntC<128>{});
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" pa_status pa_paged_attention_prefill(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
    int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t max_query_len, float scale, pa_dtype dtype, void* stream) {
  clear_error();
  if (dtype != PA_DTYPE_BF16) {
    if (!supported_dtype(dtype)) {
      set_error("dtype %d is not PA_DTYPE_F32 or PA_DTYPE_BF16", (int)dtype);
      return PA_ERR_INVALID_ARGUMENT;
    }
    set_error("prefill is built for bfloat16 only");
    return PA_ERR_UNSUPPORTED;
  }
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      num_q_heads % num_kv_heads) {
    set_error("invalid sizes: num_seqs=%d num_tokens=%d max_query_len=%d Hq=%d Hkv=%d "
              "num_blocks=%d max_blocks=%d", num_seqs, num_tokens, max_query_len,
              num_q_heads, num_kv_heads, num_blocks, max_blocks_per_seq);
    return PA_ERR_INVALID_ARGUMENT;
  }
  const int G = num_q_heads / num_kv_heads;
  if (!(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32)) {
    set_error("query heads per kv head = %d; built for 1, 2, 4, 8, 16, 32", G);
    return PA_ERR_UNSUPPORTED;
  }
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) {
    set_error("head_dim=%d block_size=%d; built for {64, 128} x {16, 32}", head_dim,
              block_size);
    return PA_ERR_UNSUPPORTED;
  }
  // Key halves per workgroup (see prefill_mfma_kernel): two when the block
  // table spans at least four times the longest query, i.e. few new rows
  // against long contexts.  PAGEDATTN_PREFILL_KSPLIT=1|2 forces either.
  int ks = (int64_t)max_blocks_per_seq * block_size >= 4 * (int64_t)max_query_len ? 2 : 1;
  if (options().prefill_ksplit) ks = options().prefill_ksplit;
  const int64_t rows_per_wg = (int64_t)kPrefillWaves * kPrefillRows / ks;
  const int64_t row_groups = ((int64_t)max_query_len * G + rows_per_wg - 1) / rows_per_wg;
  // Workgroups are numbered blockIdx.y * gridDim.x + blockIdx.x in 32 bits.
  if (row_groups > 65535 || (int64_t)num_seqs * num_kv_heads * row_groups > 0x7FFFFFFF) {
    set_error("num_seqs=%d x num_kv_heads=%d x %lld row groups (max_query_len=%d) is too "
              "large for one launch", num_seqs, num_kv_heads, (long long)row_groups,
              max_query_len);
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start) {
    set_error("a tensor pointer is NULL");
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) {
    set_error("out, q, k_cache and v_cache must be 16-byte aligned");
    return PA_ERR_INVALID_ARGUMENT;
  }
  PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.row_groups = (int32_t)row_groups;
  {
    // Cost buckets of the longest-first order: T = tokens per row group keys
    // each, widened so that the longest possible context fits the table.
    const int64_t T = std::max<int64_t>(1, rows_per_wg / G);
    const int64_t max_tokens = (int64_t)max_blocks_per_seq * block_size;
    const int64_t nb = (max_tokens + T - 1) / T;
    const int64_t widen = (nb + kMaxCostBuckets - 1) / kMaxCostBuckets;
    a.bucket_width = (int32_t)(T * std::max<int64_t>(1, widen));
    a.num_buckets = (int32_t)std::min<int64_t>(
        kMaxCostBuckets, (max_tokens + a.bucket_width - 1) / a.bucket_width + 1);
  }
  a.scale_log2 = scale * 1.4426950408889634f;
  const hipError_t err = launch_prefill(head_dim, block_size, G, a, num_seqs, ks,
                                        static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    set_error("prefill launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  return PA_OK;
}
