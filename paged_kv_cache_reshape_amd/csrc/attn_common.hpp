// Pieces shared by the decode kernels: the lane layout of a KV row, the
// per-row online-softmax state, cross-XCD publishing of partial states, and
// the log-sum-exp merge of partial states.
//
// What is computed (barellm README, feature list and paged-cache list;
// LLAISYS README, self-attention item): for sequence b and query head h,
// softmax attention of q[b,h] over the first context_lens[b] cached rows of KV
// head h / G, the rows found through the block table; float32 accumulation;
// softmax in running max / running sum form (online softmax).
#pragma once

#include "common.hpp"

#include <math.h>

namespace pa {

// Everything a decode kernel receives.  Workspace regions are laid out by the
// host for the kernel that runs.
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_acc;      // unnormalised partial outputs
  float* ws_ml;       // (max, sum) of each partial state, base-2 units
  int32_t* counters;  // arrivals per merged unit, reset by the merger
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t part_blocks;   // partition kernel: blocks per partition
  int32_t max_parts;     // partition kernel: partitions per sequence, at most
  int32_t heads_per_wg;  // consecutive kv heads one workgroup takes (1, 2 or 4)
  int32_t deferred_merge;  // 1: partitions store their states and a second kernel merges
  int32_t stream_workers;  // stream schedule: worker waves per kv head (0: fixed partitions)
  float scale_log2;      // scale * log2(e): scores are kept in base-2 units
  // Decode step with the KV write fused in: this step's token of sequence b
  // ([num_seqs, num_kv_heads, D] rows), attended as position ctx - 1 and
  // written to that cache slot.  nullptr: the caches are only read.
  const void* new_k;
  const void* new_v;
};

// Lane layout.  One KV row (one token, one kv head) is D*elt contiguous bytes
// spread over RL lanes of 16 bytes; a wave load covers ROWS rows; a block of
// BS tokens takes NI loads for K and NI for V.  A wave serves GW query heads
// of one kv head; groups larger than 8 are split over HS waves.
template <class DT, int D, int BS, int G, int NW>
struct DecodeShape {
  static constexpr int E = DT::kPerChunk;
  static constexpr int RL = D / E;
  static constexpr int ROWS = 64 / RL;
  static constexpr int NI = BS / ROWS;
  static constexpr int GW = G < 8 ? G : 8;
  static constexpr int HS = G / GW;
  static_assert(RL >= 4 && RL <= 32, "row must span 4..32 lanes");
  static_assert(BS % ROWS == 0, "block must be whole wave loads");
  static_assert(NW % HS == 0, "waves must cover every head split");
};

// q.k over one 16-byte chunk, float32 accumulation (bf16 products are exact).
__device__ __forceinline__ float chunk_dot(BF16, uint4 q, uint4 k) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.x),
                                            __builtin_bit_cast(bf16x2, k.x), 0.0f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.y),
                                      __builtin_bit_cast(bf16x2, k.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.z),
                                      __builtin_bit_cast(bf16x2, k.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.w),
                                      __builtin_bit_cast(bf16x2, k.w), s, false);
  return s;
}
__device__ __forceinline__ float chunk_dot(F32, uint4 q, uint4 k) {
  float s = __uint_as_float(q.x) * __uint_as_float(k.x);
  s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
  s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
  s = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
  return s;
}

__device__ __forceinline__ void unpack(BF16, uint4 v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
__device__ __forceinline__ void unpack(F32, uint4 v, float* f) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

__device__ __forceinline__ void store_out(BF16, void* base, size_t i, float x) {
  static_cast<uint16_t*>(base)[i] = f32_to_bf16_rne(x);
}
__device__ __forceinline__ void store_out(F32, void* base, size_t i, float x) {
  static_cast<float*>(base)[i] = x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Partial states cross XCDs, and MI355X's per-XCD L2s are not coherent with
// each other.  A device-scope fence would write back and invalidate the whole
// L2 of the XCD; instead partial states are stored and loaded with
// system-scope atomic accesses, which go around the L2s.
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float collect(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
}

// The same system-coherent policy (sc0 sc1, what a system-scope atomic
// store or load carries on gfx950) for whole 16- or 8-byte pieces of 32-bit
// words (the balanced schedule's encoded partial states), through a buffer
// resource over a wave-uniform base: partial states move in a few wide
// accesses instead of one 4-byte transaction per value.
constexpr int kBufferWord3 = 0x00020000;  // gfx9 raw buffer, 32-bit data format
constexpr int kSystemCoherent = 17;       // cache-policy operand: sc0 | sc1
constexpr int kLoadNT = 2;                // cache-policy operand of data read once: nt
struct CoherentRegion {
  __amdgpu_buffer_rsrc_t r;
  // base must be the same in every lane; accesses are range-checked against
  // `bytes` (an access past it reads 0 and writes nothing).
  __device__ __forceinline__ CoherentRegion(float* base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, kBufferWord3)) {}
  // Raw 32-bit words (encoded partial states of the balanced schedule).
  __device__ __forceinline__ void store4u(uint32_t off, const uint32_t* w) const {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const u4 v = {w[0], w[1], w[2], w[3]};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kSystemCoherent);
  }
  __device__ __forceinline__ void store2u(uint32_t off, uint32_t a, uint32_t b) const {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 v = {a, b};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kSystemCoherent);
  }
  // N consecutive words (N in {2, 4, 8, 16}) at byte offset off.
  template <int N>
  __device__ __forceinline__ void loadu(uint32_t off, uint32_t* w) const {
    if constexpr (N == 2) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kSystemCoherent);
      w[0] = v[0];
      w[1] = v[1];
    } else {
      static_assert(N % 4 == 0, "whole 16-byte pieces");
#pragma unroll
      for (int k = 0; k < N / 4; ++k) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * k, 0, kSystemCoherent);
#pragma unroll
        for (int t = 0; t < 4; ++t) w[4 * k + t] = v[t];
      }
    }
  }
};

// Running-state sentinel: finite, so exp2(sentinel - sentinel) = 1 for rows
// that have seen no token yet (their sum and output are still zero).
constexpr float kNoMax = -1.0e30f;

// Online-softmax state of one wave for GW query heads of one kv head.  Each
// row of the wave (RL lanes) keeps its own (max, sum, output slice) over the
// tokens it saw; rows are merged once at the end with lane swaps.
template <class DT, int D, int BS, int G, int NW>
struct RowAttn {
  using Sh = DecodeShape<DT, D, BS, G, NW>;
  using S = typename DT::storage;
  static constexpr int E = Sh::E, RL = Sh::RL, ROWS = Sh::ROWS, NI = Sh::NI;
  static constexpr int GW = Sh::GW;

  float m[GW], l[GW], acc[GW][E];
  uint4 qv[GW];

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      m[h] = kNoMax;
      l[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;
    }
  }

  // q rows of GW consecutive query heads starting at `q_head0` (an element
  // pointer to q[b, h0, 0]); this lane's 16-byte slice of each.
  __device__ __forceinline__ void load_q(const S* q_head0, int col) {
#pragma unroll
    for (int h = 0; h < GW; ++h) qv[h] = load_chunk(q_head0 + (size_t)h * D + col * E);
  }

  // K and V rows of one block: kb / vb point at this lane's chunk of the
  // block's first row for this kv head; rows are tok_stride elements apart.
  // Streaming (non-temporal) loads: each row is read once.
  __device__ __forceinline__ static void fetch(const S* kb, const S* vb, size_t tok_stride,
                                               uint4 (&kr)[NI], uint4 (&vr)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = load_stream(kb + (size_t)i * ROWS * tok_stride);
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = load_stream(vb + (size_t)i * ROWS * tok_stride);
  }

  // Fold one block into the state.  pos0: sequence position of this lane's
  // row in load 0; rows at or past ctx, and every row when `live` is false,
  // are masked (score -inf, value bits 0,
  // so anything stored there -- NaN included -- has no effect).  The masking
  // is branch-free: a branch here would give the compiler paths with
  // different loads outstanding, and it would then wait for all of them.
  __device__ __forceinline__ void consume(int pos0, int ctx, bool live, float scale_log2,
                                          const uint4 (&kr)[NI], const uint4 (&vr)[NI]) {
    bool valid[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) valid[i] = live && pos0 + i * ROWS < ctx;
    float s[NI][GW];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int h = 0; h < GW; ++h) {
        const float x = group_sum<RL>(chunk_dot(DT{}, qv[h], kr[i])) * scale_log2;
        s[i][h] = valid[i] ? x : -INFINITY;
      }
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      float mx = m[h];
#pragma unroll
      for (int i = 0; i < NI; ++i) mx = fmaxf(mx, s[i][h]);
      const float alpha = fast_exp2(m[h] - mx);
      m[h] = mx;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint4 z = make_uint4(0, 0, 0, 0);
      const uint4 vb = valid[i] ? vr[i] : z;
      float vf[E];
      unpack(DT{}, vb, vf);
#pragma unroll
      for (int h = 0; h < GW; ++h) {
        const float p = fast_exp2(s[i][h] - m[h]);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }
  }

  template <int kMask>
  __device__ __forceinline__ void merge_step() {
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      const float mo = lane_xor<kMask>(m[h]);
      const float lo = lane_xor<kMask>(l[h]);
      const float M = fmaxf(m[h], mo);
      const float sa = fast_exp2(m[h] - M);
      const float sb = fast_exp2(mo - M);
      l[h] = l[h] * sa + lo * sb;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float ao = lane_xor<kMask>(acc[h][e]);
        acc[h][e] = acc[h][e] * sa + ao * sb;
      }
      m[h] = M;
    }
  }

  // Rows of the wave -> one state, held by the lanes of row 0 (and the others).
  __device__ __forceinline__ void merge_rows() {
    if constexpr (RL <= 8) merge_step<8>();
    if constexpr (RL <= 16) merge_step<16>();
    merge_step<32>();
  }

  // Row 0 writes the wave's state to LDS: acc[h][d], m[h], l[h].
  __device__ __forceinline__ void to_lds(float (*s_acc)[D], float* s_m, float* s_l,
                                         int lane) const {
    if (lane < RL) {
#pragma unroll
      for (int h = 0; h < GW; ++h) {
#pragma unroll
        for (int e = 0; e < E; ++e) s_acc[h][lane * E + e] = acc[h][e];
        if (lane == 0) {
          s_m[h] = m[h];
          s_l[h] = l[h];
        }
      }
    }
  }
};

// Blocks a wave keeps in flight while it consumes one.  Throughput follows
// the bytes outstanding per compute unit, and registers are the largest
// buffer a wave has (a block of K and V rows for one kv head is 32 VGPRs at
// head_dim 128 in bf16), so the pipeline is PF blocks deep.  Measured on
// MI355X (Qwen3-shaped batch): depth 2 beats 3, 4 and 5, whose extra
// registers cost more occupancy than the extra depth returns.
#ifndef PA_PREFETCH_DEPTH
#define PA_PREFETCH_DEPTH 2
#endif

// Walk blocks jj = first, first + step, ... < n with the next PF-1 blocks'
// loads in flight while the current one is consumed.  Written so that the
// compiler keeps that overlap: the loop body has no branch (a block index at
// or past n is fetched as block n-1, which is in bounds, with `live` false
// so that the fetch can read nothing, and consumed with every row masked),
// the ring of PF buffers is indexed with constants only
// (the loop is unrolled by PF), and a scheduling barrier keeps each prefetch
// issued ahead of the arithmetic that does not need it.
template <int NL, int PF = PA_PREFETCH_DEPTH, class Fetch, class Consume>
__device__ __forceinline__ void stream_blocks(int first, int step, int n, Fetch&& fetch,
                                              Consume&& consume) {
  if (first >= n) return;
  auto clamp = [&](int j) { return j < n ? j : n - 1; };
  uint4 kr[PF][NL], vr[PF][NL];
#pragma unroll
  for (int p = 0; p < PF - 1; ++p) {
    const int j = first + p * step;
    fetch(clamp(j), j < n, kr[p], vr[p]);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads of one block together
  }
  for (int jj = first; jj < n; jj += PF * step) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int jn = jj + (u + PF - 1) * step;
      fetch(clamp(jn), jn < n, kr[(u + PF - 1) % PF], vr[(u + PF - 1) % PF]);
      __builtin_amdgcn_sched_barrier(0);
      const int j = jj + u * step;
      consume(j, j < n, kr[u], vr[u]);
    }
  }
}

// Merge stored partial states (m, l, acc) of `gh` output rows into the
// output.  `row_of(p, r)` returns the row index (into ws_ml / 2 and ws_acc /
// D) of output row r in piece p, so the rows of several kv heads, which lie
// apart in the workspace, merge in one pass.  Pieces are read in index order
// through LDS in chunks of kChunk (s_pm / s_pl hold that many), so the result
// does not depend on the order in which they were written.  Used by one whole workgroup; `gh` rows of D values
// each, output at out + out_base (rows consecutive).
//
// The partial outputs are read with system-scope loads, which go to memory:
// every thread first issues the loads of U pieces for all its output
// elements, then folds them in, so that U * EPT (about kInFlight) loads are
// in flight per thread instead of one round trip per value.
template <class DT, int D, int GH, int NT, int kInFlight = 16, int kChunk = 64, class RowFn>
__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, int npieces, int gh,
                                             RowFn row_of, size_t out_base,
                                             float (*s_pm)[GH], float (*s_pl)[GH]) {
  constexpr int EPT = (GH * D + NT - 1) / NT;  // output elements per thread, at most
  constexpr int U = EPT >= kInFlight ? 1 : kInFlight / EPT;  // pieces loaded together
  const int tid = threadIdx.x;
  const int elems = gh * D;
  float rM[EPT], rL[EPT], rA[EPT];
  int qh[EPT], dd[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    rM[k] = kNoMax;
    rL[k] = 0.0f;
    rA[k] = 0.0f;
    const int e = min(tid + k * NT, elems - 1);  // threads past the end repeat the last
    qh[k] = e / D;
    dd[k] = e % D;
  }
  float v[U][EPT];
  // Partial outputs of pieces c0 + p0 .. c0 + p0 + U - 1 (clamped to the chunk).
  auto load_batch = [&](int c0, int p0, int n) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pc = c0 + min(p0 + u, n - 1);
#pragma unroll
      for (int k = 0; k < EPT; ++k) v[u][k] = collect(a.ws_acc + row_of(pc, qh[k]) * D + dd[k]);
    }
  };
  for (int c0 = 0; c0 < npieces; c0 += kChunk) {
    const int n = min(kChunk, npieces - c0);
    // The first batch of partial outputs is requested with the chunk's
    // (m, l) pairs: one memory round trip before anything can be folded.
    load_batch(c0, 0, n);
    for (int i = tid; i < n * gh; i += NT) {
      const int pp = i / gh, h = i % gh;
      const size_t r = row_of(c0 + pp, h);
      s_pm[pp][h] = collect(a.ws_ml + r * 2);
      s_pl[pp][h] = collect(a.ws_ml + r * 2 + 1);
    }
    __syncthreads();
    float M[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      M[k] = rM[k];
      for (int pp = 0; pp < n; ++pp) M[k] = fmaxf(M[k], s_pm[pp][qh[k]]);
      const float f0 = fast_exp2(rM[k] - M[k]);
      rL[k] *= f0;
      rA[k] *= f0;
      rM[k] = M[k];
    }
    for (int p0 = 0; p0 < n; p0 += U) {
      if (p0 > 0) load_batch(c0, p0, n);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (p0 + u < n) {
#pragma unroll
          for (int k = 0; k < EPT; ++k) {
            const float f = fast_exp2(s_pm[p0 + u][qh[k]] - M[k]);
            rL[k] += s_pl[p0 + u][qh[k]] * f;
            rA[k] += v[u][k] * f;
          }
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + k * NT;
    if (e < elems) store_out(DT{}, a.out, out_base + e, rA[k] / rL[k]);
  }
  // Leave the workspace zero, as the balanced schedule's merges expect it.
  // Every piece had landed before it was read (its workgroup waited for its
  // stores before counting itself in, or it was stored by an earlier
  // launch), so once every thread has used its loads (the barrier) any
  // thread may zero any of the rows: 16-byte ordinary stores over whole
  // rows (nothing in this launch reads them again, and the end of the
  // launch writes them back before any later launch reads them).
  __syncthreads();
  static_assert(D % 4 == 0, "rows of whole 16-byte words");
  constexpr int Q = D / 4;
  for (int i = tid; i < npieces * gh * Q; i += NT) {
    const int ri = i / Q;
    const size_t r = row_of(ri / gh, ri % gh);
    reinterpret_cast<uint4*>(a.ws_acc + r * D)[i % Q] = make_uint4(0, 0, 0, 0);
  }
  for (int i = tid; i < npieces * gh; i += NT) {
    const size_t r = row_of(i / gh, i % gh);
    *reinterpret_cast<uint2*>(a.ws_ml + r * 2) = make_uint2(0, 0);
  }
}

// Publish-and-count: every thread's publish() stores must be complete before
// the workgroup counts itself in; returns true in every thread of the
// workgroup that brought the counter to `expected` (the merger), which also
// finds the counter reset for the next call.
__device__ __forceinline__ bool arrive(int32_t* counter, int expected, int* s_flag) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_SYSTEM);
    *s_flag = (prev == expected - 1);
  }
  __syncthreads();
  return *s_flag != 0;
}

__device__ __forceinline__ void reset_counter(int32_t* counter) {
  if (threadIdx.x == 0)
    __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Where a partition workgroup stands: its sequence, kv-head group and
// partition, the sequence's context length, this lane's block-table entries
// (lane l holds the partition's blocks l and 64 + l), and how many blocks it
// streams.
struct PartitionWork {
  int b, gg, part, ctx, blk0, nparts, nblk_run;
  int ent[2];
  bool poisoned;
  // Physical id of the partition's block j (j wave-uniform, below 128).
  __device__ __forceinline__ int block(int j) const {
    return __builtin_amdgcn_readlane(j < 64 ? ent[0] : ent[1], j & 63);
  }
};

// Start of a partition workgroup (grid x = (kv-head group, sequence), y =
// partition).  The context length, the block-table entries and -- through
// `load_q` -- the query rows are requested together, before anything waits
// on them.  Returns false when the workgroup has nothing to stream: its
// partition starts past the context, or the context is empty (output zeros)
// or out of range (output NaN), which the partition-0 workgroup writes.
// Workgroups are dealt to the XCDs round-robin in linear-id order; with the
// partition index slowest every partition index is spread over all XCDs.
template <class DT, int D, int BS, int G, int NT, class LoadQ>
__device__ __forceinline__ bool partition_prologue(const DecodeArgs& a, int lane,
                                                   PartitionWork& w, LoadQ&& load_q) {
  const int hpw = a.heads_per_wg;
  const int n_groups = a.num_kv_heads / hpw;
  w.gg = blockIdx.x % n_groups;
  w.b = blockIdx.x / n_groups;
  w.part = blockIdx.y;
  w.ctx = a.context_lens[w.b];
  w.blk0 = w.part * a.part_blocks;
  const int32_t* trow = a.block_tables + (size_t)w.b * a.max_blocks + w.blk0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = 64 * h + lane;
    w.ent[h] = (e < a.part_blocks && w.blk0 + e < a.max_blocks) ? trow[e] : 0;
  }
  load_q(w.b, w.gg);

  const int part_tokens = a.part_blocks * BS;
  const bool bad_ctx = w.ctx < 0 || w.ctx > a.max_blocks * BS;
  w.nparts = (bad_ctx || w.ctx == 0) ? 1 : (w.ctx + part_tokens - 1) / part_tokens;
  if (w.part >= w.nparts) return false;
  if (bad_ctx || w.ctx == 0) {
    const int wg_elems = hpw * G * D;
    const size_t out_base = ((size_t)w.b * a.num_q_heads + (size_t)w.gg * hpw * G) * D;
    const float fill = bad_ctx ? __builtin_nanf("") : 0.0f;
    for (int e = threadIdx.x; e < wg_elems; e += NT) store_out(DT{}, a.out, out_base + e, fill);
    return false;
  }
  const int nblk_seq = (w.ctx + BS - 1) / BS;
  const int nblk = min(a.part_blocks, nblk_seq - w.blk0);
  bool bad_here = false;
#pragma unroll
  for (int h = 0; h < 2; ++h)
    bad_here = bad_here || (64 * h + lane < nblk && (w.ent[h] < 0 || w.ent[h] >= a.num_blocks));
  w.poisoned = __ballot(bad_here) != 0;  // same answer in every wave
  w.nblk_run = w.poisoned ? 0 : nblk;
  return true;
}

// Fused KV write of a decode step: the
// step's token rows go from new_k / new_v ([num_seqs, num_kv_heads, D]) to
// the cache slot the block table gives for position ctx - 1 -- the slot a
// separate write would take -- unless the context is empty or out of range
// or that block lies outside the pool.  The copy is done by extra
// workgroups after the attention workgroups (of the last partition row on
// the fixed schedule), the last ones dispatched: stores issued by the
// attention workgroups themselves, interleaved with the stream, cost far
// more than their bytes (on the 256-sequence MHA batch, 12 us for 4 MiB).
// The wave that attends the token takes the new rows from new_k / new_v in
// registers, so it never needs the stored copy, and a value it reads in
// that slot meanwhile is discarded.
constexpr int kStepCopyChunks = 4;  // 16-byte chunks per thread

__host__ __device__ inline int64_t step_copy_chunks(const DecodeArgs& a, int D, int elt_bytes) {
  return (int64_t)a.num_seqs * 2 * a.num_kv_heads * D * elt_bytes / 16;
}
// Workgroups of NT threads that copy the step's rows (0 without a step),
// rounded up to a multiple of 8: workgroups are dealt to the 8 XCDs
// round-robin in linear-id order, so a grid row longer by a multiple of 8
// leaves every attention workgroup on the XCD it has without a step (on the
// 32K-token batch, 64 partition rows, any other count cost 1%).
inline int step_copy_workgroups(const DecodeArgs& a, int D, int elt_bytes, int NT) {
  if (a.new_k == nullptr) return 0;
  const int64_t per_wg = (int64_t)NT * kStepCopyChunks;
  const int64_t n = (step_copy_chunks(a, D, elt_bytes) + per_wg - 1) / per_wg;
  return (int)((n + 7) / 8 * 8);
}

// Copy workgroup `wg`: chunks (wg * kStepCopyChunks + u) * NT + thread, in
// order sequence, tensor (K, V), kv head, d.
template <class DT, int D, int BS, int NT>
__device__ __forceinline__ void step_copy(const DecodeArgs& a, int wg) {
  using S = typename DT::storage;
  constexpr int kChunk = DT::kPerChunk;  // elements per 16-byte chunk
  const int row_chunks = a.num_kv_heads * D / kChunk;  // one tensor, one sequence
  const int64_t total = step_copy_chunks(a, D, sizeof(S));
#pragma unroll
  for (int u = 0; u < kStepCopyChunks; ++u) {
    const int64_t c = ((int64_t)wg * kStepCopyChunks + u) * NT + threadIdx.x;
    if (c >= total) break;
    const int b = (int)(c / (2 * row_chunks));
    const int r = (int)(c - (int64_t)b * 2 * row_chunks);
    const bool is_v = r >= row_chunks;
    const int off = (is_v ? r - row_chunks : r) * kChunk;
    const int ctx = a.context_lens[b];
    if (ctx <= 0 || ctx > a.max_blocks * BS) continue;
    const int blk = a.block_tables[(size_t)b * a.max_blocks + (ctx - 1) / BS];
    if (blk < 0 || blk >= a.num_blocks) continue;
    const size_t src = (size_t)b * a.num_kv_heads * D + off;
    const size_t dst = ((size_t)blk * BS + (ctx - 1) % BS) * a.num_kv_heads * D + off;
    store_chunk(static_cast<S*>(const_cast<void*>(is_v ? a.v_cache : a.k_cache)) + dst,
                load_chunk(static_cast<const S*>(is_v ? a.new_v : a.new_k) + src));
  }
}

// At the start of a decode kernel whose first n_attn workgroups (in grid x)
// attend: true for the copy workgroups after them, which do their share of
// the copy in the grid's last row and return.
template <class DT, int D, int BS, int NT>
__device__ __forceinline__ bool step_copy_role(const DecodeArgs& a, int n_attn) {
  if ((int)blockIdx.x < n_attn) return false;
  if (blockIdx.y == gridDim.y - 1) step_copy<DT, D, BS, NT>(a, blockIdx.x - n_attn);
  return true;
}

// End of a partition workgroup.  Every wave has left its state in LDS, one
// slot per wave: wave w serves kv head w % hpw of the workgroup's group, head
// slice (w / hpw) % HS and token share w / (hpw * HS).  The token shares of
// each (kv head, query head) are combined; then the output is stored (the
// sequence fits one partition), or the partial state is published and the
// last workgroup of the (sequence, head group) to arrive merges every
// partition into the output.
template <class DT, int D, int G, int GW, int HS, int NW, int HPW>
__device__ __forceinline__ void finish_partition(const DecodeArgs& a, int b, int gg, int part,
                                                 int nparts, bool poisoned,
                                                 const float (*s_acc)[GW][D],
                                                 const float (*s_m)[GW],
                                                 const float (*s_l)[GW]) {
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x;
  const int hpw = a.heads_per_wg;
  const int Hkv = a.num_kv_heads;
  const int n_groups = Hkv / hpw;
  const int nwt = NW / (hpw * HS);  // waves sharing one (kv head, head slice)
  const int wg_elems = hpw * G * D;
  const size_t out_base = ((size_t)b * a.num_q_heads + (size_t)gg * hpw * G) * D;

  // Row r = hwe * G + hh of the group (the order of the output rows) is held
  // by waves w0(r) + hpw * HS * t, t < nwt, head h(r).  With large query
  // groups (many elements per thread, shares from eight waves) its maximum,
  // sum and the factor of each wave's share are worked out once per row and
  // used by the row's D elements; with small ones each element works them
  // out itself, since there the extra barrier costs more than the
  // exponentials it saves (measured on MI355X: MQA batch 25.2 -> 24.3 us,
  // Qwen3 batch 33.8 -> 34.1 us when shared).  Same operations in the same
  // order either way, so the results are the same bits.  The shared factors
  // live in the merge's LDS area, not used before the combine is over:
  // nwt * rows = NW * GW factors fit in s_pm, 2 * rows in s_pl.  HPW is the
  // most kv heads a workgroup takes, so kRows bounds its output rows.
  constexpr bool kRowFactors = G >= 8;
  constexpr int kRows = HPW * G;
  // The merge in this launch takes fewer than 16 pieces (16 or more go to the
  // merge kernel), so its LDS area holds 16 pieces' (max, sum) per row.
  constexpr int kPieces = 16;
  static_assert(NW * GW <= kPieces * kRows, "combine factors must fit the merge's LDS area");
  __shared__ float s_pm[kPieces][kRows];
  __shared__ float s_pl[kPieces][kRows];
  const int rows = hpw * G;
  float* s_fac = &s_pm[0][0];  // [t][r]: t * rows + r
  float* s_rm = &s_pl[0][0];
  float* s_rl = s_rm + rows;
  if constexpr (kRowFactors) {
    for (int r = tid; r < rows; r += NT) {
      const int hwe = r / G, hh = r % G;
      const int w0 = hwe + hpw * (hh / GW);
      const int h = hh % GW;
      float M = kNoMax;
      for (int t = 0; t < nwt; ++t) M = fmaxf(M, s_m[w0 + hpw * HS * t][h]);
      float L = 0.0f;
      for (int t = 0; t < nwt; ++t) {
        const int w = w0 + hpw * HS * t;
        const float f = fast_exp2(s_m[w][h] - M);
        s_fac[t * rows + r] = f;
        L += s_l[w][h] * f;
      }
      s_rm[r] = M;
      s_rl[r] = poisoned ? __builtin_nanf("") : L;
    }
    __syncthreads();
  }
  // Output element e (row r = e / D of the group, kv head hwe, query head hh,
  // dimension d) with combined sum A, row maximum M and row sum L: the
  // normalised output, or the partition's state for the merge.
  const auto emit = [&](int e, int hwe, int hh, int d, float A, float M, float L) {
    if (nparts == 1) {
      store_out(DT{}, a.out, out_base + e, A / L);
    } else {
      const size_t pr = (((size_t)b * Hkv + gg * hpw + hwe) * a.max_parts + part) * G + hh;
      if (a.deferred_merge) {
        // Read by the merge kernel, after this launch has ended.
        a.ws_acc[pr * D + d] = A;
        if (d == 0) {
          a.ws_ml[pr * 2 + 0] = M;
          a.ws_ml[pr * 2 + 1] = L;
        }
      } else {
        publish(a.ws_acc + pr * D + d, A);
        if (d == 0) {
          publish(a.ws_ml + pr * 2 + 0, M);
          publish(a.ws_ml + pr * 2 + 1, L);
        }
      }
    }
  };
  if constexpr (kRowFactors) {
    // Four consecutive elements of one row per thread: one 16-byte LDS read
    // per wave share (each element sums its shares in the same order).
    static_assert(D % 4 == 0, "rows split into 4-element pieces");
    for (int e = 4 * tid; e < wg_elems; e += 4 * NT) {
      const int hwe = e / (G * D), rem = e % (G * D);
      const int hh = rem / D, d = rem % D;
      const int r = e / D;
      const int w0 = hwe + hpw * (hh / GW);
      const int h = hh % GW;
      float A0 = 0.0f, A1 = 0.0f, A2 = 0.0f, A3 = 0.0f;
      for (int t = 0; t < nwt; ++t) {
        const float4 v = *reinterpret_cast<const float4*>(&s_acc[w0 + hpw * HS * t][h][d]);
        const float f = s_fac[t * rows + r];
        A0 += v.x * f;
        A1 += v.y * f;
        A2 += v.z * f;
        A3 += v.w * f;
      }
      const float M = s_rm[r], L = s_rl[r];
      emit(e, hwe, hh, d, A0, M, L);
      emit(e + 1, hwe, hh, d + 1, A1, M, L);
      emit(e + 2, hwe, hh, d + 2, A2, M, L);
      emit(e + 3, hwe, hh, d + 3, A3, M, L);
    }
  } else {
    for (int e = tid; e < wg_elems; e += NT) {
      const int hwe = e / (G * D), rem = e % (G * D);
      const int hh = rem / D, d = rem % D;
      const int w0 = hwe + hpw * (hh / GW);
      const int h = hh % GW;
      float M = kNoMax, L = 0.0f, A = 0.0f;
      for (int t = 0; t < nwt; ++t) M = fmaxf(M, s_m[w0 + hpw * HS * t][h]);
      for (int t = 0; t < nwt; ++t) {
        const int w = w0 + hpw * HS * t;
        const float f = fast_exp2(s_m[w][h] - M);
        L += s_l[w][h] * f;
        A += s_acc[w][h][d] * f;
      }
      if (poisoned) L = __builtin_nanf("");
      emit(e, hwe, hh, d, A, M, L);
    }
  }
  if (nparts == 1 || a.deferred_merge) return;

  __shared__ int s_last;
  int32_t* counter = a.counters + (size_t)b * n_groups + gg;
  if (!arrive(counter, nparts, &s_last)) return;

  // Output row r of the group is query head r % G of kv head r / G; the
  // pieces of one kv head are max_parts * G rows apart.  All the group's rows
  // merge in one pass (one round trip for every kv head's states), sized for
  // the group's own number of kv heads, so that each thread's loads cover as
  // many pieces as they can.
  const size_t head_rows = (size_t)a.max_parts * G;
  const size_t grp_base = ((size_t)b * Hkv + (size_t)gg * hpw) * head_rows;
  const auto row_of = [&](int p, int r) {
    return grp_base + (size_t)(r / G) * head_rows + (size_t)p * G + r % G;
  };
  // About eight loads in flight per thread: a sequence split inside the
  // launch has fewer than 16 pieces, mostly a few, and a smaller batch sends
  // fewer clamped repeats of its last piece (measured on MI355X: Qwen3 batch
  // 33.04 -> 32.88 us, Llama-3.2 batch 66.4 -> 66.1 us against 16).
  const auto merge = [&](auto gh) {
    constexpr int GH = decltype(gh)::value;
    merge_pieces<DT, D, GH, NT, 8, kPieces>(a, nparts, rows, row_of, out_base,
                                reinterpret_cast<float (*)[GH]>(&s_pm[0][0]),
                                reinterpret_cast<float (*)[GH]>(&s_pl[0][0]));
  };
  if (hpw == 1) {
    merge(IntC<G>{});
  } else {
    if constexpr (HPW >= 2) {
      if (hpw == 2)
        merge(IntC<2 * G>{});
      else
        merge(IntC<kRows>{});
    }
  }
  reset_counter(counter);
}

// Body of the merge kernel that follows a partition launch with deferred
// merge: one workgroup of D threads per (sequence, query head) merges that
// row's partition states into the output, one element a thread, with every
// piece of a 64-piece chunk requested in one round trip.  (One workgroup per
// (sequence, kv head) left the 32K-token batch's 8.5 MB of states to 64 CUs:
// 10 us.)  Each element folds the same values in the same order as the
// in-launch merge.  Sequences that fit one partition, and empty or
// out-of-range contexts, were finished by the partition kernel.
template <class DT, int D, int G>
__device__ __forceinline__ void merge_partitions(const DecodeArgs& a, int bs) {
  const int Hq = a.num_q_heads;
  const int b = blockIdx.x / Hq;
  const int qh = blockIdx.x % Hq;
  const int kvh = qh / G, r = qh % G;
  const int ctx = a.context_lens[b];
  if (ctx <= 0 || ctx > a.max_blocks * bs) return;
  const int part_tokens = a.part_blocks * bs;
  const int nparts = (ctx + part_tokens - 1) / part_tokens;
  if (nparts <= 1) return;
  __shared__ float s_pm[64][1];
  __shared__ float s_pl[64][1];
  const size_t base = ((size_t)b * a.num_kv_heads + kvh) * a.max_parts * G + r;
  const size_t out_base = ((size_t)b * Hq + qh) * D;
  merge_pieces<DT, D, 1, D, 64>(
      a, nparts, 1, [&](int p, int) { return base + (size_t)p * G; }, out_base, s_pm, s_pl);
}

}  // namespace pa
