// Single-token decode attention over a paged KV cache, gfx950.
//
// What is computed (barellm README, feature list and paged-cache list;
// LLAISYS README, self-attention item): for sequence b and query head h,
// softmax attention of q[b,h] over the first context_lens[b] cached rows of KV
// head h / G, the rows found through the block table.  Accumulation in
// float32; the running max / running sum form of softmax (online softmax).
//
// Work decomposition (MI355X-first, not taken from any page):
//   * one workgroup per (partition, kv head, sequence); a partition is
//     part_blocks consecutive logical blocks of one sequence;
//   * the G query heads that share a KV head are handled together, so every
//     K/V byte is fetched from HBM once per (sequence, kv head);
//   * a wavefront reads one block's rows with 128-bit loads: a row
//     (one token, one kv head, head_dim elements) is head_dim*elt bytes
//     contiguous, spread over RL = head_dim*elt/16 lanes; 64/RL rows per load;
//   * q.k partial dot products are summed over the RL lanes of a row with DPP
//     row operations; every row keeps its own online-softmax state (max, sum,
//     unnormalised output), merged across rows with lane swaps and across
//     waves through LDS at the end;
//   * a sequence with more than one partition writes each partition's state
//     to the workspace; the last workgroup of that (sequence, kv head) to
//     arrive (atomic arrival counter) merges them with a log-sum-exp
//     reduction and writes the output, so there is no second launch (the
//     last-block pattern of the LLAISYS README, CUDA argmax item).
//   * MI355X has one L2 per XCD and the L2s are not coherent with each other;
//     a device-scope fence therefore writes back and invalidates the whole L2
//     of the XCD, which costs far more than the data it protects.  Partition
//     states are instead stored and loaded with system-scope atomic accesses
//     (they bypass the non-coherent L2s), each workgroup waits for its own
//     stores to complete before it counts itself in, and the merger loads
//     only after it has seen every arrival: no cache-wide maintenance.
#include "common.hpp"

#include <math.h>

namespace pa {

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_acc;      // [B, Hkv, max_parts, G, D]  unnormalised partition outputs
  float* ws_ml;       // [B, Hkv, max_parts, G, 2]  (max, sum) per partition, log2 units
  int32_t* counters;  // [B, Hkv]                   arrivals, reset by the merger
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t part_blocks;
  int32_t max_parts;
  float scale_log2;   // scale * log2(e): scores are kept in base-2 units
};

template <class DT, int D, int BS, int G, int NW>
struct DecodeShape {
  static constexpr int E = DT::kPerChunk;      // elements per lane chunk
  static constexpr int RL = D / E;             // lanes per row
  static constexpr int ROWS = 64 / RL;         // rows per wave load
  static constexpr int NI = BS / ROWS;         // wave loads per block (per K or V)
  static constexpr int GW = G < 8 ? G : 8;     // query heads per wave
  static constexpr int HS = G / GW;            // head splits across waves
  static constexpr int NWT = NW / HS;          // waves sharing one head split
  static_assert(RL >= 4 && RL <= 32, "row must span 4..32 lanes");
  static_assert(BS % ROWS == 0, "block must be whole wave loads");
  static_assert(NW % HS == 0, "waves must cover every head split");
};

// q.k over one 16-byte chunk, float32 accumulation.
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

// Partition states cross XCDs: system-scope accesses skip the per-XCD L2s.
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float collect(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
}

// Running-state sentinel: finite, so exp2(sentinel - sentinel) = 1 for rows
// that have seen no token yet (their sum and output are still zero).
constexpr float kNoMax = -1.0e30f;

template <int kMask, int GW, int E>
__device__ __forceinline__ void merge_rows(float (&m)[GW], float (&l)[GW],
                                           float (&acc)[GW][E]) {
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

template <class DT, int D, int BS, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  using Sh = DecodeShape<DT, D, BS, G, NW>;
  using S = typename DT::storage;
  constexpr int E = Sh::E, RL = Sh::RL, ROWS = Sh::ROWS, NI = Sh::NI;
  constexpr int GW = Sh::GW, HS = Sh::HS, NWT = Sh::NWT;
  constexpr int NT = NW * 64;

  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index is the same on every lane; say so, so loops over it stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hkv = a.num_kv_heads;

  const int ctx = a.context_lens[b];
  const int part_tokens = a.part_blocks * BS;
  const bool bad_ctx = ctx < 0 || ctx > a.max_blocks * BS;
  const int nparts = (bad_ctx || ctx == 0) ? 1 : (ctx + part_tokens - 1) / part_tokens;
  if (part >= nparts) return;

  const size_t out_base = ((size_t)b * a.num_q_heads + (size_t)g * G) * D;
  if (bad_ctx || ctx == 0) {
    const float fill = bad_ctx ? __builtin_nanf("") : 0.0f;
    for (int e = tid; e < G * D; e += NT) store_out(DT{}, a.out, out_base + e, fill);
    return;
  }

  // This partition's block-table entries, one per lane.
  const int blk0 = part * a.part_blocks;
  const int nblk_seq = (ctx + BS - 1) / BS;
  const int nblk = min(a.part_blocks, nblk_seq - blk0);
  const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks + blk0;
  const int my_blk = lane < nblk ? trow[lane] : 0;
  const bool bad_here = lane < nblk && (my_blk < 0 || my_blk >= a.num_blocks);
  const bool poisoned = __ballot(bad_here) != 0;  // same answer in every wave
  const int nblk_run = poisoned ? 0 : nblk;

  const int hs = wave % HS;  // which GW-head slice of the group
  const int tw = wave / HS;  // which of the NWT waves on that slice
  const int row = lane / RL;
  const int col = lane % RL;
  const int h0 = g * G + hs * GW;

  uint4 qv[GW];
#pragma unroll
  for (int h = 0; h < GW; ++h)
    qv[h] = load_chunk(static_cast<const S*>(a.q) +
                       ((size_t)b * a.num_q_heads + h0 + h) * D + col * E);

  float m[GW], l[GW], acc[GW][E];
#pragma unroll
  for (int h = 0; h < GW; ++h) {
    m[h] = kNoMax;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;
  }

  const size_t tok_stride = (size_t)Hkv * D;   // elements between tokens
  const size_t blk_stride = tok_stride * BS;   // elements between blocks
  const int lane_off = row * Hkv * D + col * E;
  const S* kbase = static_cast<const S*>(a.k_cache) + (size_t)g * D + lane_off;
  const S* vbase = static_cast<const S*>(a.v_cache) + (size_t)g * D + lane_off;

  for (int j = tw; j < nblk_run; j += NWT) {
    const int phys = __builtin_amdgcn_readlane(my_blk, j);
    const S* kb = kbase + (size_t)phys * blk_stride;
    const S* vb = vbase + (size_t)phys * blk_stride;
    uint4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = load_chunk(kb + (size_t)i * ROWS * tok_stride);
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = load_chunk(vb + (size_t)i * ROWS * tok_stride);

    const int pos0 = (blk0 + j) * BS + row;  // position of this lane's row in load 0
    const bool full = (blk0 + j + 1) * BS <= ctx;

    float s[NI][GW];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int h = 0; h < GW; ++h)
        s[i][h] = group_sum<RL>(chunk_dot(DT{}, qv[h], kr[i])) * a.scale_log2;
    if (!full) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (pos0 + i * ROWS >= ctx)
#pragma unroll
          for (int h = 0; h < GW; ++h) s[i][h] = -INFINITY;
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
      float vf[E];
      unpack(DT{}, vr[i], vf);
      if (!full && pos0 + i * ROWS >= ctx) {
        // slots past the sequence may hold anything, NaN included
#pragma unroll
        for (int e = 0; e < E; ++e) vf[e] = 0.0f;
      }
#pragma unroll
      for (int h = 0; h < GW; ++h) {
        const float p = fast_exp2(s[i][h] - m[h]);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }
  }

  // Rows of the wave -> one state per wave (held by every row afterwards).
  if constexpr (RL <= 8) merge_rows<8, GW, E>(m, l, acc);
  if constexpr (RL <= 16) merge_rows<16, GW, E>(m, l, acc);
  merge_rows<32, GW, E>(m, l, acc);

  __shared__ float s_acc[NW][GW][D];
  __shared__ float s_m[NW][GW];
  __shared__ float s_l[NW][GW];
  __shared__ int s_last;
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < GW; ++h) {
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[wave][h][col * E + e] = acc[h][e];
      if (col == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // Waves on the same head slice -> the partition's state for each (head, d).
  const size_t bg = (size_t)b * Hkv + g;
  const size_t part_base = (bg * a.max_parts + part) * (size_t)G;
  for (int e = tid; e < G * D; e += NT) {
    const int hh = e / D, d = e % D;
    const int hsl = hh / GW, h = hh % GW;
    float M = kNoMax;
#pragma unroll
    for (int t = 0; t < NWT; ++t) M = fmaxf(M, s_m[hsl + HS * t][h]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      const int w = hsl + HS * t;
      const float f = fast_exp2(s_m[w][h] - M);
      L += s_l[w][h] * f;
      A += s_acc[w][h][d] * f;
    }
    if (poisoned) L = __builtin_nanf("");
    if (nparts == 1) {
      store_out(DT{}, a.out, out_base + e, A / L);
    } else {
      publish(a.ws_acc + part_base * D + e, A);
      if (d == 0) {
        publish(a.ws_ml + (part_base + hh) * 2 + 0, M);
        publish(a.ws_ml + (part_base + hh) * 2 + 1, L);
      }
    }
  }
  if (nparts == 1) return;

  // Count this partition in once all of its stores have completed; the
  // workgroup that brings the count to nparts merges.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(a.counters + bg, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_SYSTEM);
    s_last = (prev == nparts - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // Merge: partition maxima and sums go through LDS in chunks of up to 64
  // partitions (one system-scope load per value); each thread keeps a
  // running (max, sum, output) for the elements it owns and rescales it
  // when a chunk raises the maximum.  Chunks and partitions are visited in
  // index order, so the result does not depend on arrival order.
  constexpr int kChunk = 64;
  constexpr int EPT = (G * D + NT - 1) / NT;  // elements per thread
  __shared__ float s_pm[kChunk][G];
  __shared__ float s_pl[kChunk][G];
  const size_t seq_base = bg * a.max_parts * (size_t)G;
  float rM[EPT], rL[EPT], rA[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    rM[k] = kNoMax;
    rL[k] = 0.0f;
    rA[k] = 0.0f;
  }
  for (int c0 = 0; c0 < nparts; c0 += kChunk) {
    const int n = min(kChunk, nparts - c0);
    for (int i = tid; i < n * G; i += NT) {
      const int pp = i / G, hh = i % G;
      const size_t r = seq_base + (size_t)(c0 + pp) * G + hh;
      s_pm[pp][hh] = collect(a.ws_ml + r * 2);
      s_pl[pp][hh] = collect(a.ws_ml + r * 2 + 1);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = tid + k * NT;
      if (EPT * NT == G * D || e < G * D) {
        const int hh = e / D;
        float M = rM[k];
        for (int pp = 0; pp < n; ++pp) M = fmaxf(M, s_pm[pp][hh]);
        const float f0 = fast_exp2(rM[k] - M);
        float L = rL[k] * f0, A = rA[k] * f0;
        const float* acc_p = a.ws_acc + (seq_base + (size_t)c0 * G) * D + e;
#pragma unroll 8
        for (int pp = 0; pp < n; ++pp) {
          const float f = fast_exp2(s_pm[pp][hh] - M);
          L += s_pl[pp][hh] * f;
          A += collect(acc_p + (size_t)pp * G * D) * f;
        }
        rM[k] = M;
        rL[k] = L;
        rA[k] = A;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + k * NT;
    if (EPT * NT == G * D || e < G * D) store_out(DT{}, a.out, out_base + e, rA[k] / rL[k]);
  }
  if (tid == 0)
    __hip_atomic_store(a.counters + bg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ------------------------------------------------------------------ host
namespace {

constexpr int kWaves = 4;

struct Geometry {
  int part_blocks;
  int max_parts;
  size_t acc_bytes, ml_bytes, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool group_supported(int g) {
  return g == 1 || g == 2 || g == 4 || g == 8 || g == 16 || g == 32;
}

// Library choice of partition length (in blocks): the largest power of two
// <= 64 blocks that still gives at least ~8 workgroups per compute unit when
// every sequence is as long as its table allows.
int auto_part_blocks(int B, int Hkv, int max_blocks) {
  const long target = 8L * 256;
  int pb = kMaxPartitionBlocks;
  while (pb > 4) {
    const long parts = (max_blocks + pb - 1) / pb;
    if ((long)B * Hkv * parts >= target) break;
    pb /= 2;
  }
  return pb;
}

int resolve_part_blocks(int B, int Hkv, int max_blocks, int bs, int requested) {
  if (requested == 0) return auto_part_blocks(B, Hkv, max_blocks);
  if (requested < 0 || requested % bs != 0) return -1;
  const int pb = requested / bs;
  if (pb < 1 || pb > kMaxPartitionBlocks) return -1;
  return pb;
}

bool geometry(int B, int Hq, int Hkv, int D, int max_blocks, int bs, int requested,
              Geometry* out) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || max_blocks <= 0) return false;
  if (!supported_head_dim(D) || !supported_block_size(bs)) return false;
  const int pb = resolve_part_blocks(B, Hkv, max_blocks, bs, requested);
  if (pb < 0) return false;
  out->part_blocks = pb;
  out->max_parts = (max_blocks + pb - 1) / pb;
  if (out->max_parts <= 1 || B == 0) {
    out->acc_bytes = out->ml_bytes = out->total = 0;
    return true;
  }
  const size_t rows = (size_t)B * Hkv * out->max_parts * (size_t)(Hq / Hkv);
  out->acc_bytes = align256(rows * D * sizeof(float));
  out->ml_bytes = align256(rows * 2 * sizeof(float));
  out->total = out->acc_bytes + out->ml_bytes;
  return true;
}

template <class DT, int D, int BS, int G>
hipError_t launch(const DecodeArgs& a, int B, hipStream_t stream) {
  dim3 grid(a.max_parts, a.num_kv_heads, B);
  decode_kernel<DT, D, BS, G, kWaves><<<grid, kWaves * 64, 0, stream>>>(a);
  return hipGetLastError();
}

template <class DT, int D, int BS>
hipError_t by_group(int G, const DecodeArgs& a, int B, hipStream_t s) {
  switch (G) {
    case 1: return launch<DT, D, BS, 1>(a, B, s);
    case 2: return launch<DT, D, BS, 2>(a, B, s);
    case 4: return launch<DT, D, BS, 4>(a, B, s);
    case 8: return launch<DT, D, BS, 8>(a, B, s);
    case 16: return launch<DT, D, BS, 16>(a, B, s);
    case 32: return launch<DT, D, BS, 32>(a, B, s);
  }
  return hipErrorInvalidValue;
}

template <class DT, int D>
hipError_t by_block(int bs, int G, const DecodeArgs& a, int B, hipStream_t s) {
  return bs == 16 ? by_group<DT, D, 16>(G, a, B, s) : by_group<DT, D, 32>(G, a, B, s);
}

template <class DT>
hipError_t by_dim(int D, int bs, int G, const DecodeArgs& a, int B, hipStream_t s) {
  return D == 64 ? by_block<DT, 64>(bs, G, a, B, s) : by_block<DT, 128>(bs, G, a, B, s);
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_blocks_per_seq,
                                            int32_t block_size, int32_t requested) {
  Geometry geo;
  if (!geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                block_size, requested, &geo))
    return -1;
  return geo.part_blocks * block_size;
}

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t max_blocks_per_seq,
                                           int32_t block_size,
                                           int32_t partition_size) {
  Geometry geo;
  if (!geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                block_size, partition_size, &geo))
    return 0;
  return geo.total;
}

extern "C" pa_status pa_paged_attention_decode(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
    int32_t block_size, int32_t max_blocks_per_seq, float scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t* counters,
    int64_t num_counters, pa_dtype dtype, void* stream) {
  clear_error();
  if (!supported_dtype(dtype)) {
    set_error("dtype %d is not PA_DTYPE_F32 or PA_DTYPE_BF16", (int)dtype);
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0) {
    set_error("sizes must be positive (num_seqs may be 0): num_seqs=%d "
              "num_q_heads=%d num_kv_heads=%d num_blocks=%d max_blocks_per_seq=%d",
              num_seqs, num_q_heads, num_kv_heads, num_blocks, max_blocks_per_seq);
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (num_q_heads % num_kv_heads != 0) {
    set_error("num_q_heads=%d is not a multiple of num_kv_heads=%d", num_q_heads,
              num_kv_heads);
    return PA_ERR_INVALID_ARGUMENT;
  }
  const int G = num_q_heads / num_kv_heads;
  if (!group_supported(G)) {
    set_error("query heads per kv head = %d; built for 1, 2, 4, 8, 16, 32", G);
    return PA_ERR_UNSUPPORTED;
  }
  if (!supported_head_dim(head_dim)) {
    set_error("head_dim=%d; built for 64 and 128", head_dim);
    return PA_ERR_UNSUPPORTED;
  }
  if (!supported_block_size(block_size)) {
    set_error("block_size=%d; built for 16 and 32", block_size);
    return PA_ERR_UNSUPPORTED;
  }
  if (num_seqs > 65535 || num_kv_heads > 65535) {
    set_error("num_seqs and num_kv_heads must be <= 65535");
    return PA_ERR_UNSUPPORTED;
  }
  if ((long)max_blocks_per_seq * block_size > 0x7FFFFFFFL) {
    set_error("max_blocks_per_seq * block_size overflows int32");
    return PA_ERR_INVALID_ARGUMENT;
  }
  Geometry geo;
  if (!geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                block_size, partition_size, &geo)) {
    set_error("partition_size=%d must be 0 or a multiple of block_size=%d "
              "between 1 and 64 blocks", partition_size, block_size);
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) {
    set_error("a tensor pointer is NULL");
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) {
    set_error("out, q, k_cache and v_cache must be 16-byte aligned");
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (geo.total > 0) {
    if (workspace_bytes < geo.total) {
      set_error("workspace holds %zu bytes, needs %zu", workspace_bytes, geo.total);
      return PA_ERR_WORKSPACE_TOO_SMALL;
    }
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) {
      set_error("workspace must be non-NULL and 256-byte aligned");
      return PA_ERR_INVALID_ARGUMENT;
    }
    if (!counters || num_counters < (int64_t)num_seqs * num_kv_heads) {
      set_error("counters must hold num_seqs * num_kv_heads = %lld int32 (got %lld)",
                (long long)num_seqs * num_kv_heads, (long long)num_counters);
      return PA_ERR_WORKSPACE_TOO_SMALL;
    }
  }

  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  char* ws = static_cast<char*>(workspace);
  a.ws_acc = geo.total ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_ml = geo.total ? reinterpret_cast<float*>(ws + geo.acc_bytes) : nullptr;
  a.counters = geo.total ? counters : nullptr;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.part_blocks = geo.part_blocks;
  a.max_parts = geo.max_parts;
  a.scale_log2 = scale * 1.4426950408889634f;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err =
      dtype == PA_DTYPE_BF16
          ? by_dim<BF16>(head_dim, block_size, G, a, num_seqs, s)
          : by_dim<F32>(head_dim, block_size, G, a, num_seqs, s);
  if (err != hipSuccess) {
    set_error("decode launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  return PA_OK;
}
