// Pure-read ceilings of the decode's HBM access patterns, for the benchmark.
//
// Each kernel reads exactly the K and V bytes that a decode of the batch
// reads (every row of every used block of every sequence, once), folds them
// into a value that is kept alive, and does nothing else: no softmax, no
// merge, no output.  Its time is what the access pattern alone costs on the
// GPU, the floor under any decode that reads the cache that way.  These are
// measurements beside the library, never part of it.
//
//   mode 0, contiguous: the same byte count read as one contiguous range of
//           K and one of V (256 workgroups of 8 waves, equal shares).
//   mode 1, head rows: the decode's balanced schedule -- each kv head's block
//           list cut into equal ranges; a 4-wave workgroup reads four
//           neighbouring kv heads of one range, each wave its head's
//           head_dim-wide slice of each token row, two blocks in flight.
//   mode 2, token rows: the batch's block list cut into equal ranges, one per
//           workgroup of 8 waves, which reads whole blocks (every kv head of
//           every token: one contiguous run per block), two in flight.
//   mode 3, interleaved head rows: each kv head's block list cut into
//           256 / num_kv_heads equal ranges, one per 4-wave workgroup, whose
//           waves take every fourth block of the range (the head's slice of
//           each token row), two in flight.
//
// bfloat16 caches, head_dim 64 or 128, block_size 16 or 32, at most 2048
// sequences and 128 blocks per range.
//
// rc_stream_probe: the rate of plain streaming reads -- nwg workgroups, each
// reading its own contiguous per_wg-vector region, U 16-byte loads per lane
// in flight, non-temporal or plain -- to see what one CU, some CUs and every
// CU draw from HBM.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxSeqs = 2048;
constexpr int kMaxRange = 128;
constexpr int kWorkgroups = 256;

__device__ __forceinline__ u32x4 ld(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

struct Args {
  const char* k;
  const char* v;
  const int* tables;
  const int* ctx;
  int B, max_blocks, Hkv, row_bytes, bs;
  int ranges;            // equal ranges of the block list (per head group in mode 1)
  long long flat_bytes;  // mode 0: bytes of K (and of V) to read
  uint32_t* sink;
};

// Blocks per sequence, prefix-summed into s_cum[0..B] by the workgroup.
template <int NT>
__device__ int prefix_blocks(const Args& a, int* s_cum, int* s_part) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int c0 = 0; c0 < a.B; c0 += NT) {
    const int b = c0 + tid;
    const int nb = b < a.B ? min((a.ctx[b] + a.bs - 1) / a.bs, a.max_blocks) : 0;
    int x = nb;
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(x, o, 64);
      if (lane >= o) x += t;
    }
    if (lane == 63) s_part[wave] = x;
    __syncthreads();
    int off = carry, tot = 0;
    for (int w = 0; w < NT / 64; ++w) {
      off += w < wave ? s_part[w] : 0;
      tot += s_part[w];
    }
    if (b < a.B) s_cum[b] = off + x - nb;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) s_cum[a.B] = carry;
  __syncthreads();
  return carry;
}

// The physical block of each of the range's blocks i = lane and 64 + lane.
__device__ void range_entries(const Args& a, const int* s_cum, int s, int n, int (&ent)[2]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = 64 * h + lane;
    ent[h] = 0;
    if (i < n) {
      const int g = s + i;
      int lo = 0, hi = a.B;  // s_cum[lo] <= g < s_cum[lo + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_cum[mid] <= g) lo = mid; else hi = mid;
      }
      ent[h] = a.tables[(long long)lo * a.max_blocks + (g - s_cum[lo])];
    }
  }
}

// 8 waves, 8 loads of 16 bytes in flight per lane (64 KB per workgroup).
__global__ __launch_bounds__(512) void read_contiguous(Args a) {
  constexpr int U = 8, STEP = 512 * 16;
  const long long per = a.flat_bytes / (kWorkgroups / 2);
  const char* base = blockIdx.x < kWorkgroups / 2 ? a.k : a.v;
  const long long lo = per * (blockIdx.x % (kWorkgroups / 2));
  uint32_t acc = 0;
  for (long long o = lo + threadIdx.x * 16; o < lo + per; o += U * STEP) {
    u32x4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = o + u * STEP < lo + per ? ld(base + o + u * STEP) : u32x4{};
#pragma unroll
    for (int u = 0; u < U; ++u) acc += fold(r[u]);
  }
  if (acc == 0x9E3779B9u) a.sink[blockIdx.x] = acc;
}

// NI 16-byte loads per lane cover a head's slice of one block.
template <int NI>
__global__ __launch_bounds__(256) void read_head_rows(Args a, int heads_per_wg) {
  __shared__ int s_cum[kMaxSeqs + 1];
  __shared__ int s_part[4];
  const int T = prefix_blocks<256>(a, s_cum, s_part);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ngr = a.Hkv / heads_per_wg, rpw = 4 / heads_per_wg;
  const int gg = blockIdx.x % ngr;
  const int r = (blockIdx.x / ngr) * rpw + wave / heads_per_wg;
  const int h = gg * heads_per_wg + wave % heads_per_wg;
  const int R = a.ranges * rpw;
  const int s = (int)((long long)r * T / R), n = (int)((long long)(r + 1) * T / R) - s;
  int ent[2];
  range_entries(a, s_cum, s, n, ent);
  const int RL = a.row_bytes / 16, ROWS = 64 / RL;
  const long long tok = (long long)a.Hkv * a.row_bytes, blk = tok * a.bs;
  const long long loff = (long long)(lane / RL) * tok + (long long)h * a.row_bytes + (lane % RL) * 16;
  auto entry = [&](int i) { return __builtin_amdgcn_readlane(i < 64 ? ent[0] : ent[1], i & 63); };
  u32x4 kr[2][NI], vr[2][NI];
  auto fetch = [&](int i, u32x4 (&k)[NI], u32x4 (&v)[NI]) {
    const long long base = (long long)entry(i) * blk + loff;
#pragma unroll
    for (int t = 0; t < NI; ++t) k[t] = ld(a.k + base + t * ROWS * tok);
#pragma unroll
    for (int t = 0; t < NI; ++t) v[t] = ld(a.v + base + t * ROWS * tok);
  };
  uint32_t acc = 0;
  if (n > 0) {
    fetch(0, kr[0], vr[0]);
    for (int i = 0; i < n; i += 2) {
      fetch(min(i + 1, n - 1), kr[1], vr[1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < NI; ++t) acc += fold(kr[0][t]) + fold(vr[0][t]);
      fetch(min(i + 2, n - 1), kr[0], vr[0]);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < n) {
#pragma unroll
        for (int t = 0; t < NI; ++t) acc += fold(kr[1][t]) + fold(vr[1][t]);
      }
    }
  }
  if (acc == 0x9E3779B9u) a.sink[blockIdx.x * 4 + wave] = acc;
}

// One kv head per 4-wave workgroup, waves interleaving the blocks of one
// range (wave w takes blocks w, w + 4, ...): NI 16-byte loads per lane cover
// the head's slice of a block.
template <int NI>
__global__ __launch_bounds__(256) void read_head_interleaved(Args a) {
  __shared__ int s_cum[kMaxSeqs + 1];
  __shared__ int s_part[4];
  const int T = prefix_blocks<256>(a, s_cum, s_part);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x % a.Hkv, r = blockIdx.x / a.Hkv, R = a.ranges;
  const int s = (int)((long long)r * T / R), n = (int)((long long)(r + 1) * T / R) - s;
  // This wave's blocks of the range: i = wave + 4 k < n.
  const int nw = n > wave ? (n - wave + 3) / 4 : 0;
  int ent[2];
  {
    // entries of this wave's blocks k = lane and 64 + lane
    ent[0] = ent[1] = 0;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int k = 64 * hh + lane;
      if (k < nw) {
        const int g = s + wave + 4 * k;
        int lo = 0, hi = a.B;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_cum[mid] <= g) lo = mid; else hi = mid;
        }
        ent[hh] = a.tables[(long long)lo * a.max_blocks + (g - s_cum[lo])];
      }
    }
  }
  const int RL = a.row_bytes / 16, ROWS = 64 / RL;
  const long long tok = (long long)a.Hkv * a.row_bytes, blk = tok * a.bs;
  const long long loff = (long long)(lane / RL) * tok + (long long)h * a.row_bytes + (lane % RL) * 16;
  auto entry = [&](int i) { return __builtin_amdgcn_readlane(i < 64 ? ent[0] : ent[1], i & 63); };
  u32x4 kr[2][NI], vr[2][NI];
  auto fetch = [&](int i, u32x4 (&k)[NI], u32x4 (&v)[NI]) {
    const long long base = (long long)entry(i) * blk + loff;
#pragma unroll
    for (int t = 0; t < NI; ++t) k[t] = ld(a.k + base + t * ROWS * tok);
#pragma unroll
    for (int t = 0; t < NI; ++t) v[t] = ld(a.v + base + t * ROWS * tok);
  };
  uint32_t acc = 0;
  if (nw > 0) {
    fetch(0, kr[0], vr[0]);
    for (int i = 0; i < nw; i += 2) {
      fetch(min(i + 1, nw - 1), kr[1], vr[1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < NI; ++t) acc += fold(kr[0][t]) + fold(vr[0][t]);
      fetch(min(i + 2, nw - 1), kr[0], vr[0]);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < nw) {
#pragma unroll
        for (int t = 0; t < NI; ++t) acc += fold(kr[1][t]) + fold(vr[1][t]);
      }
    }
  }
  if (acc == 0x9E3779B9u) a.sink[blockIdx.x * 4 + wave] = acc;
}

// CPW 16-byte loads per lane of an 8-wave workgroup cover one whole block.
template <int CPW>
__global__ __launch_bounds__(512) void read_token_rows(Args a) {
  __shared__ int s_cum[kMaxSeqs + 1];
  __shared__ int s_part[8];
  const int T = prefix_blocks<512>(a, s_cum, s_part);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = blockIdx.x, R = a.ranges;
  const int s = (int)((long long)r * T / R), n = (int)((long long)(r + 1) * T / R) - s;
  int ent[2];
  range_entries(a, s_cum, s, n, ent);
  const long long blk = (long long)a.Hkv * a.row_bytes * a.bs;
  auto entry = [&](int i) { return __builtin_amdgcn_readlane(i < 64 ? ent[0] : ent[1], i & 63); };
  u32x4 kr[2][CPW], vr[2][CPW];
  auto fetch = [&](int i, u32x4 (&k)[CPW], u32x4 (&v)[CPW]) {
    const long long base = (long long)entry(i) * blk + wave * 1024 + lane * 16;
#pragma unroll
    for (int t = 0; t < CPW; ++t) k[t] = ld(a.k + base + t * 8192);
#pragma unroll
    for (int t = 0; t < CPW; ++t) v[t] = ld(a.v + base + t * 8192);
  };
  uint32_t acc = 0;
  if (n > 0) {
    fetch(0, kr[0], vr[0]);
    for (int i = 0; i < n; i += 2) {
      fetch(min(i + 1, n - 1), kr[1], vr[1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < CPW; ++t) acc += fold(kr[0][t]) + fold(vr[0][t]);
      fetch(min(i + 2, n - 1), kr[0], vr[0]);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < n) {
#pragma unroll
        for (int t = 0; t < CPW; ++t) acc += fold(kr[1][t]) + fold(vr[1][t]);
      }
    }
  }
  if (acc == 0x9E3779B9u) a.sink[blockIdx.x * 8 + wave] = acc;
}

}  // namespace

// One launch of `mode` on `stream`.  kv_bytes: the K plus V bytes a decode
// reads (mode 0 reads half of it from each cache, from the start); the
// caches must hold at least that.  sink: >= 2048 uint32 of device memory.
// Returns 0, or -1 for sizes the kernels are not built for (nothing is
// launched), or the HIP error of the launch.
// Stream probe: workgroup g reads vectors [g per_wg, (g + 1) per_wg) of p.
template <int U, bool NT>
__global__ void stream_probe(const uint4* __restrict__ p, long per_wg, uint32_t* sink) {
  const uint4* base = p + (long)blockIdx.x * per_wg;
  uint32_t acc = 0;
  const long nt = blockDim.x;
  for (long i = threadIdx.x; i < per_wg; i += nt * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long j = i + u * nt;
      v[u] = make_uint4(0, 0, 0, 0);
      if (j < per_wg) {
        if constexpr (NT) {
          typedef uint32_t u4 __attribute__((ext_vector_type(4)));
          const u4 t = __builtin_nontemporal_load(reinterpret_cast<const u4*>(base + j));
          v[u] = make_uint4(t.x, t.y, t.z, t.w);
        } else {
          v[u] = base[j];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x & 2047] = acc;  // keeps the loads alive
}

extern "C" int rc_read_ceiling(int mode, const void* k_cache, const void* v_cache,
                               const int* block_tables, const int* context_lens, int num_seqs,
                               int max_blocks, int num_kv_heads, int head_dim, int block_size,
                               long long kv_bytes, long long total_blocks, uint32_t* sink,
                               void* stream) {
  if (num_seqs < 1 || num_seqs > kMaxSeqs || (head_dim != 64 && head_dim != 128) ||
      (block_size != 16 && block_size != 32) || num_kv_heads < 1)
    return -1;
  Args a{};
  a.k = static_cast<const char*>(k_cache);
  a.v = static_cast<const char*>(v_cache);
  a.tables = block_tables;
  a.ctx = context_lens;
  a.B = num_seqs;
  a.max_blocks = max_blocks;
  a.Hkv = num_kv_heads;
  a.row_bytes = head_dim * 2;
  a.bs = block_size;
  a.sink = sink;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == 0) {
    a.flat_bytes = kv_bytes / 2 / (kWorkgroups / 2) / 16 * 16 * (kWorkgroups / 2);
    read_contiguous<<<kWorkgroups, 512, 0, s>>>(a);
  } else if (mode == 1) {
    const int hw = num_kv_heads % 4 == 0 ? 4 : num_kv_heads % 2 == 0 ? 2 : 1;
    const int ngr = num_kv_heads / hw;
    a.ranges = kWorkgroups / ngr > 0 ? kWorkgroups / ngr : 1;  // workgroups per head group
    if ((total_blocks + a.ranges * (4 / hw) - 1) / (a.ranges * (4 / hw)) > kMaxRange) return -1;
    const int ni = block_size * a.row_bytes / 1024;  // 16-byte loads per lane per block
    const dim3 grid((unsigned)(ngr * a.ranges));
    switch (ni) {
      case 2: read_head_rows<2><<<grid, 256, 0, s>>>(a, hw); break;
      case 4: read_head_rows<4><<<grid, 256, 0, s>>>(a, hw); break;
      case 8: read_head_rows<8><<<grid, 256, 0, s>>>(a, hw); break;
      default: return -1;
    }
  } else if (mode == 2) {
    a.ranges = kWorkgroups;
    if ((total_blocks + a.ranges - 1) / a.ranges > kMaxRange) return -1;
    const long long blk = (long long)num_kv_heads * a.row_bytes * block_size;
    if (blk % 8192) return -1;
    switch (blk / 8192) {
      case 1: read_token_rows<1><<<kWorkgroups, 512, 0, s>>>(a); break;
      case 2: read_token_rows<2><<<kWorkgroups, 512, 0, s>>>(a); break;
      case 4: read_token_rows<4><<<kWorkgroups, 512, 0, s>>>(a); break;
      case 8: read_token_rows<8><<<kWorkgroups, 512, 0, s>>>(a); break;
      default: return -1;
    }
  } else if (mode == 3) {
    if (kWorkgroups % num_kv_heads) return -1;
    a.ranges = kWorkgroups / num_kv_heads;  // ranges per kv head
    // each wave holds at most 128 of its range's blocks
    if ((total_blocks + a.ranges - 1) / a.ranges > 4 * kMaxRange) return -1;
    const int ni = block_size * a.row_bytes / 1024;
    switch (ni) {
      case 2: read_head_interleaved<2><<<kWorkgroups, 256, 0, s>>>(a); break;
      case 4: read_head_interleaved<4><<<kWorkgroups, 256, 0, s>>>(a); break;
      case 8: read_head_interleaved<8><<<kWorkgroups, 256, 0, s>>>(a); break;
      default: return -1;
    }
  } else {
    return -1;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}

// nwg workgroups of `threads` threads stream per_wg 16-byte vectors each from
// p (which holds nwg * per_wg); u in {1, 2, 4, 8, 16} loads in flight per
// lane; nt: non-temporal loads.  Returns 0, -1 for arguments it does not
// take, or the HIP error of the launch.
extern "C" int rc_stream_probe(const void* p, long long per_wg, int nwg, int threads, int u,
                               int nt, uint32_t* sink, void* stream) {
  if (nwg < 1 || per_wg < 1 || threads < 64 || threads > 1024 || threads % 64) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4* v = static_cast<const uint4*>(p);
  auto go = [&](auto uc, auto ntc) {
    stream_probe<decltype(uc)::value, decltype(ntc)::value><<<nwg, threads, 0, s>>>(v, per_wg, sink);
    return (int)hipGetLastError();
  };
  using F = std::integral_constant<bool, false>;
  using T = std::integral_constant<bool, true>;
  switch (u) {
    case 1: return nt ? go(std::integral_constant<int, 1>{}, T{}) : go(std::integral_constant<int, 1>{}, F{});
    case 2: return nt ? go(std::integral_constant<int, 2>{}, T{}) : go(std::integral_constant<int, 2>{}, F{});
    case 4: return nt ? go(std::integral_constant<int, 4>{}, T{}) : go(std::integral_constant<int, 4>{}, F{});
    case 8: return nt ? go(std::integral_constant<int, 8>{}, T{}) : go(std::integral_constant<int, 8>{}, F{});
    case 16: return nt ? go(std::integral_constant<int, 16>{}, T{}) : go(std::integral_constant<int, 16>{}, F{});
  }
  return -1;
}
