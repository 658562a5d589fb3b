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
// of one (sequence, kv head); rows of later tokens see more keys, so the
// grid's row groups are issued last-first.  Per K/V block (the blocks up to
// the workgroup's last row position):
//   * the whole workgroup loads 64 keys' worth of blocks (K and V rows for kv
//     head g) with full-row coalesced 16-byte loads into one of two LDS stages
//     (the next stage's loads are in flight while the current one is used);
//   * every wave folds the block into its rows' online-softmax state
//     (mfma_attn.hpp), each score masked past its row's position; a wave
//     whose rows all end before the block skips it.
// There is no split over key ranges, so no workspace and no merge: each
// wave's state ends complete and is normalised and stored directly.
#include "mfma_attn.hpp"

#include "decode_launch.hpp"

#include <stdlib.h>

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
  int32_t row_groups;  // workgroups per (sequence, kv head) along the query rows
  float scale_log2;
};

constexpr int kPrefillWaves = 8;
constexpr int kPrefillRows = 32;  // query rows per wave
// Keys per LDS stage (several blocks): 64, or 32 at head_dim 64, where the
// workgroup is held to 128 VGPRs so that two fit on a compute unit.
template <int D>
constexpr int prefill_stage_keys() { return D == 64 ? 32 : 64; }

template <int D, int BS, int G, int NW>
__global__ __launch_bounds__(NW * 64, D == 64 ? 4 : 2) void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int NR = kPrefillRows;
  constexpr int KC = 32;  // keys folded per call: two 16-token tiles, so p.v runs on
                          // v_mfma_f32_16x16x32_bf16 whatever the block size
  using Sh = TileShape<D, KC, NR>;
  using T = RowTileAttn<D, KC, NR>;
  constexpr int RL = Sh::RL, PITCH = Sh::PITCH, HT = Sh::HT;
  constexpr int NT = NW * 64;
  constexpr int kChunks = BS * RL;  // 16-byte chunks of one block's rows, K or V
  static_assert(kChunks % 64 == 0, "a wave's chunks are all K or all V");
  constexpr int NCH = (2 * kChunks + NT - 1) / NT;  // chunks per thread per block, K and V
  constexpr int KB = prefill_stage_keys<D>() / BS;              // blocks per stage
  constexpr int SK = prefill_stage_keys<D>() * PITCH;           // one stage's K (or V) rows
  // [stage][K rows | V rows]: the stage's KB blocks are consecutive logical
  // blocks, so row t of a stage is key position (first block) * BS + t.
  __shared__ __attribute__((aligned(16))) char s_kv[2][2 * SK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int b = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int rg = a.row_groups - 1 - (int)blockIdx.y;  // later rows first
  const int qs = a.query_start[b];
  const int nq = a.query_start[b + 1] - qs;
  const int ctx = a.context_lens[b];
  const int nrows = nq * G;
  const int r0 = rg * NW * NR;
  if (r0 >= nrows) return;
  const int r_end = min(nrows, r0 + NW * NR);
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

  const int wr0 = r0 + wave * NR;  // this wave's first row
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  T st;
  st.reset();
  st.load_q(
      [&](int r) -> const uint16_t* {
        const int R = wr0 + r;
        return R < nrows ? q + ((size_t)(qs + R / G) * Hq + (size_t)g * G + R % G) * D
                         : nullptr;
      },
      lane);
  int rowpos[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int R = wr0 + 16 * ht + (lane & 15);
    rowpos[ht] = R < nrows ? first + R / G : -1;
  }
  // Keys this wave's rows reach (0 if it has no rows).
  const int wave_kend = wr0 < nrows ? first + (min(nrows, wr0 + NR) - 1) / G + 1 : 0;

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
  const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks;
  bool bad = false;  // a block id outside the pool: rows become NaN
  uint4 r[KB][NCH];
  auto chunk = [&](int i) { return (tid + i * NT) % (2 * kChunks); };
  // Loads of blocks jb0 .. jb0 + KB - 1 (ids past the last block read the last
  // one again: in range, never folded in).
  auto fetch = [&](int jb0) {
    // Table entries first, all together: a vector load completes in order,
    // so waiting for an entry between K/V loads would wait for those too.
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
        r[kb][i] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(is_k ? rk : rv, off, 0, 0));
      }
    }
  };
  auto stage = [&](int s) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = chunk(i);
        const bool is_k = __builtin_amdgcn_readfirstlane(c) < kChunks;
        const int cc = is_k ? c : c - kChunks;
        *reinterpret_cast<uint4*>(s_kv[s] + (is_k ? 0 : SK) + (kb * BS + cc / RL) * PITCH +
                                  (cc % RL) * 16) = r[kb][i];
      }
  };

  fetch(0);
  stage(0);
  __builtin_amdgcn_s_waitcnt(0);  // q rows and the first blocks are in: nothing pending
  __syncthreads();
  for (int jb0 = 0; jb0 < nblk; jb0 += KB) {
    const int s = (jb0 / KB) & 1;
    // The next stage's loads are in flight while this one is folded in.
    fetch(jb0 + KB < nblk ? jb0 + KB : jb0);
    __builtin_amdgcn_sched_barrier(0);
    // 32 keys at a time; keys past the last block (stage rows loaded from
    // the last block again) sit past every row's position and are masked.
#pragma unroll
    for (int kc = 0; kc < prefill_stage_keys<D>() / KC; ++kc) {
      const int p0 = jb0 * BS + kc * KC;
      if (p0 < nblk * BS && p0 < wave_kend)
        st.consume(s_kv[s] + kc * KC * PITCH, s_kv[s] + SK + kc * KC * PITCH, p0, rowpos,
                   a.scale_log2, lane);
    }
    stage(s ^ 1);
    __syncthreads();
  }

  if (bad) {
    for (int e = lane; e < NR * D; e += 64) {
      const int R = wr0 + e / D;
      if (R < nrows) out[out_at(R, e % D)] = 0x7FC0;
    }
    return;
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
hipError_t launch_prefill_t(const PrefillArgs& a, int num_seqs, hipStream_t stream) {
  dim3 grid(num_seqs * a.num_kv_heads, a.row_groups);
  prefill_mfma_kernel<D, BS, G, kPrefillWaves><<<grid, kPrefillWaves * 64, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefill(int D, int BS, int G, const PrefillArgs& a, int num_seqs,
                          hipStream_t s) {
  auto by_g = [&](auto d, auto bs) -> hipError_t {
    constexpr int Dv = decltype(d)::value, BSv = decltype(bs)::value;
    switch (G) {
      case 1: return launch_prefill_t<Dv, BSv, 1>(a, num_seqs, s);
      case 2: return launch_prefill_t<Dv, BSv, 2>(a, num_seqs, s);
      case 4: return launch_prefill_t<Dv, BSv, 4>(a, num_seqs, s);
      case 8: return launch_prefill_t<Dv, BSv, 8>(a, num_seqs, s);
      case 16: return launch_prefill_t<Dv, BSv, 16>(a, num_seqs, s);
      case 32: return launch_prefill_t<Dv, BSv, 32>(a, num_seqs, s);
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
  const int64_t rows_per_wg = (int64_t)kPrefillWaves * kPrefillRows;
  const int64_t row_groups = ((int64_t)max_query_len * G + rows_per_wg - 1) / rows_per_wg;
  if (row_groups > 65535 || (int64_t)num_seqs * num_kv_heads > 0x7FFFFFFF) {
    set_error("max_query_len=%d too large for one launch", max_query_len);
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
  a.row_groups = (int32_t)row_groups;
  a.scale_log2 = scale * 1.4426950408889634f;
  const hipError_t err = launch_prefill(head_dim, block_size, G, a, num_seqs,
                                        static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    set_error("prefill launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  return PA_OK;
}
