// Paged KV write (reshape_and_cache), block copy (copy-on-write of shared
// blocks) and the dense debug gather, gfx950.
//
// The write is the cache's logical-to-physical write (barellm README,
// paged-cache component list): each new token's K and V rows go to the slot
// the caller assigned, slot = physical_block * block_size + offset.  Because
// the cache is [num_blocks, block_size, kv_heads, head_dim] with token before
// head, one token's rows for all KV heads are one contiguous run of
// kv_heads * head_dim elements at element offset slot * kv_heads * head_dim,
// so the write is a row copy: one lane per 16-byte chunk, 128-bit loads and
// stores, coalesced along the row.
#include "common.hpp"

namespace pa {

__global__ __launch_bounds__(256) void kv_write_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    const int64_t* __restrict__ slot_mapping, int64_t total_chunks,
    int32_t row_chunks, int64_t num_slots) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total_chunks) return;
  const int64_t tok = i / row_chunks;
  const int64_t c = i - tok * row_chunks;
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;
  const uint4 kv = key[i];
  const uint4 vv = value[i];
  k_cache[slot * row_chunks + c] = kv;
  v_cache[slot * row_chunks + c] = vv;
}

// Block dst of both caches becomes a copy of block src, for each (src, dst)
// pair; grid x = pair, grid y = slices of the block.  A block shared by
// several sequences (their tables name the same physical block for a common
// prefix: MinivLLM article, "Running It" section; nano-vllm overview,
// prefix caching in "Kernmodul: Sequence") is copied before one of them
// writes into it.
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    uint4* k_cache, uint4* v_cache, const int64_t* __restrict__ block_pairs,
    int64_t blk_chunks, int64_t num_blocks) {
  const int64_t src = block_pairs[2 * (int64_t)blockIdx.x];
  const int64_t dst = block_pairs[2 * (int64_t)blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t step = (int64_t)gridDim.y * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; c < blk_chunks; c += step) {
    const uint4 kv = k_cache[src * blk_chunks + c];
    const uint4 vv = v_cache[src * blk_chunks + c];
    k_cache[dst * blk_chunks + c] = kv;
    v_cache[dst * blk_chunks + c] = vv;
  }
}

// dense[b, t] = cache[table[b, t / bs], t % bs] for t < ctx_b, zero bytes
// after it, 0xFF bytes where the table names a block outside the pool.
__global__ __launch_bounds__(256) void gather_kernel(
    uint4* __restrict__ k_dense, uint4* __restrict__ v_dense,
    const uint4* __restrict__ k_cache, const uint4* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int64_t total_chunks, int32_t row_chunks, int32_t block_size, int32_t max_blocks,
    int32_t num_blocks) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total_chunks) return;
  const int64_t seq_tokens = (int64_t)max_blocks * block_size;
  const int64_t per_seq = seq_tokens * row_chunks;
  const int64_t b = i / per_seq;
  const int64_t rem = i - b * per_seq;
  const int64_t t = rem / row_chunks;
  const int64_t c = rem - t * row_chunks;
  int64_t ctx = context_lens[b];
  if (ctx > seq_tokens) ctx = seq_tokens;
  uint4 kz = make_uint4(0, 0, 0, 0), vz = kz;
  if (t < ctx) {
    const int32_t blk = block_tables[b * max_blocks + t / block_size];
    if (blk < 0 || blk >= num_blocks) {
      kz = vz = make_uint4(~0u, ~0u, ~0u, ~0u);
    } else {
      const int64_t src = ((int64_t)blk * block_size + t % block_size) * row_chunks + c;
      kz = k_cache[src];
      vz = v_cache[src];
    }
  }
  k_dense[i] = kz;
  v_dense[i] = vz;
}

namespace {

pa_status check_cache_args(int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                           int32_t block_size, pa_dtype dtype) {
  if (!supported_dtype(dtype)) {
    set_error("dtype %d is not PA_DTYPE_F32 or PA_DTYPE_BF16", (int)dtype);
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (num_kv_heads <= 0 || num_blocks <= 0) {
    set_error("num_kv_heads=%d and num_blocks=%d must be positive", num_kv_heads,
              num_blocks);
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (!supported_head_dim(head_dim)) {
    set_error("head_dim=%d; built for 64 and 128", head_dim);
    return PA_ERR_UNSUPPORTED;
  }
  if (!supported_block_size(block_size)) {
    set_error("block_size=%d; built for 16 and 32", block_size);
    return PA_ERR_UNSUPPORTED;
  }
  return PA_OK;
}

unsigned grid_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" pa_status pa_reshape_and_cache(const void* key, const void* value,
                                          void* k_cache, void* v_cache,
                                          const int64_t* slot_mapping,
                                          int32_t num_tokens, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t num_blocks,
                                          int32_t block_size, pa_dtype dtype,
                                          void* stream) {
  clear_error();
  pa_status st = check_cache_args(num_kv_heads, head_dim, num_blocks, block_size, dtype);
  if (st != PA_OK) return st;
  if (num_tokens < 0) {
    set_error("num_tokens=%d is negative", num_tokens);
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) {
    set_error("a tensor pointer is NULL");
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache)) {
    set_error("key, value, k_cache and v_cache must be 16-byte aligned");
    return PA_ERR_INVALID_ARGUMENT;
  }
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * dtype_bytes(dtype);
  const int32_t row_chunks = (int32_t)(row_bytes / 16);
  const int64_t total = (int64_t)num_tokens * row_chunks;
  kv_write_kernel<<<grid_for(total), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(key), static_cast<const uint4*>(value),
      static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), slot_mapping, total,
      row_chunks, (int64_t)num_blocks * block_size);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error("reshape_and_cache launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  return PA_OK;
}

extern "C" pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs,
                                    int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t num_blocks, int32_t block_size, pa_dtype dtype,
                                    void* stream) {
  clear_error();
  pa_status st = check_cache_args(num_kv_heads, head_dim, num_blocks, block_size, dtype);
  if (st != PA_OK) return st;
  if (num_pairs < 0) {
    set_error("num_pairs=%d is negative", num_pairs);
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_pairs) {
    set_error("a tensor pointer is NULL");
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (!aligned16(k_cache) || !aligned16(v_cache)) {
    set_error("k_cache and v_cache must be 16-byte aligned");
    return PA_ERR_INVALID_ARGUMENT;
  }
  const int64_t blk_chunks =
      (int64_t)block_size * num_kv_heads * head_dim * dtype_bytes(dtype) / 16;
  // Enough slices that one block's chunks are one or two passes of 256 lanes.
  const unsigned slices = (unsigned)((blk_chunks + 511) / 512);
  copy_blocks_kernel<<<dim3((unsigned)num_pairs, slices), 256, 0,
                       static_cast<hipStream_t>(stream)>>>(
      static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), block_pairs, blk_chunks,
      num_blocks);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error("copy_blocks launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  return PA_OK;
}

extern "C" pa_status pa_debug_gather_kv(void* k_dense, void* v_dense,
                                        const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t num_blocks, int32_t block_size,
                                        int32_t max_blocks_per_seq, pa_dtype dtype,
                                        void* stream) {
  clear_error();
  pa_status st = check_cache_args(num_kv_heads, head_dim, num_blocks, block_size, dtype);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq <= 0) {
    set_error("num_seqs=%d must be >= 0 and max_blocks_per_seq=%d positive", num_seqs,
              max_blocks_per_seq);
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (num_seqs == 0) return PA_OK;
  if (!k_dense || !v_dense || !k_cache || !v_cache || !block_tables || !context_lens) {
    set_error("a tensor pointer is NULL");
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (!aligned16(k_dense) || !aligned16(v_dense) || !aligned16(k_cache) ||
      !aligned16(v_cache)) {
    set_error("dense and cache tensors must be 16-byte aligned");
    return PA_ERR_INVALID_ARGUMENT;
  }
  const int32_t row_chunks =
      (int32_t)((int64_t)num_kv_heads * head_dim * dtype_bytes(dtype) / 16);
  const int64_t total =
      (int64_t)num_seqs * max_blocks_per_seq * block_size * row_chunks;
  gather_kernel<<<grid_for(total), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<uint4*>(k_dense), static_cast<uint4*>(v_dense),
      static_cast<const uint4*>(k_cache), static_cast<const uint4*>(v_cache),
      block_tables, context_lens, total, row_chunks, block_size, max_blocks_per_seq,
      num_blocks);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error("gather launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  return PA_OK;
}
