// C ABI of the decode: argument checks, the choice of kernel and schedule,
// workspace layout and the launch.
//
// The decode runs as fixed partitions: one workgroup per (kv-head group,
// sequence, partition of partition_size tokens).  Two kernels share that
// schedule, its workspace and its results: the matrix-core one
// (decode_mfma.hip) for bfloat16 with 4, 8, 16 or 32 query heads per kv head,
// the vector-ALU one (decode_partition.hip) for everything else.  When the
// caller leaves the partition size to the library it picks, by shape, the
// partition length and the kv heads per workgroup that measured fastest on
// MI355X for the decode workloads (see auto_partition_tokens).
#include "decode_launch.hpp"

#include <stdlib.h>
#include <string.h>

namespace pa {
namespace {

bool group_supported(int g) {
  return g == 1 || g == 2 || g == 4 || g == 8 || g == 16 || g == 32;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Consecutive kv heads one workgroup takes: its waves then read neighbouring
// rows of each token (one contiguous run of hpw * head_dim elements) together.
//
// Measured: two heads per workgroup at head_dim 128, one at head_dim 64 (whose
// 128-byte rows already fill a load with eight tokens).  PAGEDATTN_HEADS_PER_WG
// overrides the choice (1, 2 or 4) for experiments.
int heads_per_workgroup(int Hkv, int G, int D) {
  const int hs = G > 8 ? G / 8 : 1;
  if (const char* env = getenv("PAGEDATTN_HEADS_PER_WG")) {
    const int v = atoi(env);
    if ((v == 1 || v == 2 || v == 4) && Hkv % v == 0 && v * hs <= kDecodeWaves) return v;
  }
  if (D == 128 && Hkv % 2 == 0 && 2 * hs <= kDecodeWaves) return 2;
  return 1;
}

// Library choice of partition length, from the head size, the query group
// and the longest context the block table can describe.  Measured on MI355X
// over the decode workloads (Qwen3-, Llama-3.2-shaped, long-context,
// large-batch MHA/MQA): long partitions win -- a compute unit streams at most
// about 40 GB/s, so what counts is that the longest partitions are few and
// large ones carry no merge -- with tables of more than 4096 tokens taking
// 2048 (the 32K-token batch: 191 us at 2048, 200 us at 1024).  At head_dim 64
// the vector kernel (G <= 2) does better with 512 tokens; groups of 4 or
// more, on the matrix cores for bfloat16, take 1024 (Llama-3.2-shaped batch
// 61.0 against 61.3 us, 32-token blocks 66.4 against 73.3 us).
int auto_partition_tokens(int D, int G, int max_tokens) {
  if (D != 128) return G >= 4 ? 1024 : 512;
  return max_tokens > 4096 ? 2048 : 1024;
}

// The matrix-core kernel where it applies, except for groups of 4 over block
// tables of more than 4096 tokens.  There every compute unit streams whole
// partitions for the whole launch, and the vector kernel's two kv heads per
// workgroup move more bytes per compute unit.  Measured on MI355X, the
// 32K-token batch (G = 4) took 167 / 174 / 189 us on the vector kernel
// against 177 / 181 / 194 us on the matrix cores at 2048 / 1024 / 512-token
// partitions.  Over shorter, ragged tables the matrix cores win by 7-13% at
// G = 4 (Llama-3.2-shaped batch 61.7 against 66.1 us).
// PAGEDATTN_DECODE_KERNEL=valu forces the vector-ALU kernel (tests compare
// the two).
bool use_mfma(int dtype, int D, int bs, int G, int64_t span_tokens) {
  if (!mfma_supported(dtype, D, bs, G)) return false;
  if (G == 4 && span_tokens > 4096) return false;
  const char* env = getenv("PAGEDATTN_DECODE_KERNEL");
  return !(env && strcmp(env, "valu") == 0);
}

// PAGEDATTN_MERGE=separate / inkernel forces where split sequences are
// merged (the tests run both paths).
bool deferred_merge(int max_parts) {
  const char* env = getenv("PAGEDATTN_MERGE");
  if (env && strcmp(env, "separate") == 0) return true;
  if (env && strcmp(env, "inkernel") == 0) return false;
  return max_parts >= 16;
}

struct Plan {
  int part_blocks;
  int max_parts;
  int hpw;
  size_t acc_bytes, ml_bytes, total;
};

// The partitioning and workspace for these sizes; false if invalid.
bool make_plan(int B, int Hq, int Hkv, int D, int max_blocks, int bs, int requested,
               Plan* p) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || max_blocks <= 0) return false;
  if (!supported_head_dim(D) || !supported_block_size(bs)) return false;
  const int G = Hq / Hkv;
  if (!group_supported(G)) return false;
  p->hpw = heads_per_workgroup(Hkv, G, D);
  const int tokens = requested == 0 ? auto_partition_tokens(D, G, max_blocks * bs) : requested;
  if (tokens < 0 || tokens % bs != 0) return false;
  const int pb = tokens / bs;
  if (pb < 1 || pb > kMaxPartitionBlocks) return false;
  p->part_blocks = pb;
  p->max_parts = (max_blocks + pb - 1) / pb;
  p->acc_bytes = p->ml_bytes = p->total = 0;
  if (p->max_parts <= 1 || B == 0) return true;
  const size_t rows = (size_t)B * Hkv * p->max_parts * G;
  p->acc_bytes = align256(rows * D * sizeof(float));
  p->ml_bytes = align256(rows * 2 * sizeof(float));
  p->total = p->acc_bytes + p->ml_bytes;
  return true;
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_blocks_per_seq,
                                            int32_t block_size, int32_t requested) {
  Plan p;
  if (!make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                 block_size, requested, &p))
    return -1;
  return p.part_blocks * block_size;
}

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t max_blocks_per_seq,
                                           int32_t block_size,
                                           int32_t partition_size) {
  Plan p;
  if (!make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                 block_size, partition_size, &p))
    return 0;
  return p.total;
}

namespace {

// Both decode entry points: with `step`, the step's token rows key / value
// are written into the caches by the decode launch itself.
pa_status decode_impl(void* out, const void* q, bool step, const void* key, const void* value,
                      const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                      int32_t block_size, int32_t max_blocks_per_seq, float scale,
                      int32_t partition_size, void* workspace, size_t workspace_bytes,
                      int32_t* counters, int64_t num_counters, pa_dtype dtype, void* stream) {
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
  if ((int64_t)num_seqs * num_kv_heads > 0x7FFFFFFF ||
      (int64_t)num_seqs * num_q_heads * head_dim > 0x7FFFFFFFFFFFLL) {
    set_error("num_seqs * num_kv_heads must fit in int32");
    return PA_ERR_UNSUPPORTED;
  }
  if ((int64_t)max_blocks_per_seq * block_size > 0x7FFFFFFF) {
    set_error("max_blocks_per_seq * block_size overflows int32");
    return PA_ERR_INVALID_ARGUMENT;
  }
  Plan plan;
  if (!make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                 block_size, partition_size, &plan)) {
    set_error("partition_size=%d must be 0 or a multiple of block_size=%d "
              "between 1 and 128 blocks", partition_size, block_size);
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (plan.max_parts > 65535) {
    set_error("%d partitions per sequence (max 65535): raise partition_size",
              plan.max_parts);
    return PA_ERR_UNSUPPORTED;
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
  if (step && (!key || !value || !aligned16(key) || !aligned16(value))) {
    set_error("key and value must be non-NULL and 16-byte aligned");
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (plan.total > 0) {
    if (workspace_bytes < plan.total) {
      set_error("workspace holds %zu bytes, needs %zu", workspace_bytes, plan.total);
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
  a.ws_acc = plan.total ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_ml = plan.total ? reinterpret_cast<float*>(ws + plan.acc_bytes) : nullptr;
  a.counters = plan.total ? counters : nullptr;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.part_blocks = plan.part_blocks;
  a.max_parts = plan.max_parts;
  const bool mfma = use_mfma(dtype, head_dim, block_size, G,
                              (int64_t)max_blocks_per_seq * block_size);
  // The matrix-core kernel serves one kv head per workgroup (its eight waves
  // split the blocks).
  a.heads_per_wg = mfma ? 1 : plan.hpw;
  a.deferred_merge = plan.max_parts > 1 && deferred_merge(plan.max_parts);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.new_k = step ? key : nullptr;
  a.new_v = step ? value : nullptr;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err = mfma ? launch_mfma(head_dim, block_size, G, a, s)
                             : launch_partition(dtype, head_dim, block_size, G, a, s);
  if (err != hipSuccess) {
    set_error("decode launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  if (a.deferred_merge) {
    const hipError_t merr = launch_merge(dtype, head_dim, block_size, G, a, s);
    if (merr != hipSuccess) {
      set_error("merge launch failed: %s", hipGetErrorString(merr));
      return PA_ERR_HIP;
    }
  }
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_paged_attention_decode(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
    int32_t block_size, int32_t max_blocks_per_seq, float scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t* counters,
    int64_t num_counters, pa_dtype dtype, void* stream) {
  return decode_impl(out, q, false, nullptr, nullptr, k_cache, v_cache, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks,
                     block_size, max_blocks_per_seq, scale, partition_size, workspace,
                     workspace_bytes, counters, num_counters, dtype, stream);
}

extern "C" pa_status pa_decode_step(
    void* out, const void* q, const void* key, const void* value, void* k_cache,
    void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq, float scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t* counters,
    int64_t num_counters, pa_dtype dtype, void* stream) {
  return decode_impl(out, q, true, key, value, k_cache, v_cache, block_tables, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                     max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes,
                     counters, num_counters, dtype, stream);
}
