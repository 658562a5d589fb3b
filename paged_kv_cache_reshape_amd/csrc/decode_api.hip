// C ABI of the decode: argument checks, the choice of schedule, workspace
// layout and the launch.
//
// Two schedules compute the same function (the kernels' headers describe
// them):
//   * balanced ("stream-K"): equal shares of the batch's (sequence, kv-head
//     group, block) units for a grid that fills the GPU -- used when the
//     caller leaves the partition size to the library (partition_size 0);
//   * fixed partitions: partition_size tokens per workgroup -- used when the
//     caller names a partition size, and for batches too large for the
//     balanced kernel's per-sequence table in LDS.
#include "decode_launch.hpp"

#include <stdlib.h>

namespace pa {
namespace {

bool group_supported(int g) {
  return g == 1 || g == 2 || g == 4 || g == 8 || g == 16 || g == 32;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Consecutive kv heads one workgroup takes: up to 4, so that the workgroup's
// waves read neighbouring rows of each token (one contiguous run of
// hpw * head_dim elements) together; fewer when large query-head groups
// already need the waves.
int heads_per_workgroup(int Hkv, int G) {
  const int hs = G > 8 ? G / 8 : 1;
  if (const char* env = getenv("PAGEDATTN_HEADS_PER_WG")) {
    const int v = atoi(env);
    if ((v == 1 || v == 2 || v == 4) && Hkv % v == 0 && v * hs <= kDecodeWaves) return v;
  }
  for (int h = 4; h > 1; h /= 2)
    if (Hkv % h == 0 && h * hs <= kDecodeWaves) return h;
  return 1;
}

// Compute units of the current device (cached); 256 (MI355X) if unknown.
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Workgroups of the balanced schedule: every compute unit filled to its
// resident limit (an environment override exists for tuning).
int streamk_grid(int dtype, int D, int BS, int G) {
  int per_cu = 0;
  if (const char* env = getenv("PAGEDATTN_WGS_PER_CU")) per_cu = atoi(env);
  if (per_cu <= 0) per_cu = streamk_wgs_per_cu(dtype, D, BS, G);
  if (per_cu <= 0) per_cu = 4;
  return device_cus() * per_cu;
}

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

struct Plan {
  bool streamk;
  int part_blocks;  // fixed partitions
  int max_parts;
  int num_wg;       // balanced
  int hpw;
  size_t acc_bytes, ml_bytes, total;
};

// The schedule and workspace for these sizes; false if `requested` is invalid.
bool make_plan(int dtype, int B, int Hq, int Hkv, int D, int max_blocks, int bs,
               int requested, Plan* p) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || max_blocks <= 0) return false;
  if (!supported_head_dim(D) || !supported_block_size(bs)) return false;
  const int G = Hq / Hkv;
  if (!group_supported(G)) return false;
  p->hpw = heads_per_workgroup(Hkv, G);
  p->acc_bytes = p->ml_bytes = p->total = 0;
  p->num_wg = 0;
  p->part_blocks = 0;
  p->max_parts = 0;
  if (requested == 0 && B <= kStreamKMaxSeqs) {
    p->streamk = true;
    if (B == 0) return true;
    p->num_wg = streamk_grid(dtype, D, bs, G);
    const size_t rows = (size_t)p->num_wg * 2 * p->hpw * G;
    p->acc_bytes = align256(rows * D * sizeof(float));
    p->ml_bytes = align256(rows * 2 * sizeof(float));
    p->total = p->acc_bytes + p->ml_bytes;
    return true;
  }
  p->streamk = false;
  int pb;
  if (requested == 0) {
    pb = auto_part_blocks(B, Hkv, max_blocks);
  } else {
    if (requested < 0 || requested % bs != 0) return false;
    pb = requested / bs;
    if (pb < 1 || pb > kMaxPartitionBlocks) return false;
  }
  p->part_blocks = pb;
  p->max_parts = (max_blocks + pb - 1) / pb;
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
  if (!make_plan(PA_DTYPE_BF16, num_seqs, num_q_heads, num_kv_heads, head_dim,
                 max_blocks_per_seq, block_size, requested, &p))
    return -1;
  return p.streamk ? 0 : p.part_blocks * block_size;
}

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t max_blocks_per_seq,
                                           int32_t block_size,
                                           int32_t partition_size) {
  // The balanced schedule's grid depends on the storage type's occupancy and
  // this call does not name the type: size for the larger of the two.
  Plan p16, p32;
  if (!make_plan(PA_DTYPE_BF16, num_seqs, num_q_heads, num_kv_heads, head_dim,
                 max_blocks_per_seq, block_size, partition_size, &p16) ||
      !make_plan(PA_DTYPE_F32, num_seqs, num_q_heads, num_kv_heads, head_dim,
                 max_blocks_per_seq, block_size, partition_size, &p32))
    return 0;
  return p16.total > p32.total ? p16.total : p32.total;
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
  if (!make_plan(dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                 block_size, partition_size, &plan)) {
    set_error("partition_size=%d must be 0 or a multiple of block_size=%d "
              "between 1 and 64 blocks", partition_size, block_size);
    return PA_ERR_INVALID_ARGUMENT;
  }
  if (!plan.streamk && plan.max_parts > 65535) {
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
  a.heads_per_wg = plan.hpw;
  a.scale_log2 = scale * 1.4426950408889634f;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err =
      plan.streamk
          ? launch_streamk(dtype, head_dim, block_size, G, a, plan.num_wg, s)
          : launch_partition(dtype, head_dim, block_size, G, a, s);
  if (err != hipSuccess) {
    set_error("decode launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  return PA_OK;
}
