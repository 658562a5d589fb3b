/*
 * libpagedattn -- paged KV-cache write and single-token paged decode attention
 * for AMD Instinct MI355X (gfx950).  Plain C ABI: raw pointers and sizes only.
 *
 * Sources of the operations (web pages this library is written from):
 *   - barellm README (quanhua92/barellm), paged-cache component list: K/V live
 *     in fixed-size physical blocks of one [physical_blocks, block_size,
 *     kv_heads, head_dim] tensor per layer; a per-request block table maps
 *     logical block pos // block_size to a physical block; the cache owns the
 *     logical-to-physical writes.  Feature list: token-before-head (NHD)
 *     layout; one-token batched decode over requests of unequal length; MHA,
 *     GQA and MQA; paged storage must agree with a contiguous cache.
 *   - CUDAlab README, "Paged Attention 调用链": one forward entry point for
 *     paged multi-head attention; Benchmark section: the kv_mul (grouped
 *     heads) and block_size parameters.
 *   - LLAISYS README, implemented-features list: C++ backend behind a C API
 *     called from Python; online softmax with a running max and running sum;
 *     grouped heads by broadcasting; a multi-block reduction finished by the
 *     last block to arrive (fence + atomic counter) instead of a second launch
 *     (the fixed-partition schedule does so; the balanced schedule finishes
 *     in the launch too, by the worker holding a sequence's last block).
 *   - MinivLLM article, "What the Two Benchmark Scripts Compare": paged
 *     decode attention as its own kernel, blockwise online softmax.
 *
 * Conventions for every call:
 *   - All tensors are dense, row-major, in device memory, 16-byte aligned,
 *     and owned by the caller.  The library never allocates, frees or
 *     synchronises; it keeps no state between calls except each host
 *     thread's last error message, the PAGEDATTN_* options it read from the
 *     environment, and the static device buffer of pa_decode_step_noalloc
 *     (the other calls' arrival counters are the caller's, left at zero by
 *     every call).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     runs asynchronously; results are visible after the caller synchronises.
 *   - Arguments are checked before anything is launched.  On failure the call
 *     returns a non-zero pa_status, launches nothing, and
 *     pa_last_error_message() (per host thread) says what was wrong.
 *   - Tensor *contents* are trusted: a block id outside [0, num_blocks) or a
 *     context length outside 0 .. max_blocks_per_seq * block_size is never
 *     dereferenced -- the affected output row is written as NaN instead.
 *   - Floating-point tensors share one storage type (pa_dtype): float32 or
 *     bfloat16 (raw 16-bit patterns).  Accumulation is always float32.
 *   - No C++ exception crosses this interface.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad combination */
  PA_ERR_UNSUPPORTED = 2,        /* valid but not built: head_dim, block_size, group */
  PA_ERR_WORKSPACE_TOO_SMALL = 3,
  PA_ERR_HIP = 4                 /* the HIP runtime refused a launch or query */
} pa_status;

typedef enum pa_dtype {
  PA_DTYPE_F32 = 0,
  PA_DTYPE_BF16 = 1
} pa_dtype;

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t pa_version(void);

/*
 * Static text for a status code; never NULL.  (LLAISYS README, intro and
 * implemented-features list: a C++ backend behind a C API called from
 * Python -- errors cross that interface as status codes and text, never as
 * C++ exceptions.)
 */
const char* pa_status_string(int32_t status);

/* Detail of the last failed call made by this host thread ("" if none);
 * same source as pa_status_string. */
const char* pa_last_error_message(void);

/*
 * Re-read the PAGEDATTN_* environment overrides of the library's own choices
 * (schedule, kernel, merge path, workers; for tests and tuning runs).  They
 * are read once, at the first call that needs them, and again only here; a
 * call running on another thread meanwhile uses one whole set, old or new.
 */
void pa_reload_options(void);

/*
 * Paged KV write (the cache's logical-to-physical write; barellm README,
 * paged-cache component list).
 *
 * For each i < num_tokens with s = slot_mapping[i] and 0 <= s < num_blocks *
 * block_size: copies key[i, :, :] to k_cache[s / block_size, s % block_size,
 * :, :] and value[i, :, :] to v_cache[...] -- an exact copy of the stored
 * bits.  Rows with s < 0 are skipped (padding); rows with s past the pool are
 * skipped too.  Slots that appear twice in one call are written in no
 * particular order.
 *
 *   key, value      [num_tokens, num_kv_heads, head_dim]      (read)
 *   k_cache, v_cache[num_blocks, block_size, num_kv_heads, head_dim] (written)
 *   slot_mapping    [num_tokens] int64                        (read)
 *
 * num_tokens == 0 is a valid no-op.  head_dim in {64, 128}; block_size in
 * {16, 32}.
 */
pa_status pa_reshape_and_cache(const void* key, const void* value,
                               void* k_cache, void* v_cache,
                               const int64_t* slot_mapping,
                               int32_t num_tokens, int32_t num_kv_heads,
                               int32_t head_dim, int32_t num_blocks,
                               int32_t block_size, pa_dtype dtype,
                               void* stream);

/*
 * Paged prefill (and chunked-prefill) attention, causal: the step before
 * decode, where a prompt -- or a chunk of it after a cached prefix -- is
 * processed at once (MinivLLM article, "Engine Layout": prefilling vs
 * decoding; nano-vllm overview, "Prefill vs. Decode").
 *
 * Sequence b brings n_b = query_start[b+1] - query_start[b] new tokens, the
 * last n_b of its L_b = context_lens[b] positions; their K/V rows must
 * already be in the cache (pa_reshape_and_cache).  Row t of q for sequence
 * b (t < n_b) sits at position L_b - n_b + t; for each query head h:
 *
 *   out[query_start[b] + t, h, :] = softmax_j(scale * q[., h, :] . K[j, h/G, :])
 *                                   V[j, h/G, :]   over positions j <= L_b - n_b + t,
 *
 * with G = num_q_heads / num_kv_heads, float32 accumulation, bf16 output
 * (round to nearest even).
 *
 *   out          [num_tokens, num_q_heads, head_dim]   (written)
 *   q            [num_tokens, num_q_heads, head_dim]   (read)
 *   k_cache, v_cache, block_tables, context_lens       as for the decode
 *   query_start  [num_seqs + 1] int32, non-decreasing, query_start[0] = 0,
 *                query_start[num_seqs] = num_tokens     (read)
 *   max_query_len >= every n_b (sizes the launch; rows of a longer sequence
 *                past max_query_len are left unwritten)
 *
 * bfloat16 only (PA_ERR_UNSUPPORTED for float32); head_dim in {64, 128},
 * block_size in {16, 32}, G in {1, 2, 4, 8, 16, 32}.  No workspace.  Rows of
 * a sequence with n_b > L_b, or whose L_b exceeds max_blocks_per_seq *
 * block_size, are NaN; so are rows whose key range names a block outside the
 * pool.  num_seqs, num_tokens or max_query_len of 0 is a no-op.
 * Asynchronous on `stream`.
 */
pa_status pa_paged_attention_prefill(void* out, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens,
                                     const int32_t* query_start, int32_t num_seqs,
                                     int32_t num_tokens, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim,
                                     int32_t num_blocks, int32_t block_size,
                                     int32_t max_blocks_per_seq, int32_t max_query_len,
                                     float scale, pa_dtype dtype, void* stream);

/*
 * Block copy for copy-on-write of shared blocks.  Sequences that share a
 * prompt prefix may name the same physical block in their block tables
 * (block sharing and prefix caching: MinivLLM article, "Running It" section;
 * nano-vllm overview, "Kernmodul: Sequence"); before a sequence writes a new
 * token into a block it shares, the caller gives it a private copy.
 *
 * For each i < num_pairs with src = block_pairs[2i], dst = block_pairs[2i+1],
 * both in [0, num_blocks): block dst of k_cache and of v_cache becomes a
 * bit-exact copy of block src.  Pairs naming a block outside the pool are
 * skipped.  A block that is the destination of two pairs, or the destination
 * of one and the source of another, ends in an unspecified state.
 *
 *   k_cache, v_cache [num_blocks, block_size, num_kv_heads, head_dim] (read/written)
 *   block_pairs      [num_pairs, 2] int64, device memory            (read)
 *
 * num_pairs == 0 is a valid no-op.  Asynchronous on `stream`.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t num_blocks, int32_t block_size, pa_dtype dtype,
                         void* stream);

/*
 * The partition size (tokens) pa_paged_attention_decode will use for these
 * sizes.  Split-K over a sequence's tokens, each partition's softmax state
 * merged by a log-sum-exp reduction, is what the long-context workload
 * states (8 sequences of 32768 tokens, 512-token partitions, cross-partition
 * log-sum-exp reduce); the LLAISYS README (implemented-features list) has
 * the last block to arrive finish such a multi-block reduction.
 *
 * `requested` itself if it is a positive multiple of block_size no larger
 * than 128 * block_size.  For `requested` 0 the library's own choice: 0 when
 * the balanced schedule serves these sizes (num_seqs * num_kv_heads <= 1024
 * with 1 or 2 query heads per kv head, or with 4 at head_dim 64 over tables
 * of at most 4096 tokens: equal ranges of the batch's blocks per worker
 * instead of fixed partitions); otherwise at head_dim 64, 512
 * tokens for 1 or 2 query heads per kv head and 1024 for more; at head_dim
 * 128, 1024 tokens, or 2048 when max_blocks_per_seq * block_size exceeds
 * 4096 -- the fastest measured on MI355X for the decode workloads.  -1 if
 * `requested` is invalid.
 */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_blocks_per_seq, int32_t block_size,
                                 int32_t requested);

/*
 * Bytes of workspace pa_paged_attention_decode needs for these sizes: the
 * split-K partial results that the log-sum-exp merge reads (same sources as
 * pa_decode_partition_size): per piece of a split sequence and query head,
 * head_dim floats of unnormalised output plus the running max and sum.  With
 * fixed partitions, one piece per (sequence, KV head, partition); with the
 * balanced schedule, two per (KV head, worker range).  0 when no sequence
 * can span more than one piece, and 0 on invalid sizes.  The workspace must
 * be all zero before its first use (like the counters); every call leaves
 * what it used at zero again, so one workspace serves any later call (any
 * sizes) on the same stream.  Two calls that may run at the same time must
 * not share a workspace.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_blocks_per_seq, int32_t block_size,
                                 int32_t partition_size);

/*
 * Single-token decode attention over a paged KV cache (barellm README,
 * feature list: one-token batched decode with unequal lengths; paged-cache
 * list: position -> block table -> physical block).
 *
 * For each sequence b < num_seqs with L = context_lens[b] (the cached tokens,
 * including the one written this step) and each query head h < num_q_heads,
 * with g = h / (num_q_heads / num_kv_heads):
 *     row t < L is  k_cache[block_tables[b, t / block_size], t % block_size, g, :]
 *     s_t        =  scale * dot(q[b, h, :], k_t)
 *     out[b,h,:] =  sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s)
 * in float32 arithmetic, rounded once to the storage type (round to nearest
 * even).  L == 0 writes a zero row.  Table entries at or past
 * ceil(L / block_size) may be loaded but are never dereferenced: their
 * values are not used.
 *
 * Sequences longer than one partition are split into partitions of
 * `partition_size` tokens (0 = library choice, see
 * pa_decode_partition_size); each partition's softmax state (max, sum,
 * unnormalised output) goes to the workspace and the partitions are merged
 * with a log-sum-exp reduction.  With fewer than 16 partitions per sequence
 * the last partition of that (sequence, KV head) to finish -- found with an
 * atomic arrival counter -- merges them in the same launch; with 16 or more
 * a second kernel, launched on the same stream, merges every split sequence
 * (one long serial merge at the end of the first launch costs more than the
 * launch).  Under the balanced schedule (partition size 0 from
 * pa_decode_partition_size) each KV head's blocks, sequence after sequence,
 * are cut into equal ranges, one per worker; a sequence cut by a range
 * boundary is merged in the same launch by the worker holding its last
 * block, which waits for the other pieces' states to land (they belong to
 * workgroups dispatched no later than its own; the wait is bounded, so it
 * cannot hang); that schedule uses no arrival counters.  Results do not
 * depend on the order in which partitions finish (bit-identical reruns).
 *
 *   out            [num_seqs, num_q_heads, head_dim]                   (written)
 *   q              [num_seqs, num_q_heads, head_dim]                   (read)
 *   k_cache, v_cache [num_blocks, block_size, num_kv_heads, head_dim]  (read)
 *   block_tables   [num_seqs, max_blocks_per_seq] int32                (read)
 *   context_lens   [num_seqs] int32                                    (read)
 *   workspace      >= pa_decode_workspace_bytes(...) bytes, 256-byte
 *                  aligned, all zero before the first call; every call
 *                  leaves it all zero again (NULL allowed if that size is 0)
 *   counters       >= num_seqs * num_kv_heads int32 arrival counters; all
 *                  zero before the first call; every call leaves the
 *                  counters it used at zero again, so one counter array can
 *                  serve any later call (any sizes) on the same stream
 *                  (NULL allowed if the workspace size is 0)
 *
 * head_dim in {64, 128}; block_size in {16, 32}; num_q_heads a multiple of
 * num_kv_heads with a group of 1, 2, 4, 8, 16 or 32 query heads per KV head.
 */
pa_status pa_paged_attention_decode(void* out, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables,
                                    const int32_t* context_lens,
                                    int32_t num_seqs, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim,
                                    int32_t num_blocks, int32_t block_size,
                                    int32_t max_blocks_per_seq, float scale,
                                    int32_t partition_size,
                                    void* workspace, size_t workspace_bytes,
                                    int32_t* counters, int64_t num_counters,
                                    pa_dtype dtype, void* stream);

/*
 * One decode step in one launch: the KV write of every sequence's new token
 * (the write of the barellm README's paged-cache list: logical position ->
 * block table -> physical slot) fused into the decode above.  In a decode
 * step the new token of sequence b is the last of its L = context_lens[b]
 * positions, so its rows go to
 *     k_cache[block_tables[b, (L-1) / block_size], (L-1) % block_size, :, :] = key[b]
 * and the same for V -- exactly what pa_reshape_and_cache does with that
 * slot -- and the decode attends them as position L-1.  Out and caches are bit-identical
 * to pa_reshape_and_cache (slot_mapping[b] = that slot) followed by
 * pa_paged_attention_decode with the same arguments; this saves the write's
 * launch.  Sequences with L == 0 or L past the table write nothing, nor does
 * one whose slot names a block outside the pool.  The block that receives a
 * sequence's new token must not be read by another sequence of the same call
 * (a shared block is copied first: pa_copy_blocks).
 *
 *   key, value   [num_seqs, num_kv_heads, head_dim], 16-byte aligned (read)
 *   k_cache, v_cache                                     (read and written)
 *   every other argument as for pa_paged_attention_decode.
 */
pa_status pa_decode_step(void* out, const void* q, const void* key, const void* value,
                         void* k_cache, void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t num_blocks, int32_t block_size,
                         int32_t max_blocks_per_seq, float scale, int32_t partition_size,
                         void* workspace, size_t workspace_bytes, int32_t* counters,
                         int64_t num_counters, pa_dtype dtype, void* stream);

/*
 * pa_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc): the
 * same kernels, the same results bit for bit, with the split-K workspace and
 * the arrival counters taken from a buffer the library keeps in static
 * device memory -- 65536 counters and 16 MiB of workspace per GPU, held
 * until the process ends.  Sizes that need more (num_seqs * num_kv_heads
 * above 65536, or pa_decode_workspace_bytes(...) above 16 MiB) return
 * PA_ERR_WORKSPACE_TOO_SMALL before anything is launched.  Nothing is
 * allocated: the caller passes every input and `out`.
 *
 * The device of `stream` must be current.  The first call on a device finds
 * that device's buffer and clears it with a kernel on `stream`; it
 * must not be made under graph capture (PA_ERR_INVALID_ARGUMENT).  Every call
 * on one GPU shares that GPU's buffer, which keeps the last call's contents:
 * calls that may overlap on one GPU (other streams, other host threads) race
 * and must be serialised by the caller.
 *
 * Arguments as for pa_decode_step, without workspace and counters.
 */
pa_status pa_decode_step_noalloc(void* out, const void* q, const void* key,
                                 const void* value, void* k_cache, void* v_cache,
                                 const int32_t* block_tables,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t num_blocks,
                                 int32_t block_size, int32_t max_blocks_per_seq,
                                 float scale, int32_t partition_size, pa_dtype dtype,
                                 void* stream);

/*
 * Test and debugging aid: the exact gather a dense-attention engine would do
 * (barellm README, feature list: pages gathered into dense tensors).
 *
 * k_dense[b, t] = k_cache[block_tables[b, t / block_size], t % block_size]
 * for t < context_lens[b], all-zero bytes for t >= context_lens[b]; the same
 * for V.  Rows whose block id is outside [0, num_blocks) are filled with 0xFF
 * bytes (NaN in both storage types).
 *
 *   k_dense, v_dense [num_seqs, max_blocks_per_seq * block_size,
 *                     num_kv_heads, head_dim]                          (written)
 */
pa_status pa_debug_gather_kv(void* k_dense, void* v_dense,
                             const void* k_cache, const void* v_cache,
                             const int32_t* block_tables,
                             const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_kv_heads,
                             int32_t head_dim, int32_t num_blocks,
                             int32_t block_size, int32_t max_blocks_per_seq,
                             pa_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
