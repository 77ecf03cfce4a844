/*
 * pa.h -- libpa: paged-KV-cache decode attention for AMD Instinct MI355X
 * (gfx950), behind a plain C ABI.
 *
 * The method (pages cited by title and section):
 *  - the KV cache is cut into fixed-size physical blocks and each sequence
 *    reaches its tokens through a logical->physical block table; K and V live
 *    in pools laid out [num_blocks][block_size][num_heads][head_dim]
 *    ("LLM推理优化：vLLM PagedAttention深度解析与工程实践", §3.1 Block Table
 *    and §4.1 注意力计算的修改; here num_heads is the number of KV heads);
 *  - every decode step writes the new token's K/V into its slot and then the
 *    new token's query attends over all cached tokens, softmax(q K^T s) V
 *    (same page, §二; "vLLM 深度拆解：当大模型推理学会「分页注意力」",
 *    §2.1, §3.1 and §3.3);
 *  - a single-pass kernel for short contexts and a split-context kernel that
 *    accumulates partial results per partition and merges them afterwards
 *    (first page, §4.1: paged_attention_v1 / v2);
 *  - query heads share KV heads in contiguous groups of G = Hq / Hkv
 *    ("LLM推理优化技术地图：从KV Cache到量化与投机解码", §2.3 GQA);
 *  - a host-side block manager: a free pool, per-sequence block tables,
 *    blocks shared by reference with reference counts, copy-on-write
 *    (first page, §3.2; second page, §3.3 BlockSpaceManager).
 *
 * Conventions for every call below:
 *  - Device entry points take DEVICE pointers owned by the caller, enqueue
 *    their kernels on `stream` (NULL = the null stream) and return without
 *    synchronising.  libpa never allocates or frees device memory.
 *  - Arguments are checked on the host before anything is enqueued; a bad
 *    argument returns PA_ERR_INVALID_ARG (or PA_ERR_UNSUPPORTED for a valid
 *    but unimplemented shape) and enqueues nothing.  Device-resident values
 *    (slots, block ids, context lengths) cannot be checked on the host; the
 *    kernels clamp or skip out-of-range values so that no access leaves the
 *    caller's buffers, and the results for such inputs are unspecified.
 *  - A failure reported by the HIP runtime at launch returns PA_ERR_HIP.
 *  - pa_last_error() returns a message for the last non-OK status on the
 *    calling thread.
 *  - 16-bit float data (fp16 or bf16) is passed as raw 16-bit patterns; all
 *    device buffers must be 16-byte aligned and densely packed in the stated
 *    layout (row-major, innermost index last).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,
  PA_ERR_OOM = 2,
  PA_ERR_UNSUPPORTED = 3,
  PA_ERR_HIP = 4
} pa_status;

typedef enum pa_dtype { PA_F16 = 0, PA_BF16 = 1 } pa_dtype;

/* Message for the last non-OK status returned on this thread ("" if none).
 * The string stays valid until the next libpa call on the same thread. */
const char* pa_last_error(void);

/* Library version string. */
const char* pa_version(void);

/* ------------------------------------------------------------------------
 * Cache write (the new tokens' K/V into their slots).
 * Follows: the new token's K/V are written back into the KV cache after
 * each step ("vLLM 深度拆解：当大模型推理学会「分页注意力」", §3.1 data flow,
 * and §3.3 append_slot: into the current block, or a fresh one when full).
 *
 *   key, value        [num_tokens][num_kv_heads][head_dim]   16-bit
 *   key_cache,
 *   value_cache       [num_blocks][block_size][num_kv_heads][head_dim]
 *   slot_mapping      [num_tokens] int64; slot = block * block_size + offset.
 *                     A negative slot means "write nothing for this token".
 *
 * Token t's K row and V row are copied bit for bit to
 * cache[slot / block_size][slot % block_size][*][*].  Slots >= num_blocks *
 * block_size are skipped on the device.  The same slot twice in one call is
 * undefined (the allocator never produces it).  head_dim in {64, 128}; any
 * positive block_size and num_kv_heads.  num_tokens == 0 is a no-op.
 * ---------------------------------------------------------------------- */
pa_status pa_reshape_and_cache(const void* key, const void* value,
                               void* key_cache, void* value_cache,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks,
                               pa_dtype dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Single-pass paged decode ("v1": the whole context of a sequence in one
 * workgroup; meant for short contexts).
 * Follows: softmax(Q K^T / sqrt(d)) V over the paged cache
 * ("LLM推理优化：vLLM PagedAttention深度解析与工程实践", §二 formula and §4.1
 * paged_attention_v1), for one query token per sequence.
 *
 *   out               [num_seqs][num_q_heads][head_dim]   16-bit (written)
 *   query             [num_seqs][num_q_heads][head_dim]   16-bit
 *   key_cache,
 *   value_cache       [num_blocks][block_size][num_kv_heads][head_dim]
 *   block_tables      [num_seqs][max_blocks_per_seq] int32 physical block ids
 *   context_lens      [num_seqs] int32: tokens in the cache for each sequence,
 *                     the new token included (it sits at position L-1)
 *   max_context_len   an upper bound of every context_lens[i]
 *                     (<= max_blocks_per_seq * block_size)
 *   scale             multiplies q.k before the softmax (usually 1/sqrt(D))
 *
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * out[i][h] = sum_j softmax_j(scale * q[i][h] . K_i[j]) V_i[j] over the
 * context_lens[i] tokens of sequence i, gathered in logical order through
 * block_tables[i]; computed in fp32 and rounded to nearest even at the end.
 * A sequence with context_lens[i] == 0 gets an all-zero output row.
 * Supported: head_dim in {64, 128}; block_size in {16, 32};
 * num_q_heads % num_kv_heads == 0.
 *   start_event,
 *   stop_event        NULL, or events (created with timing) that the launch
 *                     records itself when the decode starts and ends
 *                     (hipExtLaunchKernel): times the decode without a
 *                     marker in the stream.  With nothing to launch they are
 *                     recorded at the call.
 * ---------------------------------------------------------------------- */
pa_status pa_decode(void* out, const void* query, const void* key_cache,
                    const void* value_cache, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t num_blocks,
                    int32_t max_context_len, float scale, pa_dtype dtype,
                    hipStream_t stream,
                    hipEvent_t start_event, hipEvent_t stop_event);

/* Bytes of device workspace pa_decode_partitioned needs: per (sequence,
 * q head, partition) an fp32 accumulator [head_dim], a max and a sum, for
 * ceil(max_context_len / partition_size) partitions.  Returns 0 for invalid
 * sizes. */
size_t pa_decode_partitioned_workspace_size(int32_t num_seqs,
                                            int32_t num_q_heads,
                                            int32_t head_dim,
                                            int32_t max_context_len,
                                            int32_t partition_size);

/* ------------------------------------------------------------------------
 * Split-context paged decode ("v2": partial accumulation per partition,
 * then a merge; first page, §4.1 paged_attention_v2).
 * Arguments as pa_decode, plus:
 *   partition_size    tokens per partition; a multiple of block_size,
 *                     at most 1024.  Partition p of sequence i covers tokens
 *                     [p*P, min(L_i, (p+1)*P)).
 *   work_items        NULL, or a device array [num_work_items][2] int32 of
 *                     (sequence, partition) pairs naming every partition to
 *                     compute: each p < ceil(context_lens[i] / P) of every
 *                     sequence exactly once, in any order.  A caller that
 *                     knows the context lengths on the host (a scheduler
 *                     does) passes it so that only live partitions are
 *                     launched; with NULL the kernel covers all
 *                     ceil(max_context_len / P) partitions of every sequence
 *                     and the ones past a sequence's end exit at once.
 *                     Pairs out of range are skipped; a missing or repeated
 *                     pair gives unspecified output for that sequence.  A
 *                     non-NULL list with num_work_items = 0 (and
 *                     num_seqs > 0) is rejected with PA_ERR_INVALID_ARG:
 *                     pass NULL for the full grid.
 *   workspace         device buffer of at least
 *                     pa_decode_partitioned_workspace_size(...) bytes,
 *                     16-byte aligned; its contents on entry do not matter.
 * Each partition computes, per q head, m = max of its logits,
 * l = sum exp(logit - m) and acc = sum exp(logit - m) V; a second kernel
 * merges: out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p with
 * M = max_p m_p.  Result as pa_decode up to fp32 rounding order.
 * num_q_heads * head_dim must stay below 2^23 (PA_ERR_UNSUPPORTED beyond).
 * A context_lens[i] above max_context_len breaks the caller's side of the
 * contract: only its first ceil(max_context_len / P) partitions are read
 * (every access still stays inside the caller's buffers).
 * start_event / stop_event as for pa_decode: recorded when the first kernel
 * starts and the merge ends.
 * ---------------------------------------------------------------------- */
pa_status pa_decode_partitioned(void* out, const void* query,
                                const void* key_cache, const void* value_cache,
                                const int32_t* block_tables,
                                int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, int32_t max_context_len,
                                float scale, pa_dtype dtype,
                                int32_t partition_size,
                                const int32_t* work_items,
                                int32_t num_work_items, void* workspace,
                                size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t start_event, hipEvent_t stop_event);

/* ------------------------------------------------------------------------
 * pa_decode_partitioned without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It computes exactly what
 * pa_decode_partitioned computes, with the same kernels; the split
 * workspace is a file-scope device array inside libpa of
 * pa_decode_partitioned_noalloc_max_workspace() bytes (64 MiB), one copy per
 * GPU, created when libpa's code is loaded on that GPU and held until the
 * process ends.  The call allocates nothing (no hipMalloc, no hipFree).
 *   Arguments as pa_decode_partitioned, without workspace / workspace_bytes.
 *   A call whose workspace (pa_decode_partitioned_workspace_size of the same
 *   sizes) exceeds the array is rejected with PA_ERR_INVALID_ARG before
 *   anything is enqueued.
 *   The array of the CURRENT device is used; a non-NULL stream must belong
 *   to it (PA_ERR_INVALID_ARG otherwise).  The first call on a device looks
 *   the array's address up (hipGetSymbolAddress, with that device current);
 *   a failure there returns PA_ERR_HIP.
 * Every call on one GPU shares that GPU's array and leaves its partials in
 * it: calls that overlap on one GPU (other streams, other threads) race and
 * give unspecified outputs; calls ordered on one stream are safe.  Nothing
 * in the array needs to start at zero (the merge reads only partials the
 * same call wrote).
 * ---------------------------------------------------------------------- */
size_t pa_decode_partitioned_noalloc_max_workspace(void);

pa_status pa_decode_partitioned_noalloc(void* out, const void* query,
                                        const void* key_cache,
                                        const void* value_cache,
                                        const int32_t* block_tables,
                                        int32_t max_blocks_per_seq,
                                        const int32_t* context_lens,
                                        int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t num_blocks,
                                        int32_t max_context_len, float scale,
                                        pa_dtype dtype, int32_t partition_size,
                                        const int32_t* work_items,
                                        int32_t num_work_items,
                                        hipStream_t stream,
                                        hipEvent_t start_event,
                                        hipEvent_t stop_event);

/* ------------------------------------------------------------------------
 * Decode-step update of device-resident block tables.
 * Follows: append_slot puts the new token into the sequence's current block
 * or a fresh one ("vLLM 深度拆解：当大模型推理学会「分页注意力」", §3.3), and
 * the block table maps each logical block to its physical block
 * ("LLM推理优化：vLLM PagedAttention深度解析与工程实践", §3.1).  After one
 * append per sequence, the only entry that can differ from the previous
 * table is the one holding the new token, at position L-1:
 *   block_tables[i][(context_lens[i] - 1) / block_size] = slot_mapping[i] / block_size
 * (a fresh block, a copy-on-write replacement, or the unchanged block).
 *   block_tables      [num_seqs][max_blocks_per_seq] int32, updated in place
 *   context_lens      [num_seqs] int32, the new token included
 *   slot_mapping      [num_seqs] int64, the new token's slot (< 0: skip)
 * Entries whose slot is outside [0, num_blocks * block_size), whose length
 * is <= 0 or whose index reaches max_blocks_per_seq are skipped on the
 * device.  Lets a caller keep tables on the GPU and send only 12 bytes per
 * sequence per step.
 * ---------------------------------------------------------------------- */
pa_status pa_update_block_tables(int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens,
                                 const int64_t* slot_mapping, int32_t num_seqs,
                                 int32_t block_size, int32_t num_blocks,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * One decode step's writes in one launch: the same results as copying the
 * step's staged metadata to the device, then pa_update_block_tables, then
 * pa_reshape_and_cache (the new token goes into its slot and its block into
 * the table: "vLLM 深度拆解：当大模型推理学会「分页注意力」", §3.1 and §3.3
 * append_slot; "LLM推理优化：vLLM PagedAttention深度解析与工程实践", §3.1
 * block table), without the copy launch: the kernel reads the staged arrays
 * from pinned host memory over the bus.
 *   staged_slots   [num_seqs] int64, pinned host memory (hipHostMalloc or a
 *                  pinned torch tensor; 8-byte aligned): each new token's slot
 *   staged_lens    [num_seqs] int32, pinned host memory: context lengths, the
 *                  new token included
 *   staged_items   [num_items][2] int32, pinned host memory (8-byte aligned),
 *                  or NULL with num_items = 0: a work list for
 *                  pa_decode_partitioned
 *   slot_mapping   [num_seqs] int64, device: receives staged_slots
 *   context_lens   [num_seqs] int32, device: receives staged_lens
 *   work_items     [num_items][2] int32, device: receives staged_items
 *   block_tables   [num_seqs][max_blocks_per_seq] int32, device, updated as
 *                  pa_update_block_tables does
 *   key, value     [num_seqs][num_kv_heads][head_dim] 16-bit, device
 *   key_cache, value_cache  the pools, written as pa_reshape_and_cache does
 * The staged buffers must stay unchanged until the launch has run:
 * done_event (NULL, or an event created with timing) is recorded by the
 * launch itself when its kernel ends, and a host that waits on it before
 * rewriting them needs no marker in the stream.  Copy-on-write block copies
 * (pa_copy_blocks) must be issued before this call.  Returns
 * PA_ERR_INVALID_ARG, launching nothing, when a staged pointer is not host
 * memory the device can read.
 * ---------------------------------------------------------------------- */
pa_status pa_write_step(const int64_t* staged_slots, const int32_t* staged_lens,
                        const int32_t* staged_items, int32_t num_items,
                        int64_t* slot_mapping, int32_t* context_lens,
                        int32_t* work_items, int32_t* block_tables,
                        int32_t max_blocks_per_seq, const void* key,
                        const void* value, void* key_cache, void* value_cache,
                        int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t num_blocks,
                        hipStream_t stream, hipEvent_t done_event);

/* ------------------------------------------------------------------------
 * Block copy for copy-on-write: for each pair k, block dst[k] of both pools
 * becomes a bit-exact copy of block src[k] (all slots, heads and dims).
 * Follows: a shared block is copied only when a sharer must modify it
 * ("vLLM 深度拆解：当大模型推理学会「分页注意力」", §3.3 Copy-on-Write).
 *   block_pairs       [num_pairs][2] int32 device array (src, dst)
 * Pairs with an id outside [0, num_blocks) are skipped on the device.  A dst
 * that is also another pair's src, or appears twice, is undefined.
 * ---------------------------------------------------------------------- */
pa_status pa_copy_blocks(void* key_cache, void* value_cache,
                         const int32_t* block_pairs, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks,
                         pa_dtype dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Multi-token (chunked-prefill) attention.
 * Follows: "vLLM 深度拆解：当大模型推理学会「分页注意力」", §2.3 (prefill
 * computes every prompt token at once) and §5.1 (chunked prefill: a long
 * prompt's prefill cut into chunks that run between decode steps), over the
 * paged cache of "LLM推理优化：vLLM PagedAttention深度解析与工程实践", §4.1.
 * Sequence i holds context_lens[i] tokens in the cache; its last
 * n_i = query_start[i+1] - query_start[i] tokens are its query chunk (their
 * K/V written before this call, e.g. by pa_reshape_and_cache).  Query row
 * query_start[i] + k (position context_lens[i] - n_i + k) attends causally
 * to tokens 0 .. its position:
 *   out[row][h] = sum_{j <= pos} softmax_j(scale * q[row][h] . K[j]) V[j]
 *   query, out     [num_query_tokens][num_q_heads][head_dim] 16-bit
 *   query_start    [num_seqs + 1] int32 device array, query_start[0] = 0
 *   seq_order      [num_seqs] int32 device array or NULL: the order in which
 *                  the sequences' work is dispatched (a permutation of
 *                  0..num_seqs-1; longest context first balances the launch;
 *                  entries outside [0, num_seqs) are skipped)
 *   max_query_len  >= every n_i (sizes the grid); a longer chunk is cut:
 *                  its first max_query_len rows are computed at their true
 *                  positions, the rest are left unwritten
 * Other arguments as for pa_decode; block_size must be a power of two
 * (PA_ERR_UNSUPPORTED otherwise).  Products run on the matrix cores with
 * fp32 accumulation; the softmax weights enter the P.V product as a 16-bit
 * part plus a 16-bit remainder (about 17 significant bits).  A chunk longer
 * than its context (n_i > context_lens[i]), or one whose rows fall outside
 * [0, num_query_tokens), is skipped whole on the device (its outputs are
 * left unwritten).
 * ---------------------------------------------------------------------- */
pa_status pa_prefill(void* out, const void* query, const void* key_cache,
                     const void* value_cache, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                     const int32_t* query_start, const int32_t* seq_order,
                     int32_t num_seqs,
                     int32_t num_query_tokens, int32_t max_query_len,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t num_blocks, float scale,
                     pa_dtype dtype, hipStream_t stream, hipEvent_t start_event,
                     hipEvent_t stop_event);

/* ------------------------------------------------------------------------
 * INT8 KV cache.
 * Follows: "LLM推理优化技术地图：从KV Cache到量化与投机解码", §4.3 (quantising
 * the KV cache to INT8 halves its bytes; accuracy is model-dependent).  The
 * pages fix no convention; this library's is symmetric per-row quantisation
 * with one fp32 scale per (token, KV head) row of head_dim elements:
 *   a = max |x|,  s = a / 127,  code = clamp(round_half_even(x / s), -127, 127)
 * computed in fp32 (correctly rounded division) when the row is written; the
 * row reads back as s * code.  a = 0 gives codes 0 and s = 0; a row holding
 * inf or NaN gives s = NaN and codes 0.
 *   key_cache / value_cache  [num_blocks][block_size][num_kv_heads][head_dim]
 *                            int8 codes
 *   key_scale / value_scale  [num_blocks][num_kv_heads][block_size] fp32
 * head_dim is 64 or 128.  Queries, outputs and the K/V rows handed to the
 * writes stay 16-bit (dtype); every other argument is as for the 16-bit call
 * of the same name.
 * ---------------------------------------------------------------------- */

/* pa_reshape_and_cache into INT8 pools: each token's K and V rows are
 * quantised per KV head and written with their scales.  Alignment: key /
 * value 16 bytes, codes and slot_mapping 8, scales 4. */
pa_status pa_reshape_and_cache_int8(const void* key, const void* value,
                                    int8_t* key_cache, int8_t* value_cache,
                                    float* key_scale, float* value_scale,
                                    const int64_t* slot_mapping,
                                    int32_t num_tokens, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, pa_dtype dtype,
                                    hipStream_t stream);

/* pa_write_step into INT8 pools (the step's K/V rows quantised as above). */
pa_status pa_write_step_int8(const int64_t* staged_slots,
                             const int32_t* staged_lens,
                             const int32_t* staged_items, int32_t num_items,
                             int64_t* slot_mapping, int32_t* context_lens,
                             int32_t* work_items, int32_t* block_tables,
                             int32_t max_blocks_per_seq, const void* key,
                             const void* value, int8_t* key_cache,
                             int8_t* value_cache, float* key_scale,
                             float* value_scale, int32_t num_seqs,
                             int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks,
                             pa_dtype dtype, hipStream_t stream,
                             hipEvent_t done_event);

/* pa_decode over INT8 pools: K and V rows are read as scale x code; the
 * output is as for pa_decode (fp32 arithmetic, rounded once to dtype).
 * Pools 16-byte aligned, scales 4. */
pa_status pa_decode_int8(void* out, const void* query, const int8_t* key_cache,
                         const int8_t* value_cache, const float* key_scale,
                         const float* value_scale, const int32_t* block_tables,
                         int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, int32_t max_context_len,
                         float scale, pa_dtype dtype, hipStream_t stream,
                         hipEvent_t start_event, hipEvent_t stop_event);

/* pa_decode_partitioned over INT8 pools (same workspace size). */
pa_status pa_decode_partitioned_int8(
    void* out, const void* query, const int8_t* key_cache,
    const int8_t* value_cache, const float* key_scale, const float* value_scale,
    const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_context_len, float scale, pa_dtype dtype,
    int32_t partition_size, const int32_t* work_items, int32_t num_work_items,
    void* workspace, size_t workspace_bytes, hipStream_t stream,
    hipEvent_t start_event, hipEvent_t stop_event);

/* pa_copy_blocks for INT8 pools: codes and scales of each pair's src block
 * are copied to its dst block.  head_dim a multiple of 16 and
 * num_kv_heads * block_size a multiple of 4; pools and scales 16-byte
 * aligned. */
pa_status pa_copy_blocks_int8(int8_t* key_cache, int8_t* value_cache,
                              float* key_scale, float* value_scale,
                              const int32_t* block_pairs, int32_t num_pairs,
                              int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * Host block allocator (no device memory; not thread-safe: one caller at a
 * time per handle).
 * Follows: the BlockManager of "LLM推理优化：vLLM PagedAttention深度解析与
 * 工程实践", §3.2 (free pool taken from its head, returned to its tail;
 * allocate(seq, num_tokens) grows by ceil((num_tokens - have) / block_size)
 * blocks and fails before taking any when the pool is short), with the
 * append_slot / free / shared-block rules of "vLLM 深度拆解", §3.3 (blocks
 * shared by reference carry a reference count and go back to the pool when
 * it reaches zero; a shared block is copied before a sharer writes into it).
 * Every call that returns PA_ERR_OOM or PA_ERR_INVALID_ARG leaves the
 * allocator unchanged.
 * ---------------------------------------------------------------------- */
typedef struct pa_allocator pa_allocator;

/* initial_free_order: a permutation of 0..num_blocks-1 giving the initial
 * order of the free pool, or NULL for 0, 1, ..., num_blocks-1. */
pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size,
                          const int32_t* initial_free_order,
                          pa_allocator** out);
void pa_alloc_destroy(pa_allocator* a);

/* Make sequence seq_id (created if new) hold num_tokens tokens: take
 * ceil((num_tokens - blocks_held * block_size) / block_size) blocks when its
 * blocks do not cover num_tokens.  Never shrinks. */
pa_status pa_alloc_allocate(pa_allocator* a, int64_t seq_id, int32_t num_tokens);

/* Add one token to seq_id (created if new) and return its slot
 * (block * block_size + offset).  If the token lands in a block shared with
 * another sequence, the sequence gets a fresh block and *cow_src / *cow_dst
 * name the block to copy (see pa_copy_blocks); otherwise both are -1.
 * cow_src / cow_dst may be NULL. */
pa_status pa_alloc_append_slot(pa_allocator* a, int64_t seq_id,
                               int64_t* slot_out, int32_t* cow_src,
                               int32_t* cow_dst);

/* append_slot for n distinct sequences at once; all or nothing (PA_ERR_OOM
 * before any change when the pool cannot serve the whole batch).
 * slots_out [n]; context_lens_out [n] (tokens held after the append, or
 * NULL); cow_src / cow_dst [n] or NULL. */
pa_status pa_alloc_append_slots(pa_allocator* a, const int64_t* seq_ids,
                                int32_t n, int64_t* slots_out,
                                int32_t* context_lens_out, int32_t* cow_src,
                                int32_t* cow_dst);

/* New sequence dst_seq references the first num_tokens tokens (a multiple
 * of block_size, at most src's tokens) of src_seq: the same physical
 * blocks, each reference count + 1. */
pa_status pa_alloc_share_prefix(pa_allocator* a, int64_t src_seq,
                                int64_t dst_seq, int32_t num_tokens);

/* New sequence dst_seq references every block of src_seq (a partly filled
 * last block included) and holds as many tokens. */
pa_status pa_alloc_fork(pa_allocator* a, int64_t src_seq, int64_t dst_seq);

/* Drop seq_id: each of its blocks loses a reference, in table order
 * (reverse table order while prefix caching is on), and goes to the tail of
 * the free pool when no reference is left. */
pa_status pa_alloc_free(pa_allocator* a, int64_t seq_id);

/* Automatic prefix caching.
 * Follows: "LLM推理优化：vLLM PagedAttention深度解析与工程实践", §4.2 (KV
 * blocks of a prefix that an earlier request already holds are reused), and
 * the Qwen2.5-7B vLLM 0.6.3 deployment page, §3.2 (a prompt is cut into
 * fixed-size blocks, each keyed by its token ids chained to the blocks before
 * it; a hit needs the same tokens, block-aligned, from the first token on).
 * Off by default.  Turning it on or off forgets every cached block.  While
 * on, the host memory it costs is block_size + 4 int32 per physical block
 * plus one index entry per cached block (the first page, §六 pitfall 4: the
 * table is worth its memory only when prompts share prefixes).
 * PA_ERR_OOM if that memory cannot be had. */
pa_status pa_alloc_set_prefix_caching(pa_allocator* a, int32_t enabled);

/* Create sequence seq_id (PA_ERR_INVALID_ARG if it exists) holding the
 * prompt tokens[0..num_tokens) (int32 token ids, host memory; read only
 * during the call) in ceil(num_tokens / block_size) blocks.
 * With prefix caching on, the longest cached block-aligned prefix of the
 * prompt is reused (its blocks gain a reference; a cached block waiting in
 * the free pool is taken out of it), never including the block that holds
 * the last prompt token; the other blocks come from the pool head (a cached
 * block handed out this way leaves the cache).  The prompt's full blocks
 * that were not reused are then cached, unless their prefix is cached
 * already.  *cached_tokens_out (may be NULL) = tokens whose K/V is already in
 * the cache, a multiple of block_size: the caller writes K/V only for
 * positions [*cached_tokens_out, num_tokens), whose slots pa_alloc_slots
 * gives.  Cached blocks must hold the K/V of their tokens before a later
 * prompt reuses them: write them in stream order before any later read.
 * PA_ERR_OOM (nothing changed) when the pool cannot supply the blocks not
 * reused plus the reused ones that wait in the pool.  With caching off this
 * is pa_alloc_allocate on a new sequence, with *cached_tokens_out = 0. */
pa_status pa_alloc_allocate_prompt(pa_allocator* a, int64_t seq_id,
                                   const int32_t* tokens, int32_t num_tokens,
                                   int32_t* cached_tokens_out);

/* Blocks currently cached (held or waiting in the free pool), or -1. */
int32_t pa_alloc_num_cached_blocks(const pa_allocator* a);

/* Copy seq_id's block table (physical ids in logical order) to out[0..cap);
 * *n_out = number of blocks (PA_ERR_INVALID_ARG if cap is too small). */
pa_status pa_alloc_block_table(const pa_allocator* a, int64_t seq_id,
                               int32_t* out, int32_t cap, int32_t* n_out);

/* Block tables of n sequences as a dense [n][max_blocks_per_seq] int32
 * array, unused entries set to pad; context_lens_out [n] (may be NULL)
 * receives each sequence's token count. */
pa_status pa_alloc_block_tables(const pa_allocator* a, const int64_t* seq_ids,
                                int32_t n, int32_t* out,
                                int32_t max_blocks_per_seq, int32_t pad,
                                int32_t* context_lens_out);

/* Slots of positions [begin, end) of seq_id (each < its token count). */
pa_status pa_alloc_slots(const pa_allocator* a, int64_t seq_id, int32_t begin,
                         int32_t end, int64_t* out);

/* Tokens held by seq_id, or -1 if unknown. */
int32_t pa_alloc_num_tokens(const pa_allocator* a, int64_t seq_id);

/* Blocks in the free pool. */
int32_t pa_alloc_num_free(const pa_allocator* a);

/* Reference count of a physical block, or -1 for an invalid id. */
int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block_id);

/* Blocks held by two or more sequences (reference count >= 2: shared
 * prefixes, forks, prefix-cache hits), or -1 for a NULL allocator.  Kept
 * current by every call that changes a reference count. */
int32_t pa_alloc_num_shared_blocks(const pa_allocator* a);

/* Work list for pa_decode_partitioned from the host's context lengths:
 * every live (sequence, partition) pair of partition_size tokens (at most
 * max_parts per sequence; max_parts < 0: no limit), each exactly once.
 * Order: the decode runs list position i on XCD i % 8, so the pairs are
 * dealt to 8 queues, one per XCD.  Each sequence is cut into runs of at most
 * q consecutive partitions; runs go longest first (in tokens; ties in
 * sequence order) to the queue holding the fewest tokens so far (ties: the
 * lowest queue).  q starts at ceil(N / 8) for N pairs in all (one run for all
 * but the longest contexts) and halves while the fullest queue holds more
 * than 1.01x the mean tokens, down to 1; the q with the fullest queue
 * lightest is taken (the larger q on a tie).  A queue lists its full
 * partitions in that order, then its ragged ones longest first (ties in that
 * order), so the shortest work ends the launch.  The output reads the queues round-robin: position 8j + x is
 * queue x's item j while every queue has one; after that the queues still
 * holding items take turns in the same order.  A sequence's partitions
 * thus run on one XCD and share its L2.  Splitting the context into
 * partitions follows the split-context ("v2") kernel of
 * "LLM推理优化：vLLM PagedAttention深度解析与工程实践", §4.1; the order is
 * this library's scheduling choice.
 *   context_lens  [num_seqs] int32, host memory
 *   items_out     [capacity][2] int32, host memory: (sequence, partition)
 * *n_out = the number of items; PA_ERR_INVALID_ARG if it exceeds capacity
 * (the first capacity items are written). */
pa_status pa_partition_work_items(const int32_t* context_lens, int32_t num_seqs,
                                  int32_t partition_size, int32_t max_parts,
                                  int32_t* items_out, int32_t capacity, int32_t* n_out);

/* The free pool in order (head first) into out[0..cap); *n_out = its size. */
pa_status pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap,
                             int32_t* n_out);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
