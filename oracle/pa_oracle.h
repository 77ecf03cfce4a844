/*
 * pa_oracle.h -- the CPU oracle for paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this library: only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg do.  It shares no source with the HIP
 * library (libpa) and includes none of its headers.
 *
 * What it computes is the plain definition of each step, written out slowly:
 *
 *   - 16-bit float conversions, from the IEEE 754 binary16 and the bfloat16
 *     definitions (round to nearest, ties to even, for the narrowing ones);
 *   - the cache write: each new token's K/V copied bit for bit into its slot
 *     of the paged pool [num_blocks][block_size][num_kv_heads][head_dim]
 *     (page "LLM推理优化：vLLM PagedAttention深度解析与工程实践", §4.1 for the
 *     layout; page "vLLM 深度拆解：当大模型推理学会「分页注意力」", §3.1 and
 *     §3.3 for writing the new token's K/V back into its block);
 *   - the slot of a logical position through a block table (same pages, §3.1
 *     "Block Table" of the first, §2.1 of the second);
 *   - the gather of a sequence's K/V into contiguous logical order, then
 *     softmax(q K^T * scale) V in fp32 (first page, §二 formula and §4.1;
 *     paging changes no arithmetic, first page §九);
 *   - multi-token (chunked-prefill) attention: several query tokens of a
 *     sequence, the last tokens of its cache, each attending causally to the
 *     tokens up to its own position (page "vLLM 深度拆解：当大模型推理学会
 *     「分页注意力」", §2.3: prefill computes every prompt token at once, §5.1:
 *     a long prompt's prefill cut into chunks that run between decode steps);
 *   - the split-context form (partial max / sum / accumulator per partition,
 *     then the log-sum-exp merge), used only to check itself against the
 *     single-pass form (first page §4.1, "partial accumulate, then merge");
 *   - an INT8 KV cache (page "LLM推理优化技术地图：从KV Cache到量化与投机解码",
 *     §4.3: INT8 halves the KV bytes; the pages fix no convention, so the one
 *     here is this library's): symmetric codes with one fp32 scale per
 *     (token, kv head) row, s = max|x| / 127, c = round_half_even(x / s)
 *     clamped to +-127, dequantised as s * c, then the same attention;
 *   - KV bytes per token, 2 x layers x kv_heads x head_dim x bytes (first page
 *     §二; page www.mhpq.cn/news/468822 §1.2; page
 *     "LLM推理优化技术地图：从KV Cache到量化与投机解码" §2.2).
 *
 * Build: plain C++17, host only, -O2 -ffp-contract=off (no fused multiply-add,
 * so every product and sum is rounded to fp32 on its own).
 *
 * Parity pins: every function here is pinned in tests/test_oracle_pins.py
 * (brute-force fp64 contiguous attention, library conversions, the pages'
 * worked examples and closed forms, invariances).  No function is "parity
 * unpinned".
 */
#ifndef PA_ORACLE_H
#define PA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype codes used by this oracle (its own; not shared with libpa) */
#define PAO_F16 0
#define PAO_BF16 1

/* return codes */
#define PAO_OK 0
#define PAO_BAD_ARG (-1)      /* shape / dtype / pointer error            */
#define PAO_BAD_SLOT (-2)     /* slot >= num_blocks * block_size          */
#define PAO_DUP_SLOT (-3)     /* the same slot twice in one cache write   */
#define PAO_BAD_BLOCK (-4)    /* block id outside [0, num_blocks)         */
#define PAO_BAD_LEN (-5)      /* context length <= 0 or beyond the table  */

float pao_f16_to_f32(uint16_t h);
float pao_bf16_to_f32(uint16_t b);
uint16_t pao_f32_to_f16(float x);
uint16_t pao_f32_to_bf16(float x);

/* element-wise array forms of the four conversions above */
void pao_widen(const uint16_t* in, float* out, int64_t n, int32_t dtype);
void pao_narrow(const float* in, uint16_t* out, int64_t n, int32_t dtype);

/* Cache write.  key/value: [n][hkv][d] 16-bit patterns.  Pools:
 * [nb][bs][hkv][d].  slot_mapping[t] < 0 means "no write" for token t.
 * Every other slot must be < nb*bs and appear once. */
int32_t pao_cache_write(const uint16_t* key, const uint16_t* value,
                        uint16_t* key_cache, uint16_t* value_cache,
                        const int64_t* slot_mapping, int32_t n,
                        int32_t hkv, int32_t d, int32_t bs, int32_t nb);

/* Slot of logical position pos through one block-table row. */
int64_t pao_slot(const int32_t* block_table_row, int32_t pos, int32_t bs);

/* Gather one sequence's K and V of kv head g into contiguous [L][d] fp32
 * arrays, in logical order. */
int32_t pao_gather(float* k_out, float* v_out,
                   const uint16_t* key_cache, const uint16_t* value_cache,
                   const int32_t* block_table_row, int32_t L, int32_t g,
                   int32_t hkv, int32_t d, int32_t bs, int32_t nb,
                   int32_t dtype);

/* Single-pass decode of selected (sequence, q head) pairs.
 * q: [s][hq][d]; block_tables: [s][mb]; context_lens: [s];
 * pairs: [n_pairs][2] = (seq, q head); out_f32: [n_pairs][d] (fp32 result
 * before the final rounding); out_t: [n_pairs][d] 16-bit (may be NULL).
 * nthreads <= 0 means one thread per hardware core. */
int32_t pao_decode_pairs(float* out_f32, uint16_t* out_t,
                         const uint16_t* q, const uint16_t* key_cache,
                         const uint16_t* value_cache,
                         const int32_t* block_tables, int32_t mb,
                         const int32_t* context_lens, int32_t s,
                         int32_t hq, int32_t hkv, int32_t d, int32_t bs,
                         int32_t nb, float scale, int32_t dtype,
                         const int32_t* pairs, int32_t n_pairs,
                         int32_t nthreads);

/* All pairs: out_f32 / out_t are [s][hq][d]. */
int32_t pao_decode(float* out_f32, uint16_t* out_t, const uint16_t* q,
                   const uint16_t* key_cache, const uint16_t* value_cache,
                   const int32_t* block_tables, int32_t mb,
                   const int32_t* context_lens, int32_t s, int32_t hq,
                   int32_t hkv, int32_t d, int32_t bs, int32_t nb,
                   float scale, int32_t dtype, int32_t nthreads);

/* Split-context form: partitions of partition_size tokens, per-partition
 * (max, sum, acc), then the merge.  Same argument meaning as pao_decode. */
int32_t pao_decode_partitioned(float* out_f32, uint16_t* out_t,
                               const uint16_t* q, const uint16_t* key_cache,
                               const uint16_t* value_cache,
                               const int32_t* block_tables, int32_t mb,
                               const int32_t* context_lens, int32_t s,
                               int32_t hq, int32_t hkv, int32_t d, int32_t bs,
                               int32_t nb, float scale, int32_t dtype,
                               int32_t partition_size);

/* Multi-token (chunked-prefill) attention: for each sequence i, the last
 * n_i = query_start[i+1] - query_start[i] of its context_lens[i] cached
 * tokens are its query chunk; query row query_start[i] + k (position
 * context_lens[i] - n_i + k) attends causally to tokens 0 .. that position.
 * q / out_f32 / out_t: [query_start[s]][hq][d]; query_start: [s + 1], from 0. */
int32_t pao_prefill(float* out_f32, uint16_t* out_t, const uint16_t* q,
                    const uint16_t* key_cache, const uint16_t* value_cache,
                    const int32_t* block_tables, int32_t mb, const int32_t* context_lens,
                    const int32_t* query_start, int32_t s, int32_t hq, int32_t hkv, int32_t d,
                    int32_t bs, int32_t nb, float scale, int32_t dtype, int32_t nthreads);

/* INT8 KV: quantise rows [rows][d] of 16-bit values into codes [rows][d]
 * and scales [rows] (the convention above). */
int32_t pao_quantize_rows(const uint16_t* x, int64_t rows, int32_t d, int32_t dtype,
                          int8_t* codes, float* scales);

/* INT8 cache write: token t's K and V rows [hkv][d] are quantised per kv
 * head into codes key_cache/value_cache [nb][bs][hkv][d] and scales
 * key_scale/value_scale [nb][hkv][bs] at slot_mapping[t] (< 0: no write). */
int32_t pao_cache_write_int8(const uint16_t* key, const uint16_t* value, int8_t* key_cache,
                             int8_t* value_cache, float* key_scale, float* value_scale,
                             const int64_t* slot_mapping, int32_t n, int32_t hkv, int32_t d,
                             int32_t bs, int32_t nb, int32_t dtype);

/* Gather of kv head g with each row dequantised (scale x code, fp32). */
int32_t pao_gather_int8(float* k_out, float* v_out, const int8_t* key_cache,
                        const int8_t* value_cache, const float* key_scale,
                        const float* value_scale, const int32_t* block_table_row, int32_t L,
                        int32_t g, int32_t hkv, int32_t d, int32_t bs, int32_t nb);

/* pao_decode_pairs over an INT8 cache (same arguments, plus the scales). */
int32_t pao_decode_int8_pairs(float* out_f32, uint16_t* out_t, const uint16_t* q,
                              const int8_t* key_cache, const int8_t* value_cache,
                              const float* key_scale, const float* value_scale,
                              const int32_t* block_tables, int32_t mb,
                              const int32_t* context_lens, int32_t s, int32_t hq, int32_t hkv,
                              int32_t d, int32_t bs, int32_t nb, float scale, int32_t dtype,
                              const int32_t* pairs, int32_t n_pairs, int32_t nthreads);

/* KV-cache bytes per token: 2 (K and V) x layers x kv_heads x head_dim x
 * bytes per element. */
uint64_t pao_kv_bytes_per_token(int32_t layers, int32_t kv_heads,
                                int32_t head_dim, int32_t elem_bytes);

/* Logical K+V bytes one decode call reads: sum_i L_i x 2 x hkv x d x eb. */
uint64_t pao_kv_bytes_gathered(const int32_t* context_lens, int32_t s,
                               int32_t hkv, int32_t d, int32_t elem_bytes);

#ifdef __cplusplus
}
#endif
#endif /* PA_ORACLE_H */
