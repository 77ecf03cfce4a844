// pa_internal.h -- declarations shared by libpa's translation units (not
// installed; the public interface is include/pa.h).
#pragma once

#include <cstddef>
#include <cstdint>

#include "pa.h"

namespace pa {

// thread-local last-error message
pa_status fail(pa_status st, const char* msg);
void clear_error();

// Waves of a single-pass workgroup, which owns a whole context: long contexts
// want more of them (LLaMA-13B-shaped layer, 32 sequences of 128..2048
// tokens: 4 waves 113.2 us, 8 waves 109.8 us, 16 waves 123.8 us).
constexpr int kWavesSingle = 8;
// Tokens per LDS pass of the single-pass kernel: 8 units of 16 tokens a wave.
constexpr int32_t kSingleChunk = 128 * kWavesSingle;

// Parameters of the attention kernels, passed by value as one kernel argument.
struct AttnParams {
  void* out;                  // [S][Hq][D] 16-bit (single pass) or unused
  const void* q;              // [S][Hq][D] 16-bit
  const void* k_cache;        // [NB][bs][Hkv][D]
  const void* v_cache;
  const int32_t* block_tables;  // [S][mb]
  const int32_t* context_lens;  // [S]
  float* part_acc;            // [S][nP_max][Hq][D]   (split-context only)
  float* part_max;            // [S][nP_max][Hq]
  float* part_sum;            // [S][nP_max][Hq]
  int64_t block_stride;       // elements per physical block = bs * Hkv * D
  int32_t mb;                 // row stride of block_tables
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;              // G = Hq / Hkv
  int32_t heads_per_wg;       // query heads one workgroup serves (<= 8)
  int32_t head_chunks;        // ceil(G / heads_per_wg)
  int32_t block_size;
  int32_t log2_block_size;
  int32_t num_blocks;
  int32_t chunk;              // tokens per pass over LDS (= partition size)
  int32_t num_parts;          // nP_max (split-context)
  int32_t grid_parts;         // partitions in the dense grid (nP_max rounded up to odd)
  const int32_t* work_items;  // [num_work_items][2] (seq, partition), or NULL: dense grid
  int32_t num_work_items;
  float scale_log2;           // scale * log2(e): logits live in the base-2 domain
  const float* k_scale;       // INT8 pools only: [NB][Hkv][bs] fp32 row scales
  const float* v_scale;
};

// Launchers; each returns the hipError_t of its launch.
// kind: 0 = single-pass decode, 1 = split-context partitions, 2 = merge.
// start / stop (may be NULL): events the launch itself records when the
// kernel starts / ends (hipExtLaunchKernel), with no marker in the stream.
int launch_attn_f16_d64(int kind, const AttnParams& p, hipStream_t stream, hipEvent_t start,
                        hipEvent_t stop);
int launch_attn_f16_d128(int kind, const AttnParams& p, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop);
int launch_attn_bf16_d64(int kind, const AttnParams& p, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop);
int launch_attn_bf16_d128(int kind, const AttnParams& p, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop);
// INT8 pools (codes, with the row scales in p.k_scale / p.v_scale); kind 2
// (merge) is the same kernel as for 16-bit pools.
int launch_attn_q8_f16_d64(int kind, const AttnParams& p, hipStream_t stream, hipEvent_t start,
                           hipEvent_t stop);
int launch_attn_q8_f16_d128(int kind, const AttnParams& p, hipStream_t stream, hipEvent_t start,
                            hipEvent_t stop);
int launch_attn_q8_bf16_d64(int kind, const AttnParams& p, hipStream_t stream, hipEvent_t start,
                            hipEvent_t stop);
int launch_attn_q8_bf16_d128(int kind, const AttnParams& p, hipStream_t stream, hipEvent_t start,
                             hipEvent_t stop);
// Split-context partitions over INT8 pools on the matrix cores (up to 16
// query heads per workgroup; the launcher sets p.head_chunks and
// p.heads_per_wg for it); the merge is kind 2 of the launchers above.
int launch_attn_q8_mfma_split(int dtype, int head_dim, const AttnParams& p, hipStream_t stream,
                              hipEvent_t start, hipEvent_t stop);
// Query heads per KV head from which INT8 split-context decodes use it: with
// fewer, the vector kernel keeps up with the memory stream (measured: 4 heads
// 4 % slower on the matrix cores, 5 heads 1.25x faster, 7 heads 1.55x).
constexpr int kQ8MfmaMinGroup = 5;
int launch_cache_write(const void* key, const void* value, void* k_cache, void* v_cache,
                       const int64_t* slots, int32_t n, int32_t chunks_per_tok,
                       int64_t num_slots, hipStream_t stream);
int launch_update_tables(int32_t* tables, int32_t mb, const int32_t* lens, const int64_t* slots,
                         int32_t n, int32_t bs, int64_t num_slots, hipStream_t stream);
int launch_write_step(const int64_t* staged_slots, const int32_t* staged_lens,
                      const int32_t* staged_items, int32_t num_items, int64_t* slot_mapping,
                      int32_t* context_lens, int32_t* work_items, int32_t* tables, int32_t mb,
                      int32_t bs, const void* key, const void* value, void* k_cache,
                      void* v_cache, int32_t n, int32_t chunks_per_tok, int64_t num_slots,
                      hipStream_t stream, hipEvent_t done);
int launch_cache_write_q8(const void* key, const void* value, void* k_codes, void* v_codes,
                          float* k_scale, float* v_scale, const int64_t* slots, int32_t n,
                          int32_t head_dim, int32_t chunks_per_tok, int64_t num_slots, int32_t bs,
                          int32_t bf16, hipStream_t stream);
int launch_write_step_q8(const int64_t* staged_slots, const int32_t* staged_lens,
                         const int32_t* staged_items, int32_t num_items, int64_t* slot_mapping,
                         int32_t* context_lens, int32_t* work_items, int32_t* tables, int32_t mb,
                         int32_t bs, const void* key, const void* value, void* k_codes,
                         void* v_codes, float* k_scale, float* v_scale, int32_t n,
                         int32_t head_dim, int32_t chunks_per_tok, int64_t num_slots,
                         int32_t bf16, hipStream_t stream, hipEvent_t done);
int launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                       int64_t chunks_per_block, int32_t num_blocks, hipStream_t stream);

}  // namespace pa
