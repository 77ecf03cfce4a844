// pa_cache.hip -- the cache write, the table update, the fused step write
// and the copy-on-write block copy.
//
// Cache write: the new token's K/V go into its slot of the paged pools
// ("vLLM 深度拆解：当大模型推理学会「分页注意力」", §3.1 data flow and §3.3
// append_slot).  A token row of one pool is Hkv*D 16-bit values, contiguous
// in the input [N][Hkv][D] and in the pool [NB][bs][Hkv][D] (slot s starts
// at element s*Hkv*D), so each lane moves one 16-byte chunk: a coalesced
// read and a coalesced write, no arithmetic on the values.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, const int64_t* __restrict__ slots, int64_t num_chunks,
    int32_t chunks_per_tok, int64_t num_slots) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= num_chunks) return;
  const int64_t t = gid / chunks_per_tok;
  const int64_t c = gid - t * chunks_per_tok;
  const int64_t s = slots[t];
  if (s < 0 || s >= num_slots) return;   // padding token, or out of range: no write
  const int64_t dst = s * chunks_per_tok + c;
  k_cache[dst] = key[gid];
  v_cache[dst] = value[gid];
}

// Copy-on-write: block pair k copies src -> dst in both pools, 16 bytes per
// lane; blockIdx.y selects the pair.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_cache,
                                                          uint4* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int64_t chunks_per_block,
                                                          int32_t num_blocks) {
  const int32_t src = pairs[2 * blockIdx.y];
  const int32_t dst = pairs[2 * blockIdx.y + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       c < chunks_per_block; c += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    k_cache[dst * chunks_per_block + c] = k_cache[src * chunks_per_block + c];
    v_cache[dst * chunks_per_block + c] = v_cache[src * chunks_per_block + c];
  }
}

// Decode-step table update: sequence i's new token sits at position L_i - 1
// in slot s_i, so the table entry that holds it is (L_i - 1) / bs and its
// block is s_i / bs.  Appending never moves earlier blocks, and a copy-on-write
// replaces exactly this entry, so one store per sequence keeps a
// device-resident table equal to the allocator's.
__global__ __launch_bounds__(256) void update_tables_kernel(int32_t* __restrict__ tables,
                                                            int32_t mb,
                                                            const int32_t* __restrict__ lens,
                                                            const int64_t* __restrict__ slots,
                                                            int32_t n, int32_t bs,
                                                            int64_t num_slots) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t s = slots[i];
  const int32_t L = lens[i];
  if (s < 0 || s >= num_slots || L <= 0) return;
  const int32_t idx = (L - 1) / bs;
  if (idx >= mb) return;
  tables[static_cast<int64_t>(i) * mb + idx] = static_cast<int32_t>(s / bs);
}

// One decode step's writes in one launch: blocks [0, tok_blocks) take one
// 16-byte chunk of a new token's K/V row per thread, as the cache write;
// the thread with chunk 0 of token t also copies its slot and length from
// the staging buffer to the device arrays and records the token's block in
// the table, as the table update.  Blocks past tok_blocks copy the work list.
// The staged arrays are pinned host memory read over the bus: every wave
// reads one slot (the lanes of a token share the address), so the step's
// metadata costs one round trip instead of a copy launch.
__global__ __launch_bounds__(256) void write_step_kernel(
    const int64_t* __restrict__ staged_slots, const int32_t* __restrict__ staged_lens,
    const int2* __restrict__ staged_items, int64_t* __restrict__ slot_mapping,
    int32_t* __restrict__ context_lens, int2* __restrict__ work_items, int32_t num_items,
    int32_t* __restrict__ tables, int32_t mb, int32_t bs, const uint4* __restrict__ key,
    const uint4* __restrict__ value, uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    int64_t num_chunks, int32_t chunks_per_tok, int64_t num_slots, uint32_t tok_blocks) {
  if (blockIdx.x >= tok_blocks) {
    const int64_t i = static_cast<int64_t>(blockIdx.x - tok_blocks) * blockDim.x + threadIdx.x;
    if (i < num_items) work_items[i] = staged_items[i];
    return;
  }
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= num_chunks) return;
  const int64_t t = gid / chunks_per_tok;
  const int64_t c = gid - t * chunks_per_tok;
  const int64_t s = staged_slots[t];
  if (c == 0) {
    const int32_t L = staged_lens[t];
    slot_mapping[t] = s;
    context_lens[t] = L;
    if (s >= 0 && s < num_slots && L > 0) {
      const int32_t idx = (L - 1) / bs;
      if (idx < mb) tables[t * mb + idx] = static_cast<int32_t>(s / bs);
    }
  }
  if (s < 0 || s >= num_slots) return;   // padding token, or out of range: no write
  const int64_t dst = s * chunks_per_tok + c;
  k_cache[dst] = key[gid];
  v_cache[dst] = value[gid];
}

int launch_write_step(const int64_t* staged_slots, const int32_t* staged_lens,
                      const int32_t* staged_items, int32_t num_items, int64_t* slot_mapping,
                      int32_t* context_lens, int32_t* work_items, int32_t* tables, int32_t mb,
                      int32_t bs, const void* key, const void* value, void* k_cache,
                      void* v_cache, int32_t n, int32_t chunks_per_tok, int64_t num_slots,
                      hipStream_t stream, hipEvent_t done) {
  const int64_t num_chunks = static_cast<int64_t>(n) * chunks_per_tok;
  const int64_t tok_blocks = (num_chunks + 255) / 256;
  const int64_t item_blocks = (static_cast<int64_t>(num_items) + 255) / 256;
  hipExtLaunchKernelGGL(write_step_kernel, dim3(static_cast<uint32_t>(tok_blocks + item_blocks)),
                     dim3(256), 0, stream, nullptr, done, 0, staged_slots, staged_lens,
                     reinterpret_cast<const int2*>(staged_items), slot_mapping, context_lens,
                     reinterpret_cast<int2*>(work_items), num_items, tables, mb, bs,
                     static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), num_chunks,
                     chunks_per_tok, num_slots, static_cast<uint32_t>(tok_blocks));
  return static_cast<int>(hipGetLastError());
}

int launch_update_tables(int32_t* tables, int32_t mb, const int32_t* lens, const int64_t* slots,
                         int32_t n, int32_t bs, int64_t num_slots, hipStream_t stream) {
  hipLaunchKernelGGL(update_tables_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, tables, mb,
                     lens, slots, n, bs, num_slots);
  return static_cast<int>(hipGetLastError());
}

int launch_cache_write(const void* key, const void* value, void* k_cache, void* v_cache,
                       const int64_t* slots, int32_t n, int32_t chunks_per_tok,
                       int64_t num_slots, hipStream_t stream) {
  const int64_t num_chunks = static_cast<int64_t>(n) * chunks_per_tok;
  const int64_t blocks = (num_chunks + 255) / 256;
  hipLaunchKernelGGL(cache_write_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                     static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), slots,
                     num_chunks, chunks_per_tok, num_slots);
  return static_cast<int>(hipGetLastError());
}

int launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                       int64_t chunks_per_block, int32_t num_blocks, hipStream_t stream) {
  const int64_t want = (chunks_per_block + 255) / 256;
  const uint32_t gx = static_cast<uint32_t>(want < 64 ? want : 64);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, static_cast<uint32_t>(num_pairs)), dim3(256), 0,
                     stream, static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), pairs,
                     chunks_per_block, num_blocks);
  return static_cast<int>(hipGetLastError());
}

}  // namespace pa
