// pa_cache.hip -- the cache write, the table update, the fused step write
// and the copy-on-write block copy.
//
// Cache write: the new token's K/V go into its slot of the paged pools
// ("vLLM 深度拆解：当大模型推理学会「分页注意力」", §3.1 data flow and §3.3
// append_slot).  A token row of one pool is Hkv*D 16-bit values, contiguous
// in the input [N][Hkv][D] and in the pool [NB][bs][Hkv][D] (slot s starts
// at element s*Hkv*D), so each lane moves one 16-byte chunk: a coalesced
// read and a coalesced write, no arithmetic on the values.
//
// INT8 pools: the same lanes, each holding 8 elements of one (token, KV head)
// row, quantise them: the row's D / 8 lanes form an aligned DPP group that
// takes the row's largest magnitude a, then s = a / 127 and each code is
// round_half_even(x / s) clamped to +-127, all in fp32 (correctly rounded
// division); a = 0 gives codes 0, a row holding inf or NaN gives s = NaN and
// codes 0.  Codes go to [NB][bs][Hkv][D] (8 bytes per lane), the scale to
// [NB][Hkv][bs].  ("LLM推理优化技术地图：从KV Cache到量化与投机解码", §4.3:
// INT8 halves the KV bytes; the convention is this library's.)
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cfloat>

#include "pa_internal.h"

namespace pa {

namespace {

template <int CTRL>
__device__ inline float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// max over each aligned group of N = 8 or 16 lanes; every lane gets it
template <int N>
__device__ inline float group_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));     // lane ^ 1
  x = fmaxf(x, dpp_f<0x4E>(x));     // lane ^ 2
  x = fmaxf(x, dpp_f<0x141>(x));    // quads of each 8 (row_half_mirror)
  if constexpr (N == 16) x = fmaxf(x, dpp_f<0x140>(x));   // halves of each 16 (row_mirror)
  return x;
}

__device__ inline float widen_lo(uint32_t w, bool bf16) {
  return bf16 ? __uint_as_float(w << 16)
              : static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w)));
}
__device__ inline float widen_hi(uint32_t w, bool bf16) {
  return bf16 ? __uint_as_float(w & 0xffff0000u)
              : static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// Quantise this lane's 8 elements of a row whose R lanes are an aligned
// group; every lane of the group must call it.  Returns the 8 codes (byte k
// = element k) and sets *scale to the row's scale.
template <int R>
__device__ inline uint2 quantize8(uint4 in, bool bf16, float* scale) {
  const uint32_t w[4] = {in.x, in.y, in.z, in.w};
  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = widen_lo(w[k], bf16);
    x[2 * k + 1] = widen_hi(w[k], bf16);
  }
  float a = 0.f, bad = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float m = fabsf(x[e]);
    bad = m <= FLT_MAX ? bad : 1.f;   // inf or NaN
    a = fmaxf(a, m);
  }
  a = group_max<R>(a);
  bad = group_max<R>(bad);
  const float sc = a / 127.0f;
  uint32_t lo = 0, hi = 0;
  if (bad == 0.f && a > 0.f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = fminf(fmaxf(__builtin_rintf(x[e] / sc), -127.f), 127.f);
      const uint32_t b = static_cast<uint32_t>(static_cast<int32_t>(c)) & 0xffu;
      if (e < 4) lo |= b << (8 * e);
      else hi |= b << (8 * (e - 4));
    }
  }
  *scale = bad != 0.f ? __builtin_nanf("") : sc;
  return make_uint2(lo, hi);
}

// One 16-byte input chunk per lane: chunk c of a token is elements 8c..8c+7
// of its [Hkv][D] row, i.e. lane c % R of (KV head c / R).  Writes codes and
// (lane 0 of the row) the scale to slot s; s < 0 (the caller's "no write",
// also for slots past the pool): nothing.
template <int R>
__device__ inline void write_chunk_q8(const uint4* key, const uint4* value, uint2* k_codes,
                                      uint2* v_codes, float* k_scale, float* v_scale,
                                      int64_t gid, bool live, int64_t c, int64_t s,
                                      int32_t chunks_per_tok, int32_t bs, bool bf16) {
  const uint4 kin = live ? key[gid] : make_uint4(0, 0, 0, 0);
  const uint4 vin = live ? value[gid] : make_uint4(0, 0, 0, 0);
  float ks, vs;
  const uint2 kq = quantize8<R>(kin, bf16, &ks);
  const uint2 vq = quantize8<R>(vin, bf16, &vs);
  if (!live || s < 0) return;
  const int64_t dst = s * chunks_per_tok + c;
  k_codes[dst] = kq;
  v_codes[dst] = vq;
  if (c % R == 0) {
    const int64_t hkv = chunks_per_tok / R;
    const int64_t g = c / R;
    const int64_t blk = s / bs, off = s - blk * bs;
    k_scale[(blk * hkv + g) * bs + off] = ks;
    v_scale[(blk * hkv + g) * bs + off] = vs;
  }
}

}  // namespace

template <int R>
__global__ __launch_bounds__(256) void cache_write_q8_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint2* __restrict__ k_codes,
    uint2* __restrict__ v_codes, float* __restrict__ k_scale, float* __restrict__ v_scale,
    const int64_t* __restrict__ slots, int64_t num_chunks, int32_t chunks_per_tok,
    int64_t num_slots, int32_t bs, int32_t bf16) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  // lanes past the end still take part in their (all-dead) group's reductions
  const bool in_range = gid < num_chunks;
  const int64_t t = in_range ? gid / chunks_per_tok : 0;
  const int64_t c = in_range ? gid - t * chunks_per_tok : 0;
  int64_t s = in_range ? slots[t] : -1;
  if (s >= num_slots) s = -1;            // out of range: no write
  write_chunk_q8<R>(key, value, k_codes, v_codes, k_scale, v_scale, gid, in_range, c, s,
                    chunks_per_tok, bs, bf16 != 0);
}

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

// The step write over INT8 pools: the same work, with the K/V chunks
// quantised as in cache_write_q8_kernel.
template <int R>
__global__ __launch_bounds__(256) void write_step_q8_kernel(
    const int64_t* __restrict__ staged_slots, const int32_t* __restrict__ staged_lens,
    const int2* __restrict__ staged_items, int64_t* __restrict__ slot_mapping,
    int32_t* __restrict__ context_lens, int2* __restrict__ work_items, int32_t num_items,
    int32_t* __restrict__ tables, int32_t mb, int32_t bs, const uint4* __restrict__ key,
    const uint4* __restrict__ value, uint2* __restrict__ k_codes, uint2* __restrict__ v_codes,
    float* __restrict__ k_scale, float* __restrict__ v_scale, int64_t num_chunks,
    int32_t chunks_per_tok, int64_t num_slots, uint32_t tok_blocks, int32_t bf16) {
  if (blockIdx.x >= tok_blocks) {          // uniform: whole workgroup
    const int64_t i = static_cast<int64_t>(blockIdx.x - tok_blocks) * blockDim.x + threadIdx.x;
    if (i < num_items) work_items[i] = staged_items[i];
    return;
  }
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool in_range = gid < num_chunks;
  const int64_t t = in_range ? gid / chunks_per_tok : 0;
  const int64_t c = in_range ? gid - t * chunks_per_tok : 0;
  int64_t s = in_range ? staged_slots[t] : -1;
  if (in_range && c == 0) {
    const int32_t L = staged_lens[t];
    slot_mapping[t] = s;
    context_lens[t] = L;
    if (s >= 0 && s < num_slots && L > 0) {
      const int32_t idx = (L - 1) / bs;
      if (idx < mb) tables[t * mb + idx] = static_cast<int32_t>(s / bs);
    }
  }
  if (s >= num_slots) s = -1;
  write_chunk_q8<R>(key, value, k_codes, v_codes, k_scale, v_scale, gid, in_range, c, s,
                    chunks_per_tok, bs, bf16 != 0);
}

int launch_write_step_q8(const int64_t* staged_slots, const int32_t* staged_lens,
                         const int32_t* staged_items, int32_t num_items, int64_t* slot_mapping,
                         int32_t* context_lens, int32_t* work_items, int32_t* tables, int32_t mb,
                         int32_t bs, const void* key, const void* value, void* k_codes,
                         void* v_codes, float* k_scale, float* v_scale, int32_t n,
                         int32_t head_dim, int32_t chunks_per_tok, int64_t num_slots,
                         int32_t bf16, hipStream_t stream, hipEvent_t done) {
  const int64_t num_chunks = static_cast<int64_t>(n) * chunks_per_tok;
  const int64_t tok_blocks = (num_chunks + 255) / 256;
  const int64_t item_blocks = (static_cast<int64_t>(num_items) + 255) / 256;
  const dim3 grid(static_cast<uint32_t>(tok_blocks + item_blocks));
  auto args = [&](auto kernel) {
    hipExtLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, nullptr, done, 0, staged_slots,
                          staged_lens, reinterpret_cast<const int2*>(staged_items), slot_mapping,
                          context_lens, reinterpret_cast<int2*>(work_items), num_items, tables,
                          mb, bs, static_cast<const uint4*>(key),
                          static_cast<const uint4*>(value), static_cast<uint2*>(k_codes),
                          static_cast<uint2*>(v_codes), k_scale, v_scale, num_chunks,
                          chunks_per_tok, num_slots, static_cast<uint32_t>(tok_blocks), bf16);
  };
  if (head_dim == 64) args(write_step_q8_kernel<8>);
  else args(write_step_q8_kernel<16>);
  return static_cast<int>(hipGetLastError());
}

int launch_cache_write_q8(const void* key, const void* value, void* k_codes, void* v_codes,
                          float* k_scale, float* v_scale, const int64_t* slots, int32_t n,
                          int32_t head_dim, int32_t chunks_per_tok, int64_t num_slots, int32_t bs,
                          int32_t bf16, hipStream_t stream) {
  const int64_t num_chunks = static_cast<int64_t>(n) * chunks_per_tok;
  const dim3 grid(static_cast<uint32_t>((num_chunks + 255) / 256));
  auto args = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, static_cast<const uint4*>(key),
                       static_cast<const uint4*>(value), static_cast<uint2*>(k_codes),
                       static_cast<uint2*>(v_codes), k_scale, v_scale, slots, num_chunks,
                       chunks_per_tok, num_slots, bs, bf16);
  };
  if (head_dim == 64) args(cache_write_q8_kernel<8>);
  else args(cache_write_q8_kernel<16>);
  return static_cast<int>(hipGetLastError());
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
