// pa_attn.h -- paged decode attention kernels for gfx950 (CDNA4, wave64).
//
// One query token per sequence attends over its paged K/V:
//   out[i][h] = sum_j softmax_j(scale * q[i][h] . K_i[j]) V_i[j]
// ("LLM推理优化：vLLM PagedAttention深度解析与工程实践", §二 formula; §4.1 for
// the paged layout and the v1 / v2 kernel split).  Query heads of one
// KV head (G = Hq / Hkv, "LLM推理优化技术地图", §2.3 GQA) are served by the
// same workgroup, so every K/V byte is read from HBM once for all of them.
//
// Workgroup = 4 waves = 256 lanes, one (sequence, KV head, head chunk[,
// partition]).  Its token range is processed in chunks of `chunk` tokens
// (the partition size for the split kernel), each in three phases:
//
//  1. logits.  A token's K row for one KV head is D*2 bytes; LPT = D/8 lanes
//     each load 16 bytes of it (one global_load_dwordx4), so a wave load
//     covers TPI = 64/LPT tokens that always sit in one physical block.
//     Each lane takes partial dot products of its 8 elements with the
//     matching 8 elements of every q head (v_dot2 on 16-bit pairs, fp32
//     accumulate), and DPP row operations sum the LPT partials.  Logits,
//     in the base-2 domain (scale * log2 e folded in), go to LDS.
//  2. softmax statistics.  Per-head chunk max across the workgroup, then
//     p = 2^(logit - max) written back over the logits, and their sum.
//  3. P.V.  Same load pattern over V; each lane accumulates p * V for its
//     8 dims and every head of the group in fp32 registers.
//
// The single-pass kernel ("v1") loops over all chunks of the context with a
// running max / sum / accumulator (rescaled by 2^(old max - new max)) and
// writes the normalised output.  The split kernel ("v2") handles one
// partition per workgroup and stores (max, sum, acc); the merge kernel
// combines partitions with the log-sum-exp identity.
//
// Loads use a wave-uniform (SGPR) block base and a per-lane 32-bit offset;
// block ids come from the table through scalar loads.  Tail tokens of the
// last block are masked by select (the pools' unused slots may hold NaN).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v __attribute__((ext_vector_type(2)));

template <int DT>
struct Fmt;

template <>
struct Fmt<PA_F16> {
  __device__ static inline float lo(uint32_t w) {
    return static_cast<float>(__builtin_bit_cast(half2v, w)[0]);
  }
  __device__ static inline float hi(uint32_t w) {
    return static_cast<float>(__builtin_bit_cast(half2v, w)[1]);
  }
  __device__ static inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a),
                                  __builtin_bit_cast(half2v, b), c, false);
  }
  // round to nearest even (the default rounding mode of v_cvt_f16_f32)
  __device__ static inline uint16_t narrow(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
};

template <>
struct Fmt<PA_BF16> {
  __device__ static inline float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static inline float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  __device__ static inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162v, a),
                                           __builtin_bit_cast(bf162v, b), c, false);
  }
  // round to nearest even: add 0x7fff plus the lowest kept bit, truncate
  __device__ static inline uint16_t narrow(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
    return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  }
};

// ---- cross-lane helpers ---------------------------------------------------

template <int CTRL>
__device__ inline float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over each aligned group of N lanes (N = 8 or 16, inside a DPP row);
// every lane of the group receives the total.
template <int N>
__device__ inline float group_sum(float x) {
  x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp<0x141>(x);   // row_half_mirror: quad 0 <-> quad 1 of each 8
  if constexpr (N == 16) x += dpp<0x140>(x);  // row_mirror: half 0 <-> half 1
  return x;
}

__device__ inline float wave_max_from(float x, int first_stride) {
  for (int off = first_stride; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ inline float wave_sum_from(float x, int first_stride) {
  for (int off = first_stride; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D, int GT>
struct Tile {
  static constexpr int LPT = D / 8;               // lanes per token row
  static constexpr int TPI = 64 / LPT;            // tokens per wave load
  static constexpr int GTP = GT == 1 ? 1 : (GT == 2 ? 2 : (GT <= 4 ? 4 : 8));
  static constexpr int U = 32 / TPI;              // wave loads in flight
};

// LDS (floats): probabilities [chunk][GTP], wave partial outputs
// [kWaves][GT][D], wave maxima and sums [kWaves][GTP] each.
__host__ __device__ constexpr size_t lds_floats(int D, int GT, int GTP, int chunk) {
  return static_cast<size_t>(chunk) * GTP + static_cast<size_t>(kWaves) * GT * D +
         2 * static_cast<size_t>(kWaves) * GTP;
}

template <int DT, int D, int GT, bool SPLIT>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnParams p) {
  using F = Fmt<DT>;
  using TL = Tile<D, GT>;
  constexpr int LPT = TL::LPT, TPI = TL::TPI, GTP = TL::GTP, U = TL::U;
  extern __shared__ float lds[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int row = lane / LPT;   // token of a wave load
  const int col = lane % LPT;   // 16-byte column of the head vector

  const int seq = blockIdx.z;
  const int kvh = blockIdx.y / p.head_chunks;
  const int hc = blockIdx.y - kvh * p.head_chunks;
  const int head0 = kvh * p.group + hc * GT;
  const int nact = min(GT, p.group - hc * GT);    // active heads of this chunk

  int L = p.context_lens[seq];
  L = max(0, min(L, p.mb * p.block_size));         // never past the table row
  int t_begin = 0, t_end = L;
  if constexpr (SPLIT) {
    t_begin = blockIdx.x * p.chunk;
    if (t_begin >= L) return;                       // uniform: whole workgroup
    t_end = min(L, t_begin + p.chunk);
  }

  const int64_t out_row0 = static_cast<int64_t>(seq) * p.num_q_heads + head0;
  if constexpr (!SPLIT) {
    if (L == 0) {
      uint16_t* out = static_cast<uint16_t*>(p.out);
      for (int hh = 0; hh < nact; ++hh)
        for (int d = tid; d < D; d += kThreads) out[(out_row0 + hh) * D + d] = 0;
      return;
    }
  }

  // q slices: lane (row, col) holds elements col*8 .. col*8+7 of every head
  uint4 q4[GT];
  {
    const uint16_t* q = static_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      q4[hh] = hh < nact ? *reinterpret_cast<const uint4*>(q + (out_row0 + hh) * D + col * 8)
                         : make_uint4(0, 0, 0, 0);
    }
  }

  const int32_t* bt = p.block_tables + static_cast<int64_t>(seq) * p.mb;
  const char* kbase = static_cast<const char*>(p.k_cache);
  const char* vbase = static_cast<const char*>(p.v_cache);
  const int64_t block_bytes = p.block_stride * 2;
  const uint32_t tok_bytes = static_cast<uint32_t>(p.num_kv_heads) * D * 2;
  const uint32_t lane_off =
      static_cast<uint32_t>(row) * tok_bytes + static_cast<uint32_t>(kvh * D + col * 8) * 2;
  const int bs_mask = p.block_size - 1;

  float* s_lds = lds;                                       // [chunk][GTP]
  float* red = lds + static_cast<size_t>(p.chunk) * GTP;    // [kWaves][GT][D]
  float* wmax = red + kWaves * GT * D;                      // [kWaves][GTP]
  float* wsum = wmax + kWaves * GTP;                        // [kWaves][GTP]

  float acc[GT][8];
  float m_run[GT], l_run[GT];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    m_run[hh] = -__builtin_inff();
    l_run[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  }

  for (int c0 = t_begin; c0 < t_end; c0 += p.chunk) {
    const int n = min(p.chunk, t_end - c0);
    const int ng = (n + TPI - 1) / TPI;   // wave loads covering the chunk
    const int last_g = ng - 1;

    // ---------------- phase 1: logits ----------------
    float mloc[GT];
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) mloc[hh] = -__builtin_inff();

    for (int g0 = wave * U; g0 < ng; g0 += kWaves * U) {
      uint4 kv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int g = min(g0 + u, last_g);            // clamped: loads stay in range
        const int tok0 = c0 + g * TPI;
        int blk = __builtin_amdgcn_readfirstlane(bt[tok0 >> p.log2_block_size]);
        blk = (static_cast<unsigned>(blk) < static_cast<unsigned>(p.num_blocks)) ? blk : 0;
        const char* base = kbase + blk * block_bytes +
                           static_cast<int64_t>(tok0 & bs_mask) * tok_bytes;
        kv[u] = *reinterpret_cast<const uint4*>(base + lane_off);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (g0 + u > last_g) break;                   // uniform
        const int tok = (g0 + u) * TPI + row;         // chunk-local token
        const bool valid = tok < n;
        float sv[GTP];
#pragma unroll
        for (int hh = 0; hh < GT; ++hh) {
          float a = F::dot2(q4[hh].x, kv[u].x, 0.f);
          a = F::dot2(q4[hh].y, kv[u].y, a);
          a = F::dot2(q4[hh].z, kv[u].z, a);
          a = F::dot2(q4[hh].w, kv[u].w, a);
          const float s = group_sum<LPT>(a) * p.scale_log2;
          mloc[hh] = valid ? fmaxf(mloc[hh], s) : mloc[hh];
          sv[hh] = s;
        }
#pragma unroll
        for (int hh = GT; hh < GTP; ++hh) sv[hh] = 0.f;
        if (valid && col == 0) {
          float* dst = s_lds + tok * GTP;
          if constexpr (GTP >= 4) {
#pragma unroll
            for (int k = 0; k < GTP; k += 4)
              *reinterpret_cast<float4*>(dst + k) = make_float4(sv[k], sv[k + 1], sv[k + 2], sv[k + 3]);
          } else if constexpr (GTP == 2) {
            *reinterpret_cast<float2*>(dst) = make_float2(sv[0], sv[1]);
          } else {
            dst[0] = sv[0];
          }
        }
      }
    }

    // ---------------- phase 2: chunk max, probabilities, sums ----------------
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) mloc[hh] = wave_max_from(mloc[hh], LPT);
    if (lane == 0) {
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) wmax[wave * GTP + hh] = mloc[hh];
    }
    __syncthreads();
    float m_new[GT], alpha[GT];
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      float mc = wmax[hh];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) mc = fmaxf(mc, wmax[w * GTP + hh]);
      m_new[hh] = fmaxf(m_run[hh], mc);
      alpha[hh] = fast_exp2(m_run[hh] - m_new[hh]);   // 0 on the first chunk
      m_run[hh] = m_new[hh];
    }
    float lsum[GT];
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) lsum[hh] = 0.f;
    const int npad = ng * TPI;
    for (int t = tid; t < npad; t += kThreads) {
      float v[GTP];
      float* src = s_lds + t * GTP;
      if constexpr (GTP >= 4) {
#pragma unroll
        for (int k = 0; k < GTP; k += 4) {
          const float4 f = *reinterpret_cast<const float4*>(src + k);
          v[k] = f.x; v[k + 1] = f.y; v[k + 2] = f.z; v[k + 3] = f.w;
        }
      } else if constexpr (GTP == 2) {
        const float2 f = *reinterpret_cast<const float2*>(src);
        v[0] = f.x; v[1] = f.y;
      } else {
        v[0] = src[0];
      }
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        const float pr = t < n ? fast_exp2(v[hh] - m_new[hh]) : 0.f;
        v[hh] = pr;
        lsum[hh] += pr;
      }
      if constexpr (GTP >= 4) {
#pragma unroll
        for (int k = 0; k < GTP; k += 4)
          *reinterpret_cast<float4*>(src + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
      } else if constexpr (GTP == 2) {
        *reinterpret_cast<float2*>(src) = make_float2(v[0], v[1]);
      } else {
        src[0] = v[0];
      }
    }
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) lsum[hh] = wave_sum_from(lsum[hh], 1);
    if (lane == 0) {
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) wsum[wave * GTP + hh] = lsum[hh];
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      float lc = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) lc += wsum[w * GTP + hh];
      l_run[hh] = l_run[hh] * alpha[hh] + lc;
    }
    if constexpr (!SPLIT) {
#pragma unroll
      for (int hh = 0; hh < GT; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha[hh];
    }

    // ---------------- phase 3: P . V ----------------
    for (int g0 = wave * U; g0 < ng; g0 += kWaves * U) {
      uint4 vv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int g = min(g0 + u, last_g);
        const int tok0 = c0 + g * TPI;
        int blk = __builtin_amdgcn_readfirstlane(bt[tok0 >> p.log2_block_size]);
        blk = (static_cast<unsigned>(blk) < static_cast<unsigned>(p.num_blocks)) ? blk : 0;
        const char* base = vbase + blk * block_bytes +
                           static_cast<int64_t>(tok0 & bs_mask) * tok_bytes;
        vv[u] = *reinterpret_cast<const uint4*>(base + lane_off);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (g0 + u > last_g) break;                   // uniform
        const int tok = (g0 + u) * TPI + row;
        uint4 x = vv[u];
        if (tok >= n) x = make_uint4(0, 0, 0, 0);     // unused slots may hold NaN
        float pr[GTP];
        const float* src = s_lds + tok * GTP;
        if constexpr (GTP >= 4) {
#pragma unroll
          for (int k = 0; k < GTP; k += 4) {
            const float4 f = *reinterpret_cast<const float4*>(src + k);
            pr[k] = f.x; pr[k + 1] = f.y; pr[k + 2] = f.z; pr[k + 3] = f.w;
          }
        } else if constexpr (GTP == 2) {
          const float2 f = *reinterpret_cast<const float2*>(src);
          pr[0] = f.x; pr[1] = f.y;
        } else {
          pr[0] = src[0];
        }
        float vf[8];
        vf[0] = F::lo(x.x); vf[1] = F::hi(x.x);
        vf[2] = F::lo(x.y); vf[3] = F::hi(x.y);
        vf[4] = F::lo(x.z); vf[5] = F::hi(x.z);
        vf[6] = F::lo(x.w); vf[7] = F::hi(x.w);
#pragma unroll
        for (int hh = 0; hh < GT; ++hh)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pr[hh], vf[e], acc[hh][e]);
      }
    }
    __syncthreads();   // the next chunk reuses s_lds
  }

  // ---------------- reduce over the tokens of the waves ----------------
#pragma unroll
  for (int hh = 0; hh < GT; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = wave_sum_from(acc[hh][e], LPT);
  if (row == 0) {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      float* dst = red + (wave * GT + hh) * D + col * 8;
      *reinterpret_cast<float4*>(dst) = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]);
    }
  }
  __syncthreads();

#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    if (hh >= nact) break;
    for (int d = tid; d < D; d += kThreads) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += red[(w * GT + hh) * D + d];
      if constexpr (SPLIT) {
        const int64_t slot = (out_row0 + hh) * p.num_parts + blockIdx.x;
        p.part_acc[slot * D + d] = v;
        if (d == 0) {
          p.part_max[slot] = m_run[hh];
          p.part_sum[slot] = l_run[hh];
        }
      } else {
        static_cast<uint16_t*>(p.out)[(out_row0 + hh) * D + d] = F::narrow(v / l_run[hh]);
      }
    }
  }
}

// Merge of the partitions of one (sequence, q head) per workgroup:
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p acc_p / sum_p w_p l_p
// Wave w takes partitions w, w+4, ...: the partition index is wave-uniform, so
// m_p and l_p arrive through scalar loads and each lane streams its E dims of
// acc_p, several partitions in flight at once.  The waves' sums meet in LDS.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(AttnParams p) {
  using F = Fmt<DT>;
  constexpr int E = D / 64;   // dims per lane
  constexpr int UNROLL = 4;
  __shared__ float red_acc[kWaves][D];
  __shared__ float red_l[kWaves];
  __shared__ float red_m[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = blockIdx.x;
  const int seq = pair / p.num_q_heads;
  int L = p.context_lens[seq];
  L = max(0, min(L, p.mb * p.block_size));
  const int np = min((L + p.chunk - 1) / p.chunk, p.num_parts);
  uint16_t* out = static_cast<uint16_t*>(p.out) + static_cast<int64_t>(pair) * D;
  if (np == 0) {                                   // uniform: whole workgroup
    for (int d = tid; d < D; d += kThreads) out[d] = 0;
    return;
  }
  const int64_t base = static_cast<int64_t>(pair) * p.num_parts;
  const float* pm = p.part_max + base;
  const float* ps = p.part_sum + base;
  const float* pa = p.part_acc + base * D + lane * E;

  float m = -__builtin_inff();
  for (int k = tid; k < np; k += kThreads) m = fmaxf(m, pm[k]);
  m = wave_max_from(m, 1);
  if (lane == 0) red_m[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));

  float l = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int k0 = wave; k0 < np; k0 += kWaves * UNROLL) {
    float x[UNROLL][E];
    float wk[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int k = min(k0 + u * kWaves, np - 1);  // clamped: loads stay in range
      wk[u] = (k0 + u * kWaves < np) ? fast_exp2(pm[k] - m) : 0.f;
      const float* src = pa + static_cast<int64_t>(k) * D;
      if constexpr (E == 2) {
        const float2 v = *reinterpret_cast<const float2*>(src);
        x[u][0] = v.x; x[u][1] = v.y;
      } else {
        x[u][0] = src[0];
      }
      l += wk[u] * ps[k];
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(wk[u], x[u][e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red_acc[wave][lane * E + e] = acc[e];
  if (lane == 0) red_l[wave] = l;
  __syncthreads();
  const float lt = red_l[0] + red_l[1] + red_l[2] + red_l[3];
  for (int d = tid; d < D; d += kThreads) {
    const float v = red_acc[0][d] + red_acc[1][d] + red_acc[2][d] + red_acc[3][d];
    out[d] = F::narrow(v / lt);
  }
}

template <int DT, int D, int GT>
int launch_attn_gt(int kind, const AttnParams& p, hipStream_t stream) {
  using TL = Tile<D, GT>;
  const size_t lds = lds_floats(D, GT, TL::GTP, p.chunk) * sizeof(float);
  const dim3 block(kThreads);
  if (kind == 0) {
    const dim3 grid(1, p.num_kv_heads * p.head_chunks, p.num_seqs);
    hipLaunchKernelGGL((attn_kernel<DT, D, GT, false>), grid, block, lds, stream, p);
  } else {
    const dim3 grid(p.num_parts, p.num_kv_heads * p.head_chunks, p.num_seqs);
    hipLaunchKernelGGL((attn_kernel<DT, D, GT, true>), grid, block, lds, stream, p);
  }
  return static_cast<int>(hipGetLastError());
}

template <int DT, int D>
int launch_attn(int kind, const AttnParams& p, hipStream_t stream) {
  if (kind == 2) {
    const dim3 grid(p.num_seqs * p.num_q_heads);
    hipLaunchKernelGGL((merge_kernel<DT, D>), grid, dim3(kThreads), 0, stream, p);
    return static_cast<int>(hipGetLastError());
  }
  switch (p.heads_per_wg) {
    case 1: return launch_attn_gt<DT, D, 1>(kind, p, stream);
    case 2: return launch_attn_gt<DT, D, 2>(kind, p, stream);
    case 3: return launch_attn_gt<DT, D, 3>(kind, p, stream);
    case 4: return launch_attn_gt<DT, D, 4>(kind, p, stream);
    case 5: return launch_attn_gt<DT, D, 5>(kind, p, stream);
    case 6: return launch_attn_gt<DT, D, 6>(kind, p, stream);
    case 7: return launch_attn_gt<DT, D, 7>(kind, p, stream);
    case 8: return launch_attn_gt<DT, D, 8>(kind, p, stream);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace pa
