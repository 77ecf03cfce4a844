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

// Token layout inside a workgroup.  Work is cut into units of 16 tokens (one
// block of 16, or one half of a block of 32), and wave w takes units w, w+4,
// ... of the chunk.
//  QK: 8 lanes per token, each holding KC = D/64 16-byte chunks of the K row
//      (dims c*64 + kcol*8 .. +8): a wave load covers 8 tokens x 128 bytes,
//      and a 3-step DPP sum finishes each dot product.
//  PV: VL = D/8 lanes per token, each holding 8 consecutive dims: a wave
//      load covers VTOK = 64/VL tokens; each lane accumulates its 8 dims for
//      every head of the group.
template <int D, int GT>
struct Tile {
  static constexpr int UNIT = 16;
  static constexpr int KC = D / 64;
  static constexpr int KTOK = 8;
  static constexpr int KGROUPS = UNIT / KTOK;       // 2
  static constexpr int KLOADS = KGROUPS * KC;       // 16-byte loads per lane per unit
  static constexpr int VL = D / 8;
  static constexpr int VTOK = 64 / VL;
  static constexpr int VLOADS = UNIT / VTOK;
  static constexpr int GTP = GT == 1 ? 1 : (GT == 2 ? 2 : (GT <= 4 ? 4 : 8));
};

// LDS (floats): logits / probabilities [chunk][GTP], wave partial outputs
// [kWaves][GT][D], wave maxima and sums [kWaves][GTP] each.
__host__ __device__ constexpr size_t lds_floats(int D, int GT, int GTP, int chunk) {
  return static_cast<size_t>(chunk) * GTP + static_cast<size_t>(kWaves) * GT * D +
         2 * static_cast<size_t>(kWaves) * GTP;
}

template <int N>
__device__ inline void lds_store(float* dst, const float (&v)[N]) {
  if constexpr (N >= 4) {
#pragma unroll
    for (int k = 0; k < N; k += 4)
      *reinterpret_cast<float4*>(dst + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
  } else if constexpr (N == 2) {
    *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
  } else {
    dst[0] = v[0];
  }
}

template <int N>
__device__ inline void lds_load(float (&v)[N], const float* src) {
  if constexpr (N >= 4) {
#pragma unroll
    for (int k = 0; k < N; k += 4) {
      const float4 f = *reinterpret_cast<const float4*>(src + k);
      v[k] = f.x; v[k + 1] = f.y; v[k + 2] = f.z; v[k + 3] = f.w;
    }
  } else if constexpr (N == 2) {
    const float2 f = *reinterpret_cast<const float2*>(src);
    v[0] = f.x; v[1] = f.y;
  } else {
    v[0] = src[0];
  }
}

// Buffer resource over one physical block (the base is wave-uniform).  With
// num_records = 0 every load through it is out of range: the hardware returns
// zeros without touching memory, which makes prefetches past a wave's last
// unit free.
__device__ inline __amdgpu_buffer_rsrc_t block_rsrc(const char* base, bool live) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, live ? 0x7fffffff : 0,
                                           0x00020000);
}

__device__ inline uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Wave-wide reductions that leave the result in every lane: a DPP butterfly
// inside each 16-lane row, then the four row results read back as scalars.
__device__ inline float wave_max_all(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ inline float wave_sum_all(float x) {
  x = group_sum<16>(x);
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return (a + b) + (c + d);
}

// Makes a wave's own LDS writes visible to its other lanes before they read.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Each wave runs its own softmax over its own units: logits, its running max
// m, sum l and accumulator acc (in the base-2 domain), with no workgroup
// barrier until the four waves' (m, l, acc) are combined at the end:
//   M = max_w m_w,  acc = sum_w 2^(m_w - M) acc_w,  l = sum_w 2^(m_w - M) l_w.
template <int DT, int D, int GT, bool SPLIT>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnParams p) {
  using F = Fmt<DT>;
  using TL = Tile<D, GT>;
  constexpr int UNIT = TL::UNIT, KC = TL::KC, KGROUPS = TL::KGROUPS, KLOADS = TL::KLOADS;
  constexpr int VL = TL::VL, VTOK = TL::VTOK, VLOADS = TL::VLOADS, GTP = TL::GTP;
  extern __shared__ float lds[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int krow = lane >> 3, kcol = lane & 7;      // QK: token row, 16-byte column
  const int vrow = lane / VL, vcol = lane % VL;     // PV: token row, 16-byte column

  // Which (sequence, KV head x head chunk, partition) this workgroup serves.
  //  single pass:  grid (KV heads x chunks, sequences)
  //  split, list:  1-D grid over work items x (KV heads x chunks); the KV
  //                heads of an item (one token row) land on one XCD, and
  //                items come from the caller, one per live (sequence,
  //                partition), so no workgroup is empty
  //  split, dense: grid (partitions, KV heads x chunks, sequences), partitions
  //                fastest and their count odd: workgroups go to the 8 XCDs
  //                round-robin by linear id, and an odd stride rotates each
  //                sequence's partition p across them (partition p exists only
  //                for sequences longer than p * P, so a fixed mapping would
  //                load the XCDs unevenly)
  int seq, kvhc, part = 0;
  if constexpr (!SPLIT) {
    kvhc = blockIdx.x;
    seq = blockIdx.y;
  } else {
    if (p.work_items) {
      // linear id = (item / 8) * 8 * nkv + kvhc * 8 + item % 8: ids equal mod 8
      // share an XCD, so the KV heads of one item (one token row) do
      const int nkv = p.num_kv_heads * p.head_chunks;
      const int grp = blockIdx.x / (8 * nkv);
      const int r = blockIdx.x - grp * 8 * nkv;
      kvhc = r >> 3;
      const int item = grp * 8 + (r & 7);
      if (item >= p.num_work_items) return;         // uniform: whole workgroup
      seq = p.work_items[2 * item];
      part = p.work_items[2 * item + 1];
      if (static_cast<unsigned>(seq) >= static_cast<unsigned>(p.num_seqs) ||
          static_cast<unsigned>(part) >= static_cast<unsigned>(p.num_parts))
        return;                                     // uniform: whole workgroup
    } else {
      part = blockIdx.x;
      kvhc = blockIdx.y;
      seq = blockIdx.z;
      if (part >= p.num_parts) return;
    }
  }
  const int kvh = kvhc / p.head_chunks;
  const int hc = kvhc - kvh * p.head_chunks;
  const int head0 = kvh * p.group + hc * GT;
  const int nact = min(GT, p.group - hc * GT);    // active heads of this chunk

  int L = p.context_lens[seq];
  L = max(0, min(L, p.mb * p.block_size));         // never past the table row
  int t_begin = 0, t_end = L;
  if constexpr (SPLIT) {
    t_begin = part * p.chunk;
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

  const int32_t* bt = p.block_tables + static_cast<int64_t>(seq) * p.mb;
  const char* kbase = static_cast<const char*>(p.k_cache);
  const char* vbase = static_cast<const char*>(p.v_cache);
  const int64_t block_bytes = p.block_stride * 2;
  const uint32_t tok_bytes = static_cast<uint32_t>(p.num_kv_heads) * D * 2;
  const uint32_t head_off = static_cast<uint32_t>(kvh) * D * 2;
  const uint32_t koff = static_cast<uint32_t>(krow) * tok_bytes + head_off + kcol * 16;
  const uint32_t voff = static_cast<uint32_t>(vrow) * tok_bytes + head_off + vcol * 16;
  const int bs_mask = p.block_size - 1;

  float* s_lds = lds;                                       // [chunk][GTP]
  float* red = lds + static_cast<size_t>(p.chunk) * GTP;    // [kWaves][GT][D]
  float* wmax = red + kWaves * GT * D;                      // [kWaves][GTP]
  float* wsum = wmax + kWaves * GTP;                        // [kWaves][GTP]

  float acc[GT][8];
  float m_run[GT], l_run[GT];                       // wave-uniform
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    m_run[hh] = -__builtin_inff();
    l_run[hh] = 0.f;
    if constexpr (!SPLIT) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
    }
  }

  // One chunk of n tokens from c0 for this wave's units (u = wave, wave + 4,
  // ...): logits, its own softmax statistics, P.V.  The split kernel runs it
  // once (q is dead after the logits and acc is born at the softmax, so the
  // two never share registers); the single-pass kernel loops.
  auto run_chunk = [&](const int c0, const int n) {
    const int nunits = (n + UNIT - 1) / UNIT;
    const int cnt = nunits > wave ? (nunits - wave + kWaves - 1) / kWaves : 0;
    if (cnt == 0) {                                 // uniform: this wave has no tokens
      if constexpr (SPLIT) {
#pragma unroll
        for (int hh = 0; hh < GT; ++hh)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
      }
      return;
    }

    // base of the i-th unit of this wave (clamped to its last unit; loads for
    // i >= cnt go through an empty descriptor and fetch nothing)
    auto unit_base = [&](const char* pool, int i) -> const char* {
      const int u = wave + kWaves * min(i, cnt - 1);
      const int t0 = c0 + u * UNIT;
      int blk = __builtin_amdgcn_readfirstlane(bt[t0 >> p.log2_block_size]);
      blk = (static_cast<unsigned>(blk) < static_cast<unsigned>(p.num_blocks)) ? blk : 0;
      return pool + blk * block_bytes + static_cast<int64_t>(t0 & bs_mask) * tok_bytes;
    };
    auto load_k = [&](uint4 (&dst)[KLOADS], int i) {
      const auto r = block_rsrc(unit_base(kbase, i), i < cnt);
#pragma unroll
      for (int j = 0; j < KGROUPS; ++j)
#pragma unroll
        for (int c = 0; c < KC; ++c)
          dst[j * KC + c] = load16(r, koff + c * 128, j * 8 * tok_bytes);
    };
    auto load_v = [&](uint4 (&dst)[VLOADS], int i) {
      const auto r = block_rsrc(unit_base(vbase, i), i < cnt);
#pragma unroll
      for (int j = 0; j < VLOADS; ++j) dst[j] = load16(r, voff, j * VTOK * tok_bytes);
    };

    // q slices for the QK layout: chunk c of head hh = dims c*64 + kcol*8 .. +8
    uint4 qv[GT][KC];
    {
      const uint16_t* q = static_cast<const uint16_t*>(p.q);
#pragma unroll
      for (int hh = 0; hh < GT; ++hh)
#pragma unroll
        for (int c = 0; c < KC; ++c)
          qv[hh][c] = hh < nact
                          ? *reinterpret_cast<const uint4*>(q + (out_row0 + hh) * D + c * 64 + kcol * 8)
                          : make_uint4(0, 0, 0, 0);
    }
    // logits of one unit (raw q.k; scaled in the softmax step), written by
    // the lane holding column 0 of each token
    auto qk_unit = [&](const uint4 (&kx)[KLOADS], int i) {
      const int u = wave + kWaves * i;
#pragma unroll
      for (int j = 0; j < KGROUPS; ++j) {
        float sv[GTP];
#pragma unroll
        for (int hh = 0; hh < GT; ++hh) {
          float a = 0.f;
#pragma unroll
          for (int c = 0; c < KC; ++c) {
            const uint4 k = kx[j * KC + c];
            a = F::dot2(qv[hh][c].x, k.x, a);
            a = F::dot2(qv[hh][c].y, k.y, a);
            a = F::dot2(qv[hh][c].z, k.z, a);
            a = F::dot2(qv[hh][c].w, k.w, a);
          }
          sv[hh] = group_sum<8>(a);
        }
#pragma unroll
        for (int hh = GT; hh < GTP; ++hh) sv[hh] = 0.f;
        if (kcol == 0) lds_store(s_lds + (u * UNIT + j * 8 + krow) * GTP, sv);
      }
    };
    // P.V of one unit; tokens past the chunk end get V = 0 (their p is 0 and
    // their slots may hold NaN)
    auto pv_unit = [&](const uint4 (&vx)[VLOADS], int i) {
      const int u = wave + kWaves * i;
      const bool tail = (u + 1) * UNIT > n;
#pragma unroll
      for (int j = 0; j < VLOADS; ++j) {
        const int t = u * UNIT + j * VTOK + vrow;
        uint4 x = vx[j];
        if (tail && t >= n) x = make_uint4(0, 0, 0, 0);
        float pr[GTP];
        lds_load(pr, s_lds + t * GTP);
        float vf[8];
        vf[0] = F::lo(x.x); vf[1] = F::hi(x.x);
        vf[2] = F::lo(x.y); vf[3] = F::hi(x.y);
        vf[4] = F::lo(x.z); vf[5] = F::hi(x.z);
        vf[6] = F::lo(x.w); vf[7] = F::hi(x.w);
#pragma unroll
        for (int hh = 0; hh < GT; ++hh)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pr[hh], vf[e], acc[hh][e]);
        // keep each group's probabilities and widened V short-lived
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // ---- logits of the wave's units, double-buffered ----
    uint4 va[VLOADS];
    {
      uint4 ka[KLOADS], kb[KLOADS];
      load_k(ka, 0);
      for (int i = 0; i < cnt; i += 2) {
        load_k(kb, i + 1);
        qk_unit(ka, i);
        load_k(ka, i + 2);
        if (i + 1 < cnt) qk_unit(kb, i + 1);
      }
    }
    load_v(va, 0);                         // the first V unit streams in during the softmax
    wave_lds_sync();

    // ---- the wave's softmax over its tokens (lane l: wave tokens l, l+64, ...) ----
    const int wtok = cnt * UNIT;
    auto tok_of = [&](int r) { return (wave + kWaves * (r / UNIT)) * UNIT + (r % UNIT); };
    float mloc[GT];
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) mloc[hh] = -__builtin_inff();
    for (int r = lane; r < wtok; r += 64) {
      const int t = tok_of(r);
      float v[GTP];
      lds_load(v, s_lds + t * GTP);
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        v[hh] *= p.scale_log2;
        if (t < n) mloc[hh] = v[hh] > mloc[hh] ? v[hh] : mloc[hh];
      }
      lds_store(s_lds + t * GTP, v);
    }
    float m_new[GT], alpha[GT];
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      m_new[hh] = fmaxf(m_run[hh], wave_max_all(mloc[hh]));
      alpha[hh] = fast_exp2(m_run[hh] - m_new[hh]);   // 0 on the first chunk
      m_run[hh] = m_new[hh];
    }
    float lsum[GT];
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) lsum[hh] = 0.f;
    for (int r = lane; r < wtok; r += 64) {
      const int t = tok_of(r);
      float v[GTP];
      lds_load(v, s_lds + t * GTP);
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        const float pr = t < n ? fast_exp2(v[hh] - m_new[hh]) : 0.f;
        v[hh] = pr;
        lsum[hh] += pr;
      }
      lds_store(s_lds + t * GTP, v);
    }
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      l_run[hh] = l_run[hh] * alpha[hh] + wave_sum_all(lsum[hh]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = SPLIT ? 0.f : acc[hh][e] * alpha[hh];
    }
    wave_lds_sync();

    // ---- P . V of the wave's units, double-buffered ----
    {
      uint4 vb[VLOADS];
      for (int i = 0; i < cnt; i += 2) {
        load_v(vb, i + 1);
        pv_unit(va, i);
        load_v(va, i + 2);
        if (i + 1 < cnt) pv_unit(vb, i + 1);
      }
    }
    wave_lds_sync();                       // the next chunk rewrites this wave's rows
  };

  if constexpr (SPLIT) {
    run_chunk(t_begin, t_end - t_begin);
  } else {
    for (int c0 = t_begin; c0 < t_end; c0 += p.chunk) run_chunk(c0, min(p.chunk, t_end - c0));
  }

  // ---------------- combine the waves ----------------
#pragma unroll
  for (int hh = 0; hh < GT; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = wave_sum_from(acc[hh][e], VL);
  if (vrow == 0) {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      float* dst = red + (wave * GT + hh) * D + vcol * 8;
      *reinterpret_cast<float4*>(dst) = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      wmax[wave * GTP + hh] = m_run[hh];
      wsum[wave * GTP + hh] = l_run[hh];
    }
  }
  __syncthreads();

#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    if (hh >= nact) break;
    float mw[kWaves], M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = wmax[w * GTP + hh];
      M = fmaxf(M, mw[w]);
    }
    float wt[kWaves], lt = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      wt[w] = fast_exp2(mw[w] - M);                 // 0 for a wave without tokens
      lt += wt[w] * wsum[w * GTP + hh];
    }
    for (int d = tid; d < D; d += kThreads) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += wt[w] * red[(w * GT + hh) * D + d];
      if constexpr (SPLIT) {
        const int64_t slot = (out_row0 + hh) * p.num_parts + part;
        p.part_acc[slot * D + d] = v;
        if (d == 0) {
          p.part_max[slot] = M;
          p.part_sum[slot] = lt;
        }
      } else {
        static_cast<uint16_t*>(p.out)[(out_row0 + hh) * D + d] = F::narrow(v / lt);
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
  const int nkv = p.num_kv_heads * p.head_chunks;
  if (kind == 0) {
    const dim3 grid(nkv, p.num_seqs, 1);
    hipLaunchKernelGGL((attn_kernel<DT, D, GT, false>), grid, block, lds, stream, p);
  } else {
    const dim3 grid = p.work_items ? dim3(((p.num_work_items + 7) / 8) * 8 * nkv, 1, 1)
                                   : dim3(p.grid_parts, nkv, p.num_seqs);
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
