// pa_attn.h -- paged decode attention kernels for gfx950 (CDNA4, wave64).
//
// One query token per sequence attends over its paged K/V:
//   out[i][h] = sum_j softmax_j(scale * q[i][h] . K_i[j]) V_i[j]
// ("LLM推理优化：vLLM PagedAttention深度解析与工程实践", §二 formula; §4.1 for
// the paged layout and the v1 / v2 kernel split).  Query heads of one
// KV head (G = Hq / Hkv, "LLM推理优化技术地图", §2.3 GQA) are served by the
// same workgroup, so every K/V byte is read from HBM once for all of them.
//
// Workgroup = NW waves (4 for the split kernel, 8 for the single-pass one),
// one (sequence, KV head, head chunk[, partition]).  Its tokens are cut into
// units of 16 and wave w takes units w, w + NW, ...; each wave runs its own
// softmax over its units, chunk by chunk (the partition for the split
// kernel), in three phases:
//
//  1. logits.  8 lanes per token (16 for groups of 5 or more heads, the
//     narrow layout), each holding 16-byte pieces of the K row
//     (buffer_load_dwordx4), take partial dot products with the matching q
//     elements of every head of the group (v_dot2 on 16-bit pairs, fp32
//     accumulate); a DPP reduce-scatter over each 8-lane group leaves every
//     lane the finished dot product of one head, and the lanes that own a
//     head store its logit, already in the base-2 domain
//     (scale * log2 e * q.k), to the wave's rows of LDS and keep a running
//     max of it.
//  2. softmax.  The wave takes its max per head from those running maxima,
//     overwrites the logits with p = 2^(logit - max) and sums them.
//  3. P.V.  D/8 lanes per token, each holding 8 consecutive dims of the V
//     row (D/4 lanes with 4 dims in the narrow layout), accumulate p * V for
//     every head in fp32 registers.
//
// K and V stream through a ring of unit buffers per wave, every refill
// issued on every path so that the wait counts track the ring.  At the end
// the waves' (max, sum, acc) meet in LDS and combine with the log-sum-exp
// identity.  The single-pass kernel ("v1") keeps each wave's
// running max / sum / accumulator across chunks (rescaled by
// 2^(old max - new max)) and writes the normalised output; the split kernel
// ("v2") stores (max, sum, acc) of its partition and the merge kernel
// combines the partitions.
//
// Loads use a wave-uniform block base and per-lane 32-bit offsets, with the
// non-temporal cache policy (each K/V byte is read once).  A wave's
// block ids arrive in one vector load (lane i: its unit i) and are read back
// with readlane; the tail tokens of a span's last unit get logit -inf and V
// zero (the pools' unused slots may hold NaN).
//
// INT8 pools (Q8): the pools hold one signed byte per element and the rows'
// fp32 scales sit in [NB][Hkv][bs] arrays (a row dequantises to scale x
// code; "LLM推理优化技术地图：从KV Cache到量化与投机解码", §4.3 for INT8
// halving the KV bytes, the convention being this library's).  Each lane
// widens its codes into exact 16-bit pairs (|code| <= 127) for the same v_dot2
// products and multiplies the finished dot product by the token's K scale;
// in P.V the probability is multiplied by the token's V scale before the
// accumulation.  The scales ride in the same unit rings as the codes.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pa_internal.h"

namespace pa {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// unit loads each wave keeps in flight (K, then V): the single-pass kernel
// walks whole contexts with few workgroups per CU and wants a deeper ring
#ifndef PA_DEPTH_SPLIT
#define PA_DEPTH_SPLIT 2
#endif
#ifndef PA_DEPTH_SINGLE
#define PA_DEPTH_SINGLE 4
#endif
#ifndef PA_EARLY_V
#define PA_EARLY_V 1
#endif
#ifndef PA_DEPTH_SPLIT_Q8
#define PA_DEPTH_SPLIT_Q8 3
#endif
#ifndef PA_EARLY_V_Q8
#define PA_EARLY_V_Q8 0
#endif
constexpr int kDepthSplit = PA_DEPTH_SPLIT;
constexpr bool kEarlyV = PA_EARLY_V;
// INT8 units carry half the bytes of 16-bit ones; a ring of 3 with the V ring
// issued after the logits measured 4-8 % faster than the 16-bit settings
constexpr int kDepthSplitQ8 = PA_DEPTH_SPLIT_Q8;
constexpr bool kEarlyVQ8 = PA_EARLY_V_Q8;
constexpr int kDepthSingle = PA_DEPTH_SINGLE;

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
  // dot2(a, b, 0) in the three-operand encoding with an inline 0: the
  // compiler's two-operand form needs a move to zero its accumulator first
  __device__ static inline float dot2_first(uint32_t a, uint32_t b) {
    float r;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
  }
  // round to nearest even (the default rounding mode of v_cvt_f16_f32)
  __device__ static inline uint16_t narrow(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  // two floats that are integers of magnitude <= 2048 as an exact f16 pair
  __device__ static inline uint32_t pack_int(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
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
  __device__ static inline float dot2_first(uint32_t a, uint32_t b) {
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
  }
  // round to nearest even: add 0x7fff plus the lowest kept bit, truncate
  __device__ static inline uint16_t narrow(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
    return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  }
  // two floats that are integers of magnitude <= 256 as an exact bf16 pair
  // (their low 16 bits are zero)
  __device__ static inline uint32_t pack_int(float lo, float hi) {
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
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

// Sum over the lanes l, l ^ S, l ^ 2S, ... up to 64 for S = 8, 16 or 32: lane
// xor 8 by a DPP rotate inside the 16-lane row, xor 16 and xor 32 by the
// CDNA4 row swaps.  v_permlane16_swap(a, b) exchanges the odd rows of a with
// the even rows of b, so with a = b = x the two results add up to
// x[l] + x[l ^ 16] in every lane; v_permlane32_swap does the same with the
// two 32-lane halves.
template <int S>
__device__ inline float rows_sum(float x) {
  static_assert(S == 8 || S == 16 || S == 32, "row stride");
  if constexpr (S == 8) x += dpp<0x128>(x);   // row_ror:8
  if constexpr (S <= 16) {
    const uint32_t b = __float_as_uint(x);
    const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  }
  const uint32_t c = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Token layout inside a workgroup.  Work is cut into units of 16 tokens (one
// block of 16, or one half of a block of 32), and wave w takes units w, w+4,
// ... of the chunk.
//  QK: QL lanes per token, each holding KC = D / (8 QL) 16-byte chunks of the
//      K row (dims c*8*QL + kcol*8 .. +8): a wave load covers KTOK = 64 / QL
//      tokens.  With QL = 8 a token's lanes are one aligned 8-lane group and
//      a 3-step DPP sum finishes each dot product; with QL = 16 they are 8
//      lanes of an even row plus the same 8 of the next row (WaveAttn's
//      krow / kcol), summed by 3 DPP steps and one row swap.
//  PV: VL = D / VW lanes per token, each holding VW consecutive dims (16 or
//      8 bytes): a wave load covers VTOK = 64 / VL tokens; each lane
//      accumulates its VW dims for every head of the group.
// The narrow layout (QL 16, VW 4: half the q and accumulator registers per
// lane, for the same bytes per load instruction in QK) lets more waves share
// a SIMD when the group has many heads.
template <int D, int GT, bool NARROW>
struct Tile {
  static constexpr int UNIT = 16;
  static constexpr int QL = (NARROW && D >= 128) ? 16 : 8;
  static constexpr int KC = D / (8 * QL);
  static constexpr int KTOK = 64 / QL;
  static constexpr int KGROUPS = UNIT / KTOK;
  static constexpr int KLOADS = KGROUPS * KC;       // 16-byte loads per lane per unit
  static constexpr int VW = NARROW ? 4 : 8;
  static constexpr int VL = D / VW;
  static constexpr int VTOK = 64 / VL;
  static constexpr int VLOADS = UNIT / VTOK;
  static constexpr int GTP = GT == 1 ? 1 : (GT == 2 ? 2 : (GT <= 4 ? 4 : 8));
  static_assert(KC >= 1 && VL <= 32 && KGROUPS >= 1, "layout");
};

// QK layout over INT8 pools: QL lanes per token, each holding KB bytes (= KB
// dims) of the K row in one load; q needs QC 16-byte pieces (8 dims each) per
// head.  The narrow layout halves KB (and q) for groups of many heads.  P.V
// keeps Tile's lanes (VW codes per lane), so the wave combine is shared.
template <int D, bool NARROW>
struct TileQK8 {
  static constexpr int KB = (NARROW || D < 128) ? 8 : 16;
  static constexpr int QL = D / KB;
  static constexpr int KTOK = 64 / QL;
  static constexpr int KGROUPS = 16 / KTOK;
  static constexpr int QC = KB / 8;
  static_assert(QL == 8 || QL == 16, "group_sum covers 8 or 16 lanes");
};

// One unit's loads in a wave's ring: the data words and, for INT8 pools, the
// scale of the token each lane's words belong to.
template <typename Vec, int N, int NS>
struct UnitBuf {
  Vec d[N];
  float sc[NS];
};
template <typename Vec, int N>
struct UnitBuf<Vec, N, 0> {
  Vec d[N];
};

// Query heads per workgroup from which the narrow layout is used.
#ifndef PA_NARROW_MIN_GT
#define PA_NARROW_MIN_GT 5
#endif
template <int GT>
constexpr bool kNarrow = GT >= PA_NARROW_MIN_GT;

// LDS (floats): logits / probabilities [chunk][GTP], wave partial outputs
// [nw][GT][D], wave maxima and sums [nw][GTP] each, for nw waves.
__host__ __device__ constexpr size_t lds_floats(int D, int GT, int GTP, int chunk,
                                                int nw = kWaves) {
  return static_cast<size_t>(chunk) * GTP + static_cast<size_t>(nw) * GT * D +
         2 * static_cast<size_t>(nw) * GTP;
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

// Pool loads carry the non-temporal cache policy (the `nt` bit of the
// instruction's cache-policy field): every K/V byte is read once per decode,
// and streaming them through the caches this way measured 9-13 % less time
// for the partition kernel than the default policy (the same bytes, the same
// load instructions).
constexpr int kPoolLoadPolicy = 2;

__device__ inline uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kPoolLoadPolicy);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ inline uint2 load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kPoolLoadPolicy);
  return make_uint2(v[0], v[1]);
}

__device__ inline uint32_t load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kPoolLoadPolicy);
}

template <typename Vec>
__device__ inline Vec load_vec(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (std::is_same<Vec, uint4>::value) return load16(r, voff, soff);
  else if constexpr (std::is_same<Vec, uint2>::value) return load8(r, voff, soff);
  else return load4(r, voff, soff);
}

// The 32-bit words of a lane's load, in memory order.
template <typename Vec>
struct Words;
template <>
struct Words<uint4> {
  static constexpr int N = 4;
  __device__ static inline void get(const uint4& v, uint32_t (&w)[4]) {
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
};
template <>
struct Words<uint2> {
  static constexpr int N = 2;
  __device__ static inline void get(const uint2& v, uint32_t (&w)[2]) {
    w[0] = v.x; w[1] = v.y;
  }
};
template <>
struct Words<uint32_t> {
  static constexpr int N = 1;
  __device__ static inline void get(const uint32_t& v, uint32_t (&w)[1]) { w[0] = v; }
};

// Byte k of w as a signed integer, widened to fp32 (one SDWA conversion).
template <int K>
__device__ inline float code_at(uint32_t w) {
  return static_cast<float>(static_cast<int8_t>(w >> (8 * K)));
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

// Per-wave pieces shared by the single-pass and split kernels.  Everything
// here is wave-uniform except what a lane holds of q, K, V, the block ids
// and the accumulators.
template <int DT, int D, int GT, bool Q8 = false, int NW = kWaves>
struct WaveAttn {
  using F = Fmt<DT>;
  using TL = Tile<D, GT, kNarrow<GT>>;
  using T8 = TileQK8<D, kNarrow<GT>>;
  static constexpr int UNIT = TL::UNIT;
  // QK: KC = 16-byte q pieces per head; KLOADS = K loads per lane per unit
  static constexpr int QL = Q8 ? T8::QL : TL::QL, KC = Q8 ? T8::QC : TL::KC,
                       KTOK = Q8 ? T8::KTOK : TL::KTOK,
                       KGROUPS = Q8 ? T8::KGROUPS : TL::KGROUPS,
                       KLOADS = Q8 ? T8::KGROUPS : TL::KLOADS;
  static constexpr int VW = TL::VW, VL = TL::VL, VTOK = TL::VTOK, VLOADS = TL::VLOADS,
                       GTP = TL::GTP;
  static constexpr int EB = Q8 ? 1 : 2;   // bytes per pool element
  // a lane's piece of a K row (16 bytes, or 8 for narrow INT8 rows)
  using KVec = typename std::conditional<!Q8 || T8::KB == 16, uint4, uint2>::type;
  // a lane's piece of a V row: VW elements
  using VVec = typename std::conditional<
      Q8, typename std::conditional<VW == 8, uint2, uint32_t>::type,
      typename std::conditional<VW == 8, uint4, uint2>::type>::type;
  using KBuf = UnitBuf<KVec, KLOADS, Q8 ? KGROUPS : 0>;
  using VBuf = UnitBuf<VVec, VLOADS, Q8 ? VLOADS : 0>;

  // Tokens [c0, c0 + n) of one sequence as one wave sees them: its units are
  // u = wave, wave + NW, ... below ceil(n / UNIT), cnt of them.  Lane i of blk
  // holds the physical block of the wave's unit i, fetched by one vector load
  // and read back with readlane when the unit's loads are issued.
  struct Span {
    int c0, n, cnt;
    int blk;
  };

  int wave, lane, krow, kcol, vrow, vcol;
  // QK: the head whose dot product this lane holds after the sum over its
  // aligned 8-lane group (qk_sum); lanes with (lane & 7) < GTP write it
  int qhead;
  const char* kbase;
  const char* vbase;
  const uint16_t* q;
  int64_t block_bytes;
  uint32_t tok_bytes, koff, voff;
  // INT8 scales [NB][Hkv][bs]: block stride, and per-lane offsets of the
  // lane's first token inside a unit for this KV head
  const char* ksbase;
  const char* vsbase;
  int64_t sc_block_bytes;
  uint32_t ksoff, vsoff;
  int bs_mask, log2_bs, num_blocks;
  float scale_log2;
  float* s_lds;   // [chunk][GTP]: logits, then probabilities; a unit's rows belong to its wave

  __device__ __forceinline__ WaveAttn(const AttnParams& p, int kvh, float* lds) {
    const int tid = threadIdx.x;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    lane = tid & 63;
    if constexpr (QL == 16) {
      // a token's 16 lanes: 8 in an even row and the same 8 in the next row
      // (lanes l and l + 16), so the last step of the dot-product sum is a
      // row swap that finishes two token groups at once
      krow = 2 * (lane >> 5) + ((lane >> 3) & 1);
      kcol = (lane & 7) + 8 * ((lane >> 4) & 1);
    } else {
      krow = lane / QL;
      kcol = lane % QL;
    }
    vrow = lane / VL;
    vcol = lane % VL;
    {
      const int b = lane & 7;
      qhead = GTP == 8 ? b : ((b & (GTP - 1)) ^ ((b & 4) ? GTP - 1 : 0));
    }
    kbase = static_cast<const char*>(p.k_cache);
    vbase = static_cast<const char*>(p.v_cache);
    q = static_cast<const uint16_t*>(p.q);
    block_bytes = p.block_stride * EB;
    tok_bytes = static_cast<uint32_t>(p.num_kv_heads) * D * EB;
    const uint32_t head_off = static_cast<uint32_t>(kvh) * D * EB;
    koff = static_cast<uint32_t>(krow) * tok_bytes + head_off + kcol * (Q8 ? T8::KB : 16);
    voff = static_cast<uint32_t>(vrow) * tok_bytes + head_off + vcol * VW * EB;
    if constexpr (Q8) {
      ksbase = reinterpret_cast<const char*>(p.k_scale);
      vsbase = reinterpret_cast<const char*>(p.v_scale);
      sc_block_bytes = static_cast<int64_t>(p.num_kv_heads) * p.block_size * 4;
      const uint32_t sc_head = static_cast<uint32_t>(kvh) * p.block_size * 4;
      ksoff = sc_head + static_cast<uint32_t>(krow) * 4;
      vsoff = sc_head + static_cast<uint32_t>(vrow) * 4;
    }
    bs_mask = p.block_size - 1;
    log2_bs = p.log2_block_size;
    num_blocks = p.num_blocks;
    scale_log2 = p.scale_log2;
    s_lds = lds;
  }

  // bt is the sequence's table row and c0 + n must not pass the tokens it
  // maps; n <= 0 gives an empty span that reads nothing.
  __device__ __forceinline__ Span span(const int32_t* bt, int c0, int n) const {
    Span s;
    s.c0 = c0;
    s.n = n;
    const int nunits = n > 0 ? (n + UNIT - 1) / UNIT : 0;
    s.cnt = nunits > wave ? (nunits - wave + NW - 1) / NW : 0;
    s.blk = 0;
    if (lane < s.cnt) s.blk = bt[(c0 + (wave + NW * lane) * UNIT) >> log2_bs];
    return s;
  }

  // Byte offset from a pool's start of the wave's unit i, clamped to its last
  // unit; block 0 when the wave has no unit or the entry is out of range.
  __device__ __forceinline__ int64_t unit_off(const Span& s, int i) const {
    const int j = max(0, min(i, s.cnt - 1));
    int blk = __builtin_amdgcn_readlane(s.blk, j);
    blk = static_cast<unsigned>(blk) < static_cast<unsigned>(num_blocks) ? blk : 0;
    const int t0 = s.c0 + (wave + NW * j) * UNIT;
    return blk * block_bytes + static_cast<int64_t>(t0 & bs_mask) * tok_bytes;
  }
  // The same unit in a scale array [NB][Hkv][bs] (KV head offset excluded).
  __device__ __forceinline__ int64_t unit_scale_off(const Span& s, int i) const {
    const int j = max(0, min(i, s.cnt - 1));
    int blk = __builtin_amdgcn_readlane(s.blk, j);
    blk = static_cast<unsigned>(blk) < static_cast<unsigned>(num_blocks) ? blk : 0;
    const int t0 = s.c0 + (wave + NW * j) * UNIT;
    return blk * sc_block_bytes + static_cast<int64_t>(t0 & bs_mask) * 4;
  }

  // Loads of unit i >= cnt go through an empty descriptor and fetch nothing.
  __device__ __forceinline__ void load_k(KBuf& dst, const Span& s, int i) const {
    const auto r = block_rsrc(kbase + unit_off(s, i), i < s.cnt);
    if constexpr (Q8) {
      const auto rs = block_rsrc(ksbase + unit_scale_off(s, i), i < s.cnt);
#pragma unroll
      for (int j = 0; j < KGROUPS; ++j) {
        dst.d[j] = load_vec<KVec>(r, koff, j * KTOK * tok_bytes);
        dst.sc[j] = __uint_as_float(load4(rs, ksoff, j * KTOK * 4));
      }
    } else {
#pragma unroll
      for (int j = 0; j < KGROUPS; ++j)
#pragma unroll
        for (int c = 0; c < KC; ++c)
          dst.d[j * KC + c] = load16(r, koff + c * QL * 16, j * KTOK * tok_bytes);
    }
  }
  __device__ __forceinline__ void load_v(VBuf& dst, const Span& s, int i) const {
    const auto r = block_rsrc(vbase + unit_off(s, i), i < s.cnt);
    if constexpr (Q8) {
      const auto rs = block_rsrc(vsbase + unit_scale_off(s, i), i < s.cnt);
#pragma unroll
      for (int j = 0; j < VLOADS; ++j) {
        dst.d[j] = load_vec<VVec>(r, voff, j * VTOK * tok_bytes);
        dst.sc[j] = __uint_as_float(load4(rs, vsoff, j * VTOK * 4));
      }
    } else {
#pragma unroll
      for (int j = 0; j < VLOADS; ++j) {
        if constexpr (VW == 8)
          dst.d[j] = load16(r, voff, j * VTOK * tok_bytes);
        else
          dst.d[j] = load8(r, voff, j * VTOK * tok_bytes);
      }
    }
  }

  // q slices for the QK layout: chunk c = dims c*8*QL + kcol*8 .. +8 (INT8:
  // dims kcol*KB + c*8 .. +8, the lane's codes) of the head in slot r, which
  // is head r ^ qhead (the slot order qk_sum's reduce-scatter needs).
  // Heads past nact (and slots past the group) reread the last active head:
  // their results are never used, and loads on every path keep the wait
  // counts exact.
  __device__ __forceinline__ void load_q(uint4 (&qv)[GTP][KC], int64_t row0, int nact) const {
#pragma unroll
    for (int r = 0; r < GTP; ++r)
#pragma unroll
      for (int c = 0; c < KC; ++c)
        qv[r][c] = *reinterpret_cast<const uint4*>(
            q + (row0 + min(r ^ qhead, nact - 1)) * D +
            (Q8 ? kcol * T8::KB + c * 8 : c * 8 * QL + kcol * 8));
  }

  // The lane's part of the raw q.k of its token in load group j, q slot hh.
  __device__ __forceinline__ float qk_part(const uint4 (&qv)[GTP][KC], const KBuf& kx, int j,
                                           int hh) const {
    if constexpr (Q8) {
      // the lane's codes as exact 16-bit pairs, in dim order: pair m holds
      // dims 2m, 2m + 1 of the lane's KB
      constexpr int NWD = Words<KVec>::N;
      uint32_t w[NWD], kp[2 * NWD];
      Words<KVec>::get(kx.d[j], w);
#pragma unroll
      for (int m = 0; m < NWD; ++m) {
        kp[2 * m] = F::pack_int(code_at<0>(w[m]), code_at<1>(w[m]));
        kp[2 * m + 1] = F::pack_int(code_at<2>(w[m]), code_at<3>(w[m]));
      }
      float a = F::dot2_first(qv[hh][0].x, kp[0]);
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if (c > 0) a = F::dot2(qv[hh][c].x, kp[4 * c], a);
        a = F::dot2(qv[hh][c].y, kp[4 * c + 1], a);
        a = F::dot2(qv[hh][c].z, kp[4 * c + 2], a);
        a = F::dot2(qv[hh][c].w, kp[4 * c + 3], a);
      }
      return a;
    } else {
      float a = F::dot2_first(qv[hh][0].x, kx.d[j * KC].x);
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const uint4 k = kx.d[j * KC + c];
        if (c > 0) a = F::dot2(qv[hh][c].x, k.x, a);
        a = F::dot2(qv[hh][c].y, k.y, a);
        a = F::dot2(qv[hh][c].z, k.z, a);
        a = F::dot2(qv[hh][c].w, k.w, a);
      }
      return a;
    }
  }

  // Sum over the lane's aligned 8-lane group of the products of every q
  // slot, as a reduce-scatter: slot r of lane b holds head r ^ qhead(b), so
  // each step adds half of a lane's slots to the partner lane's matching
  // slots (lane ^ 7: row_half_mirror; lane ^ 2, lane ^ 1: quad permutes) and
  // keeps the other half, and the lane ends with the group's total for its
  // own head qhead.  8 heads take 4 + 2 + 1 DPP adds instead of 3 per head;
  // with fewer slots the remaining steps are plain sums (qhead is chosen so
  // that a lane and its lane ^ 7 partner hold the same head).
  __device__ __forceinline__ float qk_sum(const float (&a)[GTP]) const {
    if constexpr (GTP == 8) {
      const float t0 = a[0] + dpp<0x141>(a[7]), t1 = a[1] + dpp<0x141>(a[6]);
      const float t2 = a[2] + dpp<0x141>(a[5]), t3 = a[3] + dpp<0x141>(a[4]);
      const float u0 = t0 + dpp<0x4E>(t2), u1 = t1 + dpp<0x4E>(t3);
      return u0 + dpp<0xB1>(u1);
    } else if constexpr (GTP == 4) {
      const float u0 = a[0] + dpp<0x4E>(a[2]), u1 = a[1] + dpp<0x4E>(a[3]);
      const float v = u0 + dpp<0xB1>(u1);
      return v + dpp<0x141>(v);
    } else if constexpr (GTP == 2) {
      float v = a[0] + dpp<0xB1>(a[1]);
      v += dpp<0x4E>(v);
      return v + dpp<0x141>(v);
    } else {
      return group_sum<8>(a[0]);
    }
  }

  // Logits of the wave's unit i in the base-2 domain (scale * log2 e * q.k),
  // one per (token, head) from the lanes that hold a head of their own
  // ((lane & 7) < GTP); tokens past the span get -inf (their slots may hold
  // NaN).  qmax gathers the lane's largest logit (of head qhead).
  __device__ __forceinline__ void qk_unit(const uint4 (&qv)[GTP][KC], const KBuf& kx, int i,
                                          const Span& s, float& qmax) const {
    const int u = wave + NW * i;
    const bool tail = (u + 1) * UNIT > s.n;     // uniform: only the span's last unit
    const bool writer = (lane & 7) < GTP;
    auto finish = [&](float v, int tok) {
      v *= scale_log2;
      if (tail) v = tok < s.n ? v : -__builtin_inff();
      qmax = fmaxf(qmax, v);
      if (writer) s_lds[tok * GTP + qhead] = v;
    };
    if constexpr (QL == 16) {
      // groups j and j + 1 together: each lane's 8-lane sum covers half of a
      // token, then v_permlane16_swap trades rows so that one add leaves
      // group j's totals in rows 0 and 2 and group j + 1's in rows 1 and 3
      static_assert(KGROUPS % 2 == 0, "QK groups come in pairs");
      const int odd = (lane >> 4) & 1;
#pragma unroll
      for (int j = 0; j < KGROUPS; j += 2) {
        // one group at a time: all GTP partial sums of a group are live
        // until its reduce-scatter
        float a[GTP];
#pragma unroll
        for (int r = 0; r < GTP; ++r) a[r] = qk_part(qv, kx, j, r);
        const float v0 = qk_sum(a);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < GTP; ++r) a[r] = qk_part(qv, kx, j + 1, r);
        const float v1 = qk_sum(a);
        const auto rr = __builtin_amdgcn_permlane16_swap(__float_as_uint(v0),
                                                         __float_as_uint(v1), false, false);
        float v = __uint_as_float(rr[0]) + __uint_as_float(rr[1]);
        if constexpr (Q8) v *= odd ? kx.sc[j + 1] : kx.sc[j];
        finish(v, u * UNIT + (j + odd) * KTOK + krow);
      }
    } else {
#pragma unroll
      for (int j = 0; j < KGROUPS; ++j) {
        float a[GTP];
#pragma unroll
        for (int r = 0; r < GTP; ++r) a[r] = qk_part(qv, kx, j, r);
        float v = qk_sum(a);
        if constexpr (Q8) v *= kx.sc[j];
        finish(v, u * UNIT + j * KTOK + krow);
      }
    }
  }

  // P.V of the wave's unit i; tokens past n get V = 0 (their p is 0 and their
  // slots may hold NaN).
  __device__ __forceinline__ void pv_unit(float (&acc)[GT][VW], VBuf& vx,
                                          const Span& s, int i) const {
    const int u = wave + NW * i;
    if ((u + 1) * UNIT > s.n) {   // uniform: only the span's last unit
      asm volatile("");   // keeps this a branch (not selects on every unit)
#pragma unroll
      for (int j = 0; j < VLOADS; ++j) {
        if (u * UNIT + j * VTOK + vrow >= s.n) {
          if constexpr (Q8)
            vx.sc[j] = 0.f;
          else
            vx.d[j] = VVec{};
        }
      }
    }
    if constexpr (Q8) {
#pragma unroll
      for (int j = 0; j < VLOADS; ++j) {
        const int t = u * UNIT + j * VTOK + vrow;
        const float vs = vx.sc[j];   // 0 past the span
        constexpr int NWD = Words<VVec>::N;
        uint32_t w[NWD];
        Words<VVec>::get(vx.d[j], w);
        float vf[VW];
#pragma unroll
        for (int m = 0; m < NWD; ++m) {
          vf[4 * m] = code_at<0>(w[m]);
          vf[4 * m + 1] = code_at<1>(w[m]);
          vf[4 * m + 2] = code_at<2>(w[m]);
          vf[4 * m + 3] = code_at<3>(w[m]);
        }
        float pr[GTP];
        lds_load(pr, s_lds + t * GTP);
#pragma unroll
        for (int hh = 0; hh < GT; ++hh) {
          const float pw = pr[hh] * vs;
#pragma unroll
          for (int e = 0; e < VW; ++e) acc[hh][e] = fmaf(pw, vf[e], acc[hh][e]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < VLOADS; ++j) {
        const int t = u * UNIT + j * VTOK + vrow;
        uint32_t w[VW / 2];
        if constexpr (VW == 8) {
          w[0] = vx.d[j].x; w[1] = vx.d[j].y; w[2] = vx.d[j].z; w[3] = vx.d[j].w;
        } else {
          w[0] = vx.d[j].x; w[1] = vx.d[j].y;
        }
        float pr[GTP];
        lds_load(pr, s_lds + t * GTP);
        float vf[VW];
#pragma unroll
        for (int e = 0; e < VW / 2; ++e) {
          vf[2 * e] = F::lo(w[e]);
          vf[2 * e + 1] = F::hi(w[e]);
        }
#pragma unroll
        for (int hh = 0; hh < GT; ++hh)
#pragma unroll
          for (int e = 0; e < VW; ++e) acc[hh][e] = fmaf(pr[hh], vf[e], acc[hh][e]);
        // keep each group's probabilities and widened V short-lived
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Logits of all the wave's units through a ring of DEPTH unit buffers:
  // units 0 .. DEPTH-1 are already on their way, and the buffer unit i was
  // consumed from refills with unit i + DEPTH.  Every refill is issued, past
  // the wave's last unit through the empty descriptor: with the loads on
  // every path the compiler's wait counts see the ring in issue order and
  // wait for one unit at a time (a skipped refill would make it wait for all).
  template <int DEPTH>
  __device__ __forceinline__ void logits(const uint4 (&qv)[GTP][KC], KBuf (&kb)[DEPTH],
                                         const Span& s, float& qmax) const {
    for (int i = 0; i < s.cnt; i += DEPTH) {
#pragma unroll
      for (int b = 0; b < DEPTH; ++b) {
        if (b == 0 || i + b < s.cnt) qk_unit(qv, kb[b], i + b, s, qmax);   // uniform
        load_k(kb[b], s, i + b + DEPTH);
      }
    }
  }

  // The wave's softmax over its tokens of the span, from the logits qk_unit
  // left in LDS (base-2 domain, -inf past the span) and each lane's qmax:
  // folds the wave's max per head into m_run, overwrites the logits with
  // p = 2^(logit - m_run) (lane l takes the wave's tokens l, l + 64, ...), and
  // sets l_run = alpha * l_run + sum p with alpha = 2^(old m_run - new
  // m_run), which it returns for the caller's accumulator.
  __device__ __forceinline__ void softmax(const Span& s, float qmax, float (&m_run)[GT],
                                          float (&l_run)[GT], float (&alpha)[GT]) const {
    const int wtok = s.cnt * UNIT;
    auto tok_of = [&](int r) { return (wave + NW * (r / UNIT)) * UNIT + (r % UNIT); };
    // lanes l, l ^ 8, ..., l ^ 56 hold the same head: the wave's max per head
    float mx = fmaxf(qmax, dpp<0x128>(qmax));   // row_ror:8
    {
      const uint32_t b = __float_as_uint(mx);
      const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
      mx = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
      const uint32_t c = __float_as_uint(mx);
      const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
      mx = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
    }
    float m_new[GT];
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      // lane hh (< 8) holds head hh
      const float mh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), hh));
      m_new[hh] = fmaxf(m_run[hh], mh);
      alpha[hh] = fast_exp2(m_run[hh] - m_new[hh]);   // 0 while m_run is -inf
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
        const float pr = fast_exp2(v[hh] - m_new[hh]);   // 0 past the span (-inf)
        v[hh] = pr;
        lsum[hh] += pr;
      }
      lds_store(s_lds + t * GTP, v);
    }
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) l_run[hh] = l_run[hh] * alpha[hh] + wave_sum_all(lsum[hh]);
  }

  // P.V over all the wave's units through a ring of DEPTH unit buffers, as
  // the logits.
  template <int DEPTH>
  __device__ __forceinline__ void values(float (&acc)[GT][VW], VBuf (&vb)[DEPTH],
                                         const Span& s) const {
    for (int i = 0; i < s.cnt; i += DEPTH) {
#pragma unroll
      for (int b = 0; b < DEPTH; ++b) {
        if (b == 0 || i + b < s.cnt) pv_unit(acc, vb[b], s, i + b);   // uniform
        load_v(vb[b], s, i + b + DEPTH);
      }
    }
  }
};

// The workgroup's result for query heads row0 .. row0 + nact - 1 of one
// sequence: the waves' (m_w, l_w, acc_w) meet in `red` and combine as
//   M = max_w m_w,  acc = sum_w 2^(m_w - M) acc_w,  l = sum_w 2^(m_w - M) l_w
// (a wave without tokens has m_w = -inf and weight 0).  Split: (acc, M, l)
// go to the partition's workspace slot; single pass: out = acc / l.
template <int DT, int D, int GT, bool SPLIT, int NW = kWaves>
__device__ __forceinline__ void combine_waves(const AttnParams& p,
                                              float (&acc)[GT][Tile<D, GT, kNarrow<GT>>::VW],
                                              const float (&m_w)[GT], const float (&l_w)[GT],
                                              float* red, int64_t row0, int nact, int part) {
  using TL = Tile<D, GT, kNarrow<GT>>;
  constexpr int VL = TL::VL, VW = TL::VW, GTP = TL::GTP;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int vrow = lane / VL, vcol = lane % VL;
  float* wmax = red + NW * GT * D;   // [NW][GTP]
  float* wsum = wmax + NW * GTP;     // [NW][GTP]
  // one head at a time: the scheduler would otherwise copy all GT * 8 values
  // before the first swap and hold twice the accumulators
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[hh][e] = rows_sum<VL>(acc[hh][e]);
    if (vrow == 0) {
      float* dst = red + (wave * GT + hh) * D + vcol * VW;
#pragma unroll
      for (int e = 0; e < VW; e += 4)
        *reinterpret_cast<float4*>(dst + e) =
            make_float4(acc[hh][e], acc[hh][e + 1], acc[hh][e + 2], acc[hh][e + 3]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      wmax[wave * GTP + hh] = m_w[hh];
      wsum[wave * GTP + hh] = l_w[hh];
    }
  }
  __syncthreads();

  // one float4 of one head per thread: GT * D / 4 <= 256 items, one pass
  constexpr int C4 = D / 4;
  for (int idx = tid; idx < GT * C4; idx += (64 * NW)) {
    const int hh = idx / C4;
    const int c = idx - hh * C4;
    if (hh >= nact) break;
    float mw[NW], M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = wmax[w * GTP + hh];
      M = fmaxf(M, mw[w]);
    }
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    float lt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = fast_exp2(mw[w] - M);
      lt += wt * wsum[w * GTP + hh];
      const float4 r = *reinterpret_cast<const float4*>(red + (w * GT + hh) * D + c * 4);
      v.x = fmaf(wt, r.x, v.x);
      v.y = fmaf(wt, r.y, v.y);
      v.z = fmaf(wt, r.z, v.z);
      v.w = fmaf(wt, r.w, v.w);
    }
    if constexpr (SPLIT) {
      // workspace rows [S][nP][Hq]: a workgroup's heads are one contiguous run
      const int64_t seq = row0 / p.num_q_heads;
      const int64_t slot = (seq * p.num_parts + part) * p.num_q_heads + (row0 - seq * p.num_q_heads) + hh;
      *reinterpret_cast<float4*>(p.part_acc + slot * D + c * 4) = v;
      if (c == 0) {
        p.part_max[slot] = M;
        p.part_sum[slot] = lt;
      }
    } else {
      using F = Fmt<DT>;
      const uint32_t lo = F::narrow(v.x / lt) | (static_cast<uint32_t>(F::narrow(v.y / lt)) << 16);
      const uint32_t hi = F::narrow(v.z / lt) | (static_cast<uint32_t>(F::narrow(v.w / lt)) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + (row0 + hh) * D + c * 4) =
          make_uint2(lo, hi);
    }
  }
}

// Single-pass decode ("v1"): workgroup = (KV head x head chunk, sequence) of
// NW waves; it walks the whole context in chunks of p.chunk tokens, each wave
// keeping its own running max / sum / accumulator across chunks (rescaled by
// alpha), and writes the normalised output.
//
// Longest context first: with up to one sequence per thread, grid row k
// serves the sequence of rank k by decreasing context length (ties by
// index), computed by every workgroup from the lengths (one per thread, ranks
// by counting).  Workgroups start in grid order, so the long contexts, whose
// workgroups set the end of the launch, start in the first wave of residency
// and the short ones fill the slots freed late (LLaMA-13B-shaped layer, 32
// sequences of 128..2048 tokens, 4 waves: 136.5 -> 113.2 us).  With more
// sequences than threads the grid keeps index order.
template <int DT, int D, int GT, bool Q8, int NW>
__global__ __launch_bounds__(64 * NW) void single_kernel(AttnParams p) {
  constexpr int NT = 64 * NW;
  using W = WaveAttn<DT, D, GT, Q8, NW>;
  extern __shared__ float lds[];
  __shared__ __attribute__((aligned(16))) int s_len[NT];
  __shared__ __attribute__((aligned(16))) int s_ord[NT];
  const int kvhc = blockIdx.x;
  int seq = blockIdx.y;
  if (p.num_seqs <= NT) {                    // uniform
    const int t = threadIdx.x;
    const int cap = p.mb * p.block_size;
    const int Lt = t < p.num_seqs ? max(0, min(p.context_lens[t], cap)) : -1;
    s_len[t] = Lt;                                 // -1 past the batch: ranks below all
    __syncthreads();
    int rank = 0;
    const int4* l4 = reinterpret_cast<const int4*>(s_len);
    for (int j4 = 0; j4 < (p.num_seqs + 3) / 4; ++j4) {
      const int4 v = l4[j4];
      const int j = 4 * j4;
      rank += (v.x > Lt) || (v.x == Lt && j < t);
      rank += (v.y > Lt) || (v.y == Lt && j + 1 < t);
      rank += (v.z > Lt) || (v.z == Lt && j + 2 < t);
      rank += (v.w > Lt) || (v.w == Lt && j + 3 < t);
    }
    if (t < p.num_seqs) s_ord[rank] = t;           // a permutation of 0 .. S - 1
    __syncthreads();
    seq = s_ord[blockIdx.y];
  }
  const int kvh = kvhc / p.head_chunks;
  const int hc = kvhc - kvh * p.head_chunks;
  const int head0 = kvh * p.group + hc * GT;
  const int nact = min(GT, p.group - hc * GT);   // active heads of this chunk
  const int64_t row0 = static_cast<int64_t>(seq) * p.num_q_heads + head0;

  int L = p.context_lens[seq];
  L = max(0, min(L, p.mb * p.block_size));         // never past the table row
  if (L == 0) {                                    // uniform: whole workgroup
    uint16_t* out = static_cast<uint16_t*>(p.out);
    for (int hh = 0; hh < nact; ++hh)
      for (int d = threadIdx.x; d < D; d += NT) out[(row0 + hh) * D + d] = 0;
    return;
  }

  const W w(p, kvh, lds);
  const int32_t* bt = p.block_tables + static_cast<int64_t>(seq) * p.mb;
  float acc[GT][W::VW], m_run[GT], l_run[GT];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    m_run[hh] = -__builtin_inff();
    l_run[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < W::VW; ++e) acc[hh][e] = 0.f;
  }
  for (int c0 = 0; c0 < L; c0 += p.chunk) {
    const typename W::Span s = w.span(bt, c0, min(p.chunk, L - c0));
    if (s.cnt == 0) continue;                      // uniform: this wave has no tokens
    float qmax = -__builtin_inff();
    {
      uint4 qv[W::GTP][W::KC];
      w.load_q(qv, row0, nact);                    // first: waiting for q must not wait for K
      typename W::KBuf kb[kDepthSingle];
#pragma unroll
      for (int b = 0; b < kDepthSingle; ++b) w.load_k(kb[b], s, b);
      w.template logits<kDepthSingle>(qv, kb, s, qmax);
    }
    typename W::VBuf vb[kDepthSingle];             // streams in during the softmax
#pragma unroll
    for (int b = 0; b < kDepthSingle; ++b) w.load_v(vb[b], s, b);
    wave_lds_sync();
    float alpha[GT];
    w.softmax(s, qmax, m_run, l_run, alpha);
#pragma unroll
    for (int hh = 0; hh < GT; ++hh)
#pragma unroll
      for (int e = 0; e < W::VW; ++e) acc[hh][e] *= alpha[hh];
    wave_lds_sync();
    w.template values<kDepthSingle>(acc, vb, s);
    wave_lds_sync();                               // the next chunk rewrites this wave's rows
  }
  combine_waves<DT, D, GT, false, NW>(p, acc, m_run, l_run, lds + static_cast<size_t>(p.chunk) * W::GTP,
                                  row0, nact, 0);
}

// Work-list grid: linear workgroup id -> (work item, KV head x chunk).  Ids
// come in groups of 8 * nkv: 8 consecutive items x the nkv KV heads (x head
// chunks), the KV heads of an item 8 ids apart, so that they share an XCD
// (workgroups go to the 8 XCDs round-robin by id) and read the same token
// rows.  Inside an XCD the dispatcher deals consecutive workgroups to its
// shader engines in turn (four of them on this part, measured), so a KV head
// fixed by the id's place in its group would put every workgroup of one head
// on the same shader engine: each engine then streams one head's slices
// only, at a fixed byte offset inside every token row.  One offset class of
// the K pool streams slower; the engine holding it became the end of the
// launch (its workgroups ~20 % longer, the last ~10 us of the launch spent on
// them).  So the KV head rotates with the group: every engine serves every
// head (Qwen2.5-7B-shaped layer: 121 -> 116 us per call).
__device__ __forceinline__ void list_item_of(int id, int nkv, int* item, int* kvhc) {
  const int grp = id / (8 * nkv);
  const int r = id - grp * 8 * nkv;
  // with 1, 2 or 4 heads the group's slots repeat every 4 workgroups of an
  // XCD, so the rotation advances once per 4 / nkv groups
  const int div = (nkv < 4 && 4 % nkv == 0) ? 4 / nkv : 1;
  *kvhc = ((r >> 3) + grp / div) % nkv;
  *item = grp * 8 + (r & 7);
}

// Split-context partitions ("v2"): one (sequence, partition) work item for
// one KV head x head chunk per workgroup; each wave runs its own softmax over
// its units of the partition and the waves combine into the partition's
// (max, sum, acc) workspace slot.
//  list:  1-D grid over work items x (KV heads x chunks), list_item_of():
//         the KV heads of one item (the same token rows) share an XCD, and
//         each shader engine serves every KV head.
//  dense: grid (partitions, KV heads x chunks, sequences), partitions fastest
//         and their count odd: workgroups go to the 8 XCDs round-robin by
//         linear id, and an odd stride rotates each sequence's partition p
//         across them (partition p exists only for sequences longer than
//         p * P, so a fixed mapping would load the XCDs unevenly).
template <int DT, int D, int GT, bool Q8>
__global__ __launch_bounds__(kThreads) void split_kernel(AttnParams p) {
  using W = WaveAttn<DT, D, GT, Q8>;
  extern __shared__ float lds[];
  int seq, kvhc, part;
  if (p.work_items) {
    int item;
    list_item_of(blockIdx.x, p.num_kv_heads * p.head_chunks, &item, &kvhc);
    if (item >= p.num_work_items) return;          // uniform: whole workgroup
    seq = __builtin_amdgcn_readfirstlane(p.work_items[2 * item]);
    part = __builtin_amdgcn_readfirstlane(p.work_items[2 * item + 1]);
  } else {
    part = blockIdx.x;
    kvhc = blockIdx.y;
    seq = blockIdx.z;
  }
  if (static_cast<unsigned>(seq) >= static_cast<unsigned>(p.num_seqs) ||
      static_cast<unsigned>(part) >= static_cast<unsigned>(p.num_parts))
    return;                                        // uniform: whole workgroup
  int L = __builtin_amdgcn_readfirstlane(p.context_lens[seq]);
  L = max(0, min(L, p.mb * p.block_size));         // never past the table row
  const int c0 = part * p.chunk;
  if (c0 >= L) return;                             // uniform: whole workgroup

  const int kvh = kvhc / p.head_chunks;
  const int hc = kvhc - kvh * p.head_chunks;
  const int head0 = kvh * p.group + hc * GT;
  const int nact = min(GT, p.group - hc * GT);     // active heads of this chunk
  const int64_t row0 = static_cast<int64_t>(seq) * p.num_q_heads + head0;
  const W w(p, kvh, lds);
  const typename W::Span s =
      w.span(p.block_tables + static_cast<int64_t>(seq) * p.mb, c0, min(p.chunk, L - c0));

  float acc[GT][W::VW], m_w[GT], l_w[GT];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    m_w[hh] = -__builtin_inff();
    l_w[hh] = 0.f;
  }
  constexpr int DEPTH = Q8 ? kDepthSplitQ8 : kDepthSplit;
  constexpr bool EARLY_V = (Q8 ? kEarlyVQ8 : kEarlyV) && !kNarrow<GT>;
  if (s.cnt > 0) {                                 // uniform: this wave has tokens
    // Issue order matters: loads complete in order for the wait counts, so q
    // goes first (waiting for it must not wait for the rings).
    typename W::VBuf vb[DEPTH];
    float qmax = -__builtin_inff();
    {
      uint4 qv[W::GTP][W::KC];
      w.load_q(qv, row0, nact);
      typename W::KBuf kb[DEPTH];
#pragma unroll
      for (int b = 0; b < DEPTH; ++b) w.load_k(kb[b], s, b);
      if constexpr (EARLY_V) {
        // the V ring fills behind the K ring: its first units are resident by
        // the time the logits are done, so the stream does not drain between
        // the two phases.  The narrow layout (many heads) skips this: the
        // registers it would hold through the logits cost a wave per SIMD.
#pragma unroll
        for (int b = 0; b < DEPTH; ++b) w.load_v(vb[b], s, b);
      }
      w.template logits<DEPTH>(qv, kb, s, qmax);
    }
    if constexpr (!EARLY_V) {
#pragma unroll
      for (int b = 0; b < DEPTH; ++b) w.load_v(vb[b], s, b);   // streams in during the softmax
    }
    wave_lds_sync();
    float alpha[GT];
    w.softmax(s, qmax, m_w, l_w, alpha);
    // acc is born here, after q is dead: the two never share registers
#pragma unroll
    for (int hh = 0; hh < GT; ++hh)
#pragma unroll
      for (int e = 0; e < W::VW; ++e) acc[hh][e] = 0.f;
    wave_lds_sync();
    w.template values<DEPTH>(acc, vb, s);
  } else {
#pragma unroll
    for (int hh = 0; hh < GT; ++hh)
#pragma unroll
      for (int e = 0; e < W::VW; ++e) acc[hh][e] = 0.f;
  }
  combine_waves<DT, D, GT, true>(p, acc, m_w, l_w, lds + static_cast<size_t>(p.chunk) * W::GTP,
                                 row0, nact, part);
}

// Merge of the partitions of one (sequence, q head) by one wave:
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p acc_p / sum_p w_p l_p
// Lane j holds the max and sum of partitions j, j + 64, ...; the partials'
// float4 columns are read PER partitions per load (lane: column lane % C4,
// partition k0 + lane / C4 + PER * r), ROWS partitions (16 or 64) per round
// trip, the first batch requested together with the maxima before M is
// known.  ROWS = 16 serves launches of up to 16 partitions per sequence with
// a quarter of the registers, so more of their (sequence, head) waves are
// resident at once.  A partition's
// weight is its max minus M from the lane that loaded it (ds_bpermute).  One
// wave per workgroup: every workgroup of a decode is resident at once and no
// barrier is needed.
template <int DT, int D, int ROWS>
__global__ __launch_bounds__(64) void merge_wave_kernel(AttnParams p) {
  using F = Fmt<DT>;
  constexpr int C4 = D / 4;            // float4 columns of one partial
  constexpr int PER = 64 / C4;         // partitions per load (2 for D 128, 4 for D 64)
  constexpr int R = ROWS / PER;        // loads per lane for ROWS partitions
  static_assert(ROWS % PER == 0 && ROWS <= 64, "batch of whole loads");
  const int lane = threadIdx.x;
  const int pair = blockIdx.x;
  const int seq = pair / p.num_q_heads;
  int L = __builtin_amdgcn_readfirstlane(p.context_lens[seq]);
  L = max(0, min(L, p.mb * p.block_size));
  const int np = min((L + p.chunk - 1) / p.chunk, p.num_parts);
  uint16_t* out = static_cast<uint16_t*>(p.out) + static_cast<int64_t>(pair) * D;
  if (np == 0) {                                   // uniform
    for (int d = lane; d < D; d += 64) out[d] = 0;
    return;
  }
  // partition k of (seq, head) sits in workspace row (seq * nP + k) * Hq + head
  const int64_t base = static_cast<int64_t>(seq) * p.num_parts * p.num_q_heads +
                       (pair - seq * p.num_q_heads);
  const int ks = p.num_q_heads;
  const float* pm = p.part_max + base;
  const float* ps = p.part_sum + base;
  const int col = lane % C4, row = lane / C4;
  // a batch of ROWS accumulator rows k0 .. k0 + ROWS - 1 of the (seq, head)
  // through one buffer resource: row k0 + j at byte j * Hq * D * 4, this
  // lane's float4 at col * 16.  The resource ends after row np - 1, so the
  // loads of rows past it fetch nothing and return zeros (the bound applies
  // to the per-lane offset, which therefore carries the row).  The host keeps
  // 64 rows under 2 GiB (Hq * D < 2^23).
  const uint32_t row_bytes = static_cast<uint32_t>(ks) * D * 4;
  const uint32_t voff = static_cast<uint32_t>(row) * row_bytes + col * 16;

  float4 x[R];
  auto load_batch = [&](int k0) {
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
        p.part_acc + (base + static_cast<int64_t>(k0) * ks) * D, 0,
        static_cast<int>(min(np - k0, ROWS) * row_bytes), 0x00020000);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(
          rsrc, voff + static_cast<uint32_t>(PER * r) * row_bytes, 0, 0);
      x[r] = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                         __uint_as_float(v[3]));
    }
  };
  load_batch(0);
  const float m0 = lane < np ? pm[lane * ks] : -__builtin_inff();
  const float l0 = lane < np ? ps[lane * ks] : 0.f;
  float mloc = m0;
  for (int k = lane + 64; k < np; k += 64) mloc = fmaxf(mloc, pm[k * ks]);
  const float M = wave_max_all(mloc);
  const float w0 = lane < np ? fast_exp2(m0 - M) : 0.f;   // weight of partition `lane`
  float lloc = w0 * l0;
  for (int k = lane + 64; k < np; k += 64) lloc += fast_exp2(pm[k * ks] - M) * ps[k * ks];
  const float lt = wave_sum_all(lloc);

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < np; k0 += ROWS) {
    float wl = w0;                                 // weights of partitions k0 + lane
    if (k0 > 0) {                                  // uniform: only past ROWS partitions
      load_batch(k0);
      wl = k0 + lane < np ? fast_exp2(pm[(k0 + lane) * ks] - M) : 0.f;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // partition k0 + row + PER r: rows past np are zeros with weight 0
      const float wk = __shfl(wl, row + PER * r);
      acc.x = fmaf(wk, x[r].x, acc.x);
      acc.y = fmaf(wk, x[r].y, acc.y);
      acc.z = fmaf(wk, x[r].z, acc.z);
      acc.w = fmaf(wk, x[r].w, acc.w);
    }
  }
  // the rows of one column: lanes col, col + C4, ...
#pragma unroll
  for (int off = C4; off < 64; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off);
    acc.y += __shfl_xor(acc.y, off);
    acc.z += __shfl_xor(acc.z, off);
    acc.w += __shfl_xor(acc.w, off);
  }
  if (row == 0) {
    const uint32_t lo = F::narrow(acc.x / lt) | (static_cast<uint32_t>(F::narrow(acc.y / lt)) << 16);
    const uint32_t hi = F::narrow(acc.z / lt) | (static_cast<uint32_t>(F::narrow(acc.w / lt)) << 16);
    *reinterpret_cast<uint2*>(out + col * 4) = make_uint2(lo, hi);
  }
}

template <int DT, int D, int GT, bool Q8>
int launch_attn_gt(int kind, const AttnParams& p, hipStream_t stream, hipEvent_t start,
                   hipEvent_t stop) {
  using TL = Tile<D, GT, kNarrow<GT>>;
  const int nkv = p.num_kv_heads * p.head_chunks;
  if (kind == 0) {
    constexpr int NW = kWavesSingle;
    const size_t lds = lds_floats(D, GT, TL::GTP, p.chunk, NW) * sizeof(float);
    const dim3 grid(nkv, p.num_seqs, 1);
    hipExtLaunchKernelGGL((single_kernel<DT, D, GT, Q8, NW>), grid, dim3(64 * NW), lds, stream,
                          start, stop, 0, p);
  } else {
    const size_t lds = lds_floats(D, GT, TL::GTP, p.chunk) * sizeof(float);
    const dim3 grid = p.work_items ? dim3(((p.num_work_items + 7) / 8) * 8 * nkv, 1, 1)
                                   : dim3(p.grid_parts, nkv, p.num_seqs);
    hipExtLaunchKernelGGL((split_kernel<DT, D, GT, Q8>), grid, dim3(kThreads), lds, stream, start,
                          stop, 0, p);
  }
  return static_cast<int>(hipGetLastError());
}

// Q8: the pools hold INT8 codes with fp32 row scales (p.k_scale, p.v_scale).
template <int DT, int D, bool Q8 = false>
int launch_attn(int kind, const AttnParams& p, hipStream_t stream, hipEvent_t start,
                hipEvent_t stop) {
  if (kind == 2) {
    const dim3 grid(p.num_seqs * p.num_q_heads);
    if (p.num_parts <= 16)
      hipExtLaunchKernelGGL((merge_wave_kernel<DT, D, 16>), grid, dim3(64), 0, stream, start, stop, 0, p);
    else
      hipExtLaunchKernelGGL((merge_wave_kernel<DT, D, 64>), grid, dim3(64), 0, stream, start, stop, 0, p);
    return static_cast<int>(hipGetLastError());
  }
  switch (p.heads_per_wg) {
    case 1: return launch_attn_gt<DT, D, 1, Q8>(kind, p, stream, start, stop);
    case 2: return launch_attn_gt<DT, D, 2, Q8>(kind, p, stream, start, stop);
    case 3: return launch_attn_gt<DT, D, 3, Q8>(kind, p, stream, start, stop);
    case 4: return launch_attn_gt<DT, D, 4, Q8>(kind, p, stream, start, stop);
    case 5: return launch_attn_gt<DT, D, 5, Q8>(kind, p, stream, start, stop);
    case 6: return launch_attn_gt<DT, D, 6, Q8>(kind, p, stream, start, stop);
    case 7: return launch_attn_gt<DT, D, 7, Q8>(kind, p, stream, start, stop);
    case 8: return launch_attn_gt<DT, D, 8, Q8>(kind, p, stream, start, stop);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace pa
