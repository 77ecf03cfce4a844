// pa_attn_q8_mfma.hip -- split-context decode over INT8 pools on the matrix
// cores, for groups of several query heads per KV head.
//
// The operation is the partition kernel's of pa_attn.h over INT8 pools: for
// one (sequence, context partition, KV head) and each query head h of the
// group, the partition's running max, sum of weights and weighted sum of V
// rows, a row reading back as scale x code ("LLM推理优化：vLLM PagedAttention
// 深度解析与工程实践", §4.1 and §4.3 for the paged decode and its partitions;
// "LLM推理优化技术地图：从KV Cache到量化与投机解码", §2.3 for GQA, §4.3 for the
// INT8 cache).  Over 16-bit pools that kernel is bound by memory; over INT8
// pools, with many heads per KV head, its vector work (widening every code,
// then G products per element) takes longer than the half-size stream, so
// here the products run on the matrix cores:
//   S^T = K Q^T      16x16x32 products: A = 16 K rows of codes widened to
//                    exact 16-bit integers (|code| <= 127), B = the group's
//                    q; a lane's 32 (or 16) codes of a row are one contiguous
//                    run, dims D/4 * (l / 16) + 8c .. +8 of product c, and
//                    its q slices follow the same order.  Lane l then holds
//                    the raw scores of tokens 4 (l / 16) + r of head l % 16,
//                    which it multiplies by those tokens' K scales (one
//                    16-byte load of the scale row).
//   online softmax   as over 16-bit pools; the weights are then multiplied
//                    by the tokens' V scales (weight 0 by select past the
//                    partition: those slots' scales may be NaN).
//   O^T += V^T P^T   16x16x16 products over the unit's 16 tokens: V^T from
//                    the wave's copy of the unit's V rows in LDS, widened to
//                    16-bit when written and read back by the gfx950
//                    transposing read; P^T as a 16-bit part plus a 16-bit
//                    remainder (two products), so the scaled weights keep
//                    ~17 significant bits.
// A workgroup of 4 waves serves up to 16 query heads of one KV head; wave w
// takes the partition's 16-token units w, w + 4, ...  The next unit's codes
// and scales (K and V together) stream in while a unit is processed: they
// are issued as soon as its V rows sit in LDS.  A deeper ring measured slower
// (its registers cost a wave per SIMD).  Loads past the wave's last unit go
// through an empty buffer descriptor and fetch nothing, so every path issues
// the same loads and the wait counts stay exact.  The waves' (max, sum, O^T)
// meet in LDS at the end and are written to the partition's workspace slot in
// the layout the merge kernel of pa_attn.h reads.
#include "pa_attn.h"
#include "pa_mfma.h"

namespace pa {
namespace {

using namespace mx;

constexpr int kWavesM = 4;
constexpr int kThreadsM = 64 * kWavesM;
constexpr int kHeadsM = 16;   // query heads per workgroup: the columns of the products
constexpr int kUnitM = 16;    // tokens per unit: the rows of K in S^T = K Q^T
constexpr int kDepthM = 1;    // units in flight ahead of the one being processed

template <int D>
struct Q8Tile {
  static constexpr int KC = D / 32;            // S^T products per unit (32 dims each)
  static constexpr int KSL = D / 4;            // codes of a K row per lane (one run)
  static constexpr int KL = KSL / 16;          // 16-byte K loads per lane per unit
  static constexpr int DB = D / 16;            // 16-dim blocks of O^T
  static constexpr int VLPT = D / 16;          // V loads: lanes per token, 16 codes each
  static constexpr int VTPI = 64 / VLPT;       // tokens per V load
  static constexpr int VI = kUnitM / VTPI;     // V loads per lane per unit
  static constexpr int ROW = D * 2 + 32;       // a widened V row in LDS, padded (bytes)
  static constexpr int VBUF = kUnitM * ROW;    // a wave's copy of its unit's V
  static constexpr int RSTR = D + 4;           // a head's row of a wave's O^T in LDS (floats)
  static constexpr int RED = kHeadsM * RSTR * 4;
  static constexpr int WAVE = VBUF > RED ? VBUF : RED;   // per-wave LDS region (bytes)
  static constexpr int LDS = kWavesM * WAVE + 2 * kWavesM * kHeadsM * 4;
  static_assert(KC >= 1 && KL >= 1 && VI >= 1 && VTPI * VI == kUnitM, "tile");
};

template <int D>
struct Q8Unit {
  uint4 k[Q8Tile<D>::KL];    // the lane's run of K codes
  uint4 v[Q8Tile<D>::VI];    // the lane's 16 V codes per load
  uint4 ks, vs;              // K and V scales of tokens 4 (l / 16) .. +4 (fp32 bits)
};

// Four codes of w (bytes 0..3) as two exact 16-bit pairs.
template <int DT>
__device__ inline void widen4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  using F = Fmt<DT>;
  lo = F::pack_int(code_at<0>(w), code_at<1>(w));
  hi = F::pack_int(code_at<2>(w), code_at<3>(w));
}

// At least 4 waves per SIMD: left to itself the compiler kept the
// accumulators in AGPRs beside 104 VGPRs (136 registers, 3 waves per SIMD);
// bound to 128 it fits everything in 114 VGPRs without spills, and the extra
// wave's loads in flight took the Qwen2.5-7B-shaped layer's partition kernel
// from 74.9 to 69.4 us (5 waves spill and run ~45 % slower).
template <int DT, int D>
__global__ __launch_bounds__(kThreadsM, 4) void q8_mfma_split_kernel(AttnParams p) {
  using T = Q8Tile<D>;
  extern __shared__ __align__(16) char lds[];
  int seq, kvhc, part;
  if (p.work_items) {
    // the work-list grid of the vector kernels (list_item_of)
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
  const int n = min(p.chunk, L - c0);

  const int kvh = kvhc / p.head_chunks;
  const int hc = kvhc - kvh * p.head_chunks;
  const int head0 = kvh * p.group + hc * kHeadsM;
  const int nact = min(kHeadsM, p.group - hc * kHeadsM);
  const int64_t row0 = static_cast<int64_t>(seq) * p.num_q_heads + head0;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane & 15, g = lane >> 4;

  // the wave's units and their physical blocks (lane i: unit wave + 4i)
  const int nunits = (n + kUnitM - 1) / kUnitM;
  const int cnt = nunits > wave ? (nunits - wave + kWavesM - 1) / kWavesM : 0;
  const int32_t* bt = p.block_tables + static_cast<int64_t>(seq) * p.mb;
  int blk = 0;
  if (lane < cnt) blk = bt[(c0 + (wave + kWavesM * lane) * kUnitM) >> p.log2_block_size];

  const char* kbase = static_cast<const char*>(p.k_cache);
  const char* vbase = static_cast<const char*>(p.v_cache);
  const char* ksbase = reinterpret_cast<const char*>(p.k_scale);
  const char* vsbase = reinterpret_cast<const char*>(p.v_scale);
  const int64_t block_bytes = p.block_stride;      // one byte per code
  const int64_t sc_block_bytes = static_cast<int64_t>(p.num_kv_heads) * p.block_size * 4;
  const uint32_t tok_bytes = static_cast<uint32_t>(p.num_kv_heads) * D;
  const uint32_t koff = static_cast<uint32_t>(h) * tok_bytes + kvh * D + T::KSL * g;
  const uint32_t voff = static_cast<uint32_t>(lane / T::VLPT) * tok_bytes + kvh * D +
                        16 * (lane % T::VLPT);
  const uint32_t soff = static_cast<uint32_t>(kvh) * p.block_size * 4 + 16 * g;
  const int bs_mask = p.block_size - 1;

  // codes and scales of the wave's unit i (clamped to its last unit; unit
  // i >= cnt goes through an empty descriptor and reads nothing)
  auto load_unit = [&](Q8Unit<D>& r, int i) {
    const int j = max(0, min(i, cnt - 1));
    int b = __builtin_amdgcn_readlane(blk, j);
    b = static_cast<unsigned>(b) < static_cast<unsigned>(p.num_blocks) ? b : 0;
    const int t0 = (c0 + (wave + kWavesM * j) * kUnitM) & bs_mask;   // first token in the block
    const bool live = i < cnt;
    const auto rk = block_rsrc(kbase + b * block_bytes + static_cast<int64_t>(t0) * tok_bytes, live);
#pragma unroll
    for (int c = 0; c < T::KL; ++c) r.k[c] = load16(rk, koff + 16 * c, 0);
    const auto rv = block_rsrc(vbase + b * block_bytes + static_cast<int64_t>(t0) * tok_bytes, live);
#pragma unroll
    for (int c = 0; c < T::VI; ++c) r.v[c] = load16(rv, voff, c * T::VTPI * tok_bytes);
    const int64_t so = b * sc_block_bytes + static_cast<int64_t>(t0) * 4;
    r.ks = load16(block_rsrc(ksbase + so, live), soff, 0);
    r.vs = load16(block_rsrc(vsbase + so, live), soff, 0);
  };

  // q first: waiting for it must not wait for the ring.  Product c takes
  // dims D/4 * g + 8c .. +8, in the order of the lane's run of K codes.
  uint4 qb[T::KC];
  {
    const uint16_t* q =
        static_cast<const uint16_t*>(p.q) + (row0 + min(h, nact - 1)) * D + T::KSL * g;
#pragma unroll
    for (int c = 0; c < T::KC; ++c) qb[c] = *reinterpret_cast<const uint4*>(q + 8 * c);
  }
  Q8Unit<D> ring[kDepthM];
#pragma unroll
  for (int b = 0; b < kDepthM; ++b) load_unit(ring[b], b);

  char* vb = lds + wave * T::WAVE;
  const float sl2 = p.scale_log2;
  float m = -__builtin_inff(), lsum = 0.f;
  f32x4 acc[T::DB];
#pragma unroll
  for (int b = 0; b < T::DB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int i = 0; i < cnt; i += kDepthM) {
#pragma unroll
    for (int b = 0; b < kDepthM; ++b) {
      const int ii = i + b;
      if (b == 0 || ii < cnt) {                    // uniform
        const Q8Unit<D>& r = ring[b];
        const int tb = (wave + kWavesM * ii) * kUnitM;   // the unit's first token in the span
        const bool tail = tb + kUnitM > n;
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < T::KC; ++c) {
          const uint4 w = r.k[c / 2];
          const uint32_t w0 = (c & 1) ? w.z : w.x, w1 = (c & 1) ? w.w : w.y;
          uint4 a;
          widen4<DT>(w0, a.x, a.y);
          widen4<DT>(w1, a.z, a.w);
          s = mma_k32<DT>(a, qb[c], s);
        }
        const float ksc[4] = {__uint_as_float(r.ks.x), __uint_as_float(r.ks.y),
                              __uint_as_float(r.ks.z), __uint_as_float(r.ks.w)};
        const float vsc[4] = {__uint_as_float(r.vs.x), __uint_as_float(r.vs.y),
                              __uint_as_float(r.vs.z), __uint_as_float(r.vs.w)};
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (s[e] * ksc[e]) * sl2;
        if (tail) {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = tb + 4 * g + e < n ? x[e] : -__builtin_inff();
        }
        const float mu = row4_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const float mn = fmaxf(m, mu);
        if (__builtin_amdgcn_ballot_w64(mn > m)) {       // some head's max moved
          const float al = fast_exp2(m - mn);            // 0 while m is -inf
          lsum *= al;
#pragma unroll
          for (int d = 0; d < T::DB; ++d) acc[d] *= al;
        }
        m = mn;
        float pr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[e] = fast_exp2(x[e] - m);
        lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        // the weights times the tokens' V scales; past the span weight 0 by
        // select (those slots' scales may be NaN)
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = pr[e] * vsc[e];
        if (tail) {
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[e] = tb + 4 * g + e < n ? pv[e] : 0.f;
        }
        uint2 phi, plo;
        split_pair<DT>(pv[0], pv[1], phi.x, plo.x);
        split_pair<DT>(pv[2], pv[3], phi.y, plo.y);
        // the unit's V rows, widened, into the wave's LDS copy (every code is
        // finite: rows past the span meet weight 0)
#pragma unroll
        for (int j = 0; j < T::VI; ++j) {
          const int t = lane / T::VLPT + j * T::VTPI;
          uint4 lo, hi;
          widen4<DT>(r.v[j].x, lo.x, lo.y);
          widen4<DT>(r.v[j].y, lo.z, lo.w);
          widen4<DT>(r.v[j].z, hi.x, hi.y);
          widen4<DT>(r.v[j].w, hi.z, hi.w);
          char* dst = vb + t * T::ROW + 32 * (lane % T::VLPT);
          *reinterpret_cast<uint4*>(dst) = lo;
          *reinterpret_cast<uint4*>(dst + 16) = hi;
        }
        // the ring slot is free: the unit DEPTH further on streams in (the
        // barrier keeps its loads from being hoisted above the stores, which
        // would hold a second copy of the slot)
        __builtin_amdgcn_sched_barrier(0);
        load_unit(ring[b], ii + kDepthM);
        // lane (h, g) addresses dims 16d + 4(h % 4) .. +4 of token 4g + h / 4;
        // the transposing read hands it dim 16d + h of tokens 4g .. 4g + 3
        uint2 a[T::DB];
#pragma unroll
        for (int d = 0; d < T::DB; ++d)
          a[d] = ds_read_tr16(vb + (4 * g + (h >> 2)) * T::ROW + (16 * d + 4 * (h & 3)) * 2);
#pragma unroll
        for (int d = 0; d < T::DB; ++d) acc[d] = mma_k16<DT>(a[d], phi, acc[d]);
#pragma unroll
        for (int d = 0; d < T::DB; ++d) acc[d] = mma_k16<DT>(a[d], plo, acc[d]);
      } else {
        load_unit(ring[b], ii + kDepthM);         // past the last unit: reads nothing
      }
    }
  }
  lsum = row4_sum(lsum);

  // the waves' (max, sum, O^T) meet in LDS: lane (h, g) holds dims
  // 16d + 4g .. +4 of head h; the wave's V copy is no longer read
  float* red = reinterpret_cast<float*>(vb);
#pragma unroll
  for (int d = 0; d < T::DB; ++d)
    *reinterpret_cast<f32x4*>(red + h * T::RSTR + 16 * d + 4 * g) = acc[d];
  float* wmax = reinterpret_cast<float*>(lds + kWavesM * T::WAVE);   // [kWavesM][kHeadsM]
  float* wsum = wmax + kWavesM * kHeadsM;
  if (g == 0) {
    wmax[wave * kHeadsM + h] = m;
    wsum[wave * kHeadsM + h] = lsum;
  }
  __syncthreads();

  // one float4 of one head per thread:
  //   M = max_w m_w,  acc = sum_w 2^(m_w - M) acc_w,  l = sum_w 2^(m_w - M) l_w
  // (a wave without units has m_w = -inf and weight 0)
  constexpr int C4 = D / 4;
  const int64_t sq = row0 / p.num_q_heads;
  const int64_t slot0 = (sq * p.num_parts + part) * p.num_q_heads + (row0 - sq * p.num_q_heads);
  for (int idx = threadIdx.x; idx < nact * C4; idx += kThreadsM) {
    const int hh = idx / C4;
    const int c = idx - hh * C4;
    float mw[kWavesM], M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWavesM; ++w) {
      mw[w] = wmax[w * kHeadsM + hh];
      M = fmaxf(M, mw[w]);
    }
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    float lt = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesM; ++w) {
      const float wt = fast_exp2(mw[w] - M);
      lt += wt * wsum[w * kHeadsM + hh];
      const float4 r = *reinterpret_cast<const float4*>(
          reinterpret_cast<const float*>(lds + w * T::WAVE) + hh * T::RSTR + c * 4);
      v.x = fmaf(wt, r.x, v.x);
      v.y = fmaf(wt, r.y, v.y);
      v.z = fmaf(wt, r.z, v.z);
      v.w = fmaf(wt, r.w, v.w);
    }
    // workspace rows [S][nP][Hq]: a workgroup's heads are one contiguous run
    const int64_t slot = slot0 + hh;
    *reinterpret_cast<float4*>(p.part_acc + slot * D + c * 4) = v;
    if (c == 0) {
      p.part_max[slot] = M;
      p.part_sum[slot] = lt;
    }
  }
}

template <int DT, int D>
int launch_q8_mfma(const AttnParams& p0, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  AttnParams p = p0;
  p.head_chunks = (p.group + kHeadsM - 1) / kHeadsM;
  p.heads_per_wg = min(p.group, kHeadsM);
  const int nkv = p.num_kv_heads * p.head_chunks;
  const dim3 grid = p.work_items ? dim3(((p.num_work_items + 7) / 8) * 8 * nkv, 1, 1)
                                 : dim3(p.grid_parts, nkv, p.num_seqs);
  hipExtLaunchKernelGGL((q8_mfma_split_kernel<DT, D>), grid, dim3(kThreadsM), Q8Tile<D>::LDS,
                        stream, start, stop, 0, p);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_attn_q8_mfma_split(int dtype, int head_dim, const AttnParams& p, hipStream_t stream,
                              hipEvent_t start, hipEvent_t stop) {
  if (dtype == PA_F16)
    return head_dim == 64 ? launch_q8_mfma<PA_F16, 64>(p, stream, start, stop)
                          : launch_q8_mfma<PA_F16, 128>(p, stream, start, stop);
  return head_dim == 64 ? launch_q8_mfma<PA_BF16, 64>(p, stream, start, stop)
                        : launch_q8_mfma<PA_BF16, 128>(p, stream, start, stop);
}

}  // namespace pa
