// pa_prefill.hip -- multi-token (chunked-prefill) attention over the paged
// cache, on the matrix cores of gfx950.
//
// Sequence i holds L_i tokens in the cache; its last n_i tokens are the
// query chunk, written to the cache before this call.  Query token k of the
// chunk sits at position p = L_i - n_i + k and attends causally to tokens
// 0 .. p ("vLLM 深度拆解：当大模型推理学会「分页注意力」", §2.3: prefill
// computes all prompt tokens at once; §5.1: chunked prefill cuts a long
// prompt's prefill into pieces that run between decode steps; the paged
// layout and the attention formula as for decode, "LLM推理优化：vLLM
// PagedAttention深度解析与工程实践", §二 and §4.1).
//
// Rows are (query token, head of the group) pairs of one (sequence, KV head),
// token-major: row r = k * G + h.  A workgroup of 8 waves takes 128
// consecutive rows; wave w's rows are the 16 "n" columns of its matrix
// products.  The workgroup walks the keys [0, 1 + the largest position among
// its rows) in tiles of 64, double-buffered in LDS (the next tile's loads in
// flight while the current one is computed; block ids one tile further
// ahead), K and V rows as they are, read by every wave.  Per tile and wave,
// in the transposed form that needs no transpose of Q or of the scores:
//   S^T = K Q^T     v_mfma_f32_16x16x32 (A = 16 keys x 32 dims of K from LDS,
//                   B = 32 dims x 16 rows of Q, resident in registers); the
//                   result holds, in lane l, keys 4(l/16)+r of row l%16 ...
//   online softmax  ... so each row's max and sum are a 4-lane exchange
//                   (row swaps); keys past the row's position get weight 0
//                   (only tiles that reach that far test it); a row's
//                   reference max follows its running max only when that
//                   passes it by more than 8 (in log2 units), so weights stay
//                   below 2^8 and the accumulators are rarely rescaled;
//   O^T += V^T P^T  v_mfma_f32_16x16x32 over 32 keys per product (A = 16 dims
//                   of V^T, taken from the row-major V tile by the gfx950
//                   transposing LDS read; B = P^T straight from the S^T
//                   registers: the 32 keys of two S^T tiles are ordered so
//                   that each lane's 8 k values are its own keys, and the V^T
//                   operand is read in the same order).  P goes in as a
//                   16-bit part plus a 16-bit remainder, two products, so the
//                   weights keep ~17 bits instead of 8.
// Products of 16-bit values are exact in the fp32 accumulators; the output
// is O / l rounded once to the 16-bit type.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "pa.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {
namespace {

using namespace mx;

constexpr int kWavesP = 8;               // waves per workgroup
constexpr int kThreadsP = 64 * kWavesP;
constexpr int kRowsP = 16 * kWavesP;     // (token, head) rows per workgroup
constexpr int kKeyTile = 64;             // keys per LDS tile
constexpr int kMT = kKeyTile / 16;       // 16-key tiles of S^T per key tile

struct PrefillParams {
  void* out;                   // [T][Hq][D] 16-bit
  const void* q;               // [T][Hq][D] 16-bit
  const void* k_cache;         // [NB][bs][Hkv][D]
  const void* v_cache;
  const int32_t* block_tables; // [S][mb]
  const int32_t* context_lens; // [S]
  const int32_t* query_start;  // [S + 1]
  const int32_t* seq_order;    // [S] dispatch order of the sequences, or NULL
  int32_t mb, num_seqs, num_tokens, max_query_len;
  int32_t num_q_heads, num_kv_heads, group, block_size, log2_block_size, num_blocks;
  int32_t row_tiles;           // ceil(max_query_len * group / kRowsP)
  float scale_log2;
};

// LDS: the K and V tiles [kKeyTile][D], both row-major, rows padded by 32
// bytes (a sweep of 0 .. 96 on the Qwen-shaped chunk step: unpadded rows ran
// 2.1x slower, 32 fastest) so that the rows one operand read touches fall in
// different banks.
#ifndef PA_PF_KPAD
#define PA_PF_KPAD 32
#endif
template <int D>
struct PrefillLds {
  static constexpr int ROW = D * 2 + PA_PF_KPAD;   // bytes per K or V row
  static constexpr int K_BYTES = kKeyTile * ROW;
  static constexpr int BUF = 2 * K_BYTES;          // one tile: K then V
  static constexpr int BYTES = 2 * BUF;            // double buffer
};

template <int DT, int D>
__global__ __launch_bounds__(kThreadsP, 4) void prefill_kernel(PrefillParams p) {
  using L = PrefillLds<D>;
  constexpr int KS = D / 32;          // k-steps of the S^T product
  constexpr int DT_TILES = D / 16;    // 16-dim tiles of O^T
  constexpr int CPK = D / 8;          // 16-byte chunks per K/V row
  constexpr int CHUNKS = kKeyTile * CPK;
  constexpr int LOADS = (CHUNKS + kThreadsP - 1) / kThreadsP;
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];

  // blockIdx -> (sequence, KV head, row tile): the tiles of one (sequence,
  // KV head) share blockIdx.x mod 8, hence an XCD and its L2; sequences go
  // in seq_order (the caller's longest-first order keeps the long ones from
  // being the tail of the launch)
  const int npairs = p.num_seqs * p.num_kv_heads;
  const int id = blockIdx.x;
  const int k8 = id >> 3;
  const int pair = (k8 / p.row_tiles) * 8 + (id & 7);
  const int tile = k8 % p.row_tiles;
  if (pair >= npairs) return;                         // uniform: whole workgroup
  const int rank = pair / p.num_kv_heads;
  const int kvh = pair - rank * p.num_kv_heads;
  const int seq = p.seq_order ? p.seq_order[rank] : rank;
  if (static_cast<unsigned>(seq) >= static_cast<unsigned>(p.num_seqs)) return;   // uniform
  const int G = p.group;

  const int q0 = p.query_start[seq];
  int L_ctx = p.context_lens[seq];
  L_ctx = max(0, min(L_ctx, p.mb * p.block_size));
  // the chunk's tokens are the last n_all of the context; a chunk longer than
  // its context, or one whose rows leave [0, num_tokens), is skipped whole; a
  // chunk longer than max_query_len keeps its positions and loses its rows
  // past that count
  const int64_t n_all64 = static_cast<int64_t>(p.query_start[seq + 1]) - q0;
  const bool chunk_ok = q0 >= 0 && n_all64 >= 0 && n_all64 <= L_ctx &&
                        static_cast<int64_t>(q0) + n_all64 <= p.num_tokens;
  const int n_all = chunk_ok ? static_cast<int>(n_all64) : 0;
  const int n = min(n_all, p.max_query_len);
  const int nrows = n * G;
  const int r0 = tile * kRowsP;
  if (r0 >= nrows) return;                            // uniform: whole workgroup
  const int base_pos = L_ctx - n_all;                 // position of query token 0
  const int last_row = min(r0 + kRowsP, nrows) - 1;
  const int kend = base_pos + last_row / G + 1;       // keys this workgroup needs

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;          // the row (n column) this lane serves
  const int lg = lane >> 4;          // its group of 4 (k rows / keys)
  const int row = r0 + wave * 16 + lr;
  const bool row_ok = row < nrows;
  const int rowc = row_ok ? row : nrows - 1;
  const int tok = rowc / G;
  const int head = kvh * G + (rowc - tok * G);
  const int pos = base_pos + tok;
  const int64_t qrow = static_cast<int64_t>(q0 + tok) * p.num_q_heads + head;

  // Q^T operands: dims 8*lg + 32*ks .. +8 of this lane's row
  uint4 qb[KS];
  const uint16_t* qp = static_cast<const uint16_t*>(p.q) + qrow * D + 8 * lg;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qb[ks] = *reinterpret_cast<const uint4*>(qp + 32 * ks);

  const int32_t* bt = p.block_tables + static_cast<int64_t>(seq) * p.mb;
  const char* kbase = static_cast<const char*>(p.k_cache) + static_cast<int64_t>(kvh) * D * 2;
  const char* vbase = static_cast<const char*>(p.v_cache) + static_cast<int64_t>(kvh) * D * 2;
  const uint32_t tok_bytes = static_cast<uint32_t>(p.num_kv_heads) * D * 2;
  const uint32_t blk_bytes = tok_bytes << p.log2_block_size;
  const int bs_mask = (1 << p.log2_block_size) - 1;
  // Thread tid moves chunks c = tid + j * kThreadsP of each tile: key c / CPK,
  // dims 8 * (c % CPK) .. +8 (a wave reads whole 256-byte rows).  Its block
  // ids run one tile ahead of its loads, so a tile's K/V loads never wait for
  // a table read.
  auto block_of = [&](int t, int j) {
    const int c = tid + j * kThreadsP;
    const int key = t * kKeyTile + c / CPK;
    if (c >= CHUNKS || key >= kend) return -1;
    const int blk = bt[key >> p.log2_block_size];
    return static_cast<unsigned>(blk) < static_cast<unsigned>(p.num_blocks) ? blk : 0;
  };
  auto load_tile = [&](int t, const int (&blk)[LOADS], uint4 (&kr)[LOADS], uint4 (&vr)[LOADS]) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int c = tid + j * kThreadsP;
      kr[j] = make_uint4(0, 0, 0, 0);       // keys past kend: zeros (their weight is 0)
      vr[j] = make_uint4(0, 0, 0, 0);
      if (blk[j] >= 0) {
        const int key = t * kKeyTile + c / CPK;
        const uint64_t at = static_cast<uint64_t>(static_cast<uint32_t>(blk[j])) * blk_bytes +
                            (static_cast<uint32_t>(key & bs_mask) * tok_bytes + (c % CPK) * 16);
        kr[j] = *reinterpret_cast<const uint4*>(kbase + at);
        vr[j] = *reinterpret_cast<const uint4*>(vbase + at);
      }
    }
  };
  auto store_tile = [&](char* buf, const uint4 (&kr)[LOADS], const uint4 (&vr)[LOADS]) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int c = tid + j * kThreadsP;
      if (c >= CHUNKS) continue;
      const int key = c / CPK, col = c % CPK;
      *reinterpret_cast<uint4*>(buf + key * L::ROW + col * 16) = kr[j];
      *reinterpret_cast<uint4*>(buf + L::K_BYTES + key * L::ROW + col * 16) = vr[j];
    }
  };

  f32x4 acc[DT_TILES];
#pragma unroll
  for (int dt = 0; dt < DT_TILES; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_lane = 0.f;                 // this lane's share of the row's sum
  // the wave's smallest position: tiles wholly at or below it need no mask
  const int wave_pos_min = base_pos + min(r0 + wave * 16, nrows - 1) / G;

  const int ntiles = (kend + kKeyTile - 1) / kKeyTile;
  uint4 kr[LOADS], vr[LOADS];
  int blk[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) blk[j] = block_of(0, j);
  load_tile(0, blk, kr, vr);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) blk[j] = block_of(1, j);
  store_tile(lds, kr, vr);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const char* buf = lds + (t & 1) * L::BUF;
    if (t + 1 < ntiles) {                  // in flight during this tile
      load_tile(t + 1, blk, kr, vr);
#pragma unroll
      for (int j = 0; j < LOADS; ++j) blk[j] = block_of(t + 2, j);
    }

    // the waves of a workgroup run each tile's phases in step (one barrier
    // per tile); a wave issuing matrix products takes priority, so the
    // products of some waves overlap the softmax of others (~2 % faster)
    __builtin_amdgcn_s_setprio(1);
    // S^T for keys t*KT + 16*mt + 4*lg + r of this lane's row
    f32x4 s[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(buf + (16 * mt + lr) * L::ROW +
                                                        (8 * lg + 32 * ks) * 2);
        s[mt] = mma_k32<DT>(a, qb[ks], s[mt]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // online softmax of the row (base 2, logits scale * log2 e * s); keys past
    // the row's position get weight 0, on the tiles that reach past the wave's
    // first row only; the max is taken on the raw scores (the scale is > 0)
    if (t * kKeyTile + kKeyTile - 1 > wave_pos_min) {          // uniform
      asm volatile("");   // keeps this a branch (not selects on every tile)
      const int lim = pos - t * kKeyTile - 4 * lg;             // last visible offset
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * mt + r > lim) s[mt][r] = -__builtin_inff();
    }
    float tmax = s[0][0];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, s[mt][r]);
    const float m_new = fmaxf(m_run, row4_max(tmax) * p.scale_log2);
    // the reference max moves only when a row's max passes it by more than
    // 8 (weights stay below 256; the normalisation at the end is exact in
    // any reference), so after the first tiles the rescale is rare
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + 8.f)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run is -inf
      l_lane *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT_TILES; ++dt) acc[dt] *= alpha;
      m_run = m_new;
    }
    float pr[4 * kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // exp2(-inf) = 0
        pr[4 * mt + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][r], p.scale_log2, -m_run));
        l_lane += pr[4 * mt + r];
      }
    __builtin_amdgcn_s_setprio(1);
    // O^T += V^T P^T on 16x16x32 products: k-step ks takes the 32 keys of
    // S^T tiles 2ks and 2ks + 1, ordered so that lane group lg's 8 k values
    // are its own keys 4lg + r of both tiles (P^T straight from registers);
    // the V^T operand follows the same order (two 8-byte reads)
    uint4 phi[kMT / 2], plo[kMT / 2];
#pragma unroll
    for (int ks = 0; ks < kMT / 2; ++ks) {
      const float* q0p = pr + 8 * ks;
      split_pair<DT>(q0p[0], q0p[1], phi[ks].x, plo[ks].x);
      split_pair<DT>(q0p[2], q0p[3], phi[ks].y, plo[ks].y);
      split_pair<DT>(q0p[4], q0p[5], phi[ks].z, plo[ks].z);
      split_pair<DT>(q0p[6], q0p[7], phi[ks].w, plo[ks].w);
    }
#pragma unroll
    for (int dt = 0; dt < DT_TILES; ++dt) {
#pragma unroll
      for (int ks = 0; ks < kMT / 2; ++ks) {
        // lane lr of group lg addresses dims 16dt + 4(lr%4) .. +4 of key
        // 32ks + 4lg + lr/4; the transposing read hands lane lr dim 16dt + lr
        // of keys 32ks + 4lg + 0..3, and a second read the same 16 keys
        // further on
        const char* vp = buf + L::K_BYTES + (32 * ks + 4 * lg + (lr >> 2)) * L::ROW +
                         (16 * dt + 4 * (lr & 3)) * 2;
        const uint2 b0 = ds_read_tr16(vp), b1 = ds_read_tr16(vp + 16 * L::ROW);
        const uint4 a = make_uint4(b0.x, b0.y, b1.x, b1.y);
        acc[dt] = mma_k32<DT>(a, phi[ks], acc[dt]);
        acc[dt] = mma_k32<DT>(a, plo[ks], acc[dt]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (t + 1 < ntiles) store_tile(lds + ((t + 1) & 1) * L::BUF, kr, vr);
    __syncthreads();   // tile t + 1 is in place; tile t's buffer may be rewritten
  }

  // out = O / l, dims 16*dt + 4*lg + r of this lane's row
  const float l_row = row4_sum(l_lane);
  if (row_ok) {
    const float inv = 1.f / l_row;
    uint16_t* op = static_cast<uint16_t*>(p.out) + qrow * D + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < DT_TILES; ++dt) {
      const uint32_t lo = narrow16<DT>(acc[dt][0] * inv) |
                          (static_cast<uint32_t>(narrow16<DT>(acc[dt][1] * inv)) << 16);
      const uint32_t hi = narrow16<DT>(acc[dt][2] * inv) |
                          (static_cast<uint32_t>(narrow16<DT>(acc[dt][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(op + 16 * dt) = make_uint2(lo, hi);
    }
  }
}

bool aligned_p(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

}  // namespace
}  // namespace pa

extern "C" pa_status pa_prefill(void* out, const void* query, const void* key_cache,
                                const void* value_cache, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                const int32_t* query_start, const int32_t* seq_order,
                                int32_t num_seqs,
                                int32_t num_query_tokens, int32_t max_query_len,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t num_blocks, float scale,
                                pa_dtype dtype, hipStream_t stream, hipEvent_t start_event,
                                hipEvent_t stop_event) {
  using pa::fail;
  pa::clear_error();
  if (dtype != PA_F16 && dtype != PA_BF16) return fail(PA_ERR_INVALID_ARG, "unknown dtype");
  if (num_seqs < 0 || num_query_tokens < 0 || max_query_len < 0)
    return fail(PA_ERR_INVALID_ARG, "negative count");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG, "block_size, num_blocks, max_blocks_per_seq must be positive");
  if ((block_size & (block_size - 1)) != 0)
    return fail(PA_ERR_UNSUPPORTED, "block_size must be a power of two");
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq * block_size overflows int32");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  const int64_t group = num_q_heads / num_kv_heads;
  const int64_t row_tiles = (static_cast<int64_t>(max_query_len) * group + pa::kRowsP - 1) /
                            pa::kRowsP;
  const int64_t pairs8 = (static_cast<int64_t>(num_seqs) * num_kv_heads + 7) / 8 * 8;
  const int64_t blocks = pairs8 * row_tiles;
  if (blocks > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "grid too large");
  if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0) {
    for (hipEvent_t e : {start_event, stop_event})
      if (e && hipEventRecord(e, stream) != hipSuccess)
        return fail(PA_ERR_HIP, "pa_prefill: hipEventRecord failed");
    return PA_OK;
  }
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
      !query_start)
    return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
  if (!pa::aligned_p(out, 16) || !pa::aligned_p(query, 16) || !pa::aligned_p(key_cache, 16) ||
      !pa::aligned_p(value_cache, 16) || !pa::aligned_p(block_tables, 4) ||
      !pa::aligned_p(context_lens, 4) || !pa::aligned_p(query_start, 4) ||
      !pa::aligned_p(seq_order, 4))
    return fail(PA_ERR_INVALID_ARG, "device buffers must be 16-byte aligned (metadata 4-byte)");
  pa::PrefillParams p{};
  p.out = out;
  p.q = query;
  p.k_cache = key_cache;
  p.v_cache = value_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start = query_start;
  p.seq_order = seq_order;
  p.mb = max_blocks_per_seq;
  p.num_seqs = num_seqs;
  p.num_tokens = num_query_tokens;
  p.max_query_len = max_query_len;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = static_cast<int32_t>(group);
  p.block_size = block_size;
  p.log2_block_size = __builtin_ctz(static_cast<unsigned>(block_size));
  p.num_blocks = num_blocks;
  p.row_tiles = static_cast<int32_t>(row_tiles);
  p.scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid(static_cast<uint32_t>(blocks)), block(pa::kThreadsP);
  if (dtype == PA_F16) {
    if (head_dim == 64)
      hipExtLaunchKernelGGL((pa::prefill_kernel<PA_F16, 64>), grid, block, 0, stream,
                            start_event, stop_event, 0, p);
    else
      hipExtLaunchKernelGGL((pa::prefill_kernel<PA_F16, 128>), grid, block, 0, stream,
                            start_event, stop_event, 0, p);
  } else {
    if (head_dim == 64)
      hipExtLaunchKernelGGL((pa::prefill_kernel<PA_BF16, 64>), grid, block, 0, stream,
                            start_event, stop_event, 0, p);
    else
      hipExtLaunchKernelGGL((pa::prefill_kernel<PA_BF16, 128>), grid, block, 0, stream,
                            start_event, stop_event, 0, p);
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(PA_ERR_HIP, hipGetErrorString(err));
  return PA_OK;
}
