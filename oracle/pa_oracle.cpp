// pa_oracle.cpp -- the CPU oracle for paged decode attention.
//
// TEST INFRASTRUCTURE ONLY: used by the tests, the package smoke check and the
// benchmark's CPU-baseline leg, never by the product path.  Plain, slow and
// written to be checked by eye against the pages; see pa_oracle.h for what
// each function follows.  Compile with -ffp-contract=off.

#include "pa_oracle.h"

#include <algorithm>
#include <atomic>
#include <cfenv>
#include <cmath>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

// ---------------------------------------------------------------------------
// 16-bit float conversions, from the format definitions.
//
// binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
//   exponent 0      -> subnormal, value = fraction * 2^-24
//   exponent 1..30  -> normal,    value = (1024 + fraction) * 2^(exponent-25)
//   exponent 31     -> inf (fraction 0) or NaN
// bfloat16: the upper 16 bits of an IEEE binary32: 1 sign, 8 exponent bits
//   (bias 127), 7 fraction bits.  Widening is exact: shift left by 16.
// Narrowing rounds to nearest, ties to even, by scaling the magnitude to an
// integer count of the target's units in the last place and rounding that
// count with nearbyint() in the default (to-nearest-even) rounding mode.
// ---------------------------------------------------------------------------

float pao_f16_to_f32(uint16_t h) {
  const uint32_t sign = h >> 15;
  const uint32_t expo = (h >> 10) & 0x1fu;
  const uint32_t frac = h & 0x3ffu;
  float v;
  if (expo == 0) {
    v = std::ldexp(static_cast<float>(frac), -24);
  } else if (expo == 31) {
    v = frac ? std::numeric_limits<float>::quiet_NaN()
             : std::numeric_limits<float>::infinity();
  } else {
    v = std::ldexp(static_cast<float>(1024u + frac), static_cast<int>(expo) - 25);
  }
  return sign ? -v : v;
}

float pao_bf16_to_f32(uint16_t b) {
  const uint32_t bits = static_cast<uint32_t>(b) << 16;
  float v;
  std::memcpy(&v, &bits, sizeof v);
  return v;
}

// Round |x| (finite, as a double, exact) to the target format with `mant`
// fraction bits, minimum normal exponent `emin` and maximum finite exponent
// `emax`.  Returns the magnitude bits (exponent field << mant | fraction), or
// the infinity pattern on overflow.
static uint32_t narrow_magnitude(double a, int mant, int emin, int emax,
                                 int bias) {
  const uint32_t inf_bits = static_cast<uint32_t>(emax + bias + 1) << mant;
  if (a == 0.0) return 0u;
  int e2;
  std::frexp(a, &e2);       // a = f * 2^e2 with f in [0.5, 1)
  int e = e2 - 1;           // a in [2^e, 2^(e+1))
  if (e < emin) {
    // subnormal range: units of 2^(emin - mant)
    const double units = std::ldexp(a, mant - emin);
    const double r = std::nearbyint(units);
    // r may reach 2^mant, which is exactly the smallest normal's bit pattern
    return static_cast<uint32_t>(r);
  }
  // normal range: a / 2^e in [1, 2); count units of 2^(e - mant)
  const double units = std::ldexp(a, mant - e);  // in [2^mant, 2^(mant+1))
  double r = std::nearbyint(units);
  if (r == std::ldexp(1.0, mant + 1)) {  // rounded up to the next binade
    r = std::ldexp(1.0, mant);
    e += 1;
  }
  if (e > emax) return inf_bits;
  const uint32_t field = static_cast<uint32_t>(e + bias);
  const uint32_t fraction = static_cast<uint32_t>(r) - (1u << mant);
  return (field << mant) | fraction;
}

uint16_t pao_f32_to_f16(float x) {
  const uint16_t sign = std::signbit(x) ? 0x8000u : 0u;
  if (std::isnan(x)) return static_cast<uint16_t>(sign | 0x7e00u);
  if (std::isinf(x)) return static_cast<uint16_t>(sign | 0x7c00u);
  const uint32_t mag = narrow_magnitude(std::fabs(static_cast<double>(x)), 10,
                                        -14, 15, 15);
  return static_cast<uint16_t>(sign | mag);
}

uint16_t pao_f32_to_bf16(float x) {
  const uint16_t sign = std::signbit(x) ? 0x8000u : 0u;
  if (std::isnan(x)) return static_cast<uint16_t>(sign | 0x7fc0u);
  if (std::isinf(x)) return static_cast<uint16_t>(sign | 0x7f80u);
  const uint32_t mag = narrow_magnitude(std::fabs(static_cast<double>(x)), 7,
                                        -126, 127, 127);
  return static_cast<uint16_t>(sign | mag);
}

static inline float widen(uint16_t v, int32_t dtype) {
  return dtype == PAO_BF16 ? pao_bf16_to_f32(v) : pao_f16_to_f32(v);
}
static inline uint16_t narrow(float v, int32_t dtype) {
  return dtype == PAO_BF16 ? pao_f32_to_bf16(v) : pao_f32_to_f16(v);
}

void pao_widen(const uint16_t* in, float* out, int64_t n, int32_t dtype) {
  for (int64_t i = 0; i < n; ++i) out[i] = widen(in[i], dtype);
}

void pao_narrow(const float* in, uint16_t* out, int64_t n, int32_t dtype) {
  for (int64_t i = 0; i < n; ++i) out[i] = narrow(in[i], dtype);
}

// ---------------------------------------------------------------------------
// Cache write: token t's K (and V) row [hkv][d] goes, bit for bit, to
// pool[b][o][*][*] with b = slot / bs and o = slot % bs.
// ---------------------------------------------------------------------------

int32_t pao_cache_write(const uint16_t* key, const uint16_t* value,
                        uint16_t* key_cache, uint16_t* value_cache,
                        const int64_t* slot_mapping, int32_t n, int32_t hkv,
                        int32_t d, int32_t bs, int32_t nb) {
  if (n < 0 || hkv <= 0 || d <= 0 || bs <= 0 || nb <= 0) return PAO_BAD_ARG;
  if (n > 0 && (!key || !value || !key_cache || !value_cache || !slot_mapping))
    return PAO_BAD_ARG;
  const int64_t num_slots = static_cast<int64_t>(nb) * bs;
  std::vector<int64_t> used;
  for (int32_t t = 0; t < n; ++t) {
    const int64_t s = slot_mapping[t];
    if (s < 0) continue;
    if (s >= num_slots) return PAO_BAD_SLOT;
    used.push_back(s);
  }
  std::sort(used.begin(), used.end());
  if (std::adjacent_find(used.begin(), used.end()) != used.end())
    return PAO_DUP_SLOT;

  const int64_t row = static_cast<int64_t>(hkv) * d;  // elements per token
  for (int32_t t = 0; t < n; ++t) {
    const int64_t s = slot_mapping[t];
    if (s < 0) continue;
    const int64_t b = s / bs;
    const int64_t o = s % bs;
    const int64_t dst = (b * bs + o) * row;
    const int64_t src = static_cast<int64_t>(t) * row;
    for (int64_t e = 0; e < row; ++e) {
      key_cache[dst + e] = key[src + e];
      value_cache[dst + e] = value[src + e];
    }
  }
  return PAO_OK;
}

int64_t pao_slot(const int32_t* block_table_row, int32_t pos, int32_t bs) {
  return static_cast<int64_t>(block_table_row[pos / bs]) * bs + pos % bs;
}

// ---------------------------------------------------------------------------
// Gather: K_i[j] = key_cache[table[j / bs]][j % bs][g][0..d) for j < L.
// ---------------------------------------------------------------------------

int32_t pao_gather(float* k_out, float* v_out, const uint16_t* key_cache,
                   const uint16_t* value_cache, const int32_t* block_table_row,
                   int32_t L, int32_t g, int32_t hkv, int32_t d, int32_t bs,
                   int32_t nb, int32_t dtype) {
  if (L <= 0) return PAO_BAD_LEN;
  if (g < 0 || g >= hkv) return PAO_BAD_ARG;
  for (int32_t j = 0; j < L; ++j) {
    const int32_t b = block_table_row[j / bs];
    if (b < 0 || b >= nb) return PAO_BAD_BLOCK;
    const int64_t base =
        ((static_cast<int64_t>(b) * bs + j % bs) * hkv + g) * d;
    for (int32_t e = 0; e < d; ++e) {
      k_out[static_cast<int64_t>(j) * d + e] = widen(key_cache[base + e], dtype);
      v_out[static_cast<int64_t>(j) * d + e] = widen(value_cache[base + e], dtype);
    }
  }
  return PAO_OK;
}

// ---------------------------------------------------------------------------
// Decode of one (sequence, q head): the plain definition.
//   s_j = scale * sum_e q[e] * K[j][e]      (ascending e)
//   m   = max_j s_j
//   e_j = exp(s_j - m)
//   l   = sum_j e_j                         (ascending j)
//   o[e] = (sum_j e_j * V[j][e]) / l        (ascending j)
// Query head h reads kv head g = h / (hq / hkv): consecutive query heads
// share one kv head.
// ---------------------------------------------------------------------------

// The definition above on gathered rows K, V [L][d] and the widened query.
static void attend(float* out, const std::vector<float>& qf, const std::vector<float>& K,
                   const std::vector<float>& V, int32_t L, int32_t d, float scale) {
  std::vector<float> s(L);
  for (int32_t j = 0; j < L; ++j) {
    float acc = 0.0f;
    for (int32_t e = 0; e < d; ++e) acc = acc + qf[e] * K[static_cast<size_t>(j) * d + e];
    s[j] = scale * acc;
  }
  float m = s[0];
  for (int32_t j = 1; j < L; ++j) m = std::max(m, s[j]);
  std::vector<float> w(L);
  float l = 0.0f;
  for (int32_t j = 0; j < L; ++j) {
    w[j] = std::exp(s[j] - m);
    l = l + w[j];
  }
  for (int32_t e = 0; e < d; ++e) {
    float acc = 0.0f;
    for (int32_t j = 0; j < L; ++j) acc = acc + w[j] * V[static_cast<size_t>(j) * d + e];
    out[e] = acc / l;
  }
}

static int32_t decode_one(float* out, const uint16_t* q_row,
                          const uint16_t* key_cache, const uint16_t* value_cache,
                          const int32_t* table_row, int32_t mb, int32_t L,
                          int32_t g, int32_t hkv, int32_t d, int32_t bs,
                          int32_t nb, float scale, int32_t dtype) {
  if (L <= 0 || L > static_cast<int64_t>(mb) * bs) return PAO_BAD_LEN;
  std::vector<float> K(static_cast<size_t>(L) * d), V(static_cast<size_t>(L) * d);
  const int32_t rc = pao_gather(K.data(), V.data(), key_cache, value_cache,
                                table_row, L, g, hkv, d, bs, nb, dtype);
  if (rc != PAO_OK) return rc;
  std::vector<float> qf(d);
  for (int32_t e = 0; e < d; ++e) qf[e] = widen(q_row[e], dtype);
  attend(out, qf, K, V, L, d, scale);
  return PAO_OK;
}

static bool shapes_ok(int32_t s, int32_t hq, int32_t hkv, int32_t d, int32_t bs,
                      int32_t nb, int32_t mb, int32_t dtype) {
  return s >= 0 && hq > 0 && hkv > 0 && hq % hkv == 0 && d > 0 && bs > 0 &&
         nb > 0 && mb > 0 && (dtype == PAO_F16 || dtype == PAO_BF16);
}

int32_t pao_decode_pairs(float* out_f32, uint16_t* out_t, const uint16_t* q,
                         const uint16_t* key_cache, const uint16_t* value_cache,
                         const int32_t* block_tables, int32_t mb,
                         const int32_t* context_lens, int32_t s, int32_t hq,
                         int32_t hkv, int32_t d, int32_t bs, int32_t nb,
                         float scale, int32_t dtype, const int32_t* pairs,
                         int32_t n_pairs, int32_t nthreads) {
  if (!shapes_ok(s, hq, hkv, d, bs, nb, mb, dtype) || n_pairs < 0)
    return PAO_BAD_ARG;
  const int32_t G = hq / hkv;
  for (int32_t p = 0; p < n_pairs; ++p) {
    if (pairs[2 * p] < 0 || pairs[2 * p] >= s || pairs[2 * p + 1] < 0 ||
        pairs[2 * p + 1] >= hq)
      return PAO_BAD_ARG;
  }
  int32_t T = nthreads > 0 ? nthreads
                           : static_cast<int32_t>(std::thread::hardware_concurrency());
  if (T < 1) T = 1;
  if (T > n_pairs) T = std::max(n_pairs, 1);

  std::atomic<int32_t> next(0);
  std::atomic<int32_t> status(PAO_OK);
  auto worker = [&]() {
    for (;;) {
      const int32_t p = next.fetch_add(1);
      if (p >= n_pairs) return;
      const int32_t i = pairs[2 * p];
      const int32_t h = pairs[2 * p + 1];
      float* o = out_f32 + static_cast<int64_t>(p) * d;
      const int32_t rc = decode_one(
          o, q + (static_cast<int64_t>(i) * hq + h) * d, key_cache, value_cache,
          block_tables + static_cast<int64_t>(i) * mb, mb, context_lens[i],
          h / G, hkv, d, bs, nb, scale, dtype);
      if (rc != PAO_OK) {
        status.store(rc);
        continue;
      }
      if (out_t)
        for (int32_t e = 0; e < d; ++e)
          out_t[static_cast<int64_t>(p) * d + e] = narrow(o[e], dtype);
    }
  };
  if (T == 1) {
    worker();
  } else {
    std::vector<std::thread> pool;
    for (int32_t t = 0; t < T; ++t) pool.emplace_back(worker);
    for (auto& th : pool) th.join();
  }
  return status.load();
}

int32_t pao_decode(float* out_f32, uint16_t* out_t, const uint16_t* q,
                   const uint16_t* key_cache, const uint16_t* value_cache,
                   const int32_t* block_tables, int32_t mb,
                   const int32_t* context_lens, int32_t s, int32_t hq,
                   int32_t hkv, int32_t d, int32_t bs, int32_t nb, float scale,
                   int32_t dtype, int32_t nthreads) {
  if (!shapes_ok(s, hq, hkv, d, bs, nb, mb, dtype)) return PAO_BAD_ARG;
  std::vector<int32_t> pairs(static_cast<size_t>(s) * hq * 2);
  for (int32_t i = 0; i < s; ++i)
    for (int32_t h = 0; h < hq; ++h) {
      pairs[2 * (static_cast<size_t>(i) * hq + h)] = i;
      pairs[2 * (static_cast<size_t>(i) * hq + h) + 1] = h;
    }
  return pao_decode_pairs(out_f32, out_t, q, key_cache, value_cache,
                          block_tables, mb, context_lens, s, hq, hkv, d, bs, nb,
                          scale, dtype, pairs.data(), s * hq, nthreads);
}

// ---------------------------------------------------------------------------
// Split-context form.  Partition p of sequence i covers tokens
// [p*P, min(L, (p+1)*P)).  Per partition and q head:
//   m_p = max s_j,  l_p = sum exp(s_j - m_p),  acc_p = sum exp(s_j - m_p) V_j
// then  M = max_p m_p,  w_p = exp(m_p - M),
//   out = (sum_p w_p acc_p) / (sum_p w_p l_p).
// ---------------------------------------------------------------------------

int32_t pao_decode_partitioned(float* out_f32, uint16_t* out_t,
                               const uint16_t* q, const uint16_t* key_cache,
                               const uint16_t* value_cache,
                               const int32_t* block_tables, int32_t mb,
                               const int32_t* context_lens, int32_t s,
                               int32_t hq, int32_t hkv, int32_t d, int32_t bs,
                               int32_t nb, float scale, int32_t dtype,
                               int32_t partition_size) {
  if (!shapes_ok(s, hq, hkv, d, bs, nb, mb, dtype) || partition_size <= 0)
    return PAO_BAD_ARG;
  const int32_t G = hq / hkv;
  const int32_t P = partition_size;
  for (int32_t i = 0; i < s; ++i) {
    const int32_t L = context_lens[i];
    if (L <= 0 || L > static_cast<int64_t>(mb) * bs) return PAO_BAD_LEN;
    for (int32_t h = 0; h < hq; ++h) {
      const int32_t g = h / G;
      std::vector<float> K(static_cast<size_t>(L) * d), V(static_cast<size_t>(L) * d);
      const int32_t rc = pao_gather(K.data(), V.data(), key_cache, value_cache,
                                    block_tables + static_cast<int64_t>(i) * mb,
                                    L, g, hkv, d, bs, nb, dtype);
      if (rc != PAO_OK) return rc;
      std::vector<float> qf(d);
      for (int32_t e = 0; e < d; ++e)
        qf[e] = widen(q[(static_cast<int64_t>(i) * hq + h) * d + e], dtype);

      const int32_t nP = (L + P - 1) / P;
      std::vector<float> mp(nP), lp(nP), accp(static_cast<size_t>(nP) * d);
      for (int32_t p = 0; p < nP; ++p) {
        const int32_t j0 = p * P;
        const int32_t j1 = std::min(L, j0 + P);
        std::vector<float> sc(j1 - j0);
        for (int32_t j = j0; j < j1; ++j) {
          float acc = 0.0f;
          for (int32_t e = 0; e < d; ++e)
            acc = acc + qf[e] * K[static_cast<size_t>(j) * d + e];
          sc[j - j0] = scale * acc;
        }
        float m = sc[0];
        for (float v : sc) m = std::max(m, v);
        float l = 0.0f;
        std::vector<float> w(j1 - j0);
        for (int32_t j = j0; j < j1; ++j) {
          w[j - j0] = std::exp(sc[j - j0] - m);
          l = l + w[j - j0];
        }
        for (int32_t e = 0; e < d; ++e) {
          float acc = 0.0f;
          for (int32_t j = j0; j < j1; ++j)
            acc = acc + w[j - j0] * V[static_cast<size_t>(j) * d + e];
          accp[static_cast<size_t>(p) * d + e] = acc;
        }
        mp[p] = m;
        lp[p] = l;
      }
      float M = mp[0];
      for (int32_t p = 1; p < nP; ++p) M = std::max(M, mp[p]);
      float den = 0.0f;
      std::vector<float> wp(nP);
      for (int32_t p = 0; p < nP; ++p) {
        wp[p] = std::exp(mp[p] - M);
        den = den + wp[p] * lp[p];
      }
      float* o = out_f32 + (static_cast<int64_t>(i) * hq + h) * d;
      for (int32_t e = 0; e < d; ++e) {
        float num = 0.0f;
        for (int32_t p = 0; p < nP; ++p)
          num = num + wp[p] * accp[static_cast<size_t>(p) * d + e];
        o[e] = num / den;
        if (out_t) out_t[(static_cast<int64_t>(i) * hq + h) * d + e] = narrow(o[e], dtype);
      }
    }
  }
  return PAO_OK;
}

// ---------------------------------------------------------------------------
// Multi-token (chunked-prefill) attention over the paged cache.  Sequence i
// holds L_i tokens in the cache, the last n_i of which are its query chunk
// (written before the attention); query token k of the chunk sits at
// position p = L_i - n_i + k and attends causally to tokens 0 .. p:
//   out[k][h] = sum_{j <= p} softmax_j(scale * q[k][h] . K[j]) V[j]
// i.e. the decode definition above with context length p + 1.
// query_start [s + 1]: the chunk of sequence i is rows [query_start[i],
// query_start[i + 1]) of q / out ([T][hq][d]).
// ---------------------------------------------------------------------------

int32_t pao_prefill(float* out_f32, uint16_t* out_t, const uint16_t* q,
                    const uint16_t* key_cache, const uint16_t* value_cache,
                    const int32_t* block_tables, int32_t mb, const int32_t* context_lens,
                    const int32_t* query_start, int32_t s, int32_t hq, int32_t hkv, int32_t d,
                    int32_t bs, int32_t nb, float scale, int32_t dtype, int32_t nthreads) {
  if (!shapes_ok(s, hq, hkv, d, bs, nb, mb, dtype) || !query_start || query_start[0] != 0)
    return PAO_BAD_ARG;
  for (int32_t i = 0; i < s; ++i) {
    const int32_t n = query_start[i + 1] - query_start[i];
    if (n < 0 || n > context_lens[i] || context_lens[i] > static_cast<int64_t>(mb) * bs)
      return PAO_BAD_LEN;
  }
  const int32_t G = hq / hkv;
  const int32_t rows = query_start[s];
  int32_t T = nthreads > 0 ? nthreads
                           : static_cast<int32_t>(std::thread::hardware_concurrency());
  T = std::max(1, std::min(T, std::max(rows * hq, 1)));
  std::atomic<int32_t> next(0), status(PAO_OK);
  auto worker = [&]() {
    for (int32_t job; (job = next.fetch_add(1)) < rows * hq;) {
      const int32_t row = job / hq, h = job % hq;
      int32_t i = 0;
      while (query_start[i + 1] <= row) ++i;
      const int32_t n = query_start[i + 1] - query_start[i];
      const int32_t pos = context_lens[i] - n + (row - query_start[i]);
      const int32_t L = pos + 1;
      std::vector<float> K(static_cast<size_t>(L) * d), V(static_cast<size_t>(L) * d), qf(d);
      const int32_t rc = pao_gather(K.data(), V.data(), key_cache, value_cache,
                                    block_tables + static_cast<int64_t>(i) * mb, L,
                                    h / G /* kv head */, hkv, d, bs, nb, dtype);
      if (rc != PAO_OK) {
        status.store(rc);
        continue;
      }
      const int64_t at = (static_cast<int64_t>(row) * hq + h) * d;
      for (int32_t e = 0; e < d; ++e) qf[e] = widen(q[at + e], dtype);
      attend(out_f32 + at, qf, K, V, L, d, scale);
      if (out_t)
        for (int32_t e = 0; e < d; ++e) out_t[at + e] = narrow(out_f32[at + e], dtype);
    }
  };
  std::vector<std::thread> pool;
  for (int32_t t = 1; t < T; ++t) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
  return status.load();
}

// ---------------------------------------------------------------------------
// INT8 KV cache.  The pages say only that quantising the KV cache to INT8
// halves its bytes ("LLM推理优化技术地图：从KV Cache到量化与投机解码", §4.3);
// the convention is this library's: symmetric, one fp32 scale per (token,
// kv head) row of d elements, all in fp32:
//   a    = max_e |x_e|                      (x widened exactly)
//   s    = a / 127
//   c_e  = clamp(round_half_even(x_e / s), -127, 127),   c = 0 when a = 0
// and the row dequantises to s * c_e (one fp32 product).  A row holding inf
// or NaN gets s = NaN and c = 0.  Codes live in the paged pools
// [nb][bs][hkv][d] (int8); scales in [nb][hkv][bs] (fp32).
// ---------------------------------------------------------------------------

static void quantize_row(const uint16_t* x, int32_t d, int32_t dtype, int8_t* c, float* s) {
  float a = 0.0f;
  bool finite = true;
  for (int32_t e = 0; e < d; ++e) {
    const float v = widen(x[e], dtype);
    if (!std::isfinite(v)) finite = false;
    a = std::max(a, std::fabs(v));
  }
  if (!finite) {
    *s = std::numeric_limits<float>::quiet_NaN();
    for (int32_t e = 0; e < d; ++e) c[e] = 0;
    return;
  }
  const float sc = a / 127.0f;
  *s = sc;
  for (int32_t e = 0; e < d; ++e) {
    if (a == 0.0f) {
      c[e] = 0;
      continue;
    }
    const float r = std::nearbyint(widen(x[e], dtype) / sc);
    c[e] = static_cast<int8_t>(std::min(127.0f, std::max(-127.0f, r)));
  }
}

int32_t pao_quantize_rows(const uint16_t* x, int64_t rows, int32_t d, int32_t dtype,
                          int8_t* codes, float* scales) {
  if (rows < 0 || d <= 0 || (dtype != PAO_F16 && dtype != PAO_BF16)) return PAO_BAD_ARG;
  if (rows > 0 && (!x || !codes || !scales)) return PAO_BAD_ARG;
  for (int64_t r = 0; r < rows; ++r) quantize_row(x + r * d, d, dtype, codes + r * d, scales + r);
  return PAO_OK;
}

int32_t pao_cache_write_int8(const uint16_t* key, const uint16_t* value, int8_t* key_cache,
                             int8_t* value_cache, float* key_scale, float* value_scale,
                             const int64_t* slot_mapping, int32_t n, int32_t hkv, int32_t d,
                             int32_t bs, int32_t nb, int32_t dtype) {
  if (n < 0 || hkv <= 0 || d <= 0 || bs <= 0 || nb <= 0 ||
      (dtype != PAO_F16 && dtype != PAO_BF16))
    return PAO_BAD_ARG;
  if (n > 0 && (!key || !value || !key_cache || !value_cache || !key_scale || !value_scale ||
                !slot_mapping))
    return PAO_BAD_ARG;
  const int64_t num_slots = static_cast<int64_t>(nb) * bs;
  std::vector<int64_t> used;
  for (int32_t t = 0; t < n; ++t) {
    if (slot_mapping[t] < 0) continue;
    if (slot_mapping[t] >= num_slots) return PAO_BAD_SLOT;
    used.push_back(slot_mapping[t]);
  }
  std::sort(used.begin(), used.end());
  if (std::adjacent_find(used.begin(), used.end()) != used.end()) return PAO_DUP_SLOT;
  for (int32_t t = 0; t < n; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    const int64_t blk = slot / bs, off = slot % bs;
    for (int32_t g = 0; g < hkv; ++g) {
      const int64_t src = (static_cast<int64_t>(t) * hkv + g) * d;
      const int64_t dst = ((blk * bs + off) * hkv + g) * d;
      const int64_t sdst = (blk * hkv + g) * bs + off;
      quantize_row(key + src, d, dtype, key_cache + dst, key_scale + sdst);
      quantize_row(value + src, d, dtype, value_cache + dst, value_scale + sdst);
    }
  }
  return PAO_OK;
}

int32_t pao_gather_int8(float* k_out, float* v_out, const int8_t* key_cache,
                        const int8_t* value_cache, const float* key_scale,
                        const float* value_scale, const int32_t* block_table_row, int32_t L,
                        int32_t g, int32_t hkv, int32_t d, int32_t bs, int32_t nb) {
  if (L <= 0) return PAO_BAD_LEN;
  if (g < 0 || g >= hkv) return PAO_BAD_ARG;
  for (int32_t j = 0; j < L; ++j) {
    const int64_t blk = block_table_row[j / bs];
    if (blk < 0 || blk >= nb) return PAO_BAD_BLOCK;
    const int64_t off = j % bs;
    const int64_t row = ((blk * bs + off) * hkv + g) * d;
    const float ks = key_scale[(blk * hkv + g) * bs + off];
    const float vs = value_scale[(blk * hkv + g) * bs + off];
    for (int32_t e = 0; e < d; ++e) {
      k_out[static_cast<int64_t>(j) * d + e] = ks * static_cast<float>(key_cache[row + e]);
      v_out[static_cast<int64_t>(j) * d + e] = vs * static_cast<float>(value_cache[row + e]);
    }
  }
  return PAO_OK;
}

int32_t pao_decode_int8_pairs(float* out_f32, uint16_t* out_t, const uint16_t* q,
                              const int8_t* key_cache, const int8_t* value_cache,
                              const float* key_scale, const float* value_scale,
                              const int32_t* block_tables, int32_t mb,
                              const int32_t* context_lens, int32_t s, int32_t hq, int32_t hkv,
                              int32_t d, int32_t bs, int32_t nb, float scale, int32_t dtype,
                              const int32_t* pairs, int32_t n_pairs, int32_t nthreads) {
  if (!shapes_ok(s, hq, hkv, d, bs, nb, mb, dtype) || n_pairs < 0) return PAO_BAD_ARG;
  for (int32_t p = 0; p < n_pairs; ++p)
    if (pairs[2 * p] < 0 || pairs[2 * p] >= s || pairs[2 * p + 1] < 0 || pairs[2 * p + 1] >= hq)
      return PAO_BAD_ARG;
  const int32_t group = hq / hkv;
  int32_t T = nthreads > 0 ? nthreads
                           : static_cast<int32_t>(std::thread::hardware_concurrency());
  T = std::max(1, std::min(T, std::max(n_pairs, 1)));
  std::atomic<int32_t> next(0), status(PAO_OK);
  auto worker = [&]() {
    for (int32_t p; (p = next.fetch_add(1)) < n_pairs;) {
      const int32_t i = pairs[2 * p], h = pairs[2 * p + 1];
      const int32_t L = context_lens[i];
      if (L <= 0 || L > static_cast<int64_t>(mb) * bs) {
        status.store(PAO_BAD_LEN);
        continue;
      }
      std::vector<float> K(static_cast<size_t>(L) * d), V(static_cast<size_t>(L) * d), qf(d);
      const int32_t rc = pao_gather_int8(K.data(), V.data(), key_cache, value_cache, key_scale,
                                         value_scale, block_tables + static_cast<int64_t>(i) * mb,
                                         L, /* kv head */ h / group, hkv, d, bs, nb);
      if (rc != PAO_OK) {
        status.store(rc);
        continue;
      }
      for (int32_t e = 0; e < d; ++e)
        qf[e] = widen(q[(static_cast<int64_t>(i) * hq + h) * d + e], dtype);
      float* o = out_f32 + static_cast<int64_t>(p) * d;
      attend(o, qf, K, V, L, d, scale);
      if (out_t)
        for (int32_t e = 0; e < d; ++e) out_t[static_cast<int64_t>(p) * d + e] = narrow(o[e], dtype);
    }
  };
  std::vector<std::thread> pool;
  for (int32_t t = 1; t < T; ++t) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
  return status.load();
}

uint64_t pao_kv_bytes_per_token(int32_t layers, int32_t kv_heads,
                                int32_t head_dim, int32_t elem_bytes) {
  return 2ull * static_cast<uint64_t>(layers) * static_cast<uint64_t>(kv_heads) *
         static_cast<uint64_t>(head_dim) * static_cast<uint64_t>(elem_bytes);
}

uint64_t pao_kv_bytes_gathered(const int32_t* context_lens, int32_t s,
                               int32_t hkv, int32_t d, int32_t elem_bytes) {
  uint64_t total = 0;
  for (int32_t i = 0; i < s; ++i)
    total += static_cast<uint64_t>(context_lens[i]) *
             pao_kv_bytes_per_token(1, hkv, d, elem_bytes);
  return total;
}
