// hogwild_oracle.cpp — plain fp64 CPU reference for Hogwild! concurrent
// attention.  TEST INFRASTRUCTURE ONLY (see hogwild_oracle.h): the product
// library never includes, links or calls this file.
//
// Build: g++ -O2 -std=c++17 -ffp-contract=off -shared -fPIC
//
// Every routine follows the pages step by step, with no blocking, fusion or
// reordering beyond what the definition states.

#include "hogwild_oracle.h"

#include <cfenv>
#include <cmath>
#include <cstring>
#include <vector>

namespace {

// The stored value of x in a pool of type dtype (scale: the plane's FP8 scale).
double store_round(int32_t dtype, double x, double scale) {
  if (dtype == HWO_BF16) return hwo_round_bf16(x);
  if (dtype == HWO_FP8) return scale * hwo_round_e4m3(x / scale);
  return static_cast<double>(static_cast<float>(x));
}

bool scales_ok(const double* s, int64_t n) {
  if (!s) return false;
  for (int64_t i = 0; i < n; ++i)
    if (!(s[i] > 0.0) || !std::isfinite(s[i])) return false;
  return true;
}

// Inverse frequency of pair i for head size D:  theta^(-2i/D)
// (omica.com.cn news 1114328, section 2.1, rotate_query: 1/base^(arange(0,dim,2)/dim)).
double inv_freq(double theta, int32_t i, int32_t D) {
  return std::pow(theta, -2.0 * static_cast<double>(i) / static_cast<double>(D));
}

// Plain dot product in fp64.
double dot(const double* a, const double* b, int32_t D) {
  double s = 0.0;
  for (int32_t d = 0; d < D; ++d) s += a[d] * b[d];
  return s;
}

}  // namespace

extern "C" {

// Round to nearest bf16 (8 significant bits, fp32 exponent range), ties to
// even, in one step from the double (no detour through float, which could
// round twice).
double hwo_round_bf16(double x) {
  if (!std::isfinite(x) || x == 0.0) return x;
  int e = 0;
  std::frexp(x, &e);  // |x| = m * 2^e, m in [0.5, 1)
  // Quantum of the bf16 grid at this magnitude: 2^(e-8) for normal numbers;
  // subnormal bf16 values share the quantum 2^-133.
  int qexp = e - 8;
  if (qexp < -133) qexp = -133;
  const int saved = std::fegetround();
  std::fesetround(FE_TONEAREST);
  const double r = std::nearbyint(std::ldexp(x, -qexp));  // ties to even
  std::fesetround(saved);
  const double y = std::ldexp(r, qexp);
  const double bf16_max = std::ldexp(255.0, 120);  // (2 - 2^-7) * 2^127
  if (std::fabs(y) > bf16_max) return std::copysign(HUGE_VAL, x);
  return y;
}

double hwo_round_f32(double x) { return static_cast<double>(static_cast<float>(x)); }

// OCP FP8 E4M3 (e4m3fn), read off its definition: sign, exponent field e
// (bias 7), mantissa m; e = 0 is subnormal; e = 15 with m = 7 is NaN.
double hwo_e4m3_value(int32_t code) {
  const int32_t c = code & 0xff;
  const int32_t e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return std::nan("");
  const double v = e == 0 ? std::ldexp(static_cast<double>(m), -9)
                          : std::ldexp(static_cast<double>(8 + m), e - 10);
  return (c & 0x80) ? -v : v;
}

// Nearest E4M3 value, ties to even, in one step from the double.  The grid
// at |x| in [2^(k-1), 2^k) has 3 fraction bits, quantum 2^(k-4); below 2^-6
// the subnormal quantum 2^-9.  Magnitudes past 448 saturate to 448 (the
// format has no infinity).
double hwo_round_e4m3(double x) {
  if (std::isnan(x) || x == 0.0) return x;
  if (std::isinf(x)) return std::copysign(448.0, x);
  int k = 0;
  std::frexp(x, &k);
  int qexp = k - 4;
  if (qexp < -9) qexp = -9;
  const int saved = std::fegetround();
  std::fesetround(FE_TONEAREST);
  const double r = std::nearbyint(std::ldexp(x, -qexp));  // ties to even
  std::fesetround(saved);
  const double y = std::ldexp(r, qexp);
  if (std::fabs(y) > 448.0) return std::copysign(448.0, x);
  return y;
}

// RoPE with rotate-half pairing: element i rotates with element i + D/2 by the
// angle pos * theta^(-2i/D)  (omica 1114328 section 2.1: q*cos + rotate_half(q)*sin,
// rotate_half(x) = (-x[D/2:], x[:D/2])).
void hwo_rope(const double* x, int32_t D, double theta, double pos, double* y) {
  const int32_t half = D / 2;
  std::vector<double> tmp(x, x + D);
  for (int32_t i = 0; i < half; ++i) {
    const double ang = pos * inv_freq(theta, i, D);
    const double c = std::cos(ang);
    const double s = std::sin(ang);
    y[i] = tmp[i] * c - tmp[i + half] * s;
    y[i + half] = tmp[i + half] * c + tmp[i] * s;
  }
}

// Combined layout (Hogwild! notes, key design 2): common cache first, then the
// other workers' unfinished steps in worker order, then the current worker's
// own step.  view_offset is where each block starts in this worker's view.
int32_t hwo_build_combined_tables(int32_t W, int32_t common_block, const int32_t* worker_block,
                                  int32_t num_blocks, const int32_t* block_len,
                                  int32_t* tbl_block, int32_t* tbl_off, int32_t* num_entries) {
  if (W <= 0 || common_block < 0 || common_block >= num_blocks) return HWO_EINVAL;
  for (int32_t w = 0; w < W; ++w) {
    const int32_t b = worker_block[w];
    if (b < 0 || b >= num_blocks || b == common_block) return HWO_EINVAL;
    for (int32_t v = 0; v < w; ++v)
      if (worker_block[v] == b) return HWO_EINVAL;
  }
  const int32_t E = W + 1;
  for (int32_t w = 0; w < W; ++w) {
    int32_t e = 0;
    int32_t off = 0;
    auto put = [&](int32_t b) {
      tbl_block[w * E + e] = b;
      tbl_off[w * E + e] = off;
      off += block_len[b];
      ++e;
    };
    put(common_block);
    for (int32_t v = 0; v < W; ++v)
      if (v != w) put(worker_block[v]);
    put(worker_block[w]);
    num_entries[w] = e;
  }
  return HWO_OK;
}

int32_t hwo_build_interleaved_tables(int32_t W, int32_t common_block, const int32_t* worker_block,
                                     int32_t num_blocks, const int32_t* block_len,
                                     int32_t* tbl_block, int32_t* tbl_off, int32_t* num_entries) {
  // same arguments and checks as the combined layout; only the entries differ
  const int32_t rc = hwo_build_combined_tables(W, common_block, worker_block, num_blocks,
                                               block_len, tbl_block, tbl_off, num_entries);
  if (rc != HWO_OK) return rc;
  const int32_t E = W + 1;
  for (int32_t w = 0; w < W; ++w) {
    for (int32_t e = 0; e < E; ++e) {
      tbl_block[w * E + e] = 0;
      tbl_off[w * E + e] = 0;
    }
    tbl_block[w * E] = common_block;
    tbl_off[w * E] = 0;
    tbl_block[w * E + 1] = worker_block[w];
    tbl_off[w * E + 1] = block_len[common_block];
    num_entries[w] = 2;
  }
  return HWO_OK;
}

// The query sits at the last position of its own view (its K/V was written
// before attention, as in ordinary decode).
int64_t hwo_query_position(int32_t n_entries, const int32_t* tbl_block, const int32_t* tbl_off,
                           const int32_t* block_len) {
  int64_t iq = -1;
  for (int32_t e = 0; e < n_entries; ++e) {
    const int32_t len = block_len[tbl_block[e]];
    if (len <= 0) continue;
    const int64_t last = static_cast<int64_t>(tbl_off[e]) + len - 1;
    if (last > iq) iq = last;
  }
  return iq;
}

// One query row at view position i_q - lag (lag = 0: the decode query), over
// the view's tokens at view positions <= that position.
static int32_t attn_row(int32_t form, int32_t D, double theta, int32_t n_entries,
                        const int32_t* tbl_block, const int32_t* tbl_off, int32_t num_blocks,
                        const int32_t* block_len, const int64_t* block_start, int32_t lag,
                        const double* q, const double* K_plane, const double* V_plane,
                        double* out) {
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  if (D <= 0 || D % 2 != 0 || (form != 0 && form != 1)) return HWO_EINVAL;
  for (int32_t e = 0; e < n_entries; ++e) {
    const int32_t b = tbl_block[e];
    if (b < 0 || b >= num_blocks) return HWO_EINVAL;
    for (int32_t f = 0; f < e; ++f)
      if (tbl_block[f] == b) return HWO_EINVAL;
  }
  const int64_t iq = hwo_query_position(n_entries, tbl_block, tbl_off, block_len) - lag;
  if (iq < 0 || lag < 0) return HWO_ENOTOKENS;

  const double scale = 1.0 / std::sqrt(static_cast<double>(D));
  std::vector<double> scores;  // concatenation over blocks, in table order
  std::vector<const double*> values;
  std::vector<double> qr(D), kr(D), kraw(D);

  if (form == 0) {
    // Definition: encode the query at its absolute position i_q ...
    hwo_rope(q, D, theta, static_cast<double>(iq), qr.data());
    for (int32_t e = 0; e < n_entries; ++e) {
      const int32_t b = tbl_block[e];
      const int64_t off = tbl_off[e];
      for (int32_t j = 0; j < block_len[b] && off + j <= iq; ++j) {
        const double* kst = K_plane + (block_start[b] + j) * static_cast<int64_t>(D);
        // ... and every key at its absolute view position off + j: undo the
        // local encoding at j (storage convention: local positions 0..len-1),
        // then encode at off + j.
        hwo_rope(kst, D, theta, -static_cast<double>(j), kraw.data());
        hwo_rope(kraw.data(), D, theta, static_cast<double>(off + j), kr.data());
        scores.push_back(dot(qr.data(), kr.data(), D) * scale);
        values.push_back(V_plane + (block_start[b] + j) * static_cast<int64_t>(D));
      }
    }
  } else {
    // Method: rho(q, i_q - off) against each block's keys as stored.
    for (int32_t e = 0; e < n_entries; ++e) {
      const int32_t b = tbl_block[e];
      const int64_t off = tbl_off[e];
      if (block_len[b] <= 0 || off > iq) continue;
      hwo_rope(q, D, theta, static_cast<double>(iq - off), qr.data());
      for (int32_t j = 0; j < block_len[b] && off + j <= iq; ++j) {
        const double* kst = K_plane + (block_start[b] + j) * static_cast<int64_t>(D);
        scores.push_back(dot(qr.data(), kst, D) * scale);
        values.push_back(V_plane + (block_start[b] + j) * static_cast<int64_t>(D));
      }
    }
  }

  // One softmax over the concatenation of every block's scores.
  double m = -HUGE_VAL;
  for (double s : scores) m = s > m ? s : m;
  double denom = 0.0;
  std::vector<double> p(scores.size());
  for (size_t t = 0; t < scores.size(); ++t) {
    p[t] = std::exp(scores[t] - m);
    denom += p[t];
  }
  if (scores.empty()) return HWO_ENOTOKENS;
  for (size_t t = 0; t < scores.size(); ++t) {
    const double w = p[t] / denom;
    for (int32_t d = 0; d < D; ++d) out[d] += w * values[t][d];
  }
  return HWO_OK;
}

int32_t hwo_attn_one(int32_t form, int32_t D, double theta, int32_t n_entries,
                     const int32_t* tbl_block, const int32_t* tbl_off, int32_t num_blocks,
                     const int32_t* block_len, const int64_t* block_start, const double* q,
                     const double* K_plane, const double* V_plane, double* out) {
  return attn_row(form, D, theta, n_entries, tbl_block, tbl_off, num_blocks, block_len,
                  block_start, 0, q, K_plane, V_plane, out);
}

int32_t hwo_attn_decode(int32_t form, int32_t W, int32_t Hq, int32_t Hkv, int32_t D, double theta,
                        int32_t E, const int32_t* tbl_block, const int32_t* tbl_off,
                        const int32_t* num_entries, int32_t num_blocks, const int32_t* block_len,
                        const int64_t* block_start, int64_t num_slots, const double* q,
                        const double* K, const double* V, double* out) {
  if (W <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return HWO_EINVAL;
  const int32_t G = Hq / Hkv;  // grouped-query attention: q-heads per kv head
  int32_t rc = HWO_OK;
  for (int32_t w = 0; w < W; ++w) {
    if (num_entries[w] < 0 || num_entries[w] > E) return HWO_EINVAL;
    for (int32_t h = 0; h < Hq; ++h) {
      const int32_t g = h / G;
      const int64_t plane = static_cast<int64_t>(g) * num_slots * D;
      const int32_t r = hwo_attn_one(form, D, theta, num_entries[w], tbl_block + w * E,
                                     tbl_off + w * E, num_blocks, block_len, block_start,
                                     q + (static_cast<int64_t>(w) * Hq + h) * D, K + plane,
                                     V + plane, out + (static_cast<int64_t>(w) * Hq + h) * D);
      if (r != HWO_OK && rc == HWO_OK) rc = r;
    }
  }
  return rc;
}

int32_t hwo_attn_chunk(int32_t form, int32_t W, int32_t n, int32_t Hq, int32_t Hkv, int32_t D,
                       double theta, int32_t E, const int32_t* tbl_block, const int32_t* tbl_off,
                       const int32_t* num_entries, int32_t num_blocks, const int32_t* block_len,
                       const int64_t* block_start, int64_t num_slots, const double* q,
                       const double* K, const double* V, double* out) {
  if (W <= 0 || n <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return HWO_EINVAL;
  const int32_t G = Hq / Hkv;
  int32_t rc = HWO_OK;
  for (int32_t w = 0; w < W; ++w) {
    if (num_entries[w] < 0 || num_entries[w] > E) return HWO_EINVAL;
    for (int32_t j = 0; j < n; ++j) {
      for (int32_t h = 0; h < Hq; ++h) {
        const int64_t plane = static_cast<int64_t>(h / G) * num_slots * D;
        const int64_t row = (static_cast<int64_t>(w) * n + j) * Hq + h;
        const int32_t r = attn_row(form, D, theta, num_entries[w], tbl_block + w * E,
                                   tbl_off + w * E, num_blocks, block_len, block_start,
                                   n - 1 - j, q + row * D, K + plane, V + plane, out + row * D);
        if (r != HWO_OK && rc == HWO_OK) rc = r;
      }
    }
  }
  return rc;
}

// Step completion: the finished step's KV is rotated and moved into the shared
// history (Hogwild! notes, key design 2).  A src key stored at local position
// j becomes dst's token len_dst + j: undo the encoding at j, encode at
// len_dst + j, round to the storage type.
int32_t hwo_block_append(int32_t L, int32_t Hkv, int32_t D, int64_t num_slots, double* K, double* V,
                         int32_t num_blocks, const int64_t* block_start, const int32_t* block_cap,
                         int32_t* block_len, int32_t src, int32_t dst, double theta, int32_t dtype,
                         const double* k_scale) {
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return HWO_EINVAL;
  if (dtype != HWO_F32 && dtype != HWO_BF16 && dtype != HWO_FP8) return HWO_EINVAL;
  if (dtype == HWO_FP8 && !scales_ok(k_scale, static_cast<int64_t>(L) * Hkv)) return HWO_EINVAL;
  const int32_t ls = block_len[src];
  const int32_t ld = block_len[dst];
  if (static_cast<int64_t>(ld) + ls > block_cap[dst]) return HWO_ECAPACITY;
  std::vector<double> raw(D), enc(D);
  for (int32_t l = 0; l < L; ++l) {
    for (int32_t g = 0; g < Hkv; ++g) {
      const int64_t plane = (static_cast<int64_t>(l) * Hkv + g) * num_slots * D;
      const double ks = dtype == HWO_FP8 ? k_scale[l * Hkv + g] : 1.0;
      for (int32_t j = 0; j < ls; ++j) {
        const int64_t s_src = plane + (block_start[src] + j) * static_cast<int64_t>(D);
        const int64_t s_dst = plane + (block_start[dst] + ld + j) * static_cast<int64_t>(D);
        hwo_rope(K + s_src, D, theta, -static_cast<double>(j), raw.data());
        hwo_rope(raw.data(), D, theta, static_cast<double>(ld) + j, enc.data());
        for (int32_t d = 0; d < D; ++d) {
          K[s_dst + d] = store_round(dtype, enc[d], ks);
          V[s_dst + d] = V[s_src + d];
        }
      }
    }
  }
  block_len[dst] = ld + ls;
  block_len[src] = 0;
  return HWO_OK;
}

int32_t hwo_block_write(int32_t Hkv, int32_t D, int64_t num_slots, double* K, double* V,
                        int32_t num_blocks, const int64_t* block_start, const int32_t* block_len,
                        int32_t n, const int32_t* blocks, const double* k_new,
                        const double* v_new, double theta, int32_t dtype, const double* k_scale,
                        const double* v_scale) {
  if (dtype != HWO_F32 && dtype != HWO_BF16 && dtype != HWO_FP8) return HWO_EINVAL;
  if (dtype == HWO_FP8 && (!scales_ok(k_scale, Hkv) || !scales_ok(v_scale, Hkv))) return HWO_EINVAL;
  for (int32_t i = 0; i < n; ++i) {
    if (blocks[i] < 0 || blocks[i] >= num_blocks) return HWO_EINVAL;
    if (block_len[blocks[i]] < 1) return HWO_ENOTOKENS;
  }
  std::vector<double> enc(D);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    const int64_t pos = block_len[b] - 1;
    for (int32_t g = 0; g < Hkv; ++g) {
      const double* kr = k_new + (static_cast<int64_t>(i) * Hkv + g) * D;
      const double* vr = v_new + (static_cast<int64_t>(i) * Hkv + g) * D;
      const int64_t s = (static_cast<int64_t>(g) * num_slots + block_start[b] + pos) * D;
      hwo_rope(kr, D, theta, static_cast<double>(pos), enc.data());
      const double ks = dtype == HWO_FP8 ? k_scale[g] : 1.0;
      const double vs = dtype == HWO_FP8 ? v_scale[g] : 1.0;
      for (int32_t d = 0; d < D; ++d) {
        K[s + d] = store_round(dtype, enc[d], ks);
        V[s + d] = store_round(dtype, vr[d], vs);
      }
    }
  }
  return HWO_OK;
}

}  // extern "C"
