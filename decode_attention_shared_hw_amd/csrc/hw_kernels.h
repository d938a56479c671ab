// hw_kernels.h — device helpers shared by the attention kernels (hw_decode.hip,
// hw_fused.hip): bf16 and DPP reductions, the RoPE rotation step, buffer
// resources and cache policies, and the MFMA tile step (K/V fragments, scores,
// online-softmax update).  Internal linkage: each source gets its own copy.
#pragma once

#include <type_traits>
#include <math.h>

#include "hw_internal.h"

namespace hw {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to bf16 (nearest even), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// cos/sin of delta * w with the angle formed and reduced mod 2*pi in fp64,
// so that positions of ~1e5 keep ~1e-7 rad of accuracy (fp32 pools).
__device__ __forceinline__ void rope_cos_sin(int64_t delta, double w, float* c, float* s) {
  const double a = static_cast<double>(delta) * w;
  const double k = rint(a * 0.15915494309189535);      // 1 / (2 pi)
  double r = fma(-k, 6.283185307179586, a);            // 2 pi, high part
  r = fma(-k, 2.4492935982947064e-16, r);              // 2 pi, low part
  sincosf(static_cast<float>(r), s, c);
}

// Same angle in revolutions, reduced exactly: frac is theta^(-2i/D)/(2 pi)
// mod 1 as a 64-bit binary fraction, so delta * frac mod 2^64 (integer
// wrap-around) is the angle's fractional revolution; its top 32 bits, as a
// signed value, give the angle in [-1/2, 1/2) revolution.  The hardware
// v_sin/v_cos take revolutions; the result carries ~1e-6 absolute error, far
// below the bf16 rounding applied to the rotated query on the MFMA path.
__device__ __forceinline__ void rope_cos_sin_fx(uint32_t delta, uint64_t frac, float* c,
                                                float* s) {
  // bits 32..63 of delta * frac (mod 2^64), delta < 2^32
  const uint32_t ph = __umulhi(delta, static_cast<uint32_t>(frac)) +
                      delta * static_cast<uint32_t>(frac >> 32);
  const float fr = static_cast<float>(static_cast<int32_t>(ph)) * 0x1p-32f;
  *s = __builtin_amdgcn_sinf(fr);
  *c = __builtin_amdgcn_cosf(fr);
}

// Lane l and lane l ^ 16 (l ^ 32) exchange values through the permlane swap
// instructions (no LDS round trip): the pair returned holds the lane's own
// value and its partner's, so a symmetric operation on the pair gives the
// same result in both lanes.
__device__ __forceinline__ float max_x16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_x16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// DPP move inside rows of 16 lanes.  The four patterns quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror and row_mirror, applied in turn with a
// symmetric combine, leave every lane with the combination of its 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppRow16[4] = {0xb1, 0x4e, 0x141, 0x140};

// max / sum over the 32 lanes of each half of the wave (every lane gets it)
__device__ __forceinline__ float half_max(float x) {
  x = fmaxf(x, dpp_mov<0xb1>(x));
  x = fmaxf(x, dpp_mov<0x4e>(x));
  x = fmaxf(x, dpp_mov<0x141>(x));
  x = fmaxf(x, dpp_mov<0x140>(x));
  return max_x16(x);
}
__device__ __forceinline__ float half_sum(float x) {
  x += dpp_mov<0xb1>(x);
  x += dpp_mov<0x4e>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return sum_x16(x);
}

constexpr int cmax(int x, int y) { return x > y ? x : y; }

// Raw buffer resource (gfx9 descriptor word 3): lane offsets are range-checked
// against `bytes`, so an offset past the end reads zero and writes nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0), bytes,
                                           0x00020000);
}

// Cache policy bits of gfx950 buffer accesses.
constexpr int kPolicySC0 = 1;   // past the CU's L1 (L2 of the XCD)
constexpr int kPolicyNT = 2;    // non-temporal: data read once (the K/V stream)
constexpr int kPolicySC1 = 16;  // device scope: coherent between all CUs of the GPU

// Phase timestamps of an instrumented build (HW_STAMPS, never in the
// library's own build): thread 0 of each workgroup (lane 0 of each wave for
// the per-wave stamps) records the 100 MHz real-time clock at fixed points.
#ifdef HW_STAMPS
__device__ uint64_t g_stamps[4096 * 32];
#define HW_STAMP(k) (g_stamps[blockIdx.x * 32 + (k)] = __builtin_amdgcn_s_memrealtime())
#define HW_MSTAMP(k) (g_stamps[(1024 + blockIdx.x) * 32 + (k)] = __builtin_amdgcn_s_memrealtime())
#else
#define HW_STAMP(k) ((void)0)
#define HW_MSTAMP(k) ((void)0)
#endif

// ------------------------------------------------------------- MFMA tile step
// Fragments (v_mfma_f32_16x16x32_bf16, lane l: i = l%16, q4 = l/16):
//   S^T[tok][row] = K[tok][:] . Q~[row][:]
//     A (K):  token i of half a, dims 8*(4s+q4)..+8  (one 16-B load)
//     B (Q~): row 16t+i, same dims
//     D:      tokens 16a + 4*q4 + v, row 16t+i
//   O^T[d][row] = V^T[d][tok] . P^T[tok][row]
//     A (V^T): dim 16m+i, tokens {4*q4+v, 16+4*q4+v} (one 16-B load)
//     B (P^T): row 16t+i, the same 8 tokens = this lane's S^T outputs
//     D:       dims 16m + 4*q4 + v, row 16t+i

// Stored K/V elements as MFMA A fragments (8 elements per lane): bf16 pools
// load 16 bytes and use them as they are; FP8 E4M3 pools load 8 bytes, which
// are widened to bf16 (exactly: every E4M3 value is a bf16 value) just before
// the product that consumes them, so the registers of a tile in flight hold
// the narrow codes.  POL is the loads' cache policy: non-temporal where every
// K/V fragment is read exactly once per call; the default (0) where two waves
// read each tile (the row groups of the run kernel), so that the second read
// finds it in L2.
template <typename E>
struct KvFrag;
template <>
struct KvFrag<uint16_t> {
  typedef u32x4 type;
  static constexpr int kBytes = 2;
  template <int POL>
  __device__ static type load(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, POL);
  }
  __device__ static u32x4 widen(const type& f) { return f; }
};
template <>
struct KvFrag<uint8_t> {
  typedef u32x2 type;
  static constexpr int kBytes = 1;
  template <int POL>
  __device__ static type load(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, POL);
  }
  template <bool HI>
  __device__ static uint32_t pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
  __device__ static u32x4 widen(const type& f) {
    return u32x4{pair<false>(f[0]), pair<true>(f[0]), pair<false>(f[1]), pair<true>(f[1])};
  }
};

// (a3) one buffer load per lane per fragment: every key load of a wave is one
// contiguous run (1 KB bf16, 512 B FP8), every value load four contiguous
// runs.  koff / voff: this lane's byte offsets inside a tile; tile: the tile's
// byte offset in the plane (wave-uniform, an SGPR operand).  The plane's
// resource range-checks the lane offsets; the tile offset is inside the plane
// by construction (a tile lies inside its block's capacity, whose slots the
// host checked against the plane).
template <int D, typename E, int POL = kPolicyNT>
__device__ __forceinline__ void load_keys(__amdgpu_buffer_rsrc_t krs, uint32_t tile, uint32_t koff,
                                          typename KvFrag<E>::type (&kf)[2][D / 32]) {
  constexpr int B = KvFrag<E>::kBytes;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      kf[h2][s] = KvFrag<E>::template load<POL>(krs, koff + (h2 * 16 * D + 4 * s * 128) * B, tile);
}

template <int D, typename E, int POL = kPolicyNT>
__device__ __forceinline__ void load_values(__amdgpu_buffer_rsrc_t vrs, uint32_t tile,
                                            uint32_t voff, typename KvFrag<E>::type (&vf)[D / 16]) {
  constexpr int B = KvFrag<E>::kBytes;
#pragma unroll
  for (int m = 0; m < D / 16; ++m)
    vf[m] = KvFrag<E>::template load<POL>(vrs, voff + 16 * m * 8 * B, tile);
}

// S^T for one tile: sc[h][t] holds tokens 16h + 4*q4 + v of rows 16t + li.
// qf: this lane's rotated-query B fragments, [NT][KS] x 64 lanes in LDS.
// Row tiles from ntv on (wave-uniform) have no fragments: their scores are 0.
template <int D, int NT, typename E>
__device__ __forceinline__ void tile_scores(const typename KvFrag<E>::type (&kf)[2][D / 32],
                                            const bf16x8* qf, int lane, f32x4 (&sc)[2][NT],
                                            int ntv = NT) {
  constexpr int KS = D / 32;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    f32x4 c0 = f32x4{0.f, 0.f, 0.f, 0.f}, c1 = c0;
#pragma unroll
    for (int s = 0; s < KS && t < ntv; ++s) {
      const bf16x8 qv = qf[(t * KS + s) * 64 + lane];
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, KvFrag<E>::widen(kf[0][s])), qv, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, KvFrag<E>::widen(kf[1][s])), qv, c1, 0, 0, 0);
    }
    sc[0][t] = c0;
    sc[1][t] = c1;
  }
}

// Online softmax of one tile's scores and the P.V update of the running
// (m, l, O^T).  Row t keeps the tile's tokens up to rowlim[t] (its causal
// limit, below `valid`); values of tokens at or past `valid` are zeroed.  The
// row sum adds the bf16-rounded weights the P.V product uses, so numerator
// and denominator carry the same weights.  Row tiles from ntv on (wave-
// uniform) are skipped.  BIG (kernels with many row tiles per wave, where
// wave-uniform branches pay for the VALU work they skip): a row tile whose
// rows all see the whole tile takes a path without the per-score masks, a
// row tile's accumulators are rescaled only when some row's maximum moved
// (the factor is otherwise exactly 1), and a whole tile's values are not
// masked.
template <int D, int NT, typename E, bool BIG = false>
__device__ __forceinline__ void tile_update(const f32x4 (&sc)[2][NT],
                                            const typename KvFrag<E>::type (&vf)[D / 16],
                                            const bool (&rowvis)[NT], const int (&rowlim)[NT],
                                            int valid, int q4,
                                            f32x4 (&acc)[D / 16][NT], float (&m_run)[NT],
                                            float (&l_run)[NT], int ntv = NT) {
  constexpr int MT = D / 16;
  bf16x8 pf[NT];
  if constexpr (!BIG) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntv) break;
      float sv[8];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tok = 16 * h2 + 4 * q4 + v;
          sv[4 * h2 + v] = (rowvis[t] && tok <= rowlim[t]) ? sc[h2][t][v] : -INFINITY;
        }
      float mt = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sv[e]);
      mt = max_x32(max_x16(mt));
      const float mn = fmaxf(m_run[t], mt);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float al = __builtin_amdgcn_exp2f(m_run[t] - mu);
      float sum = 0.f;
      bf16x8 f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f[e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(sv[e] - mu));
        sum += static_cast<float>(f[e]);
      }
      pf[t] = f;
      l_run[t] = l_run[t] * al + sum;
      m_run[t] = mn;
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m][t] *= al;
    }
    // tokens past the block's length may hold anything (even NaN): zero them
    u32x4 keep = u32x4{~0u, ~0u, ~0u, ~0u};
    if (valid < kTile) {
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int t0 = 16 * ((2 * e2) >> 2) + 4 * q4 + ((2 * e2) & 3);
        const int t1 = 16 * ((2 * e2 + 1) >> 2) + 4 * q4 + ((2 * e2 + 1) & 3);
        keep[e2] = (t0 < valid ? 0x0000ffffu : 0u) | (t1 < valid ? 0xffff0000u : 0u);
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const u32x4 v = KvFrag<E>::widen(vf[m]) & keep;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t >= ntv) break;
        acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), pf[t],
                                                            acc[m][t], 0, 0, 0);
      }
    }
  } else {
    auto row_softmax = [&](int t, auto masked_c) {
      constexpr bool masked = decltype(masked_c)::value;
      float sv[8];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tok = 16 * h2 + 4 * q4 + v;
          sv[4 * h2 + v] =
              (!masked || (rowvis[t] && tok <= rowlim[t])) ? sc[h2][t][v] : -INFINITY;
        }
      float mt = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sv[e]);
      mt = max_x32(max_x16(mt));
      const float mn = fmaxf(m_run[t], mt);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float al = __builtin_amdgcn_exp2f(m_run[t] - mu);
      float sum = 0.f;
      bf16x8 f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f[e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(sv[e] - mu));
        sum += static_cast<float>(f[e]);
      }
      pf[t] = f;
      l_run[t] = l_run[t] * al + sum;
      m_run[t] = mn;
      if (__builtin_amdgcn_ballot_w64(al != 1.f) != 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m][t] *= al;
      }
    };
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntv) break;
      if (__builtin_amdgcn_ballot_w64(!rowvis[t] || rowlim[t] < kTile - 1) == 0)
        row_softmax(t, std::false_type{});
      else
        row_softmax(t, std::true_type{});
    }
    // tokens past the block's length may hold anything (even NaN): zero them
    auto pv = [&](auto partial_c) {
      constexpr bool partial = decltype(partial_c)::value;
      u32x4 keep = u32x4{~0u, ~0u, ~0u, ~0u};
      if (partial) {
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int t0 = 16 * ((2 * e2) >> 2) + 4 * q4 + ((2 * e2) & 3);
          const int t1 = 16 * ((2 * e2 + 1) >> 2) + 4 * q4 + ((2 * e2 + 1) & 3);
          keep[e2] = (t0 < valid ? 0x0000ffffu : 0u) | (t1 < valid ? 0xffff0000u : 0u);
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        u32x4 v = KvFrag<E>::widen(vf[m]);
        if (partial) v &= keep;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t >= ntv) break;
          acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v),
                                                              pf[t], acc[m][t], 0, 0, 0);
        }
      }
    };
    if (valid < kTile)
      pv(std::true_type{});
    else
      pv(std::false_type{});
  }
}

// A group's first tile is requested after its rotated queries are published
// (0), its keys before the rotation (1), keys and values before it (2), or
// (3) keys and values before it by the upper half of the waves while the
// lower half rotates.  A
// CU takes about 64 KB of outstanding loads before a wave's next load blocks
// at issue, so requesting 8 waves' 16 KB tiles first stalls the rotation and
// the barrier behind it until the first tiles return.
}  // namespace
}  // namespace hw
