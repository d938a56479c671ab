// hw_decode.hip — fused concurrent-attention decode kernels for gfx950.
//
// One launch per layer.  Work unit = (kv head g, unit u): a contiguous range
// of 32-token tiles in the concatenation of the visible blocks of head g.
// Each workgroup
//   1. decodes the worker tables and device block lengths into a plan
//      (visibility, view offsets, i_q, tile prefix)           [prologue]
//   2. for every block its range touches, rotates the stacked W*G query rows
//      of head g by i_q - view_offset (Hogwild! notes, key design 1: only the
//      single query token is rotated, never the cache)         [a2]
//   3. streams its K/V tiles once for all rows with an online softmax in the
//      exp2 domain (Flash-Decoding split-K; news 1114328 sec. 3.2)  [a3]
//   4. writes its partial (m, l, acc) and meets the other units of head g at
//      a per-head barrier; then every unit merges its own slice of the head's
//      outputs by log-sum-exp weights in fixed unit order (deterministic)  [a4]
//
// Two main loops share the prologue and the epilogue:
//   decode_valu<T>   fp32 VALU arithmetic over LDS tiles; fp32 and bf16 pools.
//   decode_mfma<D,NT> bf16 MFMA 16x16x32: S^T = K Q~^T and O^T = V^T P^T, with
//                    tiles loaded straight into operand fragments (the pool
//                    layout matches them), rows = W*G <= 32.
#include <math.h>

#include "hw_internal.h"

namespace hw {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

// cos/sin of delta * w with the angle formed and reduced mod 2*pi in fp64,
// so that positions of ~1e5 keep ~1e-7 rad of accuracy.
__device__ __forceinline__ void rope_cos_sin(int64_t delta, double w, float* c, float* s) {
  const double a = static_cast<double>(delta) * w;
  const double k = rint(a * 0.15915494309189535);      // 1 / (2 pi)
  double r = fma(-k, 6.283185307179586, a);            // 2 pi, high part
  r = fma(-k, 2.4492935982947064e-16, r);              // 2 pi, low part
  sincosf(static_cast<float>(r), s, c);
}

// ----------------------------------------------------------------- prologue
struct Plan {
  int32_t len[HW_MAX_BLOCKS];
  uint32_t vis[HW_MAX_BLOCKS];        // bit w set: worker w sees block b
  int32_t tile0[HW_MAX_BLOCKS + 1];   // tiles of visible blocks, prefix sums
  int64_t iq[HW_MAX_WORKERS];         // query position per worker, -1: none
  int32_t off[HW_MAX_WORKERS * HW_MAX_BLOCKS];
  int32_t flags;
  int32_t head, unit, lo, hi;
};

__device__ void build_plan(const DecodeArgs& a, Plan& p) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    p.flags = 0;
    int lin = blockIdx.x;
    const int grid = gridDim.x;
    if (a.xcd_map) lin = (blockIdx.x & 7) * (grid >> 3) + (blockIdx.x >> 3);
    p.head = lin / a.P;
    p.unit = lin % a.P;
  }
  for (int i = tid; i < a.NB; i += kThreads) {
    int len = a.block_len[i];
    if (len < 0 || len > a.block_cap[i]) {
      atomicOr(&p.flags, HW_DEV_BAD_LENGTH);
      len = 0;
    }
    p.len[i] = len;
    p.vis[i] = 0u;
  }
  for (int i = tid; i < a.W * a.NB; i += kThreads) p.off[i] = 0;
  __syncthreads();
  __shared__ uint32_t bad_workers;
  if (tid == 0) bad_workers = 0u;
  __syncthreads();
  for (int i = tid; i < a.W * a.E; i += kThreads) {
    const int w = i / a.E;
    const int e = i - w * a.E;
    const int ne = a.num_entries[w];
    if (ne < 0 || ne > a.E) {
      atomicOr(&bad_workers, 1u << w);
      continue;
    }
    if (e >= ne) continue;
    const hw_entry en = a.tables[i];
    if (en.block_id < 0 || en.block_id >= a.NB) {
      atomicOr(&bad_workers, 1u << w);
      continue;
    }
    const uint32_t old = atomicOr(&p.vis[en.block_id], 1u << w);
    if (old & (1u << w)) atomicOr(&bad_workers, 1u << w);
    p.off[w * a.NB + en.block_id] = en.view_offset;
  }
  __syncthreads();
  if (bad_workers) {
    // a worker with a malformed table sees nothing: its rows come out as zeros
    for (int i = tid; i < a.NB; i += kThreads) p.vis[i] &= ~bad_workers;
    if (tid == 0) atomicOr(&p.flags, HW_DEV_BAD_ENTRY);
  }
  __syncthreads();
  if (tid < a.W) {
    int64_t iq = -1;
    for (int b = 0; b < a.NB; ++b) {
      if (((p.vis[b] >> tid) & 1u) && p.len[b] > 0) {
        const int64_t last = static_cast<int64_t>(p.off[tid * a.NB + b]) + p.len[b] - 1;
        iq = last > iq ? last : iq;
      }
    }
    p.iq[tid] = iq;
  }
  if (tid == 64) {
    int acc = 0;
    for (int b = 0; b < a.NB; ++b) {
      p.tile0[b] = acc;
      if (p.vis[b] != 0u && p.len[b] > 0) acc += (p.len[b] + kTile - 1) / kTile;
    }
    p.tile0[a.NB] = acc;
    const int64_t n = acc;
    p.lo = static_cast<int>(n * p.unit / a.P);
    p.hi = static_cast<int>(n * (p.unit + 1) / a.P);
  }
  __syncthreads();
}

// Block holding global tile j of the plan (cursor walks forward).
__device__ __forceinline__ int block_of_tile(const Plan& p, int nb, int j, int b) {
  while (b + 1 < nb && p.tile0[b + 1] <= j) ++b;
  return b;
}

// ----------------------------------------------------------------- epilogue
// Per-head barrier + merge of this unit's slice of the head's R*D outputs.
// Requires every workgroup of the launch to be resident (grid sized by the
// host from occupancy); the wait is bounded and reports kDevSyncTimeout.
__device__ void head_barrier_and_merge(const DecodeArgs& a, Plan& p, float* wgt) {
  const int tid = threadIdx.x;
  const int g = p.head, u = p.unit;
  __shared__ int timed_out;
  __syncthreads();  // every partial store of this workgroup has been issued
  if (tid == 0) {
    __threadfence();
    uint32_t* arrive = a.ws_sync + g;
    atomicAdd(arrive, 1u);
    uint32_t n = 0;
    int spins = 0;
    while ((n = __hip_atomic_load(arrive, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT)) <
               static_cast<uint32_t>(a.P) &&
           spins < (1 << 22)) {
      __builtin_amdgcn_s_sleep(2);
      ++spins;
    }
    timed_out = n < static_cast<uint32_t>(a.P);
    __threadfence();
  }
  __syncthreads();
  const int RD = a.R * a.D;
  const int o_lo = static_cast<int>(static_cast<int64_t>(RD) * u / a.P);
  const int o_hi = static_cast<int>(static_cast<int64_t>(RD) * (u + 1) / a.P);
  if (!timed_out && o_hi > o_lo) {
    const int r_lo = o_lo / a.D;
    const int r_hi = (o_hi - 1) / a.D;  // inclusive
    const int nr = r_hi - r_lo + 1;
    const float2* ml = a.ws_ml + static_cast<int64_t>(g) * a.P * a.R;
    // per-row max and normalizer over the units, in unit order
    for (int rr = tid; rr < nr; rr += kThreads) {
      const int r = r_lo + rr;
      float M = -INFINITY;
      for (int k = 0; k < a.P; ++k) M = fmaxf(M, ml[k * a.R + r].x);
      float L = 0.f;
      if (M != -INFINITY)
        for (int k = 0; k < a.P; ++k) {
          const float2 v = ml[k * a.R + r];
          L += v.y * __builtin_amdgcn_exp2f(v.x - M);
        }
      wgt[a.P * nr + 2 * rr] = M;
      wgt[a.P * nr + 2 * rr + 1] = L > 0.f ? 1.f / L : 0.f;
      if (!(L > 0.f)) atomicOr(a.status, HW_DEV_NO_TOKENS);
    }
    __syncthreads();
    for (int i = tid; i < a.P * nr; i += kThreads) {
      const int k = i / nr, rr = i - k * nr;
      const float M = wgt[a.P * nr + 2 * rr];
      const float invL = wgt[a.P * nr + 2 * rr + 1];
      const float mk = ml[k * a.R + r_lo + rr].x;
      wgt[i] = (invL > 0.f && mk != -INFINITY) ? __builtin_amdgcn_exp2f(mk - M) * invL : 0.f;
    }
    __syncthreads();
    const float* acc = a.ws_acc + static_cast<int64_t>(g) * a.P * RD;
    for (int o = o_lo + tid; o < o_hi; o += kThreads) {
      const int r = o / a.D;
      const int d = o - r * a.D;
      const int rr = r - r_lo;
      float s = 0.f;
      for (int k = 0; k < a.P; ++k) s += acc[static_cast<int64_t>(k) * RD + o] * wgt[k * nr + rr];
      const int w = r / a.G;
      const int h = g * a.G + (r - w * a.G);
      a.out[(static_cast<int64_t>(w) * a.Hq + h) * a.D + d] = s;
    }
  }
  __syncthreads();
  if (tid == 0) {
    if (timed_out) atomicOr(a.status, kDevSyncTimeout);
    if (p.flags) atomicOr(a.status, p.flags);
    uint32_t* depart = a.ws_sync + a.Hkv + g;
    const uint32_t old = atomicAdd(depart, 1u);
    if (old == static_cast<uint32_t>(a.P) - 1u) {
      // last one out: every unit of this head has passed the barrier
      __hip_atomic_store(a.ws_sync + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(depart, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------- VALU kernel
// Generic path: any dtype, rows <= HW_MAX_ROWS, D in {64, 128}.  Tiles are
// staged in LDS in logical [token][dim] order; scores, softmax and P.V run
// in fp32 on the vector ALUs.
constexpr int kValuMaxAcc = HW_MAX_ROWS * 128 / kThreads;  // 32

template <typename T>
__global__ __launch_bounds__(kThreads) void decode_valu(DecodeArgs a) {
  __shared__ Plan plan;
  __shared__ float qr[HW_MAX_ROWS * 128];
  __shared__ float ks[kTile * 129];
  __shared__ float vs[kTile * 128];
  __shared__ float ps[HW_MAX_ROWS * (kTile + 1)];
  __shared__ float m_s[HW_MAX_ROWS], l_s[HW_MAX_ROWS], al_s[HW_MAX_ROWS];
  build_plan(a, plan);
  const int tid = threadIdx.x;
  const int g = plan.head;
  const int D = a.D, R = a.R, half = D / 2;
  const T* qg = static_cast<const T*>(a.q);
  const T* kp = static_cast<const T*>(a.k) + g * a.plane_elems;
  const T* vp = static_cast<const T*>(a.v) + g * a.plane_elems;
  for (int r = tid; r < R; r += kThreads) {
    m_s[r] = -INFINITY;
    l_s[r] = 0.f;
  }
  float acc[kValuMaxAcc];
#pragma unroll
  for (int k = 0; k < kValuMaxAcc; ++k) acc[k] = 0.f;
  int b = 0, cur_b = -1;
  for (int j = plan.lo; j < plan.hi; ++j) {
    b = block_of_tile(plan, a.NB, j, b);
    if (b != cur_b) {
      __syncthreads();
      // rotate every row of head g for this block: q~ = rho(q, i_q - off)
      for (int x = tid; x < R * half; x += kThreads) {
        const int r = x / half, i = x - r * half;
        const int w = r / a.G, h = g * a.G + (r - w * a.G);
        const bool vis = (plan.vis[b] >> w) & 1u;
        float c = 0.f, s = 0.f;
        if (vis) rope_cos_sin(plan.iq[w] - plan.off[w * a.NB + b], a.inv_freq[i], &c, &s);
        const int64_t qo = (static_cast<int64_t>(w) * a.Hq + h) * D;
        const float x0 = load_elem(qg, qo + i), x1 = load_elem(qg, qo + i + half);
        qr[r * D + i] = vis ? (x0 * c - x1 * s) * a.qscale : 0.f;
        qr[r * D + i + half] = vis ? (x1 * c + x0 * s) * a.qscale : 0.f;
      }
      cur_b = b;
    }
    const int tl = j - plan.tile0[b];
    const int valid = min(kTile, plan.len[b] - tl * kTile);
    const int64_t base = (a.block_start[b] + static_cast<int64_t>(tl) * kTile) * D;
    __syncthreads();
    for (int x = tid; x < kTile * D; x += kThreads) {
      // key tile element x of the pool layout -> (token, dim)
      const int hk = x / (16 * D), rk = x - hk * 16 * D;
      const int tk = hk * 16 + ((rk & 127) >> 3), dk = (rk >> 7) * 8 + (rk & 7);
      ks[tk * 129 + dk] = load_elem(kp, base + x);
      // value tile element x -> (token, dim)
      const int gv = x / (8 * D), rv = x - gv * 8 * D;
      const int sv = rv & 7, dv = rv >> 3;
      const int tv = (sv >> 2) * 16 + gv * 4 + (sv & 3);
      vs[tv * D + dv] = tv < valid ? load_elem(vp, base + x) : 0.f;
    }
    __syncthreads();
    for (int x = tid; x < R * kTile; x += kThreads) {
      const int r = x / kTile, t = x - r * kTile;
      const int w = r / a.G;
      float s = -INFINITY;
      if (t < valid && ((plan.vis[b] >> w) & 1u)) {
        s = 0.f;
        for (int d = 0; d < D; ++d) s += qr[r * D + d] * ks[t * 129 + d];
      }
      ps[r * (kTile + 1) + t] = s;
    }
    __syncthreads();
    for (int r = tid; r < R; r += kThreads) {
      float mt = -INFINITY;
      for (int t = 0; t < kTile; ++t) mt = fmaxf(mt, ps[r * (kTile + 1) + t]);
      const float mn = fmaxf(m_s[r], mt);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float al = __builtin_amdgcn_exp2f(m_s[r] - mu);
      float sum = 0.f;
      for (int t = 0; t < kTile; ++t) {
        const float pv = __builtin_amdgcn_exp2f(ps[r * (kTile + 1) + t] - mu);
        ps[r * (kTile + 1) + t] = pv;
        sum += pv;
      }
      l_s[r] = l_s[r] * al + sum;
      m_s[r] = mn;
      al_s[r] = al;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kValuMaxAcc; ++k) {
      const int idx = tid + k * kThreads;
      if (idx < R * D) {
        const int r = idx / D, d = idx - r * D;
        float s = acc[k] * al_s[r];
        for (int t = 0; t < kTile; ++t) s += ps[r * (kTile + 1) + t] * vs[t * D + d];
        acc[k] = s;
      }
    }
  }
  __syncthreads();
  const int64_t pu = static_cast<int64_t>(g) * a.P + plan.unit;
  for (int r = tid; r < R; r += kThreads) a.ws_ml[pu * R + r] = make_float2(m_s[r], l_s[r]);
#pragma unroll
  for (int k = 0; k < kValuMaxAcc; ++k) {
    const int idx = tid + k * kThreads;
    if (idx < R * D) a.ws_acc[pu * R * D + idx] = acc[k];
  }
  head_barrier_and_merge(a, plan, ps);
}

// ------------------------------------------------------------- MFMA kernel
// bf16 pools, rows R = W*G <= 16*NT.  Each wave owns every 4th tile of the
// workgroup's range and keeps its own (m, l, O^T) for all rows; waves are
// merged in LDS at the end.
//
// Fragments (v_mfma_f32_16x16x32_bf16, lane l: i = l%16, q4 = l/16):
//   S^T[tok][row] = K[tok][:] . Q~[row][:]
//     A (K):  token i of half a, dims 8*(4s+q4)..+8  (one 16-B load)
//     B (Q~): row 16t+i, same dims
//     D:      tokens 16a + 4*q4 + v, row 16t+i
//   O^T[d][row] = V^T[d][tok] . P^T[tok][row]
//     A (V^T): dim 16m+i, tokens {4*q4+v, 16+4*q4+v} (one 16-B load)
//     B (P^T): row 16t+i, the same 8 tokens = this lane's S^T outputs
//     D:       dims 16m + 4*q4 + v, row 16t+i
struct TileRef {
  int b;          // block
  int valid;      // tokens of the tile inside the block's length
  int64_t base;   // element offset of the tile in the kv-head plane
};

template <int D>
__device__ __forceinline__ TileRef tile_ref(const Plan& p, const DecodeArgs& a, int j, int& bcur) {
  bcur = block_of_tile(p, a.NB, j, bcur);
  const int tl = j - p.tile0[bcur];
  TileRef r;
  r.b = bcur;
  r.valid = min(kTile, p.len[bcur] - tl * kTile);
  r.base = (a.block_start[bcur] + static_cast<int64_t>(tl) * kTile) * D;
  return r;
}

// (a3) one 16-byte load per lane per fragment; every load of a wave is one
// contiguous 1 KB (keys) or four contiguous 256 B runs (values).
template <int D>
__device__ __forceinline__ void load_tile(const uint16_t* kp, const uint16_t* vp, int64_t base,
                                          int li, int q4, bf16x8 (&kf)[2][D / 32],
                                          bf16x8 (&vf)[D / 16]) {
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      kf[h2][s] = *reinterpret_cast<const bf16x8*>(kp + base + h2 * 16 * D + (4 * s + q4) * 128 +
                                                   li * 8);
#pragma unroll
  for (int m = 0; m < D / 16; ++m)
    vf[m] = *reinterpret_cast<const bf16x8*>(vp + base + q4 * 8 * D + (16 * m + li) * 8);
}

// Scores, online softmax and P.V for one tile held in registers.
template <int D, int NT>
__device__ __forceinline__ void compute_tile(bf16x8 (&kf)[2][D / 32], bf16x8 (&vf)[D / 16],
                                             const bf16x8 (&qf)[NT][D / 32],
                                             const bool (&rowvis)[NT], int valid, int q4,
                                             f32x4 (&acc)[D / 16][NT], float (&m_run)[NT],
                                             float (&l_run)[NT]) {
  constexpr int KS = D / 32, MT = D / 16;
  f32x4 sc[2][NT];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[h2][s], qf[t][s], c, 0, 0, 0);
      sc[h2][t] = c;
    }
  bf16x8 pf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float sv[8];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = 16 * h2 + 4 * q4 + v;
        sv[4 * h2 + v] = (rowvis[t] && tok < valid) ? sc[h2][t][v] : -INFINITY;
      }
    float mt = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sv[e]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m_run[t], mt);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float al = __builtin_amdgcn_exp2f(m_run[t] - mu);
    float sum = 0.f;
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pv = __builtin_amdgcn_exp2f(sv[e] - mu);
      sum += pv;
      f[e] = static_cast<__bf16>(pv);
    }
    pf[t] = f;
    l_run[t] = l_run[t] * al + sum;
    m_run[t] = mn;
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m][t] *= al;
  }
  if (valid < kTile) {
    // tokens past the block's length may hold anything (even NaN): zero them
    u32x4 keep;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const int t0 = 16 * ((2 * e2) >> 2) + 4 * q4 + ((2 * e2) & 3);
      const int t1 = 16 * ((2 * e2 + 1) >> 2) + 4 * q4 + ((2 * e2 + 1) & 3);
      keep[e2] = (t0 < valid ? 0x0000ffffu : 0u) | (t1 < valid ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      u32x4 bits = __builtin_bit_cast(u32x4, vf[m]);
      bits &= keep;
      vf[m] = __builtin_bit_cast(bf16x8, bits);
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[m], pf[t], acc[m][t], 0, 0, 0);
}

template <int D, int NT>
__global__ __launch_bounds__(kThreads) void decode_mfma(DecodeArgs a) {
  constexpr int KS = D / 32;  // k-steps of the QK product
  constexpr int MT = D / 16;  // 16-dim tiles of the output
  constexpr int RP = 16 * NT; // padded rows
  constexpr int HALF = D / 2;
  constexpr int ACC_STRIDE = D + 4;
  __shared__ Plan plan;
  // per-wave rotation tables (main loop) / per-wave O^T (wave merge)
  constexpr int kCsFloats = 2 * HW_MAX_WORKERS * HALF;
  constexpr int kMergeFloats = RP * ACC_STRIDE + 2 * RP;
  constexpr int kWaveFloats = kCsFloats > kMergeFloats ? kCsFloats : kMergeFloats;
  __shared__ __attribute__((aligned(16))) float smem[kWaves * kWaveFloats];

  build_plan(a, plan);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, q4 = lane >> 4;
  const int g = plan.head;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + g * a.plane_elems;
  const uint16_t* vp = static_cast<const uint16_t*>(a.v) + g * a.plane_elems;
  float2* cs = reinterpret_cast<float2*>(smem + wave * kWaveFloats);

  bf16x8 qf[NT][KS];
  bool rowvis[NT];
  f32x4 acc[MT][NT];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
    rowvis[t] = false;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[t][s] = bf16x8{};
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // (a2) rotate the stacked query rows of head g for block b into B fragments
  auto build_qf = [&](int b) {
    for (int x = lane; x < a.W * HALF; x += 64) {
      const int w = x / HALF, i = x - w * HALF;
      float c = 0.f, s = 0.f;
      if ((plan.vis[b] >> w) & 1u)
        rope_cos_sin(plan.iq[w] - plan.off[w * a.NB + b], a.inv_freq[i], &c, &s);
      cs[x] = make_float2(c, s);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int r = 16 * t + li;
      const int w = r / a.G;
      rowvis[t] = r < a.R && ((plan.vis[b] >> w) & 1u);
      const int h = g * a.G + (r - w * a.G);
      const int64_t qo = (static_cast<int64_t>(w) * a.Hq + h) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int d0 = 8 * (4 * s + q4);
        const int p0 = d0 < HALF ? d0 + HALF : d0 - HALF;
        u32x4 xv = u32x4{0u, 0u, 0u, 0u}, yv = u32x4{0u, 0u, 0u, 0u};
        if (rowvis[t]) {
          xv = *reinterpret_cast<const u32x4*>(qg + qo + d0);
          yv = *reinterpret_cast<const u32x4*>(qg + qo + p0);
        }
        bf16x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t xw = xv[e >> 1], yw = yv[e >> 1];
          const float x = __uint_as_float((e & 1) ? (xw & 0xffff0000u) : (xw << 16));
          const float y = __uint_as_float((e & 1) ? (yw & 0xffff0000u) : (yw << 16));
          const int fi = (d0 + e) & (HALF - 1);
          const float2 csv = rowvis[t] ? cs[w * HALF + fi] : make_float2(0.f, 0.f);
          const float val = d0 < HALF ? x * csv.x - y * csv.y : x * csv.x + y * csv.y;
          f[e] = static_cast<__bf16>(val * a.qscale);
        }
        qf[t][s] = f;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };

  // Tiles lo+wave, lo+wave+4, ...; two register sets so the next tile's loads
  // are in flight while the current one is computed.
  bf16x8 kA[2][KS], kB[2][KS], vA[MT], vB[MT];
  int bcur = 0, qb = -1;
  int j = plan.lo + wave;
  if (j < plan.hi) {
    TileRef ra = tile_ref<D>(plan, a, j, bcur);
    load_tile<D>(kp, vp, ra.base, li, q4, kA, vA);
    while (true) {
      const int jb = j + kWaves;
      const bool hb = jb < plan.hi;
      TileRef rb{};
      if (hb) {
        rb = tile_ref<D>(plan, a, jb, bcur);
        load_tile<D>(kp, vp, rb.base, li, q4, kB, vB);
      }
      if (ra.b != qb) {
        build_qf(ra.b);
        qb = ra.b;
      }
      compute_tile<D, NT>(kA, vA, qf, rowvis, ra.valid, q4, acc, m_run, l_run);
      if (!hb) break;
      const int jc = jb + kWaves;
      const bool hc = jc < plan.hi;
      TileRef rc{};
      if (hc) {
        rc = tile_ref<D>(plan, a, jc, bcur);
        load_tile<D>(kp, vp, rc.base, li, q4, kA, vA);
      }
      if (rb.b != qb) {
        build_qf(rb.b);
        qb = rb.b;
      }
      compute_tile<D, NT>(kB, vB, qf, rowvis, rb.valid, q4, acc, m_run, l_run);
      if (!hc) break;
      ra = rc;
      j = jc;
    }
  }

  // wave merge in LDS, then this unit's partial
  __syncthreads();
  float* wm = smem + wave * kWaveFloats;  // [RP][ACC_STRIDE] then m[RP], l[RP]
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float lsum = l_run[t];
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    const int r = 16 * t + li;
    if (q4 == 0) {
      wm[RP * ACC_STRIDE + r] = m_run[t];
      wm[RP * ACC_STRIDE + RP + r] = lsum;
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
      *reinterpret_cast<f32x4*>(wm + r * ACC_STRIDE + 16 * m + 4 * q4) = acc[m][t];
  }
  __syncthreads();
  const int64_t pu = static_cast<int64_t>(g) * a.P + plan.unit;
  for (int x = tid; x < a.R * D; x += kThreads) {
    const int r = x / D, d = x - r * D;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, smem[wv * kWaveFloats + RP * ACC_STRIDE + r]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) {
        const float* src = smem + wv * kWaveFloats;
        const float mw = src[RP * ACC_STRIDE + r];
        const float sc2 = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L += src[RP * ACC_STRIDE + RP + r] * sc2;
        O += src[r * ACC_STRIDE + d] * sc2;
      }
    }
    a.ws_acc[pu * a.R * D + x] = O;
    if (d == 0) a.ws_ml[pu * a.R + r] = make_float2(M, L);
  }
  head_barrier_and_merge(a, plan, smem);
}

template <typename K>
int occupancy(K kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, 0) != hipSuccess) return 0;
  return n;
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs& a, int grid, hipStream_t s) {
  if ((a.D != 64 && a.D != 128) || a.R > HW_MAX_ROWS) return hipErrorInvalidValue;
  if (a.dtype == HW_F32)
    hipLaunchKernelGGL(decode_valu<float>, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(decode_valu<uint16_t>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int grid, hipStream_t s) {
  if (a.dtype != HW_BF16 || a.R > 32) return hipErrorInvalidValue;
  if (a.D == 128) {
    if (a.R <= 16)
      hipLaunchKernelGGL((decode_mfma<128, 1>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((decode_mfma<128, 2>), dim3(grid), dim3(kThreads), 0, s, a);
  } else if (a.D == 64) {
    if (a.R <= 16)
      hipLaunchKernelGGL((decode_mfma<64, 1>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((decode_mfma<64, 2>), dim3(grid), dim3(kThreads), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Resident workgroups per CU of the kernel a launch would use (0 on error).
int decode_blocks_per_cu(int path, int dtype, int D, int rows) {
  if (path == 2) {
    if (D == 128) return rows <= 16 ? occupancy(decode_mfma<128, 1>) : occupancy(decode_mfma<128, 2>);
    return rows <= 16 ? occupancy(decode_mfma<64, 1>) : occupancy(decode_mfma<64, 2>);
  }
  return dtype == HW_F32 ? occupancy(decode_valu<float>) : occupancy(decode_valu<uint16_t>);
}

}  // namespace hw
