// hw_decode.hip — run kernels of a decode call: a split launch and, when a
// kv head has several work units, a merge launch.
//
// Split launch: one workgroup per work unit (kv head g, unit u).  Each
// workgroup
//  1. reads the step's plan (hw_plan.hip), its head's query rows and the
//     rotation steps into LDS in one memory round trip;
//  2. for every block it will read, rotates the stacked rows of head g by the
//     plan's delta (i_q - view_offset - lag): only the current query tokens
//     are rotated, never the cache (Hogwild! notes, key design 1)        [a2]
//  3. streams K/V tiles once for all W*G rows with an online softmax in the
//     exp2 domain (split-K / Flash-Decoding; news 1114328 sec. 3.2)       [a3]
//     Tiles come either from the unit's contiguous range of the plan
//     (static: the result is bitwise the same on every run), or, balanced,
//     one per wave from that range and then one at a time from a per-head
//     counter, so that units on CUs that HBM serves faster take more tiles;
//  4. combines its waves' states and stores the unit's partial (m, l, acc),
//     or, with one unit per head, the final rows.
// Merge launch: one workgroup per (kv head, row): log-sum-exp merge of the
// units' partials in fixed unit order and the output row               [a4].
// The kernel boundary orders the partials' stores before their loads, so no
// workgroup waits on another.
//
// Two split kernels share the prologue and the epilogue:
//   run_valu<T>        fp32 VALU arithmetic (fp32 and bf16 pools, rows <= 64)
//   run_mfma<D,NT,E>   bf16 MFMA 16x16x32: S^T = K Q~^T and O^T = V^T P^T with
//                      tiles loaded straight into operand fragments (the pool
//                      layout matches them), rows = W*G <= 16*NT <= 80.
#include <math.h>

#include <type_traits>

#include "hw_internal.h"
#include "hw_kernels.h"

namespace hw {
namespace {

// ------------------------------------------------------------- plan in LDS
struct PlanLds {
  int32_t w[kPlanLdsWords];  // header, visible blocks, lengths (plan words [0, 340))
  int32_t flags;             // HW_DEV_* bits found by this workgroup
  int32_t tiles;             // tiles the workgroup processed
};

// Dynamic LDS: the plan's row ends [NB][qrows].
extern __shared__ int32_t rows_lds[];

// Workgroup -> (kv head, unit): consecutive workgroups take consecutive heads,
// so a head's units are Hkv workgroups apart (with 8 kv heads and the 8-XCD
// round-robin dispatch, every unit of a head runs on one XCD).
__device__ __forceinline__ void head_unit(const RunArgs& a, int* g, int* u) {
#ifdef HW_HEAD_MAJOR
  *g = fast_div(blockIdx.x, a.mP);
  *u = blockIdx.x - *g * a.P;
#else
  *u = fast_div(blockIdx.x, a.mHkv);
  *g = blockIdx.x - *u * a.Hkv;
#endif
}

// Loads issued at kernel entry: the plan words [0, 340) (85 x 16 bytes), the
// row ends (one word per thread; larger plans load the rest at commit), every
// block's current length (for the stale-plan check).
struct PlanLoads {
  int4 w;
  int32_t row;
  int32_t len;
  int32_t lo, hi;  // this unit's tile range (uniform)
};
template <int NTHR>
__device__ __forceinline__ PlanLoads issue_plan_loads(const RunArgs& a, int u) {
  const int tid = threadIdx.x;
  PlanLoads l;
  l.w = make_int4(0, 0, 0, 0);
  l.row = -1;
  l.len = 0;
  l.lo = a.plan[kPlanUnit + u];
  l.hi = a.plan[kPlanUnit + u + 1];
  if (tid < kPlanLdsWords / 4) l.w = reinterpret_cast<const int4*>(a.plan)[tid];
  if (tid < a.NB * a.qrows) l.row = a.plan[kPlanRows + tid];
  if (tid < a.NB) l.len = a.block_len[tid];
  return l;
}
template <int NTHR>
__device__ __forceinline__ void commit_plan_loads(const RunArgs& a, PlanLds& pl,
                                                  const PlanLoads& l) {
  const int tid = threadIdx.x;
  if (tid < kPlanLdsWords / 4) reinterpret_cast<int4*>(pl.w)[tid] = l.w;
  const int nrow = a.NB * a.qrows;
  if (tid < nrow) rows_lds[tid] = l.row;
#pragma unroll 1
  for (int i = tid + NTHR; i < nrow; i += NTHR) rows_lds[i] = a.plan[kPlanRows + i];
  if (tid == 0) {
    pl.flags = 0;
    pl.tiles = 0;
  }
}

// After the barrier that publishes the plan: this unit's tile range, or an
// empty one (and HW_DEV_STALE_PLAN) when the plan does not fit this call: made
// for another shape, or with visible blocks whose tiles would leave the kv-head
// plane or do not match their lengths (every wave checks, lane j block j, so
// no tile offset used below can leave the plane).  A block whose length
// changed since the plan was made also reports HW_DEV_STALE_PLAN.
template <int D, int EB>
__device__ __forceinline__ bool unit_range(const RunArgs& a, PlanLds& pl, const PlanLoads& pload,
                                           int* lo, int* hi) {
  const int32_t* w = pl.w;
  const int lane = threadIdx.x & 63;
  const int lens_loaded = pload.len;
  int l = pload.lo;
  int h = pload.hi;
  const int nvb = w[kHdrNvb];
  bool ok = w[kHdrMagic] == kPlanMagic && w[kHdrP] == a.P && w[kHdrQrows] == a.qrows &&
            w[kHdrNB] == a.NB && w[kHdrR] == a.R && nvb >= 0 && nvb <= a.NB && 0 <= l &&
            l <= h && h <= w[kHdrTiles] && w[kPlanVbTile0] == 0 &&
            w[kPlanVbTile0 + nvb] == w[kHdrTiles];
  bool bad = false;
  if (ok && lane < nvb) {
    const int64_t start = w[kPlanVbStart + lane], len = w[kPlanVbLen + lane];
    const int64_t tiles = (len + kTile - 1) / kTile;
    bad = start < 0 || len <= 0 || w[kPlanVbTile0 + lane + 1] - w[kPlanVbTile0 + lane] != tiles ||
          (start + tiles * kTile) * D * EB > a.plane_bytes;
  }
  ok = ok && __ballot(bad) == 0ull;
  if (!ok) {
    l = 0;
    h = 0;
    if (threadIdx.x == 0) {
      atomicOr(&pl.flags, HW_DEV_STALE_PLAN);
      atomicOr(&pl.tiles, 1 << 30);  // (no tile count check for this launch)
    }
  }
  if (static_cast<int>(threadIdx.x) < a.NB && lens_loaded != w[kPlanLens + threadIdx.x])
    atomicOr(&pl.flags, HW_DEV_STALE_PLAN);
  *lo = l;
  *hi = h;
  return ok;
}

// Visible blocks holding tiles lo and hi - 1 (every wave, from LDS): lane j
// tests the first tile of visible block j.
__device__ __forceinline__ void block_range(const PlanLds& pl, int lo, int hi, int* bf, int* bl) {
  const int lane = threadIdx.x & 63;
  const int nvb = pl.w[kHdrNvb];
  const int t0 = lane < nvb ? pl.w[kPlanVbTile0 + lane] : 0x7fffffff;
  *bf = __builtin_popcountll(__ballot(t0 <= lo)) - 1;
  *bl = __builtin_popcountll(__ballot(t0 <= hi - 1)) - 1;
}

// Visible block of tile j, the cursor walking forward.
__device__ __forceinline__ int block_of_tile(const PlanLds& pl, int j, int b) {
  const int nvb = pl.w[kHdrNvb];
  while (b + 1 < nvb && pl.w[kPlanVbTile0 + b + 1] <= j) ++b;
  return b;
}

struct TileRef {
  int b;          // visible block
  int valid;      // tokens of the tile inside the block's length
  int first;      // local position of the tile's first token in its block
  uint32_t byte;  // byte offset of the tile in the kv-head plane
};

template <int D, int EB>
__device__ __forceinline__ TileRef tile_ref(const PlanLds& pl, int j, int& bcur) {
  bcur = block_of_tile(pl, j, bcur);
  const int tl = j - pl.w[kPlanVbTile0 + bcur];
  TileRef r;
  r.b = bcur;
  r.valid = min(kTile, pl.w[kPlanVbLen + bcur] - tl * kTile);
  r.first = tl * kTile;
  r.byte = static_cast<uint32_t>((pl.w[kPlanVbStart + bcur] + tl * kTile) * D * EB);
  return r;
}

// ------------------------------------------------------------ unit finish
// A value the compiler must keep in SGPRs from here on.  Kernel arguments
// are otherwise reloaded at their uses (a reload is cheaper for it than a
// live register), and in the epilogue each reload is a round trip queued
// behind the chip's K/V stream.
template <typename T>
__device__ __forceinline__ T pin_sgpr(T x) {
  asm volatile("" : "+s"(x));
  return x;
}

// The epilogue's scalars, read from the arguments at kernel entry.
struct EpiArgs {
  float* out;
  float2* ws_ml;
  float* ws_acc;
  int32_t* ws_cnt;
  int32_t* status;
  int R, P, Hq, G;
  uint32_t mG;
  float vsc;  // FP8 pools: value scale of the kv head, else 1
};

// kPin: keep them in SGPRs (kernels with SGPRs to spare).
template <bool kFp8, bool kPin>
__device__ __forceinline__ EpiArgs epi_args(const RunArgs& a, int g) {
  auto pin = [](auto x) { return kPin ? pin_sgpr(x) : x; };
  EpiArgs e;
  e.out = pin(a.out);
  e.ws_ml = pin(a.ws_ml);
  e.ws_acc = pin(a.ws_acc);
  e.ws_cnt = pin(a.ws_cnt);
  e.status = pin(a.status);
  e.R = pin(a.R);
  e.P = pin(a.P);
  e.Hq = pin(a.Hq);
  e.G = pin(a.G);
  e.mG = pin(a.mG);
  e.vsc = 1.f;
  if (kFp8) {
    const float v = reinterpret_cast<const float*>(reinterpret_cast<const char*>(&a) +
                                                   offsetof(RunArgs, v_scale))[g];
    e.vsc = __int_as_float(pin(__builtin_amdgcn_readfirstlane(__float_as_int(v))));
  }
  return e;
}

// Stacked rows of kv head g: r = i * G + (h - g * G) for query row i
// (= w * nq + j) and q-head h; output row (i, h) of out [qrows][Hq][D].
template <typename A>
__device__ __forceinline__ int64_t out_row(const A& a, int g, int r) {
  const int i = fast_div(r, a.mG);
  return static_cast<int64_t>(i) * a.Hq + g * a.G + (r - i * a.G);
}

// Called by every thread once the waves' states are deposited in LDS: ns
// states of stride sstride floats, each [rc rows][ACC_STRIDE] accumulators
// then rc maxima and rc sums.  Combines them 8 outputs per item and stores
// the unit's partial ([Hkv][R][P] (m, l) pairs, [Hkv][R][P][D]
// accumulators), or, with one unit per head, the final rows out = O / L.
template <int NTHR, int D>
__device__ void emit_unit(const EpiArgs& a, PlanLds& pl, int g, int u, const float* sbuf, int ns,
                          int sstride, int rc) {
  constexpr int ACC_STRIDE = D + 4;
  constexpr int kMaxStates = 8;
  const int tid = threadIdx.x;
  const int R = a.R, P = a.P;
  const float vsc = a.vsc;
  for (int x = tid; x < R * (D / 8); x += NTHR) {
    const int r = x / (D / 8), d8 = 8 * (x - r * (D / 8));
    float mw[kMaxStates];
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kMaxStates; ++wv) {
      mw[wv] = wv < ns ? sbuf[wv * sstride + rc * ACC_STRIDE + r] : -INFINITY;
      M = fmaxf(M, mw[wv]);
    }
    float L = 0.f;
    f32x4 O0 = f32x4{0.f, 0.f, 0.f, 0.f}, O1 = O0;
    if (M != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < kMaxStates; ++wv) {
        if (wv < ns) {
          const float* src = sbuf + wv * sstride;
          const float sc = mw[wv] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[wv] - M);
          L += src[rc * ACC_STRIDE + rc + r] * sc;
          O0 += *reinterpret_cast<const f32x4*>(src + r * ACC_STRIDE + d8) * sc;
          O1 += *reinterpret_cast<const f32x4*>(src + r * ACC_STRIDE + d8 + 4) * sc;
        }
      }
    }
    if (P == 1) {
      const float inv = L > 0.f ? vsc / L : 0.f;
      float* o = a.out + out_row(a, g, r) * D + d8;
      *reinterpret_cast<f32x4*>(o) = O0 * inv;
      *reinterpret_cast<f32x4*>(o + 4) = O1 * inv;
      if (d8 == 0 && !(L > 0.f)) atomicOr(&pl.flags, HW_DEV_NO_TOKENS);
    } else {
      const int64_t pr = (static_cast<int64_t>(g) * R + r) * P + u;
      *reinterpret_cast<f32x4*>(a.ws_acc + pr * D + d8) = O0;
      *reinterpret_cast<f32x4*>(a.ws_acc + pr * D + d8 + 4) = O1;
      if (d8 == 0) a.ws_ml[pr] = make_float2(M, L);
    }
  }
  if (tid == 0) a.ws_cnt[g * P + u] = pl.tiles;
  if (P == 1) __syncthreads();
  if (tid == 0 && pl.flags) atomicOr(a.status, pl.flags);
}

// ------------------------------------------------------------- MFMA kernel
// bf16 and FP8 pools, rows R = W*G <= 16*NT.  Eight waves.  Up to 32 rows
// each wave owns every 8th tile of the workgroup's range and keeps its own
// (m, l, O^T) for all rows.  Above 32 rows the rows split into two row groups
// of ceil(NT/2) row tiles, four waves each: a wave owns every 4th tile for
// its group's rows (the other group's wave reads the same tile, mostly from
// L2), which keeps a wave's accumulators in its half of the register file.
// The waves' states are combined in LDS at the end.  Fragment layouts:
// hw_kernels.h.

#ifndef HW_ISSUE_BEFORE_ROTATION
#define HW_ISSUE_BEFORE_ROTATION 1
#endif
constexpr int kIssueBeforeRotation = HW_ISSUE_BEFORE_ROTATION;
// Rows up to which every wave's state has its own LDS slot (one-level combine).
constexpr int kOneLevelRows = 20;
// Waves of the MFMA kernel (two per SIMD) and its row groups.
constexpr int mfma_waves(int) { return 8; }
constexpr int mfma_row_groups(int NT) { return NT <= 2 ? 1 : 2; }

template <int D, int NT, typename E>
__global__ __launch_bounds__(64 * mfma_waves(NT)) void run_mfma(RunArgs a) {
  typedef typename KvFrag<E>::type Frag;
  constexpr int EB = KvFrag<E>::kBytes;
  constexpr int NWAVE = mfma_waves(NT);
  constexpr int NTHR = 64 * NWAVE;
  constexpr int RG = mfma_row_groups(NT);
  constexpr int NTG = (NT + RG - 1) / RG;  // row tiles of a wave
  constexpr int WPG = NWAVE / RG;          // waves of a row group
  // K/V cache policy: with row groups each tile is read by one wave of each
  // group, and loads with the default policy let the second read find it in
  // L2 (an 80-row call: 32.9 us, against 35.2 with non-temporal loads)
  constexpr int KV_POL = RG > 1 ? 0 : kPolicyNT;
  constexpr int NSTATE = WPG / 2;  // wave states held in LDS at once (two-level combine)
  constexpr int KS = D / 32;         // k-steps of the QK product
  constexpr int MT = D / 16;         // 16-dim tiles of the output
  constexpr int RP = 16 * NT;        // padded rows
  constexpr int HALF = D / 2;
  constexpr int ACC_STRIDE = D + 4;
  constexpr int kQf = NT <= 2 ? 6 : 1;  // blocks whose rotated queries are in LDS at once
  constexpr bool kOneLevelOk = NWAVE == 8 && RG == 1;
  constexpr int RC1 = RP < kOneLevelRows ? RP : kOneLevelRows;
  constexpr int kState1 = RC1 * ACC_STRIDE + 2 * RC1;
  constexpr int kState2 = RP * ACC_STRIDE + 2 * RP;
  constexpr int kEpiFloats = cmax(kOneLevelOk ? NWAVE * kState1 : 0, NSTATE * kState2);
  constexpr int kQfFloats = kQf * NT * KS * 64 * 4;
  __shared__ PlanLds pl;
  __shared__ uint64_t fracs[HALF];
  // the head's query rows, row stride D + 8: the rotation reads one column of
  // 16 rows at a time, which then falls into distinct LDS banks
  constexpr int QS = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t qs[RP * QS];
  __shared__ __attribute__((aligned(16))) float qbuf[kQfFloats];
  // the waves' softmax states (epilogue); apart from qbuf, so that a wave
  // done with its tiles deposits its state while the others still stream
  __shared__ __attribute__((aligned(16))) float ebuf[kEpiFloats];

  // every scalar argument, requested at entry in one round trip: otherwise
  // each first use (epilogue included) waits for its own kernel-argument load
  // behind the chip's K/V stream (kernels of up to 32 rows: the larger ones
  // have no SGPRs to spare)
  if constexpr (NT <= 2)
    asm volatile("" ::"s"(a.q), "s"(a.k), "s"(a.v), "s"(a.plan), "s"(a.block_len), "s"(a.out),
                 "s"(a.status), "s"(a.sync), "s"(a.ws_ml), "s"(a.ws_acc), "s"(a.ws_cnt),
                 "s"(a.plane_elems), "s"(a.plane_bytes), "s"(a.Hq), "s"(a.Hkv), "s"(a.G), "s"(a.R),
                 "s"(a.qrows), "s"(a.NB), "s"(a.P), "s"(a.mG), "s"(a.mHkv), "s"(a.mR),
                 "s"(a.mP), "s"(a.balance), "s"(a.dtype), "s"(a.qscale));
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, q4 = lane >> 4;
  // the wave's row group, its first row tile, its row tiles that exist and
  // its place in the group (wave-uniform)
  const int rg = RG == 1 ? 0 : __builtin_amdgcn_readfirstlane(wave) / WPG;
  const int tb = rg * NTG;
  const int ntv = RG == 1 ? NT : min(NTG, NT - tb);
  const int wl = RG == 1 ? wave : __builtin_amdgcn_readfirstlane(wave) % WPG;
  if (tid == 0) HW_STAMP(0);
  int g, u;
  head_unit(a, &g, &u);
  const EpiArgs ea = epi_args<EB == 1, (NT <= 2)>(a, g);
  // the rotation's and the loop's row scalars, kept in SGPRs likewise
  const int nrows = ea.R;
  const uint32_t mG = ea.mG;
  const int qrows = NT <= 2 ? pin_sgpr(a.qrows) : a.qrows;

  // ---- 1. one round trip: plan, lengths, rotation steps, this head's rows
  constexpr int kQVec = RP * D / 8;
  constexpr int kQRegs = (kQVec + NTHR - 1) / NTHR;
  const PlanLoads pload = issue_plan_loads<NTHR>(a, u);
  uint64_t frac = 0;
  if (tid < HALF)
    frac = reinterpret_cast<const uint64_t*>(reinterpret_cast<const char*>(&a) +
                                             offsetof(RunArgs, rope_frac))[tid];
  u32x4 qv[kQRegs];
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int k = 0; k < kQRegs; ++k) {
    const int x = tid + k * NTHR;
    const int r = (8 * x) / D, d = (8 * x) - r * D;
    qv[k] = u32x4{0u, 0u, 0u, 0u};
    if (x < kQVec && r < nrows)
      qv[k] = *reinterpret_cast<const u32x4*>(qg + out_row(ea, g, r) * D + d);
  }
  // this head's K/V plane descriptors and the query scale (FP8 pools: times
  // the key scale of the kv head)
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(
      static_cast<const char*>(a.k) + static_cast<int64_t>(g) * a.plane_elems * EB, a.plane_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(
      static_cast<const char*>(a.v) + static_cast<int64_t>(g) * a.plane_elems * EB, a.plane_bytes);
  float qsc = a.qscale;
  if (EB == 1)
    qsc *= reinterpret_cast<const float*>(reinterpret_cast<const char*>(&a) +
                                          offsetof(RunArgs, k_scale))[g];
  commit_plan_loads<NTHR>(a, pl, pload);
  if (tid < HALF) fracs[tid] = frac;
#pragma unroll
  for (int k = 0; k < kQRegs; ++k) {
    const int x = tid + k * NTHR;
    if (x < kQVec) *reinterpret_cast<u32x4*>(qs + (8 * x) / D * QS + (8 * x) % D) = qv[k];
  }
  __syncthreads();
  if (tid == 0) HW_STAMP(1);
  int lo, hi, b_first, b_last;
  const bool plan_ok = unit_range<D, EB>(a, pl, pload, &lo, &hi);
  block_range(pl, lo, hi, &b_first, &b_last);

  const uint32_t koff = (q4 * 128 + li * 8) * EB;
  const uint32_t voff = (q4 * 8 * D + li * 8) * EB;
  Frag kf[2][KS], vf[MT];
  bool rowvis[NTG];
  f32x4 acc[MT][NTG];
  float m_run[NTG], l_run[NTG];
#pragma unroll
  for (int t = 0; t < NTG; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
    rowvis[t] = false;
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // (a2) rotated queries of visible blocks gb..ge-1, shared by all waves: for
  // each block the stacked rows of head g rotated by their row end (the
  // delta), scaled, rounded to bf16 and laid out as MFMA B fragments
  // (row 16t+li, dims 8*(4s+q4)..+8 at qfs[((bi*NT + t)*KS + s)*64 + lane]).
  // Rows past R or that see nothing of the block are zero.  Item (bi, t, sh,
  // lane) rotates the 8 pairs (d0 + e, d0 + e + D/2), d0 = 8*(4*sh + q4).
  bf16x8* qfs = reinterpret_cast<bf16x8*>(qbuf);
  constexpr int IPB = NT * (KS / 2) * 64;  // items per block
  auto rotate_blocks = [&](int gb, int ge, int nthr) {
    for (int x = tid; x < (ge - gb) * IPB; x += nthr) {
      const int bi = x / IPB;
      const int slot = x - bi * IPB;
      const int ln = slot & 63;
      const int y = slot >> 6;
      const int sh = y % (KS / 2);
      const int t = y / (KS / 2);
      const int r = 16 * t + (ln & 15);
      const int d0 = 8 * (4 * sh + (ln >> 4));  // < HALF; its partner dims are d0 + HALF
      int re = -1;
      if (r < nrows) re = rows_lds[(gb + bi) * qrows + fast_div(r, mG)];
      const float sc = re >= 0 ? qsc : 0.f;
      const uint32_t delta = static_cast<uint32_t>(re >= 0 ? re : 0);
      const uint32_t* qw = reinterpret_cast<const uint32_t*>(qs + r * QS + d0);
      uint32_t* lo4 = reinterpret_cast<uint32_t*>(qfs + ((bi * NT + t) * KS + sh) * 64 + ln);
      uint32_t* hi4 = reinterpret_cast<uint32_t*>(qfs + ((bi * NT + t) * KS + sh + KS / 2) * 64 + ln);
      // (rolled: this code runs once per launch and is fetched cold)
#pragma unroll 1
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t xw = qw[e2], yw = qw[e2 + HALF / 2];
        const float x0 = __uint_as_float(xw << 16), x1 = __uint_as_float(xw & 0xffff0000u);
        const float y0 = __uint_as_float(yw << 16), y1 = __uint_as_float(yw & 0xffff0000u);
        float c0, s0, c1, s1;
        rope_cos_sin_fx(delta, fracs[d0 + 2 * e2], &c0, &s0);
        rope_cos_sin_fx(delta, fracs[d0 + 2 * e2 + 1], &c1, &s1);
        lo4[e2] = pack_bf16x2((x0 * c0 - y0 * s0) * sc, (x1 * c1 - y1 * s1) * sc);
        hi4[e2] = pack_bf16x2((y0 * c0 + x0 * s0) * sc, (y1 * c1 + x1 * s1) * sc);
      }
    }
  };

  // One tile of the loop: per-row limits from the plan when the tile's block
  // changes, scores, then the next tile's keys requested into the key
  // registers, the softmax and P.V update, the next tile's values requested.
  // Every wave keeps a tile in flight while it computes.
  int qb = -1;
  int rowend[NTG];
  const bf16x8* qf = qfs;
  // (`more` is a compile-time flag: with the next tile's loads conditional
  // the compiler cannot count the loads in flight and waits for all of them
  // before the scores, this tile's values included)
  auto step = [&](const TileRef& rt, int gb, auto more_c, uint32_t tn) {
    constexpr bool more = decltype(more_c)::value;
    if (rt.b != qb) {
      qb = rt.b;
      qf = qfs + ((qb - gb) * NT + tb) * KS * 64;
#pragma unroll
      for (int t = 0; t < NTG; ++t) {
        const int r = 16 * (tb + t) + li;
        rowend[t] = r < nrows ? rows_lds[qb * qrows + fast_div(r, mG)] : -1;
        rowvis[t] = rowend[t] >= 0;
      }
    }
    int rowlim[NTG];
#pragma unroll
    for (int t = 0; t < NTG; ++t) rowlim[t] = min(rt.valid - 1, rowend[t] - rt.first);
    f32x4 sc[2][NTG];
    tile_scores<D, NTG, E>(kf, qf, lane, sc, ntv);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (more) load_keys<D, E, KV_POL>(krs, tn, koff, kf);
    __builtin_amdgcn_sched_barrier(0);
    tile_update<D, NTG, E, (RG > 1)>(sc, vf, rowvis, rowlim, rt.valid, q4, acc, m_run, l_run,
                                     ntv);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (more) load_values<D, E, KV_POL>(vrs, tn, voff, vf);
    __builtin_amdgcn_sched_barrier(0);
  };
  const std::true_type kMore;
  const std::false_type kLast;

  int done_tiles = 0;  // tiles this wave processed
  const int nvb = pl.w[kHdrNvb];
  if (RG == 1 && a.balance && plan_ok && nvb <= kQf && a.P > 1) {
    // Balanced: every visible block rotated at once; wave w of unit u takes
    // tile u*NWAVE + w, then tiles from the head's counter (tickets start
    // after the P*NWAVE first tiles; a wave without a first tile starts with
    // a ticket).  Each wave's next ticket is requested one tile ahead, so its
    // latency hides under the current tile (the first under the rotation).
    const int T = pl.w[kHdrTiles];
    const int base = a.P * NWAVE;
    uint32_t* ctr = a.sync + static_cast<int64_t>(g) * kSyncStride;
    int j = u * NWAVE + wave;
    int bcur = 0;
    TileRef rt = {0, 0, 0, 0u};
    if (j < T) {
      rt = tile_ref<D, EB>(pl, j, bcur);
      const uint32_t t0 = __builtin_amdgcn_readfirstlane(rt.byte);
      load_keys<D, E>(krs, t0, koff, kf);
      load_values<D, E>(vrs, t0, voff, vf);
    }
    uint32_t ticket = 0;
    if (lane == 0)
      ticket = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    rotate_blocks(0, nvb, NTHR);
    __syncthreads();
    if (tid == 0) HW_STAMP(2);
    if (j >= T) {
      j = base + static_cast<int>(__builtin_amdgcn_readfirstlane(ticket));
      if (j < T) {
        if (lane == 0)
          ticket = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        rt = tile_ref<D, EB>(pl, j, bcur);
        const uint32_t t0 = __builtin_amdgcn_readfirstlane(rt.byte);
        load_keys<D, E>(krs, t0, koff, kf);
        load_values<D, E>(vrs, t0, voff, vf);
      }
    }
    while (j < T) {
      const int jn = base + static_cast<int>(__builtin_amdgcn_readfirstlane(ticket));
      ++done_tiles;
      if (jn >= T) {
        step(rt, 0, kLast, 0u);
        break;
      }
      if (lane == 0)
        ticket = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const TileRef rn = tile_ref<D, EB>(pl, jn, bcur);
      step(rt, 0, kMore, __builtin_amdgcn_readfirstlane(rn.byte));
      j = jn;
      rt = rn;
    }
  } else if (lo < hi) {
    // Static: blocks with tiles in [lo, hi) form the index range [b_first,
    // b_last], rotated kQf at a time; wave w takes tiles lo + w, lo + w +
    // NWAVE, ... of each group.  A group's first tile is requested before
    // its rotation (kIssueBeforeRotation).
    for (int gb = b_first; gb <= b_last; gb += kQf) {
      const int ge = min(gb + kQf, b_last + 1);
      const int t_lo = max(lo, pl.w[kPlanVbTile0 + gb]);
      const int t_hi = min(hi, pl.w[kPlanVbTile0 + ge]);
      int j = t_lo + wl;
      int bcur = gb;
      TileRef rt = {0, 0, 0, 0u};
      uint32_t tile0 = 0;
      // mode 3: the upper half of the waves requests its first tiles at
      // once while the lower half rotates (a CU holds ~64 KB of requests:
      // half the waves' tiles), then requests its own
      // (two row groups: not before the rotation, which reloads spilled
      // values and would wait behind the tiles' loads)
      const bool early = RG == 1 && (kIssueBeforeRotation == 3 ? wave >= NWAVE / 2
                                                                : kIssueBeforeRotation >= 1);
      const bool early_v = RG == 1 && (kIssueBeforeRotation == 3 ? early : kIssueBeforeRotation >= 2);
      if (j < t_hi) {
        rt = tile_ref<D, EB>(pl, j, bcur);
        tile0 = __builtin_amdgcn_readfirstlane(rt.byte);
        if (early) load_keys<D, E, KV_POL>(krs, tile0, koff, kf);
        if (early_v) load_values<D, E, KV_POL>(vrs, tile0, voff, vf);
      }
      if (gb != b_first) __syncthreads();  // the previous group's fragments are consumed
      if (kIssueBeforeRotation != 3 || wave < NWAVE / 2)
        rotate_blocks(gb, ge, kIssueBeforeRotation == 3 ? NTHR / 2 : NTHR);
      __syncthreads();
      if (tid == 0 && gb == b_first) HW_STAMP(2);
      qb = -1;
      if (j < t_hi) {
        if (!early) load_keys<D, E, KV_POL>(krs, tile0, koff, kf);
        if (!early_v) load_values<D, E, KV_POL>(vrs, tile0, voff, vf);
        for (;;) {
          const int jn = j + WPG;
          ++done_tiles;
          if (jn >= t_hi) {
            step(rt, gb, kLast, 0u);
            break;
          }
          const TileRef rn = tile_ref<D, EB>(pl, jn, bcur);
          step(rt, gb, kMore, __builtin_amdgcn_readfirstlane(rn.byte));
          j = jn;
          rt = rn;
        }
      }
    }
  }

  if (lane == 0) {
    HW_STAMP(3 + wave);
    if (rg == 0) atomicAdd(&pl.tiles, done_tiles);  // (each row group takes every tile)
  }
  // full row sums (the four lanes of a row hold partial sums)
#pragma unroll
  for (int t = 0; t < NTG; ++t) l_run[t] = sum_x32(sum_x16(l_run[t]));
  // Combine the waves' states (O^T rows below R, m, l) in LDS.  When every
  // wave's state fits (R <= RC1 rows, 8 waves), each wave deposits its state
  // in its own slot as soon as its tiles are done; otherwise, after a
  // barrier, half of them at a time: the upper waves deposit, each lower wave
  // folds in its partner (same fragment positions, so lane-local), and the
  // lower waves deposit (with row groups: the waves of a place in the group,
  // one per group, share a slot, each writing its group's rows).  Then every
  // thread combines its share of the unit's R*D outputs over the deposited
  // states.
  auto deposit = [&](float* buf, int rc) {
#pragma unroll
    for (int t = 0; t < NTG; ++t) {
      const int r = 16 * (tb + t) + li;
      if (r >= nrows) continue;
      if (q4 == 0) {
        buf[rc * ACC_STRIDE + r] = m_run[t];
        buf[rc * ACC_STRIDE + rc + r] = l_run[t];
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
        *reinterpret_cast<f32x4*>(buf + r * ACC_STRIDE + 16 * m + 4 * q4) = acc[m][t];
    }
  };
  int ns, sstride, rc;
  if (kOneLevelOk && nrows <= RC1) {
    deposit(ebuf + wave * kState1, RC1);
    ns = NWAVE;
    sstride = kState1;
    rc = RC1;
  } else {
    __syncthreads();
    if (wl >= NSTATE) deposit(ebuf + (wl - NSTATE) * kState2, RP);
    __syncthreads();
    if (wl < NSTATE) {
      const float* src = ebuf + wl * kState2;
#pragma unroll
      for (int t = 0; t < NTG; ++t) {
        const int r = 16 * (tb + t) + li;
        if (r >= nrows) continue;
        const float m2 = src[RP * ACC_STRIDE + r];
        const float l2 = src[RP * ACC_STRIDE + RP + r];
        const float M = fmaxf(m_run[t], m2);
        const float s1 = m_run[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[t] - M);
        const float s2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
        l_run[t] = l_run[t] * s1 + l2 * s2;
        m_run[t] = M;
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[m][t] = acc[m][t] * s1 +
                      *reinterpret_cast<const f32x4*>(src + r * ACC_STRIDE + 16 * m + 4 * q4) * s2;
      }
    }
    __syncthreads();
    if (wl < NSTATE) deposit(ebuf + wl * kState2, RP);
    ns = NSTATE;
    sstride = kState2;
    rc = RP;
  }
  __syncthreads();
  if (tid == 0) HW_STAMP(11);
  emit_unit<NTHR, D>(ea, pl, g, u, ebuf, ns, sstride, rc);
  if (lane == 0) HW_STAMP(16 + wave);
}

// ------------------------------------------------------------- VALU kernel
// Any pool dtype (fp32 or bf16), rows R = W*G <= 2*RG, fp32 arithmetic on
// the vector ALUs.  Four waves per workgroup; each wave owns every 4th tile
// of the unit's range and keeps a private (m, l, O) for all rows; the waves
// are combined in LDS at the end like the MFMA kernel's.
//
// Scores: lane (token t = lane % 32, row group rg = lane / 32) loads token
// t's key straight into registers and forms the dot products of rows
// rg*RG .. rg*RG+RG-1 against the rotated queries, read from LDS (fp32,
// broadcast to the 32 lanes of a row group).  Row max and sum over the tile
// are DPP reductions inside each 32-lane half.  P.V: lane l owns output dims
// DPL*l .. DPL*l+DPL-1 of every row and reads P and the rescale factors back
// from a per-wave LDS buffer.
template <typename T>
struct ValuTraits;
template <>
struct ValuTraits<float> {
  static constexpr int EPC = 4;  // elements per 16-byte chunk
  __device__ static float elem(const u32x4& c, int e) { return __uint_as_float(c[e]); }
  __device__ static float load(const float* p) { return *p; }
};
template <>
struct ValuTraits<uint16_t> {
  static constexpr int EPC = 8;
  __device__ static float elem(const u32x4& c, int e) {
    const uint32_t w = c[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ static float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
};

template <typename T, int D, int RG>
__global__ __launch_bounds__(kThreads) void run_valu(RunArgs a) {
  constexpr int NTHR = kThreads, NWAVE = kWaves;
  constexpr int EPC = ValuTraits<T>::EPC;
  constexpr int KC = D / EPC;     // key chunks per token
  constexpr int DPL = D / 64;     // output dims per lane
  constexpr int RM = 2 * RG;      // rows held
  constexpr int HALF = D / 2;
  constexpr int PS = 36;          // P row stride (floats), keeps float4 reads aligned
  constexpr int kPWave = RM * PS + RM;  // one wave's P and rescale factors
  constexpr int ACC_STRIDE = D + 4;
  constexpr int kState = RM * ACC_STRIDE + 2 * RM;
  constexpr int kQBlock = RM * D;      // rotated queries of one block (floats)
  constexpr int kQfFloats = 40960 / 4;  // 40 KB of rotated queries per group
  constexpr int kQf = kQfFloats / kQBlock > 0 ? kQfFloats / kQBlock : 1;
  constexpr int kUnion = cmax(kQf * kQBlock, 2 * kState);
  __shared__ PlanLds pl;
  __shared__ double invf[HALF];
  __shared__ __attribute__((aligned(16))) float qs[RM * D];  // raw query rows
  // rotated queries during the loop; the waves' softmax states at the end
  __shared__ __attribute__((aligned(16))) float ubuf[kUnion];
  __shared__ __attribute__((aligned(16))) float pbuf_all[NWAVE * kPWave];  // P, rescale factors

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int tl = lane & 31, rg = lane >> 5;
  int g, u;
  head_unit(a, &g, &u);
  const EpiArgs ea = epi_args<false, false>(a, g);
  int lo, hi, b_first, b_last;
  {
    constexpr int kQVec = RM * D / 4;  // float4 of staged query
    constexpr int kQRegs = (kQVec + NTHR - 1) / NTHR;
    const PlanLoads pload = issue_plan_loads<NTHR>(a, u);
    double w = 0.0;
    if (tid < HALF)
      w = reinterpret_cast<const double*>(reinterpret_cast<const char*>(&a) +
                                          offsetof(RunArgs, inv_freq))[tid];
    float4 qv[kQRegs];
    const T* qg = static_cast<const T*>(a.q);
#pragma unroll
    for (int k = 0; k < kQRegs; ++k) {
      const int x = tid + k * NTHR;
      const int r = (4 * x) / D, d = 4 * x - r * D;
      qv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (x < kQVec && r < a.R) {
        const T* src = qg + out_row(a, g, r) * D + d;
        qv[k] = make_float4(ValuTraits<T>::load(src), ValuTraits<T>::load(src + 1),
                            ValuTraits<T>::load(src + 2), ValuTraits<T>::load(src + 3));
      }
    }
    commit_plan_loads<NTHR>(a, pl, pload);
    if (tid < HALF) invf[tid] = w;
#pragma unroll
    for (int k = 0; k < kQRegs; ++k) {
      const int x = tid + k * NTHR;
      if (x < kQVec) *reinterpret_cast<float4*>(qs + 4 * x) = qv[k];
    }
    __syncthreads();
    (void)unit_range<D, static_cast<int>(sizeof(T))>(a, pl, pload, &lo, &hi);
  }
  block_range(pl, lo, hi, &b_first, &b_last);
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(static_cast<const T*>(a.k) + static_cast<int64_t>(g) * a.plane_elems, a.plane_bytes);
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(static_cast<const T*>(a.v) + static_cast<int64_t>(g) * a.plane_elems, a.plane_bytes);
  float* pbuf = pbuf_all + wave * kPWave;

  float acc[RM][DPL];
  float m_run[RG], l_run[RG];
#pragma unroll
  for (int i = 0; i < RG; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) acc[r][dd] = 0.f;

  // (a2) rotated, scaled queries of visible blocks gb..ge-1:
  // ubuf[(b-gb)*RM*D + r*D + d]; rows that see nothing of a block are zero
  auto rotate_blocks = [&](int gb, int ge) {
    const int items = (ge - gb) * RM * HALF;
    for (int x = tid; x < items; x += NTHR) {
      const int i = x % HALF;
      const int r = (x / HALF) % RM;
      const int bi = x / (HALF * RM);
      int re = -1;
      if (r < a.R) re = rows_lds[(gb + bi) * a.qrows + fast_div(r, a.mG)];
      float c = 0.f, s = 0.f;
      if (re >= 0) rope_cos_sin(re, invf[i], &c, &s);
      const float x0 = qs[r * D + i], x1 = qs[r * D + i + HALF];
      float* dst = ubuf + bi * kQBlock + r * D;
      dst[i] = re >= 0 ? (x0 * c - x1 * s) * a.qscale : 0.f;
      dst[i + HALF] = re >= 0 ? (x1 * c + x0 * s) * a.qscale : 0.f;
    }
  };

  // this lane's key chunks (token tl) and value chunks (dims DPL*lane..)
  auto load_k = [&](uint32_t tile, u32x4 (&kc)[KC]) {
    const uint32_t base = ((tl >> 4) * 16 * D + (tl & 15) * 8) * sizeof(T);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      // chunk c covers dims EPC*c..: group (EPC*c)/8, offset (EPC*c)%8
      const int d0 = EPC * c;
      kc[c] = __builtin_amdgcn_raw_buffer_load_b128(
          krs, base + ((d0 >> 3) * 128 + (d0 & 7)) * sizeof(T), tile, 0);
    }
  };
  constexpr int VC = 8 / EPC;  // chunks per (group, dim): 1 (bf16) or 2 (fp32)
  auto load_v = [&](uint32_t tile, u32x4 (&vc)[DPL][4][VC]) {
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
#pragma unroll
        for (int h = 0; h < VC; ++h) {
          const int d = DPL * lane + dd;
          vc[dd][gq][h] = __builtin_amdgcn_raw_buffer_load_b128(
              vrs, (gq * 8 * D + d * 8 + h * EPC) * sizeof(T), tile, 0);
        }
  };

  // last local position of visible block b that row rg*RG+i may see (-1: none)
  auto row_ends = [&](int b, int (&rowend)[RG]) {
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int r = rg * RG + i;
      rowend[i] = r < a.R ? rows_lds[b * a.qrows + fast_div(r, a.mG)] : -1;
    }
  };
  auto compute = [&](const u32x4 (&kc)[KC], const u32x4 (&vc)[DPL][4][VC], const float* qblk,
                     const int (&rowend)[RG], int valid, int first) {
    // ---- scores of rows rg*RG+i against token tl, into the P buffer (the
    // row loop stays rolled so the queries are read from LDS as they are used)
    float kv[D];
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int e = 0; e < EPC; ++e) kv[EPC * c + e] = ValuTraits<T>::elem(kc[c], e);
#pragma unroll 1
    for (int i = 0; i < RG; ++i) {
      const int r = rg * RG + i;
      const float* qr = qblk + r * D;
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int d = 0; d < D; d += 8) {
        const float4 qa = *reinterpret_cast<const float4*>(qr + d);
        const float4 qb = *reinterpret_cast<const float4*>(qr + d + 4);
        s0 += qa.x * kv[d] + qa.y * kv[d + 1] + qa.z * kv[d + 2] + qa.w * kv[d + 3];
        s1 += qb.x * kv[d + 4] + qb.y * kv[d + 5] + qb.z * kv[d + 6] + qb.w * kv[d + 7];
      }
      pbuf[r * PS + tl] = s0 + s1;
    }
    // ---- online softmax per row (exp2 domain), P and rescale factors to LDS
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int r = rg * RG + i;
      const bool ok = tl <= min(valid - 1, rowend[i] - first);
      const float sv = ok ? pbuf[r * PS + tl] : -INFINITY;
      const float mt = half_max(sv);
      const float mn = fmaxf(m_run[i], mt);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float al = __builtin_amdgcn_exp2f(m_run[i] - mu);
      const float p = __builtin_amdgcn_exp2f(sv - mu);
      l_run[i] = l_run[i] * al + half_sum(p);
      m_run[i] = mn;
      pbuf[r * PS + tl] = p;
      if (tl == 0) pbuf[RM * PS + r] = al;
    }
    // ---- P.V for every row on this lane's dims (tokens past `valid` are
    // dropped from V: they may hold anything, even NaN)
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r >= a.R) continue;  // (uniform; keeps the trip count constant)
      const float al = pbuf[RM * PS + r];
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) acc[r][dd] *= al;
    }
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        // chunk elements 4*hh..4*hh+3 of group gq hold tokens 16*hh + 4*gq + v
        float vv[4][DPL];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int e = 4 * hh + v;
          const int t = 16 * hh + 4 * gq + v;
#pragma unroll
          for (int dd = 0; dd < DPL; ++dd) {
            const float x = ValuTraits<T>::elem(vc[dd][gq][e / EPC], e % EPC);
            vv[v][dd] = t < valid ? x : 0.f;
          }
        }
#pragma unroll
        for (int r = 0; r < RM; ++r) {
          if (r >= a.R) continue;  // (uniform; keeps the trip count constant)
          const float4 p4 = *reinterpret_cast<const float4*>(pbuf + r * PS + 16 * hh + 4 * gq);
#pragma unroll
          for (int dd = 0; dd < DPL; ++dd)
            acc[r][dd] += p4.x * vv[0][dd] + p4.y * vv[1][dd] + p4.z * vv[2][dd] + p4.w * vv[3][dd];
        }
      }
    }
  };

  int done_tiles = 0;  // tiles this wave processed
  if (lo < hi) {
    for (int gb = b_first; gb <= b_last; gb += kQf) {
      const int ge = min(gb + kQf, b_last + 1);
      const int t_lo = max(lo, pl.w[kPlanVbTile0 + gb]);
      const int t_hi = min(hi, pl.w[kPlanVbTile0 + ge]);
      int j = t_lo + wave;
      int bcur = gb;
      TileRef rt = {0, 0, 0, 0u};
      u32x4 kc[KC], vc[DPL][4][VC];
      if (j < t_hi) {
        rt = tile_ref<D, static_cast<int>(sizeof(T))>(pl, j, bcur);
        const uint32_t tile = __builtin_amdgcn_readfirstlane(rt.byte);
        load_k(tile, kc);
        load_v(tile, vc);
      }
      if (gb != b_first) __syncthreads();  // the previous group's queries are consumed
      rotate_blocks(gb, ge);
      __syncthreads();
      if (j < t_hi) {
        for (;;) {
          const float* qblk = ubuf + (rt.b - gb) * kQBlock;
          int rowend[RG];
          row_ends(rt.b, rowend);
          const int jn = j + NWAVE;
          ++done_tiles;
          if (jn >= t_hi) {
            compute(kc, vc, qblk, rowend, rt.valid, rt.first);
            break;
          }
          const TileRef rn = tile_ref<D, static_cast<int>(sizeof(T))>(pl, jn, bcur);
          const uint32_t tn = __builtin_amdgcn_readfirstlane(rn.byte);
          compute(kc, vc, qblk, rowend, rt.valid, rt.first);
          load_k(tn, kc);
          load_v(tn, vc);
          j = jn;
          rt = rn;
        }
      }
    }
  }

  // ---- combine the waves' states (two at a time) into the unit's partial
  // state of row r: acc on every lane (dims), (m, l) on the row group's lanes
  auto deposit = [&](float* buf) {
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r >= a.R) continue;  // (uniform; keeps the trip count constant)
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) buf[r * ACC_STRIDE + DPL * lane + dd] = acc[r][dd];
    }
    if (tl == 0) {
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        const int r = rg * RG + i;
        if (r < a.R) {
          buf[RM * ACC_STRIDE + r] = m_run[i];
          buf[RM * ACC_STRIDE + RM + r] = l_run[i];
        }
      }
    }
  };
  if (lane == 0) atomicAdd(&pl.tiles, done_tiles);
  __syncthreads();  // every wave is done with the queries and its P buffer
  if (wave >= 2) deposit(ubuf + (wave - 2) * kState);
  __syncthreads();
  if (wave < 2) {
    // fold in the partner wave's state: m, l of every row from LDS, acc by dims
    const float* src = ubuf + wave * kState;
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r >= a.R) continue;  // (uniform; keeps the trip count constant)
      // own (m, l) of row r: held by the lanes of row group r / RG
      float mo = -INFINITY, lo2 = 0.f;
#pragma unroll
      for (int k = 0; k < RG; ++k)
        if (k == r % RG) {
          mo = m_run[k];
          lo2 = l_run[k];
        }
      // lanes of the other half hold another row: take row r's from lane (r/RG)*32
      mo = __shfl(mo, (r / RG) * 32);
      lo2 = __shfl(lo2, (r / RG) * 32);
      const float m2 = src[RM * ACC_STRIDE + r];
      const float l2 = src[RM * ACC_STRIDE + RM + r];
      const float M = fmaxf(mo, m2);
      const float s1 = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - M);
      const float s2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd)
        acc[r][dd] = acc[r][dd] * s1 + src[r * ACC_STRIDE + DPL * lane + dd] * s2;
      // the merged (m, l) go back to the row group's registers
      const float lm = lo2 * s1 + l2 * s2;
#pragma unroll
      for (int k = 0; k < RG; ++k)
        if (k == r % RG && rg == r / RG) {
          m_run[k] = M;
          l_run[k] = lm;
        }
    }
  }
  __syncthreads();
  if (wave < 2) deposit(ubuf + wave * kState);
  __syncthreads();
  emit_unit<NTHR, D>(ea, pl, g, u, ubuf, 2, kState, RM);
}

// ----------------------------------------------------------- merge kernel
// (a4) One workgroup per (kv head g, row r), one thread per output dim:
// out = sum_u acc_u 2^(m_u - M) / L with M = max_u m_u and
// L = sum_u l_u 2^(m_u - M), units in fixed order.  Units are taken
// kMergeChunk at a time: lane k of every wave loads unit u0+k's (m, l) and
// forms its weight, which the lanes read back with readlane while summing
// their accumulators, so the kernel has neither LDS nor barriers; the
// running (M, L, sum) is rescaled when a later chunk raises M.  The
// workgroup of row 0 of each head also checks that the head's units
// processed every tile of the plan once and resets the head's tile counter.
constexpr int kMergeChunk = 32;  // units whose loads are in flight together

// Lane k's value of x (the builtin moves 32-bit integers: pass the bits).
__device__ __forceinline__ float readlane_f32(float x, int k) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), k));
}

template <int D>
__global__ __launch_bounds__(D) void merge_kernel(RunArgs a) {
  // every scalar argument, requested at entry in one round trip
  asm volatile("" ::"s"(a.ws_ml), "s"(a.ws_acc), "s"(a.out), "s"(a.status), "s"(a.R), "s"(a.P),
               "s"(a.G), "s"(a.Hq), "s"(a.dtype), "s"(a.mR), "s"(a.mG));
  const int tid = threadIdx.x;  // output dim
  const int lane = tid & 63;
  if (tid == 0) HW_MSTAMP(0);
  const int g = fast_div(blockIdx.x, a.mR);
  const int r = blockIdx.x - g * a.R;
  const int P = a.P;
  // FP8 pools: values are code * scale of the kv head (requested early)
  const float vsc = a.dtype == HW_FP8
                        ? reinterpret_cast<const float*>(reinterpret_cast<const char*>(&a) +
                                                         offsetof(RunArgs, v_scale))[g]
                        : 1.f;
  // this (kv head, row)'s partials as buffers over its P units: unit u's
  // accumulators at byte u * D * 4, its (m, l) at byte u * 8.  Units past the
  // last lie outside the buffers, read as zero and get zero weight.
  const int64_t row0 = (static_cast<int64_t>(g) * a.R + r) * P;
  const __amdgpu_buffer_rsrc_t accrs = make_rsrc(a.ws_acc + row0 * D, P * D * 4);
  const __amdgpu_buffer_rsrc_t mlrs = make_rsrc(a.ws_ml + row0, P * 8);
  float M = -INFINITY, L = 0.f, s = 0.f;
  for (int u0 = 0; u0 < P; u0 += kMergeChunk) {
    const int uk = u0 + (lane & (kMergeChunk - 1));
    const float2 mv = __builtin_bit_cast(
        float2, __builtin_amdgcn_raw_buffer_load_b64(mlrs, static_cast<uint32_t>(uk) * 8u, 0, 0));
    float av[kMergeChunk];
#pragma unroll
    for (int k8 = 0; k8 < kMergeChunk; k8 += 8) {
      // eight units per base offset: the rest in the instructions' offset field
      uint32_t vo = static_cast<uint32_t>(tid + (u0 + k8) * D) * 4u;
      asm volatile("" : "+v"(vo));  // (keeps the unit offsets in the offset field)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        av[k8 + k] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(accrs, vo + k * D * 4, 0, 0));
    }
    const float mk = uk < P ? mv.x : -INFINITY;
    // (each 32-lane half of the wave holds the chunk's units: DPP reductions)
    const float Mc = fmaxf(M, half_max(mk));
    // while no unit has tokens every weight is 0 and (L, sum) stay 0
    const float Mu = Mc == -INFINITY ? 0.f : Mc;
    const float wk = mk == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mk - Mu);
    const float lk = uk < P ? mv.y * wk : 0.f;
    const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mu);
    L = L * sc + half_sum(lk);
    s *= sc;
#pragma unroll
    for (int k = 0; k < kMergeChunk; ++k) s += av[k] * readlane_f32(wk, k);
    M = Mc;
  }
  const float o = L > 0.f ? s / L * vsc : 0.f;
  a.out[out_row(a, g, r) * D + tid] = o;
  if (tid == 0 && !(L > 0.f)) atomicOr(a.status, HW_DEV_NO_TOKENS);
  if (a.balance && r == 0 && tid < 64) {
    // balanced runs: every tile of the head taken exactly once (lane k sums
    // units k, k + 64, ...), then the head's ticket counter back to zero
    int n = 0;
    for (int uu = tid; uu < P; uu += 64) n += a.ws_cnt[g * P + uu];
    n = static_cast<int>(half_sum(static_cast<float>(n)));  // < 2^24: exact
    n += __shfl_xor(n, 32);
    if (tid == 0) {
      if (n < (1 << 30) && n != a.plan[kHdrTiles]) atomicOr(a.status, HW_DEV_WORKSPACE);
      __hip_atomic_store(a.sync + static_cast<int64_t>(g) * kSyncStride, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (lane == 0) HW_MSTAMP(1 + (tid >> 6));
}

template <typename K>
int occupancy(K kernel, int threads, size_t dyn) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, dyn) != hipSuccess) return 0;
  return n;
}

// Dynamic LDS of a launch: the plan's row ends.
size_t rows_bytes(const RunArgs& a) { return static_cast<size_t>(a.NB) * a.qrows * 4; }

}  // namespace

template <typename T, int D>
hipError_t launch_valu_rows(const RunArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.Hkv * a.P));
  const size_t dyn = rows_bytes(a);
  if (a.R <= 8)
    hipLaunchKernelGGL((run_valu<T, D, 4>), grid, dim3(kThreads), dyn, s, a);
  else if (a.R <= 16)
    hipLaunchKernelGGL((run_valu<T, D, 8>), grid, dim3(kThreads), dyn, s, a);
  else if (a.R <= 20)
    hipLaunchKernelGGL((run_valu<T, D, 10>), grid, dim3(kThreads), dyn, s, a);
  else if (a.R <= 32)
    hipLaunchKernelGGL((run_valu<T, D, 16>), grid, dim3(kThreads), dyn, s, a);
  else
    hipLaunchKernelGGL((run_valu<T, D, 32>), grid, dim3(kThreads), dyn, s, a);
  return hipGetLastError();
}

hipError_t launch_run_valu(const RunArgs& a, hipStream_t s) {
  if ((a.D != 64 && a.D != 128) || a.R > kValuMaxRows || a.dtype == HW_FP8)
    return hipErrorInvalidValue;
  if (a.dtype == HW_F32)
    return a.D == 128 ? launch_valu_rows<float, 128>(a, s) : launch_valu_rows<float, 64>(a, s);
  return a.D == 128 ? launch_valu_rows<uint16_t, 128>(a, s) : launch_valu_rows<uint16_t, 64>(a, s);
}

template <int D, typename E>
hipError_t launch_mfma_d(const RunArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.Hkv * a.P));
  const size_t dyn = rows_bytes(a);
  if (a.R <= 16)
    hipLaunchKernelGGL((run_mfma<D, 1, E>), grid, dim3(64 * mfma_waves(1)), dyn, s, a);
  else if (a.R <= 32)
    hipLaunchKernelGGL((run_mfma<D, 2, E>), grid, dim3(64 * mfma_waves(2)), dyn, s, a);
  else if (a.R <= 48)
    hipLaunchKernelGGL((run_mfma<D, 3, E>), grid, dim3(64 * mfma_waves(3)), dyn, s, a);
  else if (a.R <= 64)
    hipLaunchKernelGGL((run_mfma<D, 4, E>), grid, dim3(64 * mfma_waves(4)), dyn, s, a);
  else
    hipLaunchKernelGGL((run_mfma<D, 5, E>), grid, dim3(64 * mfma_waves(5)), dyn, s, a);
  return hipGetLastError();
}

hipError_t launch_run_mfma(const RunArgs& a, hipStream_t s) {
  if (a.R > kMfmaMaxRows) return hipErrorInvalidValue;
  if (a.D == 128) {
    if (a.dtype == HW_BF16) return launch_mfma_d<128, uint16_t>(a, s);
    if (a.dtype == HW_FP8) return launch_mfma_d<128, uint8_t>(a, s);
  } else if (a.D == 64) {
    if (a.dtype == HW_BF16) return launch_mfma_d<64, uint16_t>(a, s);
    if (a.dtype == HW_FP8) return launch_mfma_d<64, uint8_t>(a, s);
  }
  return hipErrorInvalidValue;
}

// Resident workgroups per CU of the kernel a launch would use (0 on error),
// with the dynamic LDS of the largest plan (64 blocks, the rows given).
template <int D, typename E>
int mfma_occ(int rows) {
  const size_t dyn = static_cast<size_t>(HW_MAX_BLOCKS) * rows * 4;
  if (rows <= 16) return occupancy(run_mfma<D, 1, E>, 64 * mfma_waves(1), dyn);
  if (rows <= 32) return occupancy(run_mfma<D, 2, E>, 64 * mfma_waves(2), dyn);
  if (rows <= 48) return occupancy(run_mfma<D, 3, E>, 64 * mfma_waves(3), dyn);
  if (rows <= 64) return occupancy(run_mfma<D, 4, E>, 64 * mfma_waves(4), dyn);
  return occupancy(run_mfma<D, 5, E>, 64 * mfma_waves(5), dyn);
}
template <typename T, int D>
int valu_occ(int rows) {
  const size_t dyn = static_cast<size_t>(HW_MAX_BLOCKS) * rows * 4;
  if (rows <= 8) return occupancy(run_valu<T, D, 4>, kThreads, dyn);
  if (rows <= 16) return occupancy(run_valu<T, D, 8>, kThreads, dyn);
  if (rows <= 20) return occupancy(run_valu<T, D, 10>, kThreads, dyn);
  if (rows <= 32) return occupancy(run_valu<T, D, 16>, kThreads, dyn);
  return occupancy(run_valu<T, D, 32>, kThreads, dyn);
}

hipError_t launch_merge(const RunArgs& a, hipStream_t s) {
  if (a.P > kMaxUnits || (a.D != 64 && a.D != 128)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(a.Hkv * a.R));
  if (a.D == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

int run_blocks_per_cu(int path, int dtype, int D, int rows) {
  if (path == 2) {
    if (D == 128) return dtype == HW_FP8 ? mfma_occ<128, uint8_t>(rows) : mfma_occ<128, uint16_t>(rows);
    return dtype == HW_FP8 ? mfma_occ<64, uint8_t>(rows) : mfma_occ<64, uint16_t>(rows);
  }
  if (D == 128) return dtype == HW_F32 ? valu_occ<float, 128>(rows) : valu_occ<uint16_t, 128>(rows);
  return dtype == HW_F32 ? valu_occ<float, 64>(rows) : valu_occ<uint16_t, 64>(rows);
}

}  // namespace hw

#ifdef HW_STAMPS
extern "C" int hw_debug_stamps(uint64_t* host, size_t n) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(hw::g_stamps), n * sizeof(uint64_t), 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? 0 : 1;
}
#endif
