// hw_decode.hip — concurrent-attention decode kernels for gfx950.
//
// One decode call = two launches on the caller's stream:
//
//  split kernel, one workgroup per work unit (kv head g, unit u); a unit owns
//  a contiguous range of 32-token tiles in the concatenation of the blocks
//  that some worker sees.  Each workgroup
//   1. decodes the worker tables and the device block lengths into a plan
//      (visibility, view offsets, i_q, tile prefix)                  [prologue]
//   2. for every block its range touches, rotates the stacked W*G query rows
//      of head g by i_q - view_offset: only the single current query token is
//      rotated, never the cache (Hogwild! notes, key design 1)        [a2]
//   3. streams its K/V tiles once for all rows with an online softmax in the
//      exp2 domain (split-K / Flash-Decoding; news 1114328 sec. 3.2)   [a3]
//   4. writes its partial (m, l, acc) with plain stores.
//  merge kernel, one workgroup per (kv head, row): log-sum-exp merge of the
//  units' partials in fixed unit order (deterministic) and the output row [a4].
//
// The kernel boundary orders the partials' stores before their loads, so no
// workgroup ever waits on another and no cache maintenance is needed inside
// a kernel.
//
// Two split kernels share the prologue:
//   decode_valu<T>    fp32 VALU arithmetic over LDS-staged tiles (fp32 and
//                     bf16 pools, rows <= 64).
//   decode_mfma<D,NT> bf16 MFMA 16x16x32: S^T = K Q~^T and O^T = V^T P^T with
//                     tiles loaded straight into operand fragments (the pool
//                     layout matches them), rows = W*G <= 16*NT <= 32.
#include <math.h>

#include <type_traits>

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

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
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

// Stacked rows of kv head g: r = (w * nq + j) * G + (h - g * G) for worker w,
// query token j < nq and q-head h.  Query j of worker w sits lag = nq - 1 - j
// positions before the worker's query position i_q (n = 1: the decode query).
// The plan holds each row's worker and lag (row_w, row_lag), so the kernels
// divide by G and nq once.

// ----------------------------------------------------------------- prologue
struct Plan {
  int32_t len[HW_MAX_BLOCKS];
  uint32_t vis[HW_MAX_BLOCKS];        // bit w set: worker w sees block b
  int32_t tile0[HW_MAX_BLOCKS + 1];   // tiles of visible blocks, prefix sums
  long long iq[HW_MAX_WORKERS];       // query position per worker, -1: none
  int32_t row_w[HW_MAX_ROWS];         // worker of each stacked row (0 past R)
  int32_t row_lag[HW_MAX_ROWS];       // positions before i_q of each row's query
  int32_t off[HW_MAX_WORKERS * HW_MAX_BLOCKS];
  int64_t start[HW_MAX_BLOCKS];       // first slot of each block
  double invf[kMaxHalf];              // theta^(-2i/D)
  uint64_t rope_frac[kMaxHalf];       // theta^(-2i/D) / (2 pi) mod 1, 64-bit fixed point
  uint32_t bad_workers;
  int32_t flags;
  int32_t head, unit, lo, hi;
  int32_t b_first, b_last;  // blocks holding tiles lo and hi - 1
};

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by
// 1, 2, 4 and 8 lanes inside each row of 16, then the last lane of row 0
// (row 2) is added to row 1 (row 3), and the last lane of row 1 to rows 2
// and 3.  Lanes shifted in from outside a row read 0.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return x;
}

// Workgroup -> (kv head, work unit): the units of a head are consecutive
// workgroups.
__device__ __forceinline__ void plan_head_unit(const DecodeArgs& a, int* head, int* unit) {
  *head = fast_div(blockIdx.x, a.mP);
  *unit = blockIdx.x - *head * a.P;
}

// Table entry i (worker i / E, slot i % E): marks its block visible to the
// worker and records the view offset.  A malformed table (entry count out of
// range, block id out of range, a block listed twice) marks its worker bad.
__device__ __forceinline__ void plan_entry(const DecodeArgs& a, Plan& p, int i, hw_entry e,
                                           int ne) {
  const int w = fast_div(i, a.mE), slot = i - w * a.E;
  const uint32_t bit = 1u << w;
  if (ne < 0 || ne > a.E) {
    atomicOr(&p.bad_workers, bit);
    return;
  }
  if (slot >= ne) return;
  const int b = e.block_id;
  if (b < 0 || b >= a.NB) {
    atomicOr(&p.bad_workers, bit);
    return;
  }
  if (atomicOr(&p.vis[b], bit) & bit) atomicOr(&p.bad_workers, bit);
  p.off[w * a.NB + b] = e.view_offset;
}

// The plan costs one memory round trip: every global load is issued before
// the first wait.  A kernel's code is fetched cold at every launch, so the
// prologue is kept short and rolled: block-level work runs on waves 0 and 1
// with one lane per block, table entries on one thread each.
// issue(): the kernel's own loads, issued with the plan's; commit(): their
// LDS stores, run once they have arrived.  NTHR threads (the first NTHR of
// the workgroup) take part; sync() is their barrier.
struct WorkgroupBarrier {
  __device__ void operator()() const { __syncthreads(); }
};

template <int NTHR, typename Issue, typename Commit, typename Sync>
__device__ void build_plan(const DecodeArgs& a, Plan& p, Issue issue, Commit commit, Sync& sync) {
  const int tid = threadIdx.x;
  const int WE = a.W * a.E;
  // ---- loads: per block (lanes of waves 0 and 1) length and capacity, and
  // (wave 0) first slot;
  // per frequency its two forms; one table entry per thread.  The per-call
  // arrays are read from the kernel-argument segment through a pointer
  // (indexing the argument itself would copy it to scratch).
  const char* tabp = reinterpret_cast<const char*>(&a.tab);
  int len = 0, cap = 0;
  int64_t start = 0;
  // (lane b of waves 0 and 1: block b's length and capacity; wave 0 its start)
  if (tid < 128 && (tid & 63) < a.NB) {
    len = a.block_len[tid & 63];
    cap = reinterpret_cast<const int32_t*>(tabp + offsetof(DecodeTables, block_cap))[tid & 63];
    if (tid < 64)
      start = reinterpret_cast<const int64_t*>(tabp + offsetof(DecodeTables, block_start))[tid];
  }
  double invf = 0.0;
  uint64_t frac = 0u;
  if (tid < a.D / 2) {
    invf = reinterpret_cast<const double*>(tabp + offsetof(DecodeTables, inv_freq))[tid];
    frac = reinterpret_cast<const uint64_t*>(tabp + offsetof(DecodeTables, rope_frac))[tid];
  }
  hw_entry ent = {-1, 0};
  int ne = 0;
  if (tid < WE) {
    ent = a.tables[tid];
    ne = a.num_entries[fast_div(tid, a.mE)];
  }
  issue();
  // ---- state that needs none of the loads
  if (tid < a.NB) p.vis[tid] = 0u;
  if (tid < a.W) p.iq[tid] = -1;
  if (tid < HW_MAX_ROWS) {
    const bool row = tid < a.R;
    const int w = fast_div(tid, a.mGnq);
    p.row_w[tid] = row ? w : 0;
    p.row_lag[tid] = row ? a.nq - 1 - (fast_div(tid, a.mG) - w * a.nq) : 0;
  }
  for (int i = tid; i < a.W * a.NB; i += NTHR) p.off[i] = 0;
  if (tid == 0) {
    p.flags = 0;
    p.bad_workers = 0u;
    plan_head_unit(a, &p.head, &p.unit);
  }
  sync();
  // ---- visibility and view offsets from the tables
  commit();
  if (tid < WE) plan_entry(a, p, tid, ent, ne);
#pragma unroll 1
  for (int i = tid + NTHR; i < WE; i += NTHR)
    plan_entry(a, p, i, a.tables[i], a.num_entries[fast_div(i, a.mE)]);
  if (tid < a.D / 2) {
    p.invf[tid] = invf;
    p.rope_frac[tid] = frac;
  }
  if (tid < a.NB) p.start[tid] = start;
  sync();
  // ---- wave 0, lane b = block b: checked length, visibility without the
  // bad workers and the tile prefix over the visible blocks; at the same
  // time wave 1, lane b = block b: each worker's query position (the last
  // position of any block it sees)
  if (tid < 64) {
    const int b = tid;
    int v = 0;
    // (opaque until here: otherwise the compiler compares right after the
    // loads and waits for them before the rest of the plan's loads are issued)
    asm volatile("" : "+v"(len), "+v"(cap));
    if (b < a.NB) {
      if (len < 0 || len > cap) {
        atomicOr(&p.flags, HW_DEV_BAD_LENGTH);
        len = 0;
      }
      const uint32_t vis = p.vis[b] & ~p.bad_workers;
      p.vis[b] = vis;
      p.len[b] = len;
      if (vis != 0u && len > 0) v = (len + kTile - 1) / kTile;
    }
    const int incl = wave_inclusive_scan(v);
    const int nt = __builtin_amdgcn_readlane(incl, 63);
    if (b < a.NB) p.tile0[b] = incl - v;
    // The units split the tiles by cost: a tile costs 1 and every visible
    // block after the first kBlockCost more (a unit that reaches another
    // block rotates its queries before its front waves stream, measured at
    // about five tiles' time).  Cost position x maps to tile
    // sum_b clamp(x - cs_b, 0, tiles_b), cs_b being the cost position of
    // block b's first tile.  C * (unit + 1) < 2^31: a plane holds under 2^31
    // bytes, so under 2^18 tiles, and there are at most kMaxUnits units.
    const int cv = v + ((v > 0 && incl > v) ? kBlockCost : 0);
    const int cincl = wave_inclusive_scan(cv);
    const uint32_t C = static_cast<uint32_t>(__builtin_amdgcn_readlane(cincl, 63));
    const int cs = cincl - v;
    // x / P for x < 2^31: the fp64 product is within 2^-21 of the quotient,
    // so its truncation is exact except when P divides x, where it may be
    // one short (the correction)
    auto div_p = [&](uint32_t x) {
      const uint32_t q = static_cast<uint32_t>(static_cast<double>(x) * a.rP);
      return static_cast<int>(q + ((q + 1u) * static_cast<uint32_t>(a.P) <= x ? 1u : 0u));
    };
    const int xlo = div_p(C * p.unit);
    const int xhi = div_p(C * (p.unit + 1));
    const int lo = __builtin_amdgcn_readlane(wave_inclusive_scan(min(max(xlo - cs, 0), v)), 63);
    const int hi = __builtin_amdgcn_readlane(wave_inclusive_scan(min(max(xhi - cs, 0), v)), 63);
    // block of tile j: the last b < NB with tile0[b] <= j (tile0 does not
    // decrease, so these blocks are a prefix)
    const int t0 = incl - v;
    const int bf = __builtin_popcountll(__ballot(b < a.NB && t0 <= lo)) - 1;
    const int bl = __builtin_popcountll(__ballot(b < a.NB && t0 <= hi - 1)) - 1;
    if (b == 0) {
      p.tile0[a.NB] = nt;
      p.lo = lo;
      p.hi = hi;
      p.b_first = bf;
      p.b_last = bl;
      if (p.bad_workers) atomicOr(&p.flags, HW_DEV_BAD_ENTRY);
    }
  } else if (tid < 128) {
    const int b = tid - 64;
    asm volatile("" : "+v"(len), "+v"(cap));
    // (the same checks as wave 0; the visibility read here is the raw or the
    // already cleaned word, the same once the bad workers are masked out)
    if (b < a.NB && len > 0 && len <= cap) {
      const uint32_t vis = p.vis[b] & ~p.bad_workers;
#pragma unroll 1
      for (uint32_t m = vis; m != 0u; m &= m - 1u) {
        const int w = __builtin_ctz(m);
        atomicMax(&p.iq[w], static_cast<long long>(p.off[w * a.NB + b]) + len - 1);
      }
    }
  }
  sync();
}

template <int NTHR, typename Issue, typename Commit>
__device__ void build_plan(const DecodeArgs& a, Plan& p, Issue issue, Commit commit) {
  WorkgroupBarrier sync;
  build_plan<NTHR>(a, p, issue, commit, sync);
}

// Waves of one workgroup that synchronize through a counter in LDS instead of
// s_barrier, so that the other waves of the workgroup never have to join:
// each wave's LDS writes complete (release fence on LDS), lane 0 adds one,
// and the wave waits until the counter reaches count * phase.  The counter
// only grows; it must be zero before the first phase.  Every wave of the
// group reaches every phase (no early exits), so every wait ends.
struct LdsWaveBarrier {
  uint32_t* ctr;
  uint32_t count;
  uint32_t phase;
  __device__ void operator()() {
    ++phase;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if ((threadIdx.x & 63) == 0)
      __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < count * phase)
      __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }
};

// Waits until an LDS counter that other waves advance reaches `target`.
__device__ __forceinline__ void lds_wait_at_least(uint32_t* ctr, uint32_t target) {
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target)
    __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Block holding global tile j of the plan (cursor walks forward).
__device__ __forceinline__ int block_of_tile(const Plan& p, int nb, int j, int b) {
  while (b + 1 < nb && p.tile0[b + 1] <= j) ++b;
  return b;
}

// Per-unit partial: (m, l) per row and the unnormalised accumulator.
__device__ __forceinline__ int64_t partial_index(const DecodeArgs& a, const Plan& p) {
  return static_cast<int64_t>(p.head) * a.R * a.P + p.unit;
}

// ------------------------------------------------------------- MFMA kernel
// bf16 and FP8 pools, rows R = W*G <= 16*NT.  Each of the eight waves owns
// every 8th tile of the workgroup's range and keeps its own (m, l, O^T) for
// all rows; the waves' states are combined in LDS at the end.
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
  int first;      // local position of the tile's first token in its block
  int64_t base;   // element offset of the tile in the kv-head plane
};

template <int D>
__device__ __forceinline__ TileRef tile_ref(const Plan& p, int nb, int j, int& bcur) {
  bcur = block_of_tile(p, nb, j, bcur);
  const int tl = j - p.tile0[bcur];
  TileRef r;
  r.b = bcur;
  r.valid = min(kTile, p.len[bcur] - tl * kTile);
  r.first = tl * kTile;
  r.base = (p.start[bcur] + static_cast<int64_t>(tl) * kTile) * D;
  return r;
}

constexpr int cmax(int x, int y) { return x > y ? x : y; }
constexpr int kOneLevelRows = 24;  // rows up to which every wave's state has its own LDS slot

// Raw buffer resource over one kv-head plane (gfx9 descriptor word 3).  The
// lane offsets are range-checked against the plane; the tile offset (an SGPR
// operand) is in range by construction: a tile lies inside its block's
// capacity, whose slots the host checked against the plane.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const void* p, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0), bytes,
                                           0x00020000);
}

// Stored K/V elements as MFMA A fragments (8 elements per lane): bf16 pools
// load 16 bytes and use them as they are; FP8 E4M3 pools load 8 bytes, which
// are widened to bf16 (exactly: every E4M3 value is a bf16 value) just before
// the product that consumes them, so the registers of a tile in flight hold
// the narrow codes.
// K/V fragments are read exactly once per call: their loads carry the
// non-temporal cache policy (aux bit 1, `nt`), which measured 1.5 us faster per
// 76 MB call than the default policy.
constexpr int kStreamLoad = 2;
template <typename E>
struct KvFrag;
template <>
struct KvFrag<uint16_t> {
  typedef u32x4 type;
  static constexpr int kBytes = 2;
  __device__ static type load(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kStreamLoad);
  }
  __device__ static u32x4 widen(const type& f) { return f; }
};
template <>
struct KvFrag<uint8_t> {
  typedef u32x2 type;
  static constexpr int kBytes = 1;
  __device__ static type load(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, kStreamLoad);
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
// byte offset in the plane (wave-uniform, kept in an SGPR).
template <int D, typename E>
__device__ __forceinline__ void load_keys(__amdgpu_buffer_rsrc_t krs, uint32_t tile, uint32_t koff,
                                          typename KvFrag<E>::type (&kf)[2][D / 32]) {
  constexpr int B = KvFrag<E>::kBytes;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      kf[h2][s] = KvFrag<E>::load(krs, koff + (h2 * 16 * D + 4 * s * 128) * B, tile);
}

template <int D, typename E>
__device__ __forceinline__ void load_values(__amdgpu_buffer_rsrc_t vrs, uint32_t tile,
                                            uint32_t voff, typename KvFrag<E>::type (&vf)[D / 16]) {
  constexpr int B = KvFrag<E>::kBytes;
#pragma unroll
  for (int m = 0; m < D / 16; ++m) vf[m] = KvFrag<E>::load(vrs, voff + 16 * m * 8 * B, tile);
}

// The same loads with the tile offset in the range-checked lane offset: a
// tile offset past the plane reads zeros, so any value may be passed (used
// for the speculative first tile, whose offset comes from the last call).
template <int D, typename E>
__device__ __forceinline__ void load_tile_checked(__amdgpu_buffer_rsrc_t krs,
                                                  __amdgpu_buffer_rsrc_t vrs, uint32_t tile,
                                                  uint32_t koff, uint32_t voff,
                                                  typename KvFrag<E>::type (&kf)[2][D / 32],
                                                  typename KvFrag<E>::type (&vf)[D / 16]) {
  load_keys<D, E>(krs, 0, koff + tile, kf);
  load_values<D, E>(vrs, 0, voff + tile, vf);
}

// S^T for one tile: sc[h][t] holds tokens 16h + 4*q4 + v of rows 16t + li.
// qf: this lane's rotated-query B fragments, [NT][KS] x 64 lanes in LDS.
template <int D, int NT, typename E>
__device__ __forceinline__ void tile_scores(const typename KvFrag<E>::type (&kf)[2][D / 32],
                                            const bf16x8* qf, int lane, f32x4 (&sc)[2][NT]) {
  constexpr int KS = D / 32;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    f32x4 c0 = f32x4{0.f, 0.f, 0.f, 0.f}, c1 = c0;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
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
// limit, below `valid`); values of tokens at or past `valid` are zeroed.
template <int D, int NT, typename E>
__device__ __forceinline__ void tile_update(const f32x4 (&sc)[2][NT],
                                            const typename KvFrag<E>::type (&vf)[D / 16],
                                            const bool (&rowvis)[NT], const int (&rowlim)[NT],
                                            int valid, int q4,
                                            f32x4 (&acc)[D / 16][NT], float (&m_run)[NT],
                                            float (&l_run)[NT]) {
  constexpr int MT = D / 16;
  bf16x8 pf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
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
    for (int t = 0; t < NT; ++t)
      acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), pf[t],
                                                          acc[m][t], 0, 0, 0);
  }
}

template <int D, int NT, typename E>
__global__ __launch_bounds__(kMfmaThreads) void decode_mfma(DecodeArgs a) {
  typedef typename KvFrag<E>::type Frag;
  constexpr int EB = KvFrag<E>::kBytes;
  constexpr int NTHR = kMfmaThreads;
  constexpr int NWAVE = kMfmaWaves;
  constexpr int NSTATE = NWAVE / 2;  // wave states held in LDS at once
  constexpr int KS = D / 32;  // k-steps of the QK product
  constexpr int MT = D / 16;  // 16-dim tiles of the output
  constexpr int RP = 16 * NT; // padded rows
  constexpr int HALF = D / 2;
  constexpr int ACC_STRIDE = D + 4;
  // one wave's (O^T, m, l) with room for RC1 rows (all waves at once) or RP
  // rows (half of the waves at a time)
  constexpr int RC1 = RP < kOneLevelRows ? RP : kOneLevelRows;
  constexpr int kState1 = RC1 * ACC_STRIDE + 2 * RC1;
  constexpr int kState2 = RP * ACC_STRIDE + 2 * RP;
  constexpr int kQfFloats = kQfBlocks * NT * KS * 64 * 4;  // rotated-query fragments
  constexpr int kEpiFloats = cmax(NWAVE * kState1, NSTATE * kState2);
  __shared__ Plan plan;
  __shared__ __attribute__((aligned(16))) uint16_t qs[RP * D];
  // the rotated-query fragments of up to kQfBlocks blocks (main loop)
  __shared__ __attribute__((aligned(16))) float qbuf[kQfFloats];
  // the waves' softmax states (epilogue); apart from qbuf, so that a wave
  // done with its tiles deposits its state while the others still stream
  __shared__ __attribute__((aligned(16))) float ebuf[kEpiFloats];

  // every scalar argument of the prologue, requested at entry in one round
  // trip (otherwise each use site waits for its own kernel-argument load)
  asm volatile("" ::"s"(a.q), "s"(a.k), "s"(a.v), "s"(a.block_len), "s"(a.tables),
               "s"(a.num_entries), "s"(a.ws_hint), "s"(a.plane_elems), "s"(a.plane_bytes),
               "s"(a.W), "s"(a.Hq), "s"(a.G), "s"(a.R), "s"(a.E), "s"(a.NB), "s"(a.P), "s"(a.D), "s"(a.nq),
               "s"(a.qscale), "s"(a.mP), "s"(a.mE), "s"(a.mG), "s"(a.mGnq), "s"(a.rP));
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, q4 = lane >> 4;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  // The waves split for the prologue.
  //  front (waves < kFront): load the tables, lengths and this head's query
  //    rows, build the plan and the first group's rotated queries, and
  //    synchronize among themselves through an LDS counter;
  //  back: once the front waves' loads are back, request their speculative
  //    first tile (the tile each started with in the previous call with this
  //    workspace: within a decode step every layer's call has the same plan),
  //    then wait for the rotated queries and keep the tile if the plan
  //    confirms it.
  // A wave whose tile requests stall on a full memory queue (a CU accepts
  // about 64 KB before issue blocks) thus never holds a barrier the plan
  // needs.  The front waves request their first tiles after the rotation.
  constexpr int kFront = 4;
  constexpr int NF = kFront * 64;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool front = wave_u < kFront;  // wave-uniform: one side of each branch per wave
  __shared__ uint32_t sync_ctr[3];  // front barrier, front loads issued, rotation done
  if (tid < 3) sync_ctr[tid] = 0u;
  // publishes the zeroed counters; each wave passes it once, the front waves
  // right after requesting the plan's loads, the back waves first
  auto init_barrier = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  // this head's query rows, staged in LDS so that the main loop issues no
  // vector memory operations other than the K/V stream
  constexpr int kQVec = RP * D / 8;
  constexpr int kQRegs = (kQVec + NF - 1) / NF;
  int h0, u0;
  plan_head_unit(a, &h0, &u0);
  const uint32_t koff = (q4 * 128 + li * 8) * EB;
  const uint32_t voff = (q4 * 8 * D + li * 8) * EB;
  // this head's K/V plane descriptors, the query scale (FP8 pools: times the
  // key scale of the kv head) and this wave's hint slot; set up by the front
  // waves while their plan loads are in flight, by the back waves first
  __amdgpu_buffer_rsrc_t krs, vrs;
  float qsc;
  uint32_t* hint;
  auto kv_setup = [&] {
    krs = plane_rsrc(static_cast<const char*>(a.k) + static_cast<int64_t>(h0) * a.plane_elems * EB,
                     a.plane_bytes);
    vrs = plane_rsrc(static_cast<const char*>(a.v) + static_cast<int64_t>(h0) * a.plane_elems * EB,
                     a.plane_bytes);
    qsc = a.qscale;
    if (EB == 1) qsc *= reinterpret_cast<const float*>(reinterpret_cast<const char*>(&a.tab) +
                                                       offsetof(DecodeTables, k_scale))[h0];
    hint = a.ws_hint + (static_cast<int64_t>(h0) * a.P + u0) * NWAVE + wave_u;
  };
  uint32_t spec = 0xffffffffu;  // back waves: the hinted first tile
  Frag kf[2][KS], vf[MT];
  LdsWaveBarrier front_sync{&sync_ctr[0], kFront, 0u};
  if (front) {
    u32x4 qv[kQRegs];
    auto issue = [&] {
#pragma unroll
      for (int k = 0; k < kQRegs; ++k) {
        const int x = tid + k * NF;
        const int r = (8 * x) / D, d = (8 * x) - r * D;
        qv[k] = u32x4{0u, 0u, 0u, 0u};
        if (x < kQVec && r < a.R) {
          const int w = fast_div(r, a.mG), h = h0 * a.G + (r - w * a.G);
          qv[k] =
              *reinterpret_cast<const u32x4*>(qg + (static_cast<int64_t>(w) * a.Hq + h) * D + d);
        }
      }
      init_barrier();
      kv_setup();
    };
    auto commit = [&] {
#pragma unroll
      for (int k = 0; k < kQRegs; ++k) {
        const int x = tid + k * NF;
        if (x < kQVec) *reinterpret_cast<u32x4*>(qs + 8 * x) = qv[k];
      }
      // the plan's loads are back: the back waves' tiles may now fill the
      // memory queues (issued earlier, they delay these small loads by the
      // whole chip's burst)
      if (lane == 0) __hip_atomic_fetch_add(&sync_ctr[1], 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    build_plan<NF>(a, plan, issue, commit, front_sync);
  } else {
    kv_setup();
    const uint32_t hv = *hint;  // (loaded by the back waves only)
    init_barrier();
    spec = __builtin_amdgcn_readfirstlane(hv);
    lds_wait_at_least(&sync_ctr[1], kFront);
    load_tile_checked<D, E>(krs, vrs, spec, koff, voff, kf, vf);
  }
  bool rowvis[NT];
  f32x4 acc[MT][NT];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
    rowvis[t] = false;
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // (a2) rotated queries of blocks gb..ge-1, shared by all waves: for each
  // block the stacked rows of head g rotated by i_q - view_offset of their
  // worker, scaled, rounded to bf16 and laid out as MFMA B fragments
  // (row 16t+li, dims 8*(4s+q4)..+8 at qfs[((blk*NT + t)*KS + s)*64 + lane]).
  // Rows past R or of workers that do not see the block are zero.  nthr: the
  // threads taking part.
  bf16x8* qfs = reinterpret_cast<bf16x8*>(qbuf);
  // A thread's item (row, dims) is the same in every block (nthr is a
  // multiple of IPB): its query values, frequencies, worker and i_q - lag are
  // read from LDS once; per block only the view offset and visibility.
  constexpr int IPB = NT * (KS / 2) * 64;  // items per block
  auto rotate_blocks = [&](int gb, int ge, int nthr) {
    const int slot = tid & (IPB - 1);
    const int ln = slot & 63;
    const int y = slot >> 6;
    const int sh = y % (KS / 2);
    const int t = y / (KS / 2);
    const int r = 16 * t + (ln & 15);
    const int w = plan.row_w[r];
    const long long iq_lag = plan.iq[w] - plan.row_lag[r];
    const int d0 = 8 * (4 * sh + (ln >> 4));  // < HALF; its partner dims are d0 + HALF
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(qs + r * D + d0);
    uint32_t xw[4], yw[4];
    uint64_t fr[8];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      xw[e2] = qw[e2];
      yw[e2] = qw[e2 + HALF / 2];
      fr[2 * e2] = plan.rope_frac[d0 + 2 * e2];
      fr[2 * e2 + 1] = plan.rope_frac[d0 + 2 * e2 + 1];
    }
#pragma unroll 1
    for (int bi = tid / IPB; bi < ge - gb; bi += nthr / IPB) {
      const int b = gb + bi;
      const bool vis = r < a.R && ((plan.vis[b] >> w) & 1u);
      const uint32_t delta = static_cast<uint32_t>(iq_lag - plan.off[w * a.NB + b]);
      const float sc = vis ? qsc : 0.f;
      u32x4 lo, hi;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float x0 = __uint_as_float(xw[e2] << 16), x1 = __uint_as_float(xw[e2] & 0xffff0000u);
        const float y0 = __uint_as_float(yw[e2] << 16), y1 = __uint_as_float(yw[e2] & 0xffff0000u);
        float c0, s0, c1, s1;
        rope_cos_sin_fx(delta, fr[2 * e2], &c0, &s0);
        rope_cos_sin_fx(delta, fr[2 * e2 + 1], &c1, &s1);
        lo[e2] = pack_bf16x2((x0 * c0 - y0 * s0) * sc, (x1 * c1 - y1 * s1) * sc);
        hi[e2] = pack_bf16x2((y0 * c0 + x0 * s0) * sc, (y1 * c1 + x1 * s1) * sc);
      }
      *reinterpret_cast<u32x4*>(qfs + ((bi * NT + t) * KS + sh) * 64 + ln) = lo;
      *reinterpret_cast<u32x4*>(qfs + ((bi * NT + t) * KS + sh + KS / 2) * 64 + ln) = hi;
    }
  };

  // Blocks with tiles in [lo, hi) form the index range [b_first, b_last];
  // they are rotated kQfBlocks at a time.  Within a group, a software
  // pipeline runs over this wave's tiles j, j + NWAVE, ...: the next tile's
  // keys are loaded into the key registers as soon as the current scores are
  // formed, its values into the value registers right after the P.V products,
  // so every wave keeps a tile in flight while it computes.  A later group's
  // first tile is requested before its rotation; in the first group the back
  // waves keep their speculative tile when the plan confirms it.
  uint32_t first = 0xffffffffu;  // this wave's first tile (byte offset), none: all ones
  // the first group's rotation (front waves), published to the back waves
  if (front) {
    if (plan.lo < plan.hi) {
      const int b_first = plan.b_first;
      const int b_last = plan.b_last;
      rotate_blocks(b_first, min(b_first + kQfBlocks, b_last + 1), NF);
    }
    front_sync();
    if (lane == 0)
      __hip_atomic_fetch_add(&sync_ctr[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    lds_wait_at_least(&sync_ctr[2], kFront);
  }
  if (plan.lo < plan.hi) {
    const int b_first = plan.b_first;
    const int b_last = plan.b_last;
    for (int gb = b_first; gb <= b_last; gb += kQfBlocks) {
      const int ge = min(gb + kQfBlocks, b_last + 1);
      const int t_lo = max(plan.lo, plan.tile0[gb]);
      const int t_hi = min(plan.hi, plan.tile0[ge]);
      int j = t_lo + wave;
      int bcur = gb;
      TileRef rt = {0, 0, 0, 0};
      if (j < t_hi) {
        rt = tile_ref<D>(plan, a.NB, j, bcur);
        const uint32_t tile = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(rt.base * EB));
        if (gb == b_first) first = tile;
        if (gb != b_first || front || tile != spec) {
          load_keys<D, E>(krs, tile, koff, kf);
          load_values<D, E>(vrs, tile, voff, vf);
        }
      }
      if (gb != b_first) {
        __syncthreads();  // the previous group's fragments are consumed
        rotate_blocks(gb, ge, NTHR);
        __syncthreads();
      }
      if (j < t_hi) {
        int qb = -1;
        int rowend[NT];
        const bf16x8* qf = qfs;
        for (;;) {
          if (rt.b != qb) {
            qb = rt.b;
            qf = qfs + (qb - gb) * NT * KS * 64;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const int r = 16 * t + li;
              const int w = plan.row_w[r];
              rowvis[t] = r < a.R && ((plan.vis[qb] >> w) & 1u);
              // last local position row r may see in this block (causal limit)
              rowend[t] = rowvis[t]
                              ? static_cast<int>(plan.iq[w] - plan.row_lag[r] - plan.off[w * a.NB + qb])
                              : -1;
            }
          }
          int rowlim[NT];
#pragma unroll
          for (int t = 0; t < NT; ++t) rowlim[t] = min(rt.valid - 1, rowend[t] - rt.first);
          f32x4 sc[2][NT];
          const int jn = j + NWAVE;
          if (jn >= t_hi) {
            tile_scores<D, NT, E>(kf, qf, lane, sc);
            tile_update<D, NT, E>(sc, vf, rowvis, rowlim, rt.valid, q4, acc, m_run, l_run);
            break;
          }
          const TileRef rn = tile_ref<D>(plan, a.NB, jn, bcur);
          const uint32_t tn = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(rn.base * EB));
          tile_scores<D, NT, E>(kf, qf, lane, sc);
          __builtin_amdgcn_sched_barrier(0);
          load_keys<D, E>(krs, tn, koff, kf);
          __builtin_amdgcn_sched_barrier(0);
          tile_update<D, NT, E>(sc, vf, rowvis, rowlim, rt.valid, q4, acc, m_run, l_run);
          __builtin_amdgcn_sched_barrier(0);
          load_values<D, E>(vrs, tn, voff, vf);
          __builtin_amdgcn_sched_barrier(0);
          j = jn;
          rt = rn;
        }
      }
    }
  }

  // full row sums (the four lanes of a row hold partial sums)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    l_run[t] = sum_x32(sum_x16(l_run[t]));
  }
  // Combine the waves' softmax states (O^T rows below R, m, l) in LDS.  When
  // every wave's state fits (R <= RC1 rows), each wave deposits its state in
  // its own slot as soon as its tiles are done; otherwise, after a barrier,
  // half of them at a time: the upper waves deposit, each lower wave folds in
  // its partner (same fragment positions, so lane-local), and the lower
  // waves deposit.  Then every thread combines its share of the unit's R*D
  // outputs over the deposited states and stores the partial.
  auto deposit = [&](float* buf, int rc) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int r = 16 * t + li;
      if (r >= a.R) continue;
      if (q4 == 0) {
        buf[rc * ACC_STRIDE + r] = m_run[t];
        buf[rc * ACC_STRIDE + rc + r] = l_run[t];
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
        *reinterpret_cast<f32x4*>(buf + r * ACC_STRIDE + 16 * m + 4 * q4) = acc[m][t];
    }
  };
  const int64_t pu = partial_index(a, plan);
  auto combine_store = [&](auto nstate_c, int state, int rc) {
    constexpr int NS = decltype(nstate_c)::value;
    // 8 outputs per item: R * D / 8 items (320 at 20 rows), one per thread
    for (int x = tid; x < a.R * (D / 8); x += NTHR) {
      const int r = x / (D / 8), d8 = 8 * (x - r * (D / 8));
      float mw[NS];
      float M = -INFINITY;
#pragma unroll
      for (int wv = 0; wv < NS; ++wv) {
        mw[wv] = ebuf[wv * state + rc * ACC_STRIDE + r];
        M = fmaxf(M, mw[wv]);
      }
      float L = 0.f;
      f32x4 O0 = f32x4{0.f, 0.f, 0.f, 0.f}, O1 = O0;
      if (M != -INFINITY) {
#pragma unroll
        for (int wv = 0; wv < NS; ++wv) {
          const float* src = ebuf + wv * state;
          const float sc = mw[wv] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[wv] - M);
          L += src[rc * ACC_STRIDE + rc + r] * sc;
          O0 += *reinterpret_cast<const f32x4*>(src + r * ACC_STRIDE + d8) * sc;
          O1 += *reinterpret_cast<const f32x4*>(src + r * ACC_STRIDE + d8 + 4) * sc;
        }
      }
      const int64_t pr = pu + static_cast<int64_t>(r) * a.P;
      *reinterpret_cast<f32x4*>(a.ws_acc + pr * D + d8) = O0;
      *reinterpret_cast<f32x4*>(a.ws_acc + pr * D + d8 + 4) = O1;
      if (d8 == 0) a.ws_ml[pr] = make_float2(M, L);
    }
  };
  if (a.R <= RC1) {
    deposit(ebuf + wave * kState1, RC1);
    __syncthreads();
    combine_store(std::integral_constant<int, NWAVE>{}, kState1, RC1);
  } else {
    __syncthreads();
    if (wave >= NSTATE) deposit(ebuf + (wave - NSTATE) * kState2, RP);
    __syncthreads();
    if (wave < NSTATE) {
      const float* src = ebuf + wave * kState2;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int r = 16 * t + li;
        if (r >= a.R) continue;
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
    if (wave < NSTATE) deposit(ebuf + wave * kState2, RP);
    __syncthreads();
    combine_store(std::integral_constant<int, NSTATE>{}, kState2, RP);
  }
  if (lane == 0) *hint = first;
  if (tid == 0 && plan.flags) atomicOr(a.status, plan.flags);
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
};
template <>
struct ValuTraits<uint16_t> {
  static constexpr int EPC = 8;
  __device__ static float elem(const u32x4& c, int e) {
    const uint32_t w = c[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};

// max / sum over the 32 lanes of each half of the wave (every lane gets it)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float half_max(float x) {
  x = fmaxf(x, dpp_mov<0xb1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_mov<0x4e>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_mov<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_mov<0x140>(x));  // row_mirror
  return max_x16(x);
}
__device__ __forceinline__ float half_sum(float x) {
  x += dpp_mov<0xb1>(x);
  x += dpp_mov<0x4e>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return sum_x16(x);
}

template <typename T, int D, int RG>
__global__ __launch_bounds__(kThreads) void decode_valu(DecodeArgs a) {
  constexpr int NTHR = kThreads, NWAVE = kWaves;
  constexpr int EPC = ValuTraits<T>::EPC;
  constexpr int KC = D / EPC;     // key chunks per token
  constexpr int DPL = D / 64;     // output dims per lane
  constexpr int RM = 2 * RG;      // rows held
  constexpr int PS = 36;          // P row stride (floats), keeps float4 reads aligned
  constexpr int kPWave = RM * PS + RM;  // one wave's P and rescale factors
  constexpr int ACC_STRIDE = D + 4;
  constexpr int kState = RM * ACC_STRIDE + 2 * RM;
  constexpr int kQBlock = RM * D;      // rotated queries of one block (floats)
  constexpr int kQfFloats = 40960 / 4;  // 40 KB of rotated queries per group
  constexpr int kQfBlocks = kQfFloats / kQBlock > 0 ? kQfFloats / kQBlock : 1;
  constexpr int kUnion = cmax(kQfBlocks * kQBlock, 2 * kState);
  __shared__ Plan plan;
  __shared__ __attribute__((aligned(16))) float qs[RM * D];  // raw query rows
  // rotated queries during the loop; the waves' softmax states at the end
  __shared__ __attribute__((aligned(16))) float ubuf[kUnion];
  __shared__ __attribute__((aligned(16))) float pbuf_all[NWAVE * kPWave];  // P, rescale factors

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int tl = lane & 31, rg = lane >> 5;
  {
    int h0, u0;
    plan_head_unit(a, &h0, &u0);
    constexpr int kQVec = RM * D / 4;  // float4 of staged query
    constexpr int kQRegs = (kQVec + NTHR - 1) / NTHR;
    float4 qv[kQRegs];
    const T* qg = static_cast<const T*>(a.q);
    auto issue = [&] {
#pragma unroll
      for (int k = 0; k < kQRegs; ++k) {
        const int x = tid + k * NTHR;
        const int r = (4 * x) / D, d = 4 * x - r * D;
        qv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (x < kQVec && r < a.R) {
          const int w = fast_div(r, a.mG), h = h0 * a.G + (r - w * a.G);
          const T* src = qg + (static_cast<int64_t>(w) * a.Hq + h) * D + d;
          qv[k] = make_float4(load_elem(src, 0), load_elem(src, 1), load_elem(src, 2),
                              load_elem(src, 3));
        }
      }
    };
    auto commit = [&] {
#pragma unroll
      for (int k = 0; k < kQRegs; ++k) {
        const int x = tid + k * NTHR;
        if (x < kQVec) *reinterpret_cast<float4*>(qs + 4 * x) = qv[k];
      }
    };
    build_plan<NTHR>(a, plan, issue, commit);
  }
  const int g = plan.head;
  const __amdgpu_buffer_rsrc_t krs =
      plane_rsrc(static_cast<const T*>(a.k) + static_cast<int64_t>(g) * a.plane_elems, a.plane_bytes);
  const __amdgpu_buffer_rsrc_t vrs =
      plane_rsrc(static_cast<const T*>(a.v) + static_cast<int64_t>(g) * a.plane_elems, a.plane_bytes);
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

  // (a2) rotated, scaled queries of blocks gb..ge-1: qr[(b-gb)*RM*D + r*D + d]
  auto rotate_blocks = [&](int gb, int ge) {
    const int half = D / 2;
    const int items = (ge - gb) * RM * half;
    for (int x = tid; x < items; x += NTHR) {
      const int i = x % half;
      const int r = (x / half) % RM;
      const int bi = x / (half * RM);
      const int b = gb + bi;
      const int w = plan.row_w[r];
      const bool vis = r < a.R && ((plan.vis[b] >> w) & 1u);
      float c = 0.f, s = 0.f;
      if (vis) rope_cos_sin(plan.iq[w] - plan.row_lag[r] - plan.off[w * a.NB + b], plan.invf[i], &c, &s);
      const float x0 = qs[r * D + i], x1 = qs[r * D + i + half];
      float* dst = ubuf + bi * kQBlock + r * D;
      dst[i] = vis ? (x0 * c - x1 * s) * a.qscale : 0.f;
      dst[i + half] = vis ? (x1 * c + x0 * s) * a.qscale : 0.f;
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

  // last local position of block b that row rg*RG+i may see (-1: none)
  auto row_ends = [&](int b, int (&rowend)[RG]) {
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int r = rg * RG + i;
      const int w = plan.row_w[r];
      const bool vis = r < a.R && ((plan.vis[b] >> w) & 1u);
      rowend[i] = vis ? static_cast<int>(plan.iq[w] - plan.row_lag[r] - plan.off[w * a.NB + b]) : -1;
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

  if (plan.lo < plan.hi) {
    const int bq = kQfBlocks;
    const int b_first = plan.b_first;
    const int b_last = plan.b_last;
    for (int gb = b_first; gb <= b_last; gb += bq) {
      const int ge = min(gb + bq, b_last + 1);
      const int t_lo = max(plan.lo, plan.tile0[gb]);
      const int t_hi = min(plan.hi, plan.tile0[ge]);
      int j = t_lo + wave;
      int bcur = gb;
      TileRef rt = {0, 0, 0, 0};
      u32x4 kc[KC], vc[DPL][4][VC];
      if (j < t_hi) {
        rt = tile_ref<D>(plan, a.NB, j, bcur);
        const uint32_t tile =
            __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(rt.base * sizeof(T)));
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
          if (jn >= t_hi) {
            compute(kc, vc, qblk, rowend, rt.valid, rt.first);
            break;
          }
          const TileRef rn = tile_ref<D>(plan, a.NB, jn, bcur);
          const uint32_t tn =
              __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(rn.base * sizeof(T)));
          compute(kc, vc, qblk, rowend, rt.valid, rt.first);
          load_k(tn, kc);
          load_v(tn, vc);
          j = jn;
          rt = rn;
        }
      }
    }
  }

  // ---- combine the waves' states (two at a time) and store the partial
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
      float mo = -INFINITY, lo = 0.f;
#pragma unroll
      for (int k = 0; k < RG; ++k)
        if (k == r % RG) {
          mo = m_run[k];
          lo = l_run[k];
        }
      // lanes of the other half hold another row: take row r's from lane (r/RG)*32
      mo = __shfl(mo, (r / RG) * 32);
      lo = __shfl(lo, (r / RG) * 32);
      const float m2 = src[RM * ACC_STRIDE + r];
      const float l2 = src[RM * ACC_STRIDE + RM + r];
      const float M = fmaxf(mo, m2);
      const float s1 = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - M);
      const float s2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd)
        acc[r][dd] = acc[r][dd] * s1 + src[r * ACC_STRIDE + DPL * lane + dd] * s2;
      // the merged (m, l) go back to the row group's registers
      const float lm = lo * s1 + l2 * s2;
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
  const int64_t pu = partial_index(a, plan);
  for (int x = tid; x < a.R * (D / 4); x += NTHR) {
    const int r = x / (D / 4), d4 = 4 * (x - r * (D / 4));
    const float m0 = ubuf[RM * ACC_STRIDE + r], m1 = ubuf[kState + RM * ACC_STRIDE + r];
    const float M = fmaxf(m0, m1);
    float L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < 2; ++wv) {
        const float* src = ubuf + wv * kState;
        const float mw = wv ? m1 : m0;
        const float sc = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L += src[RM * ACC_STRIDE + RM + r] * sc;
        const float4 v = *reinterpret_cast<const float4*>(src + r * ACC_STRIDE + d4);
        O.x += v.x * sc;
        O.y += v.y * sc;
        O.z += v.z * sc;
        O.w += v.w * sc;
      }
    }
    const int64_t pr = pu + static_cast<int64_t>(r) * a.P;
    *reinterpret_cast<float4*>(a.ws_acc + pr * D + d4) = O;
    if (d4 == 0) a.ws_ml[pr] = make_float2(M, L);
  }
  if (tid == 0 && plan.flags) atomicOr(a.status, plan.flags);
}

// ----------------------------------------------------------- merge kernel
// (a4) One workgroup per (kv head g, row r), one thread per output dim:
// out = sum_u acc_u 2^(m_u - M) / L with M = max_u m_u and
// L = sum_u l_u 2^(m_u - M), units in fixed order.  Units are taken
// kMergeChunk at a time: lane k of every wave loads unit u0+k's (m, l) and
// forms its weight, which the lanes read back with readlane while summing
// their accumulators, so the kernel has neither LDS nor barriers; the
// running (M, L, sum) is rescaled when a later chunk raises M.
constexpr int kMergeChunk = 32;  // units whose loads are in flight together

// Lane k's value of x (the builtin moves 32-bit integers: pass the bits).
__device__ __forceinline__ float readlane_f32(float x, int k) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), k));
}

template <int D>
__global__ __launch_bounds__(D) void merge_kernel(DecodeArgs a) {
  // every scalar argument, requested at entry in one round trip
  asm volatile("" ::"s"(a.ws_ml), "s"(a.ws_acc), "s"(a.out), "s"(a.status), "s"(a.R), "s"(a.P),
               "s"(a.G), "s"(a.Hq), "s"(a.dtype), "s"(a.mR), "s"(a.mG));
  const int tid = threadIdx.x;  // output dim
  const int lane = tid & 63;
  const int g = fast_div(blockIdx.x, a.mR);
  const int r = blockIdx.x - g * a.R;
  const int P = a.P;
  // FP8 pools: values are code * scale of the kv head (requested early)
  const float vsc = a.dtype == HW_FP8
                        ? reinterpret_cast<const float*>(reinterpret_cast<const char*>(&a.tab) +
                                                         offsetof(DecodeTables, v_scale))[g]
                        : 1.f;
  // this (kv head, row)'s partials as buffers over its P units: unit u's
  // accumulators at byte u * D * 4, its (m, l) at byte u * 8.  Units past the
  // last lie outside the buffers, read as zero and get zero weight.
  const int64_t row0 = (static_cast<int64_t>(g) * a.R + r) * P;
  const __amdgpu_buffer_rsrc_t accrs = __builtin_amdgcn_make_buffer_rsrc(
      a.ws_acc + row0 * D, static_cast<short>(0), P * D * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t mlrs = __builtin_amdgcn_make_buffer_rsrc(
      a.ws_ml + row0, static_cast<short>(0), P * 8, 0x00020000);
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
  const int w = fast_div(r, a.mG), h = g * a.G + (r - w * a.G);
  const float o = L > 0.f ? s / L * vsc : 0.f;
  a.out[(static_cast<int64_t>(w) * a.Hq + h) * D + tid] = o;
  if (tid == 0 && !(L > 0.f)) atomicOr(a.status, HW_DEV_NO_TOKENS);
}

template <typename K>
int occupancy(K kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess) return 0;
  return n;
}

}  // namespace

template <typename T, int D>
hipError_t launch_valu_rows(const DecodeArgs& a, int grid, hipStream_t s) {
  if (a.R <= 8)
    hipLaunchKernelGGL((decode_valu<T, D, 4>), dim3(grid), dim3(kThreads), 0, s, a);
  else if (a.R <= 16)
    hipLaunchKernelGGL((decode_valu<T, D, 8>), dim3(grid), dim3(kThreads), 0, s, a);
  else if (a.R <= 20)
    hipLaunchKernelGGL((decode_valu<T, D, 10>), dim3(grid), dim3(kThreads), 0, s, a);
  else if (a.R <= 32)
    hipLaunchKernelGGL((decode_valu<T, D, 16>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((decode_valu<T, D, 32>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_valu(const DecodeArgs& a, int grid, hipStream_t s) {
  if ((a.D != 64 && a.D != 128) || a.R > HW_MAX_ROWS || a.dtype == HW_FP8)
    return hipErrorInvalidValue;
  if (a.dtype == HW_F32)
    return a.D == 128 ? launch_valu_rows<float, 128>(a, grid, s) : launch_valu_rows<float, 64>(a, grid, s);
  return a.D == 128 ? launch_valu_rows<uint16_t, 128>(a, grid, s)
                    : launch_valu_rows<uint16_t, 64>(a, grid, s);
}

template <typename E>
hipError_t launch_mfma_elem(const DecodeArgs& a, int grid, hipStream_t s) {
  if (a.D == 128) {
    if (a.R <= 16)
      hipLaunchKernelGGL((decode_mfma<128, 1, E>), dim3(grid), dim3(kMfmaThreads), 0, s, a);
    else
      hipLaunchKernelGGL((decode_mfma<128, 2, E>), dim3(grid), dim3(kMfmaThreads), 0, s, a);
  } else if (a.D == 64) {
    if (a.R <= 16)
      hipLaunchKernelGGL((decode_mfma<64, 1, E>), dim3(grid), dim3(kMfmaThreads), 0, s, a);
    else
      hipLaunchKernelGGL((decode_mfma<64, 2, E>), dim3(grid), dim3(kMfmaThreads), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int grid, hipStream_t s) {
  if (a.R > 32) return hipErrorInvalidValue;
  if (a.dtype == HW_BF16) return launch_mfma_elem<uint16_t>(a, grid, s);
  if (a.dtype == HW_FP8) return launch_mfma_elem<uint8_t>(a, grid, s);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
  if (a.P > kMaxUnits || (a.D != 64 && a.D != 128)) return hipErrorInvalidValue;
  if (a.D == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(a.Hkv * a.R), dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3(a.Hkv * a.R), dim3(64), 0, s, a);
  return hipGetLastError();
}

// Resident workgroups per CU of the kernel a launch would use (0 on error).
template <typename E>
int mfma_blocks_per_cu(int D, int rows) {
  const int t = kMfmaThreads;
  if (D == 128)
    return rows <= 16 ? occupancy(decode_mfma<128, 1, E>, t) : occupancy(decode_mfma<128, 2, E>, t);
  return rows <= 16 ? occupancy(decode_mfma<64, 1, E>, t) : occupancy(decode_mfma<64, 2, E>, t);
}

int decode_blocks_per_cu(int path, int dtype, int D, int rows) {
  if (path == 2)
    return dtype == HW_FP8 ? mfma_blocks_per_cu<uint8_t>(D, rows)
                           : mfma_blocks_per_cu<uint16_t>(D, rows);
  return dtype == HW_F32 ? occupancy(decode_valu<float, 128, 10>, kThreads)
                         : occupancy(decode_valu<uint16_t, 128, 10>, kThreads);
}

}  // namespace hw
