// hw_fused.hip — the split launch of decode calls of up to 32 stacked rows on
// bf16 and FP8 pools (hw_attn_decode, hw_attn_chunk): the same attention as the
// plan + run kernels (hw_plan.hip, hw_decode.hip), with the plan built inside
// every workgroup from the call's tables instead of read from a plan buffer.
//
// One workgroup per work unit (kv head, unit), 8 waves:
//  1. the front waves (0-3) load the tables, the block lengths and the head's
//     query rows in one round trip and build the plan in LDS: visible blocks,
//     each worker's query position i_q and view offsets, the unit's tile range
//     (Hogwild! notes, key design 2: the cache is shared, each worker sees the
//     blocks its table lists at its own offsets);
//     the back waves (4-7) meanwhile request the first tile they took in the
//     previous call with this workspace (a hint: within a decode step every
//     layer's call has the same plan), through range-checked offsets, and keep
//     it when the plan confirms it;
//  2. all eight waves rotate the stacked query rows of each visible block by
//     their delta i_q - lag - view_offset once the plan is complete (key
//     design 1: only the queries are rotated, never the cache)          [a2]
//  3. every wave streams its tiles (every 8th tile of the unit's range) with an
//     online softmax in the exp2 domain (split-K / Flash-Decoding)      [a3]
//  4. the waves' states are combined in LDS and the unit's partial (m, l, acc)
//     is stored; merge_kernel (hw_decode.hip) combines the units      [a4].
//
// A/B on the QwQ-32B-shaped step (4 workers, 16K common block, 64 layers): the
// per-call plan built here costs less end to end than reading the plan that
// hw_attn_plan wrote once per step (18.3 vs 19.9 us per call), so decode calls
// of up to 32 rows take this kernel.
#include <math.h>

#include <type_traits>

#include "hw_internal.h"
#include "hw_kernels.h"

namespace hw {
namespace {

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
        if (w < a.W)  // (always, unless a wait gave up and the mask is half built)
          atomicMax(&p.iq[w], static_cast<long long>(p.off[w * a.NB + b]) + len - 1);
      }
    }
  }
  sync();
}

// Waves of one workgroup that synchronize through a counter in LDS instead of
// s_barrier, so that the other waves of the workgroup never have to join:
// each wave's LDS writes complete (release fence on LDS), lane 0 adds one,
// and the wave waits until the counter reaches count * phase.  The counter
// only grows; it must be zero before the first phase.  Every wave of the
// group reaches every phase (no early exits), so every wait ends.
//
// Every wait between waves is bounded: after `limit` polls (the argument
// spin_limit, 2^22 by default: about 0.25 s, against microseconds for any
// wait of a healthy launch) the wave stops waiting and sets HW_DEV_SPIN_LIMIT
// in the plan's flags.  A wave uses the plan only after a wait that either
// succeeded (and so is ordered after any bit set before the waited-for
// arrivals) or set the bit itself, and checks the bit first: an aborted workgroup
// loads no tile through a plan offset, stores its partial from its own
// (head, unit) and reports HW_DEV_SPIN_LIMIT, so a lost arrival ends the
// launch with a flagged wrong result instead of a hang or a stray access.
struct LdsWaveBarrier {
  uint32_t* ctr;
  uint32_t count;
  uint32_t phase;
  int32_t* flags;  // the plan's HW_DEV_* bits (HW_DEV_SPIN_LIMIT when a wait gives up)
  uint32_t limit;
  __device__ void operator()() {
    ++phase;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if ((threadIdx.x & 63) == 0)
      __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    uint32_t left = limit;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < count * phase) {
      if (left-- == 0u) {
        __hip_atomic_fetch_or(flags, HW_DEV_SPIN_LIMIT, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }
};

// Waits until an LDS counter that other waves advance reaches `target`, at
// most `limit` polls (then records HW_DEV_SPIN_LIMIT, as above).
__device__ __forceinline__ void lds_wait_at_least(uint32_t* ctr, uint32_t target, int32_t* flags,
                                                  uint32_t limit) {
  uint32_t left = limit;
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
    if (left-- == 0u) {
      __hip_atomic_fetch_or(flags, HW_DEV_SPIN_LIMIT, __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_WORKGROUP);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Block holding global tile j of the plan (cursor walks forward).
__device__ __forceinline__ int block_of_tile(const Plan& p, int nb, int j, int b) {
  while (b + 1 < nb && p.tile0[b + 1] <= j) ++b;
  return b;
}

// Per-unit partial: (m, l) per row and the unnormalised accumulator.
// ------------------------------------------------------------- MFMA kernel
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

constexpr int kOneLevelRows = 24;  // rows up to which every wave's state has its own LDS slot

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
  // the head's query rows, row stride D + 8: the rotation reads one column of
  // 16 rows at a time, which then falls into distinct LDS banks
  constexpr int QS = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t qs[RP * QS];
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
  if (tid == 0) HW_STAMP(0);
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
  // (with the plan's flags, in one store: zeroed before the barrier that every
  // wave passes once, so a wave that gives up a later wait records
  // HW_DEV_SPIN_LIMIT there)
  if (tid < 4) *(tid < 3 ? &sync_ctr[tid] : reinterpret_cast<uint32_t*>(&plan.flags)) = 0u;
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
    krs = make_rsrc(static_cast<const char*>(a.k) + static_cast<int64_t>(h0) * a.plane_elems * EB,
                     a.plane_bytes);
    vrs = make_rsrc(static_cast<const char*>(a.v) + static_cast<int64_t>(h0) * a.plane_elems * EB,
                     a.plane_bytes);
    qsc = a.qscale;
    if (EB == 1) qsc *= reinterpret_cast<const float*>(reinterpret_cast<const char*>(&a.tab) +
                                                       offsetof(DecodeTables, k_scale))[h0];
    hint = a.ws_hint + (static_cast<int64_t>(h0) * a.P + u0) * NWAVE + wave_u;
  };
  uint32_t spec = 0xffffffffu;  // back waves: the hinted first tile
  Frag kf[2][KS], vf[MT];
  LdsWaveBarrier front_sync{&sync_ctr[0], kFront, 0u, &plan.flags, a.spin_limit};
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
        if (x < kQVec) *reinterpret_cast<u32x4*>(qs + (8 * x) / D * QS + (8 * x) % D) = qv[k];
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
    lds_wait_at_least(&sync_ctr[1], kFront, &plan.flags, a.spin_limit);
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
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(qs + r * QS + d0);
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
  // the first group's rotation by all eight waves once the plan is complete
  // (build_plan ends with the front waves' barrier): the front waves publish
  // it, the back waves (their speculative tiles requested) wait for it
  if (front) {
    if (lane == 0)
      __hip_atomic_fetch_add(&sync_ctr[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    lds_wait_at_least(&sync_ctr[2], kFront, &plan.flags, a.spin_limit);
  }
  if (plan.lo < plan.hi && !(plan.flags & HW_DEV_SPIN_LIMIT)) {
    const int b_first = plan.b_first;
    const int b_last = plan.b_last;
    rotate_blocks(b_first, min(b_first + kQfBlocks, b_last + 1), NTHR);
  }
  __syncthreads();  // the rotated queries are in LDS
  if (plan.lo < plan.hi && !(plan.flags & HW_DEV_SPIN_LIMIT)) {
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
  const int64_t pu = static_cast<int64_t>(h0) * a.R * a.P + u0;  // (not from the plan)
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
  if (lane == 0) HW_STAMP(16 + wave);
}


template <typename K>
int occupancy(K kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess) return 0;
  return n;
}

template <int D, typename E>
hipError_t launch_fused_d(const DecodeArgs& a, int grid, hipStream_t s) {
  if (a.R <= 16)
    hipLaunchKernelGGL((decode_mfma<D, 1, E>), dim3(grid), dim3(kMfmaThreads), 0, s, a);
  else
    hipLaunchKernelGGL((decode_mfma<D, 2, E>), dim3(grid), dim3(kMfmaThreads), 0, s, a);
  return hipGetLastError();
}

template <typename E>
int fused_occ(int D, int rows) {
  const int t = kMfmaThreads;
  if (D == 128)
    return rows <= 16 ? occupancy(decode_mfma<128, 1, E>, t) : occupancy(decode_mfma<128, 2, E>, t);
  return rows <= 16 ? occupancy(decode_mfma<64, 1, E>, t) : occupancy(decode_mfma<64, 2, E>, t);
}

}  // namespace

hipError_t launch_fused_mfma(const DecodeArgs& a, int grid, hipStream_t s) {
  if (a.R < 1 || a.R > kFusedMaxRows || (a.D != 64 && a.D != 128)) return hipErrorInvalidValue;
  if (a.dtype == HW_BF16)
    return a.D == 128 ? launch_fused_d<128, uint16_t>(a, grid, s) : launch_fused_d<64, uint16_t>(a, grid, s);
  if (a.dtype == HW_FP8)
    return a.D == 128 ? launch_fused_d<128, uint8_t>(a, grid, s) : launch_fused_d<64, uint8_t>(a, grid, s);
  return hipErrorInvalidValue;
}

int fused_blocks_per_cu(int dtype, int D, int rows) {
  return dtype == HW_FP8 ? fused_occ<uint8_t>(D, rows) : fused_occ<uint16_t>(D, rows);
}

}  // namespace hw
