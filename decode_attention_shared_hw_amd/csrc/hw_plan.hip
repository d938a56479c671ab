// hw_plan.hip — the plan of a decode call: everything that depends on the
// views and the block lengths but not on the layer (Hogwild! Inference notes,
// key design 1: each block is scored with the query rotated by i_q minus the
// block's start in the worker's view; key design 2: the combined layout's
// blocks are shared by every worker).  One workgroup builds it; every layer's
// run kernel of the step reads it.
#include "hw_internal.h"

namespace hw {
namespace {

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

constexpr int kPlanThreads = 256;

// Steps:
//  1. lengths: a length outside [0, capacity] is reported (HW_DEV_BAD_LENGTH)
//     and taken as 0; table entries: a worker whose entry count is out of
//     range, or whose table lists a block id out of range or one block twice,
//     is malformed (HW_DEV_BAD_ENTRY) and sees nothing.
//  2. i_q[w] = max over w's listed blocks with tokens of view_offset + len - 1
//     (the query's own K/V is the last token of its view); a worker for whom
//     some listed block's delta i_q - view_offset reaches 2^31 is malformed.
//  3. visible blocks: length > 0 and listed by a valid worker, in block-id
//     order, with their tiles.
//  4. units: the tiles are split into P contiguous ranges by cost, a tile
//     costing 1 and each visible block after the first kBlockCost more (a
//     unit reaching another block rotates that block's queries first).
//  5. row ends: query row i = w * nq + j sits lag = nq - 1 - j positions
//     before i_q[w]; for visible block b its row end is
//     i_q[w] - lag - view_offset[w][b] when w lists b and that is >= 0, else -1.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ uint32_t vis[HW_MAX_BLOCKS];  // bit w: worker w lists block b
  __shared__ int32_t off[HW_MAX_WORKERS * HW_MAX_BLOCKS];
  __shared__ int32_t len[HW_MAX_BLOCKS];
  __shared__ long long iq[HW_MAX_WORKERS];
  __shared__ int32_t vb_block[HW_MAX_BLOCKS], vb_cs[HW_MAX_BLOCKS], vb_tiles[HW_MAX_BLOCKS];
  __shared__ uint32_t bad;
  __shared__ int32_t flags, nvb_s, C_s;
  const int tid = threadIdx.x;
  const int W = a.W, NB = a.NB, E = a.E;
  int32_t* plan = a.plan;

  int raw = 0;
  if (tid < NB) raw = a.block_len[tid];
  if (tid < HW_MAX_BLOCKS) vis[tid] = 0u;
  for (int i = tid; i < W * NB; i += kPlanThreads) off[i] = 0;
  if (tid == 0) {
    bad = 0u;
    flags = 0;
  }
  __syncthreads();
  // ---- 1. lengths and table entries
  if (tid < HW_MAX_BLOCKS) {
    int l = 0;
    if (tid < NB) {
      l = raw;
      if (l < 0 || l > a.block_cap[tid]) {
        atomicOr(&flags, HW_DEV_BAD_LENGTH);
        l = 0;
      }
    }
    len[tid] = l;
    plan[kPlanLens + tid] = tid < NB ? raw : 0;
  }
  for (int i = tid; i < W * E; i += kPlanThreads) {
    const int w = i / E, slot = i - w * E;
    const uint32_t bit = 1u << w;
    const int ne = a.num_entries[w];
    if (ne < 0 || ne > E) {
      atomicOr(&bad, bit);
      continue;
    }
    if (slot >= ne) continue;
    const hw_entry e = a.tables[i];
    if (e.block_id < 0 || e.block_id >= NB) {
      atomicOr(&bad, bit);
      continue;
    }
    if (atomicOr(&vis[e.block_id], bit) & bit) atomicOr(&bad, bit);
    off[w * NB + e.block_id] = e.view_offset;
  }
  __syncthreads();
  // ---- 2. query positions
  if (tid < W) {
    const int w = tid;
    long long m = -1;
    for (int b = 0; b < NB; ++b)
      if (((vis[b] >> w) & 1u) && len[b] > 0)
        m = max(m, static_cast<long long>(off[w * NB + b]) + len[b] - 1);
    iq[w] = m;
    for (int b = 0; b < NB; ++b)
      if (((vis[b] >> w) & 1u) && len[b] > 0 && m - off[w * NB + b] >= (1ll << 31))
        atomicOr(&bad, 1u << w);
  }
  __syncthreads();
  // ---- 3. visible blocks (wave 0, lane b = block b)
  if (tid < 64) {
    const int b = tid;
    const uint32_t v = b < NB ? (vis[b] & ~bad) : 0u;
    const bool visible = v != 0u && len[b] > 0;
    const int tiles = visible ? (len[b] + kTile - 1) / kTile : 0;
    const uint64_t mask = __ballot(visible);
    const int idx = __builtin_popcountll(mask & ((1ull << b) - 1ull));
    const int incl = wave_inclusive_scan(tiles);
    const int cost = tiles + ((visible && idx > 0) ? kBlockCost : 0);
    const int cincl = wave_inclusive_scan(cost);
    const int nvb = __builtin_popcountll(mask);
    if (visible) {
      vb_block[idx] = b;
      vb_cs[idx] = cincl - tiles;  // cost position of the block's first tile
      vb_tiles[idx] = tiles;
      plan[kPlanVbBlock + idx] = b;
      plan[kPlanVbLen + idx] = len[b];
      plan[kPlanVbTile0 + idx] = incl - tiles;
      plan[kPlanVbStart + idx] = a.block_start[b];
    }
    // unused entries zeroed (the run kernels copy the whole region)
    if (b >= nvb) {
      plan[kPlanVbBlock + b] = 0;
      plan[kPlanVbLen + b] = 0;
      plan[kPlanVbTile0 + b + 1] = 0;
      plan[kPlanVbStart + b] = 0;
    }
    if (b == 0) {
      plan[kPlanVbTile0 + nvb] = __builtin_amdgcn_readlane(incl, 63);
      nvb_s = nvb;
      C_s = __builtin_amdgcn_readlane(cincl, 63);
    }
    const int ntiles = __builtin_amdgcn_readlane(incl, 63);
    if (b == 0) {
      plan[kHdrMagic] = kPlanMagic;
      plan[kHdrNvb] = nvb;
      plan[kHdrTiles] = ntiles;
      plan[kHdrP] = a.P;
      plan[kHdrQrows] = W * a.nq;
      plan[kHdrNB] = NB;
      plan[kHdrR] = W * a.nq * a.G;
    }
    if (b >= 8 && b < 16) plan[b] = 0;
  }
  __syncthreads();
  const int nvb = nvb_s;
  // ---- 4. unit boundaries: unit u starts at cost position floor(C u / P),
  // i.e. at tile sum_j clamp(x - cs_j, 0, tiles_j)
  for (int u = tid; u <= a.P; u += kPlanThreads) {
    const long long x = static_cast<long long>(C_s) * u / a.P;
    int t = 0;
    for (int j = 0; j < nvb; ++j) {
      const long long d = x - vb_cs[j];
      t += static_cast<int>(d < 0 ? 0 : (d > vb_tiles[j] ? vb_tiles[j] : d));
    }
    plan[kPlanUnit + u] = t;
  }
  // ---- 5. row ends
  const int qrows = W * a.nq;
  for (int i = tid; i < NB * qrows; i += kPlanThreads) {
    const int j = i / qrows, qr = i - j * qrows;
    int re = -1;
    if (j < nvb) {
      const int w = qr / a.nq;
      const int lag = a.nq - 1 - (qr - w * a.nq);
      const int b = vb_block[j];
      if (!((bad >> w) & 1u) && ((vis[b] >> w) & 1u)) {
        const long long d = iq[w] - lag - off[w * NB + b];
        if (d >= 0) re = static_cast<int>(d);
      }
    }
    plan[kPlanRows + i] = re;
  }
  if (tid == 0) {
    int f = flags;
    if (bad) f |= HW_DEV_BAD_ENTRY;
    plan[kHdrFlags] = f;
    if (f) atomicOr(a.status, f);
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hw
