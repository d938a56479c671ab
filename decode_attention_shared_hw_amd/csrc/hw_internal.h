// hw_internal.h — shared definitions of libhogwild_attn's HIP sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hogwild_attn.h"

namespace hw {

constexpr int kTile = HW_TILE_TOKENS;  // tokens per pool tile
constexpr int kThreads = 256;          // threads per VALU decode workgroup (4 waves)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxHalf = 64;           // head_dim / 2 upper bound
constexpr int kMaxUnits = 256;         // split-K work units per kv head
constexpr int kBlockCost = 5;          // extra cost, in tiles, of each visible block after the first
constexpr int kValuMaxRows = 64;       // stacked rows of the VALU kernel
constexpr int kMfmaMaxRows = 80;       // stacked rows of the MFMA kernel (HW_MAX_ROWS)

// Element offset of key (slot, d) inside one (layer, kv head) plane.  Tiles of
// 32 slots; inside a tile: [half t/16][chunk d/8][token t%16][d%8].
__host__ __device__ inline int64_t key_offset(int64_t slot, int d, int D) {
  const int64_t tile = slot >> 5;
  const int t = static_cast<int>(slot & 31);
  return tile * 32 * D + (t >> 4) * 16 * D + (d >> 3) * 128 + (t & 15) * 8 + (d & 7);
}

// Element offset of value (slot, d): [group (t%16)/4][d][8 tokens], token
// order inside a group (t/16)*4 + t%4.
__host__ __device__ inline int64_t value_offset(int64_t slot, int d, int D) {
  const int64_t tile = slot >> 5;
  const int t = static_cast<int>(slot & 31);
  return tile * 32 * D + ((t & 15) >> 2) * 8 * D + d * 8 + ((t >> 4) << 2) + (t & 3);
}

// x / d for 0 <= x < 2^16 and 1 <= d <= 256 with one multiply: the host
// passes m = div_magic(d) = ceil(2^24 / d), and (x * 2^8 * m) >> 32 equals
// floor(x / d) over that whole range (checked exhaustively).
inline uint32_t div_magic(uint32_t d) { return ((1u << 24) + d - 1u) / d; }
__device__ __forceinline__ int fast_div(int x, uint32_t m) {
  return static_cast<int>(__umulhi(static_cast<uint32_t>(x) << 8, m));
}

// Bytes per stored element of a pool type.
__host__ __device__ inline int elem_bytes(int dtype) {
  return dtype == HW_F32 ? 4 : (dtype == HW_BF16 ? 2 : 1);
}

// ------------------------------------------------------------------ plan
// A plan is the part of a decode call that depends only on the views (tables,
// entry counts) and the block lengths, not on the layer: which blocks are
// visible, how their tiles are split into work units, and, for every visible
// block and query row, the row's position delta.  Within one decode step all
// layers share it, so it is built once (plan_kernel) and read by every layer's
// call.  Layout (int32 words):
constexpr int kPlanMagic = 0x48575031;  // "HWP1"
constexpr int kPlanHdr = 0;        // [16] header, fields below
constexpr int kHdrMagic = 0;       //   kPlanMagic
constexpr int kHdrFlags = 1;       //   HW_DEV_* bits the plan found
constexpr int kHdrNvb = 2;         //   visible blocks (length > 0, seen by a valid worker)
constexpr int kHdrTiles = 3;       //   their tiles
constexpr int kHdrP = 4;           //   work units per kv head
constexpr int kHdrQrows = 5;       //   query rows (workers * query tokens)
constexpr int kHdrNB = 6;          //   pool blocks
constexpr int kHdrR = 7;           //   stacked rows per kv head (query rows * G)
constexpr int kPlanVbBlock = 16;   // [64] block id of visible block j, in block-id order
constexpr int kPlanVbLen = 80;     // [64] its length
constexpr int kPlanVbTile0 = 144;  // [65] first tile of visible block j; [nvb] = tiles
constexpr int kPlanVbStart = 212;  // [64] its first slot (a plane holds < 2^31 bytes)
constexpr int kPlanLens = 276;     // [64] every block's length as the plan read it
constexpr int kPlanLdsWords = 340; // words [0, 340) are copied to LDS by the run kernels
constexpr int kPlanUnit = 340;     // [kMaxUnits + 1] first tile of each unit
constexpr int kPlanRows = 600;     // [NB][qrows] row end of visible block j, query row i
// Row end: the last local position of the block that the query row sees
// (i_q - lag - view_offset, clipped to the block by the tile masks), -1 when
// it sees none.  When >= 0 it is also the rotation delta of the row's query
// for that block (key design 1: rho(q, i_q - i_k)).
inline int plan_words(int num_blocks, int qrows) { return kPlanRows + num_blocks * qrows; }

struct alignas(16) PlanArgs {
  const hw_entry* tables;     // [W][E]
  const int32_t* num_entries; // [W]
  const int32_t* block_len;   // [NB]
  int32_t* status;
  int32_t* plan;
  int32_t W, nq, G, E, NB, P;
  int32_t block_start[HW_MAX_BLOCKS];
  int32_t block_cap[HW_MAX_BLOCKS];
};

// ------------------------------------------------------------------ run
// Workspace of a run (device, caller-owned), in this order:
//   sync    [Hkv][kSyncStride] uint32: word 0 is each kv head's tile counter
//           of the balanced split; zero before first use, every call leaves
//           it zero (the merge launch resets it)
//   plan    the plan of hw_attn_decode / hw_attn_chunk
//   ml      [Hkv][R][P] (m, l) float pairs of the units' partial states
//   acc     [Hkv][R][P][D] float accumulators
//   cnt     [Hkv][P] int32 tiles each unit processed (checked by the merge)
constexpr int kSyncStride = 16;           // words per kv head (one 64-byte line)
constexpr int kMaxSyncHeads = 256;        // kv heads covered by the sync region
constexpr size_t kSyncBytes = static_cast<size_t>(kMaxSyncHeads) * kSyncStride * 4;

struct alignas(16) RunArgs {
  const void* q;             // [qrows][Hq][D] (fp32 pools fp32, else bf16)
  const void* k;             // plane (layer, kv head 0)
  const void* v;
  const int32_t* plan;
  const int32_t* block_len;  // [NB]: checked against the plan's copy
  float* out;                // [qrows][Hq][D] fp32
  int32_t* status;
  uint32_t* sync;            // [Hkv][kSyncStride]
  float2* ws_ml;             // [Hkv][R][P]
  float* ws_acc;             // [Hkv][R][P][D]
  int32_t* ws_cnt;           // [Hkv][P]
  int64_t plane_elems;       // num_slots * D
  int32_t plane_bytes;       // plane_elems * element size (< 2^31)
  int32_t Hq, Hkv, G, R, qrows, NB, P, D;
  uint32_t mG, mHkv, mR, mP; // div_magic of G, Hkv, R and P
  int32_t balance;           // 1: tiles after the first per wave from the head's counter
  int32_t dtype;             // HW_F32 / HW_BF16 / HW_FP8
  float qscale;              // log2(e) / sqrt(D): scores in the exp2 domain
  uint64_t rope_frac[kMaxHalf];  // frac(theta^(-2i/D) / (2 pi)) * 2^64, i < D/2
  double inv_freq[kMaxHalf];     // theta^(-2i/D)
  float k_scale[HW_MAX_FP8_KV_HEADS];  // FP8 pools: this layer's scales per kv head
  float v_scale[HW_MAX_FP8_KV_HEADS];
};

// Split launch of decode calls with the plan built in-kernel (hw_fused.hip).
constexpr int kMfmaThreads = 512;  // threads per workgroup (8 waves)
constexpr int kMfmaWaves = kMfmaThreads / 64;
constexpr int kQfBlocks = 4;       // blocks whose rotated queries are held in LDS at once
constexpr int kFusedMaxRows = 32;  // stacked rows of the fused kernel

// Per-call arrays of the fused kernel, passed in the kernel arguments and read
// at kernel start with one load per array element per thread.
struct alignas(16) DecodeTables {
  int64_t block_start[HW_MAX_BLOCKS];
  int32_t block_cap[HW_MAX_BLOCKS];
  double inv_freq[kMaxHalf];     // theta^(-2i/D), i < D/2
  uint64_t rope_frac[kMaxHalf];  // frac(theta^(-2i/D) / (2 pi)) * 2^64, i < D/2
  float k_scale[HW_MAX_FP8_KV_HEADS];  // FP8 pools: this layer's scales per kv head
  float v_scale[HW_MAX_FP8_KV_HEADS];
};

struct alignas(16) DecodeArgs {
  const void* q;            // [W * nq][Hq][D] bf16
  const void* k;            // plane of (layer, kv head 0)
  const void* v;
  const int32_t* block_len; // [NB]
  const hw_entry* tables;   // [W][E]
  const int32_t* num_entries;
  float* out;               // [W * nq][Hq][D]
  int32_t* status;
  float2* ws_ml;            // [Hkv][R][P] (m, l) partials
  float* ws_acc;            // [Hkv][R][P][D] partial accumulators
  uint32_t* ws_hint;        // [Hkv][P][kMfmaWaves] first tile (byte offset) of the last call
  int64_t plane_elems;      // num_slots * D
  int32_t plane_bytes;      // plane_elems * element size (< 2^31)
  int32_t W, Hq, Hkv, G, R, E, NB, P, D;
  int32_t nq;               // query tokens per worker; rows are (w*nq + j)*G + h
  uint32_t mP, mE, mG, mGnq, mR;  // div_magic of P, E, G, G * nq and R (indices < 2^16)
  int32_t dtype;            // HW_BF16 / HW_FP8
  float qscale;             // log2(e) / sqrt(D): scores in the exp2 domain
  double rP;                // 1 / P (rounded)
  uint32_t spin_limit;      // polls before a wait between waves gives up
  DecodeTables tab;
};

hipError_t launch_fused_mfma(const DecodeArgs& a, int grid, hipStream_t s);
int fused_blocks_per_cu(int dtype, int D, int rows);

// Launchers (hw_plan.hip, hw_decode.hip).
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_run_valu(const RunArgs& a, hipStream_t s);
hipError_t launch_run_mfma(const RunArgs& a, hipStream_t s);
hipError_t launch_merge(const RunArgs& a, hipStream_t s);
int run_blocks_per_cu(int path, int dtype, int D, int rows);
int run_lds_bytes(int path, int NB, int qrows, int rows);

// Launchers (hw_cache.hip).
hipError_t launch_build_tables(int32_t* block_len, int32_t layout, int32_t W, int32_t common,
                               const int32_t* worker_block, hw_entry* tables,
                               int32_t* num_entries, int32_t num_blocks, hipStream_t s);
hipError_t launch_append(const hw_pool& pool, int32_t src, int32_t dst, double theta,
                         hipStream_t s);
hipError_t launch_reset(int32_t* block_len, int32_t block, hipStream_t s);
hipError_t launch_advance(const hw_pool& pool, int32_t n, const int32_t* blocks, hipStream_t s);
hipError_t launch_write(const hw_pool& pool, int32_t layer, int32_t n, const int32_t* blocks,
                        const float* k_new, const float* v_new, double theta, hipStream_t s);

}  // namespace hw
