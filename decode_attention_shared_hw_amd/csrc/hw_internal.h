// hw_internal.h — shared definitions of libhogwild_attn's HIP sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hogwild_attn.h"

namespace hw {

constexpr int kTile = HW_TILE_TOKENS;  // tokens per pool tile
constexpr int kThreads = 256;          // threads per decode workgroup (4 waves)
constexpr int kWaves = kThreads / 64;
constexpr int kMfmaThreads = 512;      // threads per MFMA decode workgroup (8 waves)
constexpr int kMfmaWaves = kMfmaThreads / 64;
constexpr int kQfBlocks = 4;           // blocks whose rotated queries are held in LDS at once
constexpr int kMaxHalf = 64;           // head_dim / 2 upper bound
constexpr int kMaxUnits = 256;         // split-K work units per kv head
constexpr int kBlockCost = 5;          // extra cost, in tiles, of each visible block after the first

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

// Per-call arrays of the decode kernels, passed in the kernel arguments and
// read at kernel start with one load per array element per thread.
struct alignas(16) DecodeTables {
  int64_t block_start[HW_MAX_BLOCKS];
  int32_t block_cap[HW_MAX_BLOCKS];
  double inv_freq[kMaxHalf];  // theta^(-2i/D), i < D/2
  uint64_t rope_frac[kMaxHalf];  // frac(theta^(-2i/D) / (2 pi)) * 2^64, i < D/2
  float k_scale[HW_MAX_FP8_KV_HEADS];  // FP8 pools: this layer's scales per kv head
  float v_scale[HW_MAX_FP8_KV_HEADS];
};

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

// Kernel arguments of the fused decode kernels (passed by value).
struct alignas(16) DecodeArgs {
  const void* q;            // [W][Hq][D] pool dtype
  const void* k;            // plane of (layer, kv head 0)
  const void* v;
  const int32_t* block_len; // [NB]
  const hw_entry* tables;   // [W][E]
  const int32_t* num_entries;
  float* out;               // [W][Hq][D]
  int32_t* status;
  float2* ws_ml;            // [Hkv][R][P] (m, l) partials
  float* ws_acc;            // [Hkv][R][P][D] partial accumulators
  uint32_t* ws_hint;        // [Hkv][P][kMfmaWaves] first tile (byte offset) of the last call
  int64_t plane_elems;      // num_slots * D
  int32_t plane_bytes;      // plane_elems * element size (< 2^31)
  int32_t W, Hq, Hkv, G, R, E, NB, P, D;
  int32_t nq;               // query tokens per worker (1: decode); rows are (w*nq + j)*G + h
  uint32_t mP, mE, mG, mGnq, mR;  // div_magic of P, E, G, G * nq and R (indices < 2^16)
  int32_t dtype;            // HW_F32 / HW_BF16 / HW_FP8
  float qscale;             // log2(e) / sqrt(D): scores in the exp2 domain
  double rP;                // 1 / P (rounded)
  DecodeTables tab;
};

// Launchers (hw_decode.hip).
hipError_t launch_decode_valu(const DecodeArgs& a, int grid, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, int grid, hipStream_t s);
hipError_t launch_merge(const DecodeArgs& a, hipStream_t s);
int decode_blocks_per_cu(int path, int dtype, int D, int rows);

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
