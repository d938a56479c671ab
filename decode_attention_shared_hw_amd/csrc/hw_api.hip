// hw_api.hip — the C ABI of libhogwild_attn: argument validation, launch
// geometry, workspace layout.  Every host-visible error is returned before
// anything is enqueued.
#include <math.h>
#include <string.h>

#include <mutex>

#include "hw_internal.h"

namespace hw {
namespace {

constexpr int kMaxUnitsPerHead = kMaxUnits;
constexpr int kTargetWorkgroups = 256;  // one workgroup on each of MI355X's 256 CUs

int g_path = 0;            // 0 auto, 1 VALU, 2 MFMA
int g_units_per_head = 0;  // 0 automatic

struct DeviceInfo {
  int cus = 0;
  int occ[3][3][2][2] = {};  // [path][dtype][D==128][rows>16] resident workgroups per CU
};
std::mutex g_dev_mu;
DeviceInfo g_dev[64];
bool g_dev_ready[64] = {};

hw_status device_info(DeviceInfo** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return HW_EHIP;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_dev_ready[dev]) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return HW_EHIP;
    DeviceInfo& d = g_dev[dev];
    d.cus = p.multiProcessorCount;
    for (int path = 1; path <= 2; ++path)
      for (int dt = 0; dt < 3; ++dt)
        for (int dd = 0; dd < 2; ++dd)
          for (int rr = 0; rr < 2; ++rr) {
            if (path == 2 && dt == HW_F32) continue;
            if (path == 1 && dt == HW_FP8) continue;
            d.occ[path][dt][dd][rr] = decode_blocks_per_cu(path, dt, dd ? 128 : 64, rr ? 32 : 16);
          }
    g_dev_ready[dev] = true;
  }
  *out = &g_dev[dev];
  return HW_OK;
}

hw_status check_pool(const hw_pool* p) {
  if (!p) return HW_EINVAL;
  if (p->dtype != HW_F32 && p->dtype != HW_BF16 && p->dtype != HW_FP8) return HW_EUNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return HW_EUNSUPPORTED;
  if (p->num_layers < 1 || p->num_kv_heads < 1 || p->reserved != 0) return HW_EINVAL;
  if (p->num_blocks < 1 || p->num_blocks > HW_MAX_BLOCKS) return HW_ERANGE;
  if (p->num_slots <= 0 || p->num_slots % HW_TILE_TOKENS != 0) return HW_EINVAL;
  // one (layer, kv head) plane is addressed with 32-bit byte offsets
  if (p->num_slots * p->head_dim * elem_bytes(p->dtype) >= (int64_t(1) << 31)) return HW_ERANGE;
  if (!p->k || !p->v || !p->block_len || !p->status || !p->block_start || !p->block_cap)
    return HW_EINVAL;
  if (p->dtype == HW_FP8) {
    if (p->num_kv_heads > HW_MAX_FP8_KV_HEADS) return HW_ERANGE;
    if (!p->k_scale || !p->v_scale) return HW_EINVAL;
    const int64_t n = static_cast<int64_t>(p->num_layers) * p->num_kv_heads;
    for (int64_t i = 0; i < n; ++i)
      if (!(p->k_scale[i] > 0.f) || !isfinite(p->k_scale[i]) || !(p->v_scale[i] > 0.f) ||
          !isfinite(p->v_scale[i]))
        return HW_EINVAL;
  }
  for (int b = 0; b < p->num_blocks; ++b) {
    const int64_t s = p->block_start[b];
    const int32_t c = p->block_cap[b];
    if (s < 0 || c < 0 || s % HW_TILE_TOKENS != 0 || c % HW_TILE_TOKENS != 0) return HW_EINVAL;
    if (s + c > p->num_slots) return HW_EINVAL;
    for (int o = 0; o < b; ++o) {
      const int64_t so = p->block_start[o];
      const int32_t co = p->block_cap[o];
      if (c > 0 && co > 0 && s < so + co && so < s + c) return HW_EINVAL;  // overlap
    }
  }
  return HW_OK;
}

// frac(w / (2 pi)) as a 64-bit binary fraction (rounded): the per-dimension
// rotation step in revolutions, for exact integer angle reduction on the GPU.
uint64_t rope_fraction(double w) {
  const double f = w * 0.15915494309189535;  // 1 / (2 pi)
  const double fr = f - floor(f);
  const double scaled = ldexp(fr, 64);
  if (!(scaled < 18446744073709551616.0)) return 0;  // rounds up to a whole turn
  return static_cast<uint64_t>(scaled);
}

int select_path(const hw_pool* p, int rows) {
  if (g_path == 1) return 1;
  if (g_path == 2) return 2;
  if (p->dtype == HW_FP8) return 2;
  return (p->dtype == HW_BF16 && rows <= 32) ? 2 : 1;
}

int units_per_head_setting(int num_kv_heads) {
  if (g_units_per_head > 0) return g_units_per_head;
  int u = kTargetWorkgroups / num_kv_heads;
  if (u < 1) u = 1;
  if (u > kMaxUnitsPerHead) u = kMaxUnitsPerHead;
  return u;
}

struct WsLayout {
  size_t ml_off, acc_off, hint_off, total;
};

// [Hkv][rows][units] (m, l) pairs, then [Hkv][rows][units][D] accumulators,
// then [Hkv][units][kMfmaWaves] first-tile hints.
WsLayout ws_layout(int hkv, int units, int rows, int D) {
  WsLayout w;
  w.ml_off = 0;
  const size_t ml = static_cast<size_t>(hkv) * units * rows * sizeof(float2);
  w.acc_off = 256 * ((ml + 255) / 256);
  const size_t acc = static_cast<size_t>(hkv) * units * rows * D * sizeof(float);
  w.hint_off = 256 * ((w.acc_off + acc + 255) / 256);
  const size_t hint = static_cast<size_t>(hkv) * units * kMfmaWaves * sizeof(uint32_t);
  w.total = w.hint_off + hint;
  return w;
}

}  // namespace
}  // namespace hw

using namespace hw;

extern "C" {

int32_t hw_abi_version(void) { return HW_ABI_VERSION; }

const char* hw_status_str(hw_status s) {
  switch (s) {
    case HW_OK: return "ok";
    case HW_EINVAL: return "invalid argument";
    case HW_ERANGE: return "value outside supported limits";
    case HW_ECAPACITY: return "block capacity exceeded";
    case HW_EUNSUPPORTED: return "unsupported dtype or head_dim";
    case HW_EWORKSPACE: return "workspace missing or too small";
    case HW_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

hw_status hw_set_tuning(int32_t path, int32_t units_per_head) {
  if (path < 0 || path > 2 || units_per_head < 0 || units_per_head > kMaxUnitsPerHead)
    return HW_EINVAL;
  g_path = path;
  g_units_per_head = units_per_head;
  return HW_OK;
}

size_t hw_attn_workspace_bytes(const hw_pool* pool, int32_t num_workers, int32_t num_q_heads) {
  if (check_pool(pool) != HW_OK) return 0;
  if (num_workers < 1 || num_workers > HW_MAX_ROWS || num_q_heads < 1 ||
      num_q_heads % pool->num_kv_heads != 0)
    return 0;
  const int rows = num_workers * (num_q_heads / pool->num_kv_heads);
  if (rows > HW_MAX_ROWS) return 0;
  return ws_layout(pool->num_kv_heads, units_per_head_setting(pool->num_kv_heads), rows,
                   pool->head_dim)
      .total;
}

static hw_status attn_call(const hw_pool* pool, int32_t layer, const void* q, int32_t num_workers,
                           int32_t nq, int32_t num_q_heads, const hw_entry* tables,
                           int32_t max_entries, const int32_t* num_entries, double rope_theta,
                           float* out, void* workspace, size_t workspace_bytes, void* stream);

hw_status hw_attn_decode(const hw_pool* pool, int32_t layer, const void* q, int32_t num_workers,
                         int32_t num_q_heads, const hw_entry* tables, int32_t max_entries,
                         const int32_t* num_entries, double rope_theta, float* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return attn_call(pool, layer, q, num_workers, 1, num_q_heads, tables, max_entries, num_entries,
                   rope_theta, out, workspace, workspace_bytes, stream);
}

hw_status hw_attn_chunk(const hw_pool* pool, int32_t layer, const void* q, int32_t num_workers,
                        int32_t chunk, int32_t num_q_heads, const hw_entry* tables,
                        int32_t max_entries, const int32_t* num_entries, double rope_theta,
                        float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (chunk < 1 || chunk > HW_MAX_ROWS) return HW_ERANGE;
  return attn_call(pool, layer, q, num_workers, chunk, num_q_heads, tables, max_entries,
                   num_entries, rope_theta, out, workspace, workspace_bytes, stream);
}

static hw_status attn_call(const hw_pool* pool, int32_t layer, const void* q, int32_t num_workers,
                           int32_t nq, int32_t num_q_heads, const hw_entry* tables,
                           int32_t max_entries, const int32_t* num_entries, double rope_theta,
                           float* out, void* workspace, size_t workspace_bytes, void* stream) {
  hw_status st = check_pool(pool);
  if (st != HW_OK) return st;
  if (!q || !tables || !num_entries || !out) return HW_EINVAL;
  if (layer < 0 || layer >= pool->num_layers) return HW_EINVAL;
  if (num_workers < 1 || num_workers > HW_MAX_WORKERS) return HW_ERANGE;
  if (num_q_heads < 1 || num_q_heads % pool->num_kv_heads != 0) return HW_EINVAL;
  if (max_entries < 1 || max_entries > HW_MAX_ENTRIES) return HW_ERANGE;
  if (!(rope_theta > 0.0) || !isfinite(rope_theta)) return HW_EINVAL;
  const int G = num_q_heads / pool->num_kv_heads;
  if (static_cast<int64_t>(num_workers) * nq * G > HW_MAX_ROWS) return HW_ERANGE;
  const int rows = num_workers * nq * G;
  if (rows > HW_MAX_ROWS) return HW_ERANGE;
  const int path = select_path(pool, rows);
  if (path == 2 && (pool->dtype == HW_F32 || rows > 32)) return HW_EUNSUPPORTED;
  if (path == 1 && pool->dtype == HW_FP8) return HW_EUNSUPPORTED;
  const int P_ws = units_per_head_setting(pool->num_kv_heads);
  const WsLayout wl = ws_layout(pool->num_kv_heads, P_ws, rows, pool->head_dim);
  if (!workspace || workspace_bytes < wl.total) return HW_EWORKSPACE;

  // units per head: the setting, bounded by the tiles the blocks can hold
  int64_t max_tiles = 0;
  for (int b = 0; b < pool->num_blocks; ++b) max_tiles += pool->block_cap[b] / HW_TILE_TOKENS;
  int64_t P = P_ws;
  if (P > max_tiles) P = max_tiles;
  if (P < 1) P = 1;
  // workgroup indices stay below 2^16 (fast_div's range)
  if (P * pool->num_kv_heads >= 65536) return HW_ERANGE;

  DeviceInfo* di = nullptr;
  st = device_info(&di);
  if (st != HW_OK) return st;

  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  const size_t esz = elem_bytes(pool->dtype);
  const int64_t plane = pool->num_slots * pool->head_dim;
  a.q = q;
  a.k = static_cast<const char*>(pool->k) +
        static_cast<int64_t>(layer) * pool->num_kv_heads * plane * esz;
  a.v = static_cast<const char*>(pool->v) +
        static_cast<int64_t>(layer) * pool->num_kv_heads * plane * esz;
  a.block_len = pool->block_len;
  a.tables = tables;
  a.num_entries = num_entries;
  a.out = out;
  a.status = pool->status;
  char* ws = static_cast<char*>(workspace);
  a.ws_ml = reinterpret_cast<float2*>(ws + wl.ml_off);
  a.ws_acc = reinterpret_cast<float*>(ws + wl.acc_off);
  a.ws_hint = reinterpret_cast<uint32_t*>(ws + wl.hint_off);
  a.plane_elems = plane;
  a.plane_bytes = static_cast<int32_t>(plane * static_cast<int64_t>(esz));
  a.W = num_workers;
  a.Hq = num_q_heads;
  a.Hkv = pool->num_kv_heads;
  a.G = G;
  a.R = rows;
  a.nq = nq;
  a.E = max_entries;
  a.NB = pool->num_blocks;
  a.P = static_cast<int32_t>(P);
  a.D = pool->head_dim;
  a.dtype = pool->dtype;
  a.mP = div_magic(static_cast<uint32_t>(a.P));
  a.rP = 1.0 / a.P;
  a.mE = div_magic(static_cast<uint32_t>(a.E));
  a.mG = div_magic(static_cast<uint32_t>(a.G));
  a.mGnq = div_magic(static_cast<uint32_t>(a.G * a.nq));
  a.mR = div_magic(static_cast<uint32_t>(a.R));
  const int64_t grid = P * pool->num_kv_heads;
  a.qscale = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(pool->head_dim)));
  for (int b = 0; b < pool->num_blocks; ++b) {
    a.tab.block_start[b] = pool->block_start[b];
    a.tab.block_cap[b] = pool->block_cap[b];
  }
  for (int i = 0; i < pool->head_dim / 2; ++i) {
    const double w = pow(rope_theta, -2.0 * i / static_cast<double>(pool->head_dim));
    a.tab.inv_freq[i] = w;
    a.tab.rope_frac[i] = rope_fraction(w);
  }
  if (pool->dtype == HW_FP8) {
    const int64_t l0 = static_cast<int64_t>(layer) * pool->num_kv_heads;
    for (int g = 0; g < pool->num_kv_heads; ++g) {
      a.tab.k_scale[g] = pool->k_scale[l0 + g];
      a.tab.v_scale[g] = pool->v_scale[l0 + g];
    }
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = path == 2 ? launch_decode_mfma(a, static_cast<int>(grid), hs)
                           : launch_decode_valu(a, static_cast<int>(grid), hs);
  if (e == hipSuccess) e = launch_merge(a, hs);
  return e == hipSuccess ? HW_OK : HW_EHIP;
}

hw_status hw_block_append(const hw_pool* pool, int32_t src_block, int32_t dst_block,
                          double rope_theta, void* stream) {
  hw_status st = check_pool(pool);
  if (st != HW_OK) return st;
  if (src_block < 0 || src_block >= pool->num_blocks || dst_block < 0 ||
      dst_block >= pool->num_blocks || src_block == dst_block)
    return HW_EINVAL;
  if (!(rope_theta > 0.0) || !isfinite(rope_theta)) return HW_EINVAL;
  const hipError_t e = launch_append(*pool, src_block, dst_block, rope_theta,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HW_OK : HW_EHIP;
}

hw_status hw_block_reset(const hw_pool* pool, int32_t block, void* stream) {
  hw_status st = check_pool(pool);
  if (st != HW_OK) return st;
  if (block < 0 || block >= pool->num_blocks) return HW_EINVAL;
  return launch_reset(pool->block_len, block, static_cast<hipStream_t>(stream)) == hipSuccess
             ? HW_OK
             : HW_EHIP;
}

// Block lists of the token write: 1..HW_MAX_WORKERS distinct valid ids.
static hw_status check_block_list(const hw_pool* pool, int32_t n, const int32_t* blocks) {
  if (!blocks) return HW_EINVAL;
  if (n < 1 || n > HW_MAX_WORKERS) return HW_ERANGE;
  for (int i = 0; i < n; ++i) {
    if (blocks[i] < 0 || blocks[i] >= pool->num_blocks) return HW_EINVAL;
    for (int j = 0; j < i; ++j)
      if (blocks[j] == blocks[i]) return HW_EINVAL;
  }
  return HW_OK;
}

hw_status hw_block_advance(const hw_pool* pool, int32_t n, const int32_t* blocks, void* stream) {
  hw_status st = check_pool(pool);
  if (st != HW_OK) return st;
  st = check_block_list(pool, n, blocks);
  if (st != HW_OK) return st;
  return launch_advance(*pool, n, blocks, static_cast<hipStream_t>(stream)) == hipSuccess
             ? HW_OK
             : HW_EHIP;
}

hw_status hw_block_write(const hw_pool* pool, int32_t layer, int32_t n, const int32_t* blocks,
                         const float* k_new, const float* v_new, double rope_theta,
                         void* stream) {
  hw_status st = check_pool(pool);
  if (st != HW_OK) return st;
  st = check_block_list(pool, n, blocks);
  if (st != HW_OK) return st;
  if (!k_new || !v_new) return HW_EINVAL;
  if (layer < 0 || layer >= pool->num_layers) return HW_EINVAL;
  if (!(rope_theta > 0.0) || !isfinite(rope_theta)) return HW_EINVAL;
  return launch_write(*pool, layer, n, blocks, k_new, v_new, rope_theta,
                      static_cast<hipStream_t>(stream)) == hipSuccess
             ? HW_OK
             : HW_EHIP;
}

hw_status hw_build_combined_tables(const hw_pool* pool, int32_t num_workers, int32_t common_block,
                                   const int32_t* worker_block, hw_entry* tables,
                                   int32_t* num_entries, void* stream) {
  return hw_build_view_tables(pool, HW_LAYOUT_COMBINED, num_workers, common_block, worker_block,
                              tables, num_entries, stream);
}

hw_status hw_build_view_tables(const hw_pool* pool, int32_t layout, int32_t num_workers,
                               int32_t common_block, const int32_t* worker_block,
                               hw_entry* tables, int32_t* num_entries, void* stream) {
  if (layout != HW_LAYOUT_COMBINED && layout != HW_LAYOUT_INTERLEAVED &&
      layout != HW_LAYOUT_CONTIGUOUS)
    return HW_EINVAL;
  hw_status st = check_pool(pool);
  if (st != HW_OK) return st;
  if (!worker_block || !tables || !num_entries) return HW_EINVAL;
  if (num_workers < 1 || num_workers > HW_MAX_WORKERS) return HW_ERANGE;
  if (num_workers + 1 > HW_MAX_ENTRIES) return HW_ERANGE;
  if (common_block < 0 || common_block >= pool->num_blocks) return HW_EINVAL;
  for (int w = 0; w < num_workers; ++w) {
    const int32_t b = worker_block[w];
    if (b < 0 || b >= pool->num_blocks || b == common_block) return HW_EINVAL;
    for (int v = 0; v < w; ++v)
      if (worker_block[v] == b) return HW_EINVAL;
  }
  const hipError_t e = launch_build_tables(pool->block_len, layout, num_workers, common_block,
                                           worker_block,
                                           tables, num_entries, pool->num_blocks,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HW_OK : HW_EHIP;
}

hw_status hw_pool_status(const hw_pool* pool, int32_t* flags, int32_t clear) {
  if (!pool || !pool->status || !flags) return HW_EINVAL;
  if (hipDeviceSynchronize() != hipSuccess) return HW_EHIP;
  if (hipMemcpy(flags, pool->status, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return HW_EHIP;
  if (clear) {
    const int32_t zero = 0;
    if (hipMemcpy(pool->status, &zero, sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess)
      return HW_EHIP;
  }
  return HW_OK;
}

}  // extern "C"
