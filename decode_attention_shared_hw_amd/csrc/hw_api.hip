// hw_api.hip — the C ABI of libhogwild_attn: argument validation, launch
// geometry, workspace layout.  Every host-visible error is returned before
// anything is enqueued.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "hw_internal.h"

namespace hw {
namespace {

// Workspace of hw_attn_decode_noalloc: one array per GPU, held from the
// library's load until the process ends.  Host code uses its device address
// (scratch_address), never the name: on the host the name is a stand-in.
constexpr size_t kScratchBytes = HW_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_addr[64];  // per device, from hipGetSymbolAddress on its first call

// The device address of the current device's scratch, looked up once per
// device with that device current.
hw_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return HW_EHIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HW_EHIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return HW_OK;
}

int g_path = 0;            // 0 auto, 1 VALU, 2 MFMA
int g_units_per_head = 0;  // 0 automatic
int g_balance = 0;         // 1: balanced tile order in the split launch

// Per device: compute units, and resident run-kernel workgroups per CU for
// each (path, dtype, head_dim, row class), filled on first use.
struct DeviceInfo {
  bool ready = false;
  int cus = 0;
  int occ[4][3][2][5] = {};  // [path: -, VALU, MFMA, fused][dtype][D == 128][rows class: <=16, 32, 48, 64, 80]
};
std::mutex g_dev_mu;
DeviceInfo g_dev[64];

int row_class(int rows) { return rows <= 16 ? 0 : rows <= 32 ? 1 : rows <= 48 ? 2 : rows <= 64 ? 3 : 4; }

// Resident split-launch workgroups of the whole device for this launch shape
// (path 3: the fused kernel).  Where
// no device answers (a host without a GPU: only argument checks and sizes
// are asked for there), an MI355X with one workgroup per CU is assumed.
constexpr int kDefaultCUs = 256;
int device_capacity(int path, int dtype, int D, int rows) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kDefaultCUs;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.ready) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return kDefaultCUs;
    d.cus = p.multiProcessorCount;
    d.ready = true;
  }
  int& o = d.occ[path][dtype][D == 128 ? 1 : 0][row_class(rows)];
  if (o == 0) o = path == 3 ? fused_blocks_per_cu(dtype, D, rows) : run_blocks_per_cu(path, dtype, D, rows);
  return d.cus * (o > 0 ? o : 1);
}

// Rotation steps for (theta, D): theta^(-2i/D) and its fraction of a turn as
// a 64-bit binary fraction, cached for the last few (theta, D) seen.
struct RopeTables {
  double theta = 0.0;
  int D = 0;
  double inv_freq[kMaxHalf];
  uint64_t frac[kMaxHalf];
};
std::mutex g_rope_mu;
RopeTables g_rope[4];
int g_rope_next = 0;

// frac(w / (2 pi)) as a 64-bit binary fraction (rounded): the per-dimension
// rotation step in revolutions, for exact integer angle reduction on the GPU.
uint64_t rope_fraction(double w) {
  const double f = w * 0.15915494309189535;  // 1 / (2 pi)
  const double fr = f - floor(f);
  const double scaled = ldexp(fr, 64);
  if (!(scaled < 18446744073709551616.0)) return 0;  // rounds up to a whole turn
  return static_cast<uint64_t>(scaled);
}

void rope_tables(double theta, int D, double* inv_freq, uint64_t* frac) {
  std::lock_guard<std::mutex> lk(g_rope_mu);
  for (RopeTables& t : g_rope)
    if (t.D == D && t.theta == theta) {
      memcpy(inv_freq, t.inv_freq, sizeof(double) * D / 2);
      memcpy(frac, t.frac, sizeof(uint64_t) * D / 2);
      return;
    }
  RopeTables& t = g_rope[g_rope_next];
  g_rope_next = (g_rope_next + 1) % 4;
  t.theta = theta;
  t.D = D;
  for (int i = 0; i < D / 2; ++i) {
    t.inv_freq[i] = pow(theta, -2.0 * i / static_cast<double>(D));
    t.frac[i] = rope_fraction(t.inv_freq[i]);
  }
  memcpy(inv_freq, t.inv_freq, sizeof(double) * D / 2);
  memcpy(frac, t.frac, sizeof(uint64_t) * D / 2);
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

// The FP8 scales of one layer: positive and finite.
hw_status check_scales(const hw_pool* p, int layer) {
  if (p->dtype != HW_FP8) return HW_OK;
  const int64_t l0 = static_cast<int64_t>(layer) * p->num_kv_heads;
  for (int g = 0; g < p->num_kv_heads; ++g) {
    const float ks = p->k_scale[l0 + g], vs = p->v_scale[l0 + g];
    if (!(ks > 0.f) || !isfinite(ks) || !(vs > 0.f) || !isfinite(vs)) return HW_EINVAL;
  }
  return HW_OK;
}

int select_path(const hw_pool* p, int rows) {
  if (g_path == 1) return 1;
  if (g_path == 2) return 2;
  if (p->dtype == HW_FP8) return 2;
  return p->dtype == HW_BF16 ? 2 : 1;
}

// Call shape shared by the plan, the run and the workspace size.
struct Shape {
  int W, nq, Hq, G, qrows, R, path, P;
};

// Validates the shape and derives the path and the units per kv head: the
// device's resident workgroups of that kernel divided by the kv heads (one
// wave of workgroups fills the GPU once), or the tuning's value lowered to
// that; at most one unit per tile the blocks can hold.
hw_status call_shape(const hw_pool* pool, int W, int nq, int Hq, Shape* s) {
  if (W < 1 || W > HW_MAX_WORKERS || nq < 1 || nq > HW_MAX_ROWS) return HW_ERANGE;
  if (Hq < 1 || Hq % pool->num_kv_heads != 0) return HW_EINVAL;
  s->W = W;
  s->nq = nq;
  s->Hq = Hq;
  s->G = Hq / pool->num_kv_heads;
  if (static_cast<int64_t>(W) * nq * s->G > HW_MAX_ROWS) return HW_ERANGE;
  s->qrows = W * nq;
  s->R = s->qrows * s->G;
  s->path = select_path(pool, s->R);
  if (s->path == 2 && pool->dtype == HW_F32) return HW_EUNSUPPORTED;
  if (s->path == 1 && pool->dtype == HW_FP8) return HW_EUNSUPPORTED;
  if (s->path == 1 && s->R > kValuMaxRows) return HW_ERANGE;
  const bool fused = s->path == 2 && pool->dtype != HW_F32 && s->R <= kFusedMaxRows;
  const int cap = device_capacity(fused ? 3 : s->path, pool->dtype, pool->head_dim, s->R);
  int64_t P = cap / pool->num_kv_heads;
  if (g_units_per_head > 0 && g_units_per_head < P) P = g_units_per_head;
  if (P > kMaxUnits) P = kMaxUnits;
  int64_t max_tiles = 0;
  for (int b = 0; b < pool->num_blocks; ++b) max_tiles += pool->block_cap[b] / HW_TILE_TOKENS;
  if (P > max_tiles) P = max_tiles;
  if (pool->num_kv_heads > kMaxSyncHeads) P = 1;  // (the tile counters cover kMaxSyncHeads heads)
  if (P < 1) P = 1;
  // workgroup indices stay below 2^16 (fast_div's range)
  if (P * pool->num_kv_heads >= 65536) return HW_ERANGE;
  s->P = static_cast<int>(P);
  return HW_OK;
}

// The run kernels read the plan, q and out with 16-byte vector accesses.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t plan_bytes(const hw_pool* pool, const Shape& s) {
  return static_cast<size_t>(plan_words(pool->num_blocks, s.qrows)) * 4;
}

struct WsLayout {
  size_t plan_off, ml_off, acc_off, cnt_off, hint_off, total;
};

// [tile counters][plan][Hkv][R][P] (m, l) pairs [Hkv][R][P][D] accumulators
// [Hkv][P] tile counts [Hkv][P][kMfmaWaves] first-tile hints (fused path).
WsLayout ws_layout(const hw_pool* pool, const Shape& s) {
  WsLayout w;
  auto up = [](size_t x) { return 256 * ((x + 255) / 256); };
  const size_t units = static_cast<size_t>(pool->num_kv_heads) * s.P;
  w.plan_off = kSyncBytes;
  w.ml_off = up(w.plan_off + plan_bytes(pool, s));
  const size_t rows = units * s.R;
  w.acc_off = up(w.ml_off + rows * sizeof(float2));
  w.cnt_off = up(w.acc_off + rows * pool->head_dim * sizeof(float));
  w.hint_off = up(w.cnt_off + units * sizeof(int32_t));
  w.total = w.hint_off + units * kMfmaWaves * sizeof(uint32_t);
  return w;
}

// Decode calls that take the fused kernel (plan built in-kernel): MFMA path,
// bf16 or FP8 pool, up to 32 stacked rows.
bool fused_path(const hw_pool* pool, const Shape& s) {
  return s.path == 2 && pool->dtype != HW_F32 && s.R <= kFusedMaxRows;
}

hw_status plan_call(const hw_pool* pool, const Shape& s, const hw_entry* tables,
                    int32_t max_entries, const int32_t* num_entries, void* plan, size_t pbytes,
                    hipStream_t stream) {
  if (!tables || !num_entries || !plan) return HW_EINVAL;
  if (!aligned16(plan)) return HW_EINVAL;
  if (max_entries < 1 || max_entries > HW_MAX_ENTRIES) return HW_ERANGE;
  if (pbytes < plan_bytes(pool, s)) return HW_EWORKSPACE;
  PlanArgs a;
  memset(&a, 0, sizeof(a));
  a.tables = tables;
  a.num_entries = num_entries;
  a.block_len = pool->block_len;
  a.status = pool->status;
  a.plan = static_cast<int32_t*>(plan);
  a.W = s.W;
  a.nq = s.nq;
  a.G = s.G;
  a.E = max_entries;
  a.NB = pool->num_blocks;
  a.P = s.P;
  for (int b = 0; b < pool->num_blocks; ++b) {
    a.block_start[b] = static_cast<int32_t>(pool->block_start[b]);
    a.block_cap[b] = pool->block_cap[b];
  }
  return launch_plan(a, stream) == hipSuccess ? HW_OK : HW_EHIP;
}

// balance: 1 for the balanced tile order (tiles after each wave's first from
// the head's counter in the workspace), 0 for fixed tile ranges.
hw_status run_call(const hw_pool* pool, int32_t layer, const void* q, const Shape& s,
                   const void* plan, size_t pbytes, double theta, float* out, void* workspace,
                   size_t ws_bytes, hipStream_t stream, int balance) {
  if (!q || !out || !plan) return HW_EINVAL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(plan)) return HW_EINVAL;
  if (layer < 0 || layer >= pool->num_layers) return HW_EINVAL;
  if (!(theta > 0.0) || !isfinite(theta)) return HW_EINVAL;
  if (pbytes < plan_bytes(pool, s)) return HW_EWORKSPACE;
  const WsLayout wl = ws_layout(pool, s);
  if (!workspace || ws_bytes < wl.total) return HW_EWORKSPACE;
  if (!aligned16(workspace)) return HW_EINVAL;
  const hw_status st = check_scales(pool, layer);
  if (st != HW_OK) return st;

  RunArgs a;
  memset(&a, 0, sizeof(a));
  const size_t esz = elem_bytes(pool->dtype);
  const int64_t plane = pool->num_slots * pool->head_dim;
  const int64_t layer_off = static_cast<int64_t>(layer) * pool->num_kv_heads * plane;
  a.q = q;
  a.k = static_cast<const char*>(pool->k) + layer_off * esz;
  a.v = static_cast<const char*>(pool->v) + layer_off * esz;
  a.plan = static_cast<const int32_t*>(plan);
  a.block_len = pool->block_len;
  a.out = out;
  a.status = pool->status;
  char* ws = static_cast<char*>(workspace);
  a.sync = reinterpret_cast<uint32_t*>(ws);
  a.ws_ml = reinterpret_cast<float2*>(ws + wl.ml_off);
  a.ws_acc = reinterpret_cast<float*>(ws + wl.acc_off);
  a.ws_cnt = reinterpret_cast<int32_t*>(ws + wl.cnt_off);
  a.plane_elems = plane;
  a.plane_bytes = static_cast<int32_t>(plane * static_cast<int64_t>(esz));
  a.Hq = s.Hq;
  a.Hkv = pool->num_kv_heads;
  a.G = s.G;
  a.R = s.R;
  a.qrows = s.qrows;
  a.NB = pool->num_blocks;
  a.P = s.P;
  a.D = pool->head_dim;
  a.mG = div_magic(static_cast<uint32_t>(s.G));
  a.mHkv = div_magic(static_cast<uint32_t>(a.Hkv));
  a.mR = div_magic(static_cast<uint32_t>(s.R));
  a.mP = div_magic(static_cast<uint32_t>(s.P));
  a.balance = balance;
  a.dtype = pool->dtype;
  a.qscale = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(pool->head_dim)));
  rope_tables(theta, pool->head_dim, a.inv_freq, a.rope_frac);
  if (pool->dtype == HW_FP8) {
    const int64_t l0 = static_cast<int64_t>(layer) * pool->num_kv_heads;
    for (int g = 0; g < pool->num_kv_heads; ++g) {
      a.k_scale[g] = pool->k_scale[l0 + g];
      a.v_scale[g] = pool->v_scale[l0 + g];
    }
  }
  // workgroup w -> (head w % Hkv, unit w / Hkv) with fast_div, exact for
  // Hkv <= 256; more kv heads run one unit per head (call_shape), and a zero
  // multiplier gives unit 0 for every workgroup
  if (a.Hkv > 256) a.mHkv = 0;
  hipError_t e = s.path == 2 ? launch_run_mfma(a, stream) : launch_run_valu(a, stream);
  if (e == hipSuccess && s.P > 1) e = launch_merge(a, stream);
  return e == hipSuccess ? HW_OK : HW_EHIP;
}

// Polls before a wait between the waves of a work unit gives up: 2^22 (about
// 0.25 s), or HW_SPIN_LIMIT from the environment (tests force the limit).
uint32_t spin_limit() {
  const char* e = getenv("HW_SPIN_LIMIT");
  if (e && *e) {
    char* end = nullptr;
    const unsigned long long v = strtoull(e, &end, 10);
    if (end && *end == 0) return v > 0xffffffffull ? 0xffffffffu : static_cast<uint32_t>(v);
  }
  return 1u << 22;
}

// Split launch with the plan built in-kernel (hw_fused.hip), then the merge.
// The caller has validated the shape, the pointers and the workspace.
hw_status fused_call(const hw_pool* pool, int32_t layer, const void* q, const Shape& s,
                     const hw_entry* tables, int32_t max_entries, const int32_t* num_entries,
                     double theta, float* out, void* workspace, const WsLayout& wl,
                     hipStream_t stream) {
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  const size_t esz = elem_bytes(pool->dtype);
  const int64_t plane = pool->num_slots * pool->head_dim;
  const int64_t layer_off = static_cast<int64_t>(layer) * pool->num_kv_heads * plane;
  a.q = q;
  a.k = static_cast<const char*>(pool->k) + layer_off * esz;
  a.v = static_cast<const char*>(pool->v) + layer_off * esz;
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
  a.W = s.W;
  a.Hq = s.Hq;
  a.Hkv = pool->num_kv_heads;
  a.G = s.G;
  a.R = s.R;
  a.nq = s.nq;
  a.E = max_entries;
  a.NB = pool->num_blocks;
  a.P = s.P;
  a.D = pool->head_dim;
  a.dtype = pool->dtype;
  a.mP = div_magic(static_cast<uint32_t>(a.P));
  a.rP = 1.0 / a.P;
  a.mE = div_magic(static_cast<uint32_t>(a.E));
  a.mG = div_magic(static_cast<uint32_t>(a.G));
  a.mGnq = div_magic(static_cast<uint32_t>(a.G * a.nq));
  a.mR = div_magic(static_cast<uint32_t>(a.R));
  a.spin_limit = spin_limit();
  a.qscale = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(pool->head_dim)));
  for (int b = 0; b < pool->num_blocks; ++b) {
    a.tab.block_start[b] = pool->block_start[b];
    a.tab.block_cap[b] = pool->block_cap[b];
  }
  rope_tables(theta, pool->head_dim, a.tab.inv_freq, a.tab.rope_frac);
  if (pool->dtype == HW_FP8) {
    const int64_t l0 = static_cast<int64_t>(layer) * pool->num_kv_heads;
    for (int g = 0; g < pool->num_kv_heads; ++g) {
      a.tab.k_scale[g] = pool->k_scale[l0 + g];
      a.tab.v_scale[g] = pool->v_scale[l0 + g];
    }
  }
  hipError_t e = launch_fused_mfma(a, s.P * pool->num_kv_heads, stream);
  if (e == hipSuccess) {
    // the merge reads the partials in the same [Hkv][R][P] layout
    RunArgs m;
    memset(&m, 0, sizeof(m));
    m.out = out;
    m.status = pool->status;
    m.ws_ml = a.ws_ml;
    m.ws_acc = a.ws_acc;
    m.Hq = s.Hq;
    m.Hkv = pool->num_kv_heads;
    m.G = s.G;
    m.R = s.R;
    m.qrows = s.qrows;
    m.NB = pool->num_blocks;
    m.P = s.P;
    m.D = pool->head_dim;
    m.mG = a.mG;
    m.mR = a.mR;
    m.dtype = pool->dtype;
    memcpy(m.v_scale, a.tab.v_scale, sizeof(m.v_scale));
    e = launch_merge(m, stream);
  }
  return e == hipSuccess ? HW_OK : HW_EHIP;
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
    case HW_EUNSUPPORTED: return "unsupported dtype, head_dim or path";
    case HW_EWORKSPACE: return "workspace or plan missing or too small";
    case HW_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

hw_status hw_set_tuning(int32_t path, int32_t units_per_head, int32_t balance) {
  if (path < 0 || path > 2 || units_per_head < 0 || units_per_head > kMaxUnits ||
      (balance != 0 && balance != 1))
    return HW_EINVAL;
  g_path = path;
  g_units_per_head = units_per_head;
  g_balance = balance;
  return HW_OK;
}

size_t hw_attn_plan_bytes(const hw_pool* pool, int32_t num_workers, int32_t chunk,
                          int32_t num_q_heads) {
  if (check_pool(pool) != HW_OK) return 0;
  Shape s;
  if (call_shape(pool, num_workers, chunk, num_q_heads, &s) != HW_OK) return 0;
  return plan_bytes(pool, s);
}

size_t hw_attn_workspace_bytes(const hw_pool* pool, int32_t num_workers, int32_t num_q_heads) {
  if (check_pool(pool) != HW_OK) return 0;
  // num_workers query rows: the layout of one worker with that many query
  // tokens (a chunk call's W * chunk rows may exceed HW_MAX_WORKERS)
  Shape s;
  if (call_shape(pool, 1, num_workers, num_q_heads, &s) != HW_OK) return 0;
  return ws_layout(pool, s).total;
}

hw_status hw_attn_plan(const hw_pool* pool, int32_t num_workers, int32_t chunk,
                       int32_t num_q_heads, const hw_entry* tables, int32_t max_entries,
                       const int32_t* num_entries, void* plan, size_t plan_bytes_,
                       void* stream) {
  hw_status st = check_pool(pool);
  if (st != HW_OK) return st;
  Shape s;
  st = call_shape(pool, num_workers, chunk, num_q_heads, &s);
  if (st != HW_OK) return st;
  return plan_call(pool, s, tables, max_entries, num_entries, plan, plan_bytes_,
                   static_cast<hipStream_t>(stream));
}

hw_status hw_attn_run(const hw_pool* pool, int32_t layer, const void* q, int32_t num_workers,
                      int32_t chunk, int32_t num_q_heads, const void* plan, size_t plan_bytes_,
                      double rope_theta, float* out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  hw_status st = check_pool(pool);
  if (st != HW_OK) return st;
  Shape s;
  st = call_shape(pool, num_workers, chunk, num_q_heads, &s);
  if (st != HW_OK) return st;
  return run_call(pool, layer, q, s, plan, plan_bytes_, rope_theta, out, workspace,
                  workspace_bytes, static_cast<hipStream_t>(stream), g_balance);
}

static hw_status attn_call(const hw_pool* pool, int32_t layer, const void* q, int32_t num_workers,
                           int32_t nq, int32_t num_q_heads, const hw_entry* tables,
                           int32_t max_entries, const int32_t* num_entries, double rope_theta,
                           float* out, void* workspace, size_t workspace_bytes, void* stream,
                           int balance) {
  hw_status st = check_pool(pool);
  if (st != HW_OK) return st;
  Shape s;
  st = call_shape(pool, num_workers, nq, num_q_heads, &s);
  if (st != HW_OK) return st;
  if (!q || !out || !tables || !num_entries) return HW_EINVAL;
  if (!aligned16(q) || !aligned16(out)) return HW_EINVAL;
  if (layer < 0 || layer >= pool->num_layers) return HW_EINVAL;
  if (!(rope_theta > 0.0) || !isfinite(rope_theta)) return HW_EINVAL;
  if (max_entries < 1 || max_entries > HW_MAX_ENTRIES) return HW_ERANGE;
  // (the same layout as hw_attn_workspace_bytes(pool, W * nq, Hq))
  const WsLayout wl = ws_layout(pool, s);
  if (!workspace || workspace_bytes < wl.total) return HW_EWORKSPACE;
  if (!aligned16(workspace)) return HW_EINVAL;
  st = check_scales(pool, layer);
  if (st != HW_OK) return st;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (fused_path(pool, s))
    return fused_call(pool, layer, q, s, tables, max_entries, num_entries, rope_theta, out,
                      workspace, wl, hs);
  char* plan = static_cast<char*>(workspace) + wl.plan_off;
  const size_t pb = wl.ml_off - wl.plan_off;
  st = plan_call(pool, s, tables, max_entries, num_entries, plan, pb, hs);
  if (st != HW_OK) return st;
  return run_call(pool, layer, q, s, plan, pb, rope_theta, out, workspace, workspace_bytes, hs,
                  balance);
}

hw_status hw_attn_decode(const hw_pool* pool, int32_t layer, const void* q, int32_t num_workers,
                         int32_t num_q_heads, const hw_entry* tables, int32_t max_entries,
                         const int32_t* num_entries, double rope_theta, float* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return attn_call(pool, layer, q, num_workers, 1, num_q_heads, tables, max_entries, num_entries,
                   rope_theta, out, workspace, workspace_bytes, stream, g_balance);
}

hw_status hw_attn_chunk(const hw_pool* pool, int32_t layer, const void* q, int32_t num_workers,
                        int32_t chunk, int32_t num_q_heads, const hw_entry* tables,
                        int32_t max_entries, const int32_t* num_entries, double rope_theta,
                        float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (chunk < 1 || chunk > HW_MAX_ROWS) return HW_ERANGE;
  return attn_call(pool, layer, q, num_workers, chunk, num_q_heads, tables, max_entries,
                   num_entries, rope_theta, out, workspace, workspace_bytes, stream, g_balance);
}

hw_status hw_attn_decode_noalloc(const hw_pool* pool, int32_t layer, const void* q,
                                 int32_t num_workers, int32_t num_q_heads, const hw_entry* tables,
                                 int32_t max_entries, const int32_t* num_entries,
                                 double rope_theta, float* out, void* stream) {
  hw_status st = check_pool(pool);
  if (st != HW_OK) return st;
  Shape s;
  st = call_shape(pool, num_workers, 1, num_q_heads, &s);
  if (st != HW_OK) return st;
  // the call's workspace must fit the scratch (checked before any device call)
  if (ws_layout(pool, s).total > kScratchBytes) return HW_ERANGE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != HW_OK) return st;
  // fixed tile ranges: no region of the scratch has to start at zero
  return attn_call(pool, layer, q, num_workers, 1, num_q_heads, tables, max_entries, num_entries,
                   rope_theta, out, ws, kScratchBytes, stream, 0);
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
  st = check_scales(pool, layer);
  if (st != HW_OK) return st;
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

hw_status hw_pool_status(const hw_pool* pool, int32_t* flags, int32_t clear, void* stream) {
  if (!pool || !pool->status || !flags) return HW_EINVAL;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  if (hipMemcpyAsync(&v, pool->status, sizeof(int32_t), hipMemcpyDeviceToHost, hs) != hipSuccess)
    return HW_EHIP;
  if (clear) {
    static const int32_t zero = 0;
    if (hipMemcpyAsync(pool->status, &zero, sizeof(int32_t), hipMemcpyHostToDevice, hs) !=
        hipSuccess)
      return HW_EHIP;
  }
  if (hipStreamSynchronize(hs) != hipSuccess) return HW_EHIP;
  *flags = v;
  return HW_OK;
}

}  // extern "C"
