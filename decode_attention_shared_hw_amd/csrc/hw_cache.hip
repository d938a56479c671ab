// hw_cache.hip — cache-manager kernels: combined-layout tables, step append,
// block reset.  (Hogwild! Inference notes, key design 2.)
#include <math.h>

#include <type_traits>

#include "hw_internal.h"

namespace hw {
namespace {

// ------------------------------------------------------------- tables (a1)
struct TableArgs {
  const int32_t* block_len;
  hw_entry* tables;  // [W][W+1]
  int32_t* num_entries;
  int32_t W, common, num_blocks, layout;
  int32_t worker_block[HW_MAX_WORKERS];
};

// Thread w writes worker w's view; view_offset = running length sum.
//   combined / contiguous: common cache, the other workers' blocks in
//     increasing worker id, its own block last;
//   interleaved: common cache, its own block (the others' current steps are
//     not visible); unused entries are zeroed.
__global__ void build_tables_kernel(TableArgs a) {
  const int w = threadIdx.x;
  if (w >= a.W) return;
  const int E = a.W + 1;
  hw_entry* row = a.tables + static_cast<int64_t>(w) * E;
  int e = 0;
  int32_t off = 0;
  auto put = [&](int32_t b) {
    row[e].block_id = b;
    row[e].view_offset = off;
    const int32_t len = a.block_len[b];
    off += len > 0 ? len : 0;
    ++e;
  };
  put(a.common);
  if (a.layout != HW_LAYOUT_INTERLEAVED)
    for (int v = 0; v < a.W; ++v)
      if (v != w) put(a.worker_block[v]);
  put(a.worker_block[w]);
  a.num_entries[w] = e;
  for (int k = e; k < E; ++k) {
    row[k].block_id = 0;
    row[k].view_offset = 0;
  }
}

// ------------------------------------------------------------- append (a5)
struct AppendArgs {
  void* k;
  void* v;
  int32_t* block_len;
  int64_t plane_elems;  // num_slots * D
  int64_t start_src, start_dst;
  int32_t cap_src, cap_dst;
  int32_t src, dst;
  int32_t D, dtype;
  int32_t tiles_per_plane;  // dst tiles a run of up to cap_src tokens can touch
  int32_t xcd_map;          // 1: consecutive tiles of a plane on one XCD
  int64_t planes;           // layers * kv heads
  double inv_freq[kMaxHalf];
};

// Correctly rounded double -> bf16 (ties to even), as raw bits.
__device__ uint16_t f64_to_bf16_bits(double x) {
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t e = static_cast<uint32_t>((u >> 52) & 0x7ffu);
  if (e == 0x7ffu) return static_cast<uint16_t>(__float_as_uint(static_cast<float>(x)) >> 16);
  double y;
  if (e < 1023u - 126u) {
    // below the smallest normal bf16: the grid step is 2^-133
    y = rint(x * 0x1p133) * 0x1p-133;
  } else {
    // keep 8 significant bits: drop 45 of the 52 fraction bits, ties to even
    const uint64_t lsb = (u >> 45) & 1u;
    u += 0x00000FFFFFFFFFFFull + lsb;  // 2^44 - 1 + lsb
    u &= ~0x00001FFFFFFFFFFFull;       // clear the 45 dropped bits
    y = __longlong_as_double(static_cast<long long>(u));
  }
  // y is a bf16 value (or beyond its range, which float turns into inf)
  return static_cast<uint16_t>(__float_as_uint(static_cast<float>(y)) >> 16);
}

// Nearest OCP FP8 E4M3 code (ties to even) in one step from the double.  The
// grid at |x| in [2^(k-1), 2^k) has 3 fraction bits (quantum 2^(k-4)); below
// 2^-6 the subnormal quantum 2^-9.  The format has no infinity: magnitudes
// from 448 up saturate to 448 (code 0x7e; 464 is the tie between 448 and the
// unrepresentable 480 and goes to the even code 0x7e).  Codes are monotonic in
// the magnitude, so the code is the exponent field and the rounded mantissa
// added together.
__device__ uint8_t f64_to_e4m3(double x) {
  if (x != x) return 0x7f;
  const uint32_t sign = signbit(x) ? 0x80u : 0u;
  const double a = fabs(x);
  if (a >= 448.0) return static_cast<uint8_t>(sign | 0x7eu);
  if (a == 0.0) return static_cast<uint8_t>(sign);
  int k = 0;
  frexp(a, &k);
  const int qexp = k - 4 < -9 ? -9 : k - 4;
  const int r = static_cast<int>(rint(ldexp(a, -qexp)));  // 0..16
  const int code = qexp == -9 ? r : ((qexp + 10) << 3) + r - 8;
  return static_cast<uint8_t>(sign | static_cast<uint32_t>(code));
}

// Value of an E4M3 code (bias 7, 3 mantissa bits, subnormals below 2^-6).
__device__ __forceinline__ double e4m3_to_f64(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return __longlong_as_double(0x7ff8000000000000ll);
  const double v = e == 0 ? ldexp(static_cast<double>(m), -9)
                          : ldexp(static_cast<double>(8 + m), e - 10);
  return (c & 0x80) ? -v : v;
}

__device__ __forceinline__ double to_f64(float x) { return x; }
__device__ __forceinline__ double to_f64(uint16_t b) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(b) << 16));
}
__device__ __forceinline__ double to_f64(uint8_t c) { return e4m3_to_f64(c); }
template <typename T>
__device__ __forceinline__ T round_to(double x);
template <>
__device__ __forceinline__ float round_to<float>(double x) { return static_cast<float>(x); }
template <>
__device__ __forceinline__ uint16_t round_to<uint16_t>(double x) { return f64_to_bf16_bits(x); }
template <>
__device__ __forceinline__ uint8_t round_to<uint8_t>(double x) { return f64_to_e4m3(x); }

// Data moves in chunks of consecutive elements of one layout unit (a key
// token's dims, a value dim's tokens): 16 bytes, or 8 for FP8 pools, whose
// 16-byte runs would span two units.
template <typename T>
struct ChunkOf {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  static constexpr int kBytes = sizeof(T) == 1 ? 8 : 16;
  static constexpr int kElems = kBytes / static_cast<int>(sizeof(T));
  typedef typename std::conditional<kBytes == 16, u32x4, u32x2>::type type;
};

// A chunk's elements as doubles (exact).  FP8 codes widen through the
// hardware's exact E4M3 -> bf16 conversion (unit scale).
template <typename T, typename Chunk, int N>
__device__ __forceinline__ void widen_chunk(const Chunk& c, double (&x)[N]) {
  const T* e = reinterpret_cast<const T*>(&c);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = to_f64(e[i]);
}
template <>
__device__ __forceinline__ void widen_chunk<uint8_t>(const ChunkOf<uint8_t>::type& c,
                                                       double (&x)[8]) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t lo = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[w], 1.0f, false));
    const uint32_t hi = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[w], 1.0f, true));
    x[4 * w + 0] = __uint_as_float(lo << 16);
    x[4 * w + 1] = __uint_as_float(lo & 0xffff0000u);
    x[4 * w + 2] = __uint_as_float(hi << 16);
    x[4 * w + 3] = __uint_as_float(hi & 0xffff0000u);
  }
}


// One workgroup per (layer*kv head plane, destination tile).  A src key at
// local position j moves to dst position len_dst + j: rotating it by len_dst
// re-encodes it there (rho(rho(x, j), n) = rho(x, j + n)).
//
// Data move in chunks (kChunk elements, ChunkOf).  In the key layout a chunk
// holds consecutive dims of one token, so a lane loads a chunk and its
// rotate-half partner chunk (dims + D/2) of one src token, rotates the pairs
// in fp64 and stores both rounded.  In the value layout a chunk holds one dim
// of several tokens, and the shift by len_dst mixes tokens of two src tiles:
// the run's src values are staged in LDS (token-major), then every dst chunk
// the run touches is rebuilt, keeping the tokens outside the run, and stored
// whole.  FP8 pools: src and dst share the plane's scale, so the codes
// themselves are rotated and rounded.
template <typename T, int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
#pragma clang fp contract(off)
  typedef typename ChunkOf<T>::type Chunk;
  constexpr int kChunk = ChunkOf<T>::kElems;
  const int tid = threadIdx.x;
  // consecutive dst tiles of one plane on one XCD (they share src tiles)
  int lin = blockIdx.x;
  if (a.xcd_map) lin = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int64_t plane = lin / a.tiles_per_plane;
  const int k = lin - static_cast<int>(plane * a.tiles_per_plane);  // dst tile of the run
  if (plane >= a.planes) return;
  const int32_t ls = a.block_len[a.src];
  const int32_t ld = a.block_len[a.dst];
  if (ls <= 0 || ld < 0 || ls > a.cap_src || static_cast<int64_t>(ld) + ls > a.cap_dst) return;
  const int64_t first = a.start_dst + ld;  // first destination slot
  const int64_t last = first + ls;
  const int64_t t0 = ((first >> 5) + k) << 5;  // the dst tile's first slot
  const int64_t s_begin = first > t0 ? first : t0;
  const int64_t s_end = last < t0 + 32 ? last : t0 + 32;
  if (s_begin >= s_end) return;  // the run ends before this tile
  // (D a template parameter: the chunk index arithmetic below is shifts and masks)
  constexpr int half = D / 2;
  __shared__ double cs[2 * kMaxHalf];
  __shared__ T vstage[32 * D];  // run values, [token - s_begin][dim]
  if (tid < half) {
    double s, c;
    sincos(static_cast<double>(ld) * a.inv_freq[tid], &s, &c);
    cs[2 * tid] = c;
    cs[2 * tid + 1] = s;
  }
  T* kp = static_cast<T*>(a.k) + plane * a.plane_elems;
  T* vp = static_cast<T*>(a.v) + plane * a.plane_elems;
  constexpr int cpt = 32 * D / kChunk;  // chunks per tile
  constexpr int cph = half / kChunk;    // key chunks per half
  const int n = static_cast<int>(s_end - s_begin);
  const int64_t ss0 = a.start_src + (s_begin - first);  // src slot of the first token
  // In the value layout element i of the chunk at element offset off of a tile
  // holds token (r8 / 4) * 16 + 4 g + r8 % 4 and dim d, where g = off / (8 D),
  // d = (off / 8) % D and r8 = off % 8 + i.
  // ---- values, phase 1: src chunks of the (at most two) src tiles the run
  // reads, scattered into LDS
  const int64_t st_lo = ss0 >> 5, st_hi = (ss0 + n - 1) >> 5;
  const int lo_j = static_cast<int>(st_lo * 32 - ss0);  // run position of the first src tile's slot 0
  for (int x = tid; x < static_cast<int>(st_hi - st_lo + 1) * cpt; x += 256) {
    const int tl = x / cpt;              // src tile of the run (0 or 1)
    const int off = (x % cpt) * kChunk;  // element offset inside the tile
    const int g = off / (8 * D), d = (off / 8) % D, r0 = off % 8;
    const Chunk raw = *reinterpret_cast<const Chunk*>(vp + (st_lo + tl) * 32 * D + off);
    const T* e = reinterpret_cast<const T*>(&raw);
    const int jb = lo_j + tl * 32 + 4 * g;
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int r8 = r0 + i;
      const int j = jb + (r8 >> 2) * 16 + (r8 & 3);
      if (j >= 0 && j < n) vstage[j * D + d] = e[i];
    }
  }
  __syncthreads();
  // ---- keys: chunk pairs (token, dims c*kChunk.. and + D/2)
  for (int x = tid; x < n * cph; x += 256) {
    const int j = x / cph;
    const int d0 = (x % cph) * kChunk;
    const Chunk r0 = *reinterpret_cast<const Chunk*>(kp + key_offset(ss0 + j, d0, D));
    const Chunk r1 = *reinterpret_cast<const Chunk*>(kp + key_offset(ss0 + j, d0 + half, D));
    Chunk w0, w1;
    T* o0 = reinterpret_cast<T*>(&w0);
    T* o1 = reinterpret_cast<T*>(&w1);
    double x0[kChunk], x1[kChunk];
    widen_chunk<T>(r0, x0);
    widen_chunk<T>(r1, x1);
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const double c = cs[2 * (d0 + i)], s = cs[2 * (d0 + i) + 1];
      o0[i] = round_to<T>(x0[i] * c - x1[i] * s);
      o1[i] = round_to<T>(x1[i] * c + x0[i] * s);
    }
    *reinterpret_cast<Chunk*>(kp + key_offset(s_begin + j, d0, D)) = w0;
    *reinterpret_cast<Chunk*>(kp + key_offset(s_begin + j, d0 + half, D)) = w1;
  }
  // ---- values, phase 2: every chunk of the dst tile holding a run token
  const int tb = static_cast<int>(s_begin - t0), te = static_cast<int>(s_end - t0);
  for (int x = tid; x < cpt; x += 256) {
    const int off = x * kChunk;
    const int g = off / (8 * D), d = (off / 8) % D, r0 = off % 8;
    bool any = false, whole = true;
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int r8 = r0 + i;
      const int t = (r8 >> 2) * 16 + 4 * g + (r8 & 3);
      const bool in = t >= tb && t < te;
      any = any || in;
      whole = whole && in;
    }
    if (!any) continue;  // no run token in this chunk
    T* dst = vp + t0 * D + off;
    Chunk raw = {};
    if (!whole) raw = *reinterpret_cast<const Chunk*>(dst);  // keep tokens outside the run
    T* e = reinterpret_cast<T*>(&raw);
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int r8 = r0 + i;
      const int t = (r8 >> 2) * 16 + 4 * g + (r8 & 3);
      if (t >= tb && t < te) e[i] = vstage[(t - tb) * D + d];
    }
    *reinterpret_cast<Chunk*>(dst) = raw;
  }
}

// Runs after the copy on the same stream: moves the lengths, or reports.
__global__ void append_finish_kernel(int32_t* block_len, int32_t* status, int32_t src,
                                     int32_t dst, int32_t cap_src, int32_t cap_dst) {
  if (threadIdx.x != 0) return;
  const int32_t ls = block_len[src];
  const int32_t ld = block_len[dst];
  if (ls < 0 || ld < 0 || ls > cap_src || ld > cap_dst) {
    atomicOr(status, HW_DEV_BAD_LENGTH);
    return;
  }
  if (static_cast<int64_t>(ld) + ls > cap_dst) {
    atomicOr(status, HW_DEV_APPEND_OVERFLOW);
    return;
  }
  block_len[dst] = ld + ls;
  block_len[src] = 0;
}

__global__ void reset_kernel(int32_t* block_len, int32_t block) {
  if (threadIdx.x == 0) block_len[block] = 0;
}

// ------------------------------------------------------------ token write
struct TokenArgs {
  void* k;
  void* v;
  int32_t* block_len;
  int32_t* status;
  const float* k_new;  // [n][Hkv][D]
  const float* v_new;
  int64_t plane_elems;
  int32_t n, Hkv, D;
  int32_t blocks[HW_MAX_WORKERS];
  int64_t start[HW_MAX_WORKERS];
  int32_t cap[HW_MAX_WORKERS];
  double inv_freq[kMaxHalf];
  float k_scale[HW_MAX_FP8_KV_HEADS];  // FP8 pools: this layer's scales per kv head
  float v_scale[HW_MAX_FP8_KV_HEADS];
};

// Thread i reserves the next slot of block blocks[i].
__global__ void advance_kernel(TokenArgs a) {
  const int i = threadIdx.x;
  if (i >= a.n) return;
  const int32_t b = a.blocks[i];
  const int32_t len = a.block_len[b];
  if (len < 0 || len >= a.cap[i]) {
    atomicOr(a.status, HW_DEV_WRITE_OVERFLOW);
    return;
  }
  a.block_len[b] = len + 1;
}

// One workgroup per (listed block i, kv head g); thread t < D/2 writes the
// rotate-half pair (t, t + D/2) of the key and of the value.  FP8 pools store
// the codes nearest to x / scale (the division in fp64).
template <typename T>
__global__ void write_kernel(TokenArgs a) {
#pragma clang fp contract(off)
  const int i = blockIdx.x / a.Hkv;
  const int g = blockIdx.x - i * a.Hkv;
  const int t = threadIdx.x;
  const int half = a.D / 2;
  const int32_t p = a.block_len[a.blocks[i]] - 1;
  if (p < 0 || p >= a.cap[i]) {
    if (t == 0) atomicOr(a.status, HW_DEV_WRITE_OVERFLOW);
    return;
  }
  if (t >= half) return;
  const int64_t slot = a.start[i] + p;
  const float* kr = a.k_new + (static_cast<int64_t>(i) * a.Hkv + g) * a.D;
  const float* vr = a.v_new + (static_cast<int64_t>(i) * a.Hkv + g) * a.D;
  double s, c;
  sincos(static_cast<double>(p) * a.inv_freq[t], &s, &c);
  const double x0 = kr[t], x1 = kr[t + half];
  T* kp = static_cast<T*>(a.k) + g * a.plane_elems;
  T* vp = static_cast<T*>(a.v) + g * a.plane_elems;
  const bool f8 = sizeof(T) == 1;
  const double ks = f8 ? static_cast<double>(a.k_scale[g]) : 1.0;
  const double vs = f8 ? static_cast<double>(a.v_scale[g]) : 1.0;
  const double k0 = x0 * c - x1 * s, k1 = x1 * c + x0 * s;
  const double v0 = vr[t], v1 = vr[t + half];
  kp[key_offset(slot, t, a.D)] = round_to<T>(f8 ? k0 / ks : k0);
  kp[key_offset(slot, t + half, a.D)] = round_to<T>(f8 ? k1 / ks : k1);
  vp[value_offset(slot, t, a.D)] = round_to<T>(f8 ? v0 / vs : v0);
  vp[value_offset(slot, t + half, a.D)] = round_to<T>(f8 ? v1 / vs : v1);
}

}  // namespace

hipError_t launch_advance(const hw_pool& pool, int32_t n, const int32_t* blocks, hipStream_t s) {
  TokenArgs a{};
  a.block_len = pool.block_len;
  a.status = pool.status;
  a.n = n;
  for (int i = 0; i < n; ++i) {
    a.blocks[i] = blocks[i];
    a.cap[i] = pool.block_cap[blocks[i]];
  }
  hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_write(const hw_pool& pool, int32_t layer, int32_t n, const int32_t* blocks,
                        const float* k_new, const float* v_new, double theta, hipStream_t s) {
  TokenArgs a{};
  const size_t esz = elem_bytes(pool.dtype);
  a.plane_elems = pool.num_slots * pool.head_dim;
  const int64_t layer_off = static_cast<int64_t>(layer) * pool.num_kv_heads * a.plane_elems;
  a.k = static_cast<char*>(pool.k) + layer_off * esz;
  a.v = static_cast<char*>(pool.v) + layer_off * esz;
  a.block_len = pool.block_len;
  a.status = pool.status;
  a.k_new = k_new;
  a.v_new = v_new;
  a.n = n;
  a.Hkv = pool.num_kv_heads;
  a.D = pool.head_dim;
  for (int i = 0; i < n; ++i) {
    a.blocks[i] = blocks[i];
    a.start[i] = pool.block_start[blocks[i]];
    a.cap[i] = pool.block_cap[blocks[i]];
  }
  for (int i = 0; i < pool.head_dim / 2; ++i)
    a.inv_freq[i] = pow(theta, -2.0 * i / static_cast<double>(pool.head_dim));
  if (pool.dtype == HW_FP8) {
    const int64_t l0 = static_cast<int64_t>(layer) * pool.num_kv_heads;
    for (int g = 0; g < pool.num_kv_heads; ++g) {
      a.k_scale[g] = pool.k_scale[l0 + g];
      a.v_scale[g] = pool.v_scale[l0 + g];
    }
  }
  const dim3 grid(static_cast<unsigned>(n * pool.num_kv_heads));
  if (pool.dtype == HW_F32)
    hipLaunchKernelGGL(write_kernel<float>, grid, dim3(64), 0, s, a);
  else if (pool.dtype == HW_BF16)
    hipLaunchKernelGGL(write_kernel<uint16_t>, grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(write_kernel<uint8_t>, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_build_tables(int32_t* block_len, int32_t layout, int32_t W, int32_t common,
                               const int32_t* worker_block, hw_entry* tables,
                               int32_t* num_entries, int32_t num_blocks, hipStream_t s) {
  TableArgs a{};
  a.block_len = block_len;
  a.layout = layout;
  a.tables = tables;
  a.num_entries = num_entries;
  a.W = W;
  a.common = common;
  a.num_blocks = num_blocks;
  for (int w = 0; w < W; ++w) a.worker_block[w] = worker_block[w];
  hipLaunchKernelGGL(build_tables_kernel, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append(const hw_pool& pool, int32_t src, int32_t dst, double theta,
                         hipStream_t s) {
  AppendArgs a{};
  a.k = pool.k;
  a.v = pool.v;
  a.block_len = pool.block_len;
  a.plane_elems = pool.num_slots * pool.head_dim;
  a.start_src = pool.block_start[src];
  a.start_dst = pool.block_start[dst];
  a.cap_src = pool.block_cap[src];
  a.cap_dst = pool.block_cap[dst];
  a.src = src;
  a.dst = dst;
  a.D = pool.head_dim;
  a.dtype = pool.dtype;
  a.tiles_per_plane = a.cap_src / kTile + 1;
  for (int i = 0; i < pool.head_dim / 2; ++i)
    a.inv_freq[i] = pow(theta, -2.0 * i / static_cast<double>(pool.head_dim));
  const int64_t planes = static_cast<int64_t>(pool.num_layers) * pool.num_kv_heads;
  a.planes = planes;
  int64_t grid = planes * a.tiles_per_plane;
  if (grid >= 8) {
    grid = (grid + 7) / 8 * 8;  // whole rounds of the 8 XCDs; the excess exits at once
    a.xcd_map = 1;
  }
  if (a.cap_src > 0 && grid > 0) {
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 g(static_cast<unsigned>(grid));
    const bool d128 = pool.head_dim == 128;
    if (pool.dtype == HW_F32) {
      if (d128) hipLaunchKernelGGL((append_kernel<float, 128>), g, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((append_kernel<float, 64>), g, dim3(256), 0, s, a);
    } else if (pool.dtype == HW_BF16) {
      if (d128) hipLaunchKernelGGL((append_kernel<uint16_t, 128>), g, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((append_kernel<uint16_t, 64>), g, dim3(256), 0, s, a);
    } else {
      if (d128) hipLaunchKernelGGL((append_kernel<uint8_t, 128>), g, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((append_kernel<uint8_t, 64>), g, dim3(256), 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(append_finish_kernel, dim3(1), dim3(64), 0, s, pool.block_len, pool.status,
                     src, dst, a.cap_src, a.cap_dst);
  return hipGetLastError();
}

hipError_t launch_reset(int32_t* block_len, int32_t block, hipStream_t s) {
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(64), 0, s, block_len, block);
  return hipGetLastError();
}

}  // namespace hw
