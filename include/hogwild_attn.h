/*
 * hogwild_attn.h — libhogwild_attn: Hogwild! concurrent-attention decode and
 * step-completion block append on AMD Instinct MI355X (gfx950).
 *
 * What the library computes (Hogwild! Inference, NeurIPS 2025 notes):
 *  - Several workers share one KV cache made of blocks.  Worker w's view is a
 *    list of (block, view_offset) entries; in the combined layout (key design
 *    2) it is [common cache, the other workers' unfinished steps in worker
 *    order, w's own step].
 *  - Every block stores its keys at local positions 0..len-1 (storage
 *    convention in the method list); the real position of token j of a block
 *    in w's view is view_offset + j.
 *  - Attention rotates only the single query token (key design 1):
 *      rho(q, i_q)[rho(A,i_A) (+) rho(B,i_B) ...]
 *        = rho(q, i_q - i_A) A (+) rho(q, i_q - i_B) B ...
 *    i.e. each block is scored with the query rotated by i_q - view_offset,
 *    and one softmax runs over the concatenation of all blocks' scores
 *    (omica.com.cn news 1114328, sec. 3.2: scores / sqrt(dim), softmax over
 *    concat, weighted sum of V).
 *  - A finished step's KV is rotated and moved into the shared history
 *    (key design 2, last paragraph).
 *
 * Conventions fixed where the pages are silent:
 *  - RoPE pairs element i with i + D/2 (rotate-half, news 1114328 sec. 2.1),
 *    angle = position * theta^(-2i/D), theta passed by the caller.
 *  - i_q[w] = max over w's entries with len > 0 of (view_offset + len) - 1:
 *    the query's own K/V is already in its block, as in ordinary decode.
 *  - Softmax scale 1/sqrt(D); no mask inside a view; kv head of q-head h is
 *    h / (Hq / Hkv).
 *  - `out` is fp32 whatever the pool type.
 *
 * Memory: every pointer marked (device) is device memory on the current HIP
 * device; (host) is host memory read during the call.  The caller owns every
 * buffer.  q, out, plans and workspaces are 16-byte aligned (HW_EINVAL
 * otherwise).  No call allocates, frees or synchronizes, except hw_pool_status()
 * (which synchronizes its stream).  All device work is enqueued on `stream`
 * (a hipStream_t; NULL = default stream) and calls return after enqueueing.
 *
 * Errors: problems visible on the host are reported by the return code and
 * then nothing is enqueued.  Problems only visible on the device (lengths
 * read from device memory, device-resident tables) set bits in the pool's
 * sticky status word (HW_DEV_*) and the affected work is skipped: decode rows
 * of an affected worker are written as zeros, an overflowing append moves
 * nothing.  hw_pool_status() reads and optionally clears that word.
 */
#ifndef HOGWILD_ATTN_H
#define HOGWILD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HW_ABI_VERSION 3

/* Tokens per tile of the pool layout; block starts and capacities are multiples of it. */
#define HW_TILE_TOKENS 32
#define HW_MAX_BLOCKS 64   /* blocks per pool                          */
#define HW_MAX_WORKERS 32  /* workers per decode call                  */
#define HW_MAX_ROWS 80     /* num_workers * chunk * (num_q_heads / num_kv_heads);
                              64 for fp32 pools and the VALU path      */
#define HW_MAX_ENTRIES 64  /* entries per worker table                 */
#define HW_MAX_FP8_KV_HEADS 64 /* kv heads of an HW_FP8 pool             */

typedef int32_t hw_status;
#define HW_OK 0
#define HW_EINVAL 1        /* null pointer, bad shape, bad id, src == dst      */
#define HW_ERANGE 2        /* a value outside the supported limits above       */
#define HW_ECAPACITY 3     /* (reserved; capacities are checked on the device) */
#define HW_EUNSUPPORTED 4  /* dtype / head_dim / path combination not built    */
#define HW_EWORKSPACE 5    /* workspace or plan missing or smaller than required */
#define HW_EHIP 6          /* a HIP runtime call failed                        */

/* Device-detected conditions (sticky bits of the pool status word). */
#define HW_DEV_BAD_ENTRY 1       /* table entry with block id out of range, a block listed twice,
                                    or a view whose positions i_q - view_offset reach 2^31  */
#define HW_DEV_BAD_LENGTH 2      /* block_len < 0 or > capacity                                      */
#define HW_DEV_NO_TOKENS 4       /* a worker sees no token; its rows are written as zeros            */
#define HW_DEV_APPEND_OVERFLOW 8 /* len_dst + len_src > cap_dst at run time; nothing was moved        */
#define HW_DEV_WRITE_OVERFLOW 16 /* advance past a block's capacity, or a token write into an empty block */
#define HW_DEV_STALE_PLAN 32     /* hw_attn_run: the plan was made for another call shape or pool
                                    (its units are skipped and their rows written as zeros), or a
                                    block length changed since the plan was made                   */
#define HW_DEV_WORKSPACE 64      /* a run's work units did not cover every tile exactly once: the
                                    workspace's counters were not zero when the call started       */
#define HW_DEV_SPIN_LIMIT 128    /* a wait between the waves of one work unit of a decode call gave up
                                    after its limit (about 0.25 s; HW_SPIN_LIMIT in the environment
                                    sets it in polls, for tests): that unit skipped its tiles, so the
                                    call's outputs are wrong, but the launch ended                 */

/* Storage types. */
#define HW_F32 0
#define HW_BF16 1
/*
 * HW_FP8: OCP FP8 E4M3 ("e4m3fn": bias 7, 3 mantissa bits, subnormals, no
 * infinity, 0x7f/0xff NaN, largest finite 448), one byte per element, with a
 * per-(layer, kv head) scale for keys and one for values: the stored value
 * is code * scale.  This is the FP8 attention of the mixed-precision item of
 * news 1114328 sec. 6; the pages give no format, so OCP E4M3, the FP8 format
 * of the MI355X matrix cores, is used.  Queries stay bf16.
 */
#define HW_FP8 2

/* One entry of a worker's view: block id and where the block starts in the view. */
typedef struct {
  int32_t block_id;
  int32_t view_offset;
} hw_entry;

/*
 * A K/V block pool spanning all layers of a model.
 *
 * Storage.  k and v each hold num_layers * num_kv_heads planes of num_slots
 * slots of head_dim elements of `dtype`; plane (layer l, kv head g) starts at
 * element (l * num_kv_heads + g) * num_slots * head_dim.  Block b owns slots
 * [block_start[b], block_start[b] + block_cap[b]) of every plane; its token j
 * (local position j, 0 <= j < block_len[b]) is slot block_start[b] + j.
 *
 * Within a plane, slots are grouped in tiles of 32 (tile T = slot / 32,
 * t = slot % 32, tile base = T * 32 * head_dim elements) laid out to match the
 * gfx950 16x16x32 bf16 MFMA operand fragments, so that every wave load is one
 * contiguous 16-byte vector per lane:
 *   key   element (slot, d) at tile base + (t / 16) * 16 * D + (d / 8) * 128
 *                                       + (t % 16) * 8 + d % 8
 *   value element (slot, d) at tile base + ((t % 16) / 4) * 8 * D + d * 8
 *                                       + (t / 16) * 4 + t % 4
 * The same layout is used for fp32 and FP8 pools (element offsets are equal;
 * an FP8 fragment is 8 bytes).
 *
 * block_len is device memory and is changed by hw_block_append /
 * hw_block_reset / hw_block_advance; block_start and block_cap are host
 * arrays and fixed for the pool's lifetime.  status is a device int32 holding
 * the sticky HW_DEV_* bits; the caller zeroes it once.
 */
typedef struct {
  int32_t dtype;        /* HW_F32, HW_BF16 or HW_FP8                       */
  int32_t num_layers;   /* >= 1                                            */
  int32_t num_kv_heads; /* >= 1 (FP8 pools: <= HW_MAX_FP8_KV_HEADS)       */
  int32_t head_dim;     /* 64 or 128                                       */
  int32_t num_blocks;   /* 1 .. HW_MAX_BLOCKS                              */
  int32_t reserved;     /* must be 0                                       */
  int64_t num_slots;    /* slots per plane, multiple of 32                 */
  void* k;              /* (device) key planes                             */
  void* v;              /* (device) value planes                           */
  int32_t* block_len;   /* (device) [num_blocks] current lengths           */
  int32_t* status;      /* (device) sticky HW_DEV_* bits                   */
  const int64_t* block_start; /* (host) [num_blocks], multiples of 32      */
  const int32_t* block_cap;   /* (host) [num_blocks], multiples of 32      */
  /* (host) [num_layers][num_kv_heads] positive finite scales of an HW_FP8
   * pool (key and value); NULL for the other types.  A call reads the
   * scales of the layer it works on. */
  const float* k_scale;
  const float* v_scale;
} hw_pool;

/* Returns HW_ABI_VERSION. */
int32_t hw_abi_version(void);

/* Static text for a hw_status code. */
const char* hw_status_str(hw_status status);

/*
 * Decode in two parts (key design 1 and 2: within one decode step every
 * layer sees the same views, so everything that depends on the views and
 * the block lengths but not on the layer is built once per step):
 *
 *   hw_attn_plan   reads the worker tables and the device block lengths and
 *                  writes a plan: which blocks are visible, how their tiles
 *                  are split into work units, and for every visible block
 *                  and query row the row's rotation delta
 *                  i_q - lag - view_offset.  One small launch.
 *   hw_attn_run    one layer's attention from a plan: one launch.
 *
 * hw_attn_decode / hw_attn_chunk give the same result from the tables on
 * every call (up to 32 stacked rows on bf16 and FP8 pools with the plan built
 * inside the attention launch itself, otherwise plan then run; on the QwQ
 * step with 4 workers and a 16K shared history the in-launch plan measured
 * 18.3 us per call against 19.8 us for run from a plan).  A plan stays valid
 * while the tables, entry counts and block lengths it was made from are
 * unchanged (token writes into already reserved slots do not change them);
 * a run whose plan does not fit its call, or whose pool's lengths changed,
 * reports HW_DEV_STALE_PLAN.
 */

/* Bytes of a plan for `num_workers` workers with `chunk` query tokens each
 * (chunk = 1: decode).  0 if the shape is invalid. */
size_t hw_attn_plan_bytes(const hw_pool* pool, int32_t num_workers, int32_t chunk,
                          int32_t num_q_heads);

/*
 *   tables       (device) [num_workers][max_entries] views; worker w uses its
 *                first num_entries[w] entries.  A block not listed is invisible
 *                to w; a block may be listed at most once per worker.
 *   num_entries  (device) [num_workers].
 *   plan         (device) >= hw_attn_plan_bytes(...) bytes, written.
 * Host-checked errors: HW_EINVAL (null pointers, num_q_heads % num_kv_heads,
 * max_entries < 1), HW_ERANGE (limits above, chunk < 1), HW_EUNSUPPORTED,
 * HW_EWORKSPACE (plan too small), HW_EHIP (launch failure).  Malformed tables
 * and lengths set HW_DEV_BAD_ENTRY / HW_DEV_BAD_LENGTH when the plan is built.
 */
hw_status hw_attn_plan(const hw_pool* pool, int32_t num_workers, int32_t chunk,
                       int32_t num_q_heads, const hw_entry* tables, int32_t max_entries,
                       const int32_t* num_entries, void* plan, size_t plan_bytes, void* stream);

/*
 * Bytes of device workspace a call needs for this pool and call shape under
 * the current tuning and device (for chunks pass num_workers * chunk): the
 * per-kv-head tile counters, a plan (used by hw_attn_decode / hw_attn_chunk)
 * and the work units' partial states.  Returns 0 if the shape is invalid.
 * The first 16 KB (the tile counters) must be zero before the workspace's
 * first use; every call leaves them zero, so one workspace serves any
 * sequence of calls on one stream (a call that finds them otherwise reports
 * HW_DEV_WORKSPACE).  Calls that may overlap need distinct workspaces.
 */
size_t hw_attn_workspace_bytes(const hw_pool* pool, int32_t num_workers, int32_t num_q_heads);

/*
 * One layer of attention from a plan made by hw_attn_plan with the same
 * pool, num_workers, chunk and num_q_heads.
 *   q    (device) [num_workers][chunk][num_q_heads][head_dim], fp32 for fp32
 *        pools, bf16 for bf16 and FP8 pools: the current query tokens of each
 *        worker, before RoPE.
 *   out  (device) [num_workers][chunk][num_q_heads][head_dim] fp32.
 *   workspace (device) >= hw_attn_workspace_bytes(pool, num_workers * chunk,
 *        num_q_heads) bytes.
 * For each worker w, query token j and q-head h (kv head g = h / (Hq/Hkv)),
 * with query j at view position i_q[w] - (chunk - 1 - j):
 *   out[w][j][h] = sum over entries (b, off) and positions p < len_b with
 *       off + p <= i_q[w] - (chunk - 1 - j) of
 *       softmax_p( rho(q[w][j][h], i_q[w] - (chunk - 1 - j) - off) . K_b[g][p] / sqrt(D) ) V_b[g][p]
 * (chunk = 1: every listed token, no mask).  FP8 pools: K and V are
 * code * scale of their (layer, kv head); the products run on the bf16
 * matrix cores with the codes widened exactly.  Rows that see no token are
 * written as zeros and set HW_DEV_NO_TOKENS.
 * A call is one launch of work units (split-K over the visible tiles) and,
 * with several units per kv head, one launch merging their partials.
 * Host-checked errors: HW_EINVAL (null pointers, num_q_heads % num_kv_heads,
 * layer out of range, theta), HW_ERANGE (limits above), HW_EUNSUPPORTED
 * (head_dim; FP8 pools with the VALU path forced; fp32 pools with the MFMA
 * path forced or more than 64 rows), HW_EWORKSPACE, HW_EHIP.
 */
hw_status hw_attn_run(const hw_pool* pool, int32_t layer, const void* q, int32_t num_workers,
                      int32_t chunk, int32_t num_q_heads, const void* plan, size_t plan_bytes,
                      double rope_theta, float* out, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * One layer of concurrent-attention decode (key design 1; news 1114328 sec.
 * 3.2), the output of hw_attn_plan + hw_attn_run with chunk = 1.  bf16 and
 * FP8 pools with up to 32 stacked rows (num_workers * num_q_heads /
 * num_kv_heads) on the MFMA path take one launch that builds the plan inside
 * every work unit, then the merge launch (measured faster than reading a
 * plan made once per step); other calls run hw_attn_plan into the workspace,
 * then hw_attn_run.
 *   q            (device) [num_workers][num_q_heads][head_dim].
 *   tables, num_entries as hw_attn_plan.
 *   out          (device) [num_workers][num_q_heads][head_dim] fp32.
 *   workspace    (device) >= hw_attn_workspace_bytes(pool, W, Hq) bytes.
 * Errors as hw_attn_plan and hw_attn_run.  Malformed tables and lengths set
 * HW_DEV_BAD_ENTRY / HW_DEV_BAD_LENGTH on every call.
 */
hw_status hw_attn_decode(const hw_pool* pool, int32_t layer, const void* q, int32_t num_workers,
                         int32_t num_q_heads, const hw_entry* tables, int32_t max_entries,
                         const int32_t* num_entries, double rope_theta, float* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * hw_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation).  The call's workspace is a static array of
 * HW_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held until the
 * process ends; the call allocates nothing and always uses the fixed tile
 * order (bitwise the same result as hw_attn_decode with balance 0).
 * Every call on one GPU shares that GPU's scratch: calls that may overlap
 * (on different streams) race and must be ordered by the caller.
 * Errors as hw_attn_decode, and HW_ERANGE when the call's workspace
 * (hw_attn_workspace_bytes(pool, num_workers, num_q_heads)) exceeds the
 * scratch.
 */
#define HW_NOALLOC_SCRATCH_BYTES (16u << 20)
hw_status hw_attn_decode_noalloc(const hw_pool* pool, int32_t layer, const void* q,
                                 int32_t num_workers, int32_t num_q_heads, const hw_entry* tables,
                                 int32_t max_entries, const int32_t* num_entries,
                                 double rope_theta, float* out, void* stream);

/*
 * Multi-token query chunk: every worker attends with its last `chunk` tokens
 * at once (a prompt injected into, or a header prefilled in, its own block,
 * whose K/V are already stored; key design 2's "\n\n + worker" header, key
 * design 3's periodic self-check prompt).  Executed as hw_attn_decode: up to
 * 32 stacked rows (num_workers * chunk * num_q_heads / num_kv_heads) in one
 * launch with the plan built in-launch, otherwise hw_attn_plan then
 * hw_attn_run.
 *   q    (device) [num_workers][chunk][num_q_heads][head_dim], dtype as for decode.
 *   out  (device) [num_workers][chunk][num_q_heads][head_dim] fp32.
 *   workspace: hw_attn_workspace_bytes(pool, num_workers * chunk, num_q_heads).
 */
hw_status hw_attn_chunk(const hw_pool* pool, int32_t layer, const void* q, int32_t num_workers,
                        int32_t chunk, int32_t num_q_heads, const hw_entry* tables,
                        int32_t max_entries, const int32_t* num_entries, double rope_theta,
                        float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Step completion (key design 2: a finished step's KV is rotated and moved
 * into the shared history), for every layer and kv head of the pool.
 * With n = block_len[src] and m = block_len[dst] read on the device: for
 * j < n, dst token m + j receives the src key re-encoded at local position
 * m + j (rotated by m with fp64 intermediates, rounded to nearest-even in the
 * pool type) and the src value unchanged; then block_len[dst] = m + n and
 * block_len[src] = 0.  src data is left in place.  FP8 pools: src and dst
 * share the plane's key scale, so the codes are rotated and rounded to the
 * nearest E4M3 code (saturating at 448).
 * Host-checked: HW_EINVAL (ids, src == dst, theta).  Capacities are checked
 * on the device against the run-time lengths (HW_DEV_APPEND_OVERFLOW).
 */
hw_status hw_block_append(const hw_pool* pool, int32_t src_block, int32_t dst_block,
                          double rope_theta, void* stream);

/*
 * Sets block_len[block] = 0 on the device: a worker whose step was moved into
 * the shared history starts its next step in an empty block (key design 2,
 * last paragraph).  Host-checked: HW_EINVAL (id).
 */
hw_status hw_block_reset(const hw_pool* pool, int32_t block, void* stream);

/*
 * Token write, part 1: reserves the next slot of every listed block for the
 * decode step's new token: block_len[b] += 1 on the device.  A block already
 * at capacity keeps its length and sets HW_DEV_WRITE_OVERFLOW.
 *   blocks (host) [n], 1 <= n <= HW_MAX_WORKERS, distinct ids.
 * Host-checked: HW_EINVAL (null, ids out of range or repeated), HW_ERANGE (n).
 */
hw_status hw_block_advance(const hw_pool* pool, int32_t n, const int32_t* blocks, void* stream);

/*
 * Token write, part 2, for one layer: stores each listed block's new token in
 * the slot reserved by hw_block_advance, p = block_len[b] - 1, read on the
 * device.  Keys are stored encoded at their local position (Hogwild! notes,
 * key design 1: a block holds its keys at positions 0..len-1): key slot p of
 * kv head h receives rho(k_new[i][h], p), computed with fp64 intermediates and
 * rounded to nearest even in the pool type; value slot p receives v_new[i][h]
 * rounded the same way (FP8 pools: the codes nearest to x / scale of the
 * layer's kv head, saturating at 448).  Lengths are not changed.  A listed block of length 0
 * is skipped and sets HW_DEV_WRITE_OVERFLOW.
 *   blocks (host) [n], as for hw_block_advance.
 *   k_new, v_new (device) [n][num_kv_heads][head_dim] fp32.
 * Host-checked: HW_EINVAL (null, ids, layer, theta), HW_ERANGE (n).
 */
hw_status hw_block_write(const hw_pool* pool, int32_t layer, int32_t n, const int32_t* blocks,
                         const float* k_new, const float* v_new, double rope_theta,
                         void* stream);

/*
 * Combined layout (key design 2) built on the device from the current
 * block lengths: for worker w the entries are common_block at offset 0, then
 * worker_block[v] for v != w in increasing v, then worker_block[w]; each
 * view_offset is the running sum of the preceding blocks' lengths.
 *   worker_block (host) [num_workers], distinct, != common_block.
 *   tables       (device) [num_workers][num_workers + 1] written.
 *   num_entries  (device) [num_workers] written (= num_workers + 1).
 */
hw_status hw_build_combined_tables(const hw_pool* pool, int32_t num_workers, int32_t common_block,
                                   const int32_t* worker_block, hw_entry* tables,
                                   int32_t* num_entries, void* stream);

/*
 * The cache layouts of the Hogwild! notes' layout ablation, as view tables
 * built on the device (same arguments and table shape as
 * hw_build_combined_tables; entries past num_entries[w] are zeroed):
 *   HW_LAYOUT_COMBINED     token-wise sync plus step history: the combined
 *                          layout above.
 *   HW_LAYOUT_INTERLEAVED  step-level sync only: [common_block @ 0,
 *                          worker_block[w] @ len(common)]; the other workers'
 *                          current steps are not visible until appended.
 *   HW_LAYOUT_CONTIGUOUS   token-level sync only: each worker's whole output
 *                          stays in its own block (no step history is ever
 *                          appended); the tables have the combined order.
 * Host-checked: as hw_build_combined_tables, plus HW_EINVAL for the layout.
 */
#define HW_LAYOUT_COMBINED 0
#define HW_LAYOUT_INTERLEAVED 1
#define HW_LAYOUT_CONTIGUOUS 2
hw_status hw_build_view_tables(const hw_pool* pool, int32_t layout, int32_t num_workers,
                               int32_t common_block, const int32_t* worker_block,
                               hw_entry* tables, int32_t* num_entries, void* stream);

/*
 * Reads the pool's sticky HW_DEV_* bits into *flags (host) once the work
 * enqueued on `stream` so far has completed (synchronizes that stream only).
 * clear != 0 zeroes the word afterwards (on the same stream, completed
 * before the call returns).
 */
hw_status hw_pool_status(const hw_pool* pool, int32_t* flags, int32_t clear, void* stream);

/*
 * Process-wide tuning (not thread-safe against concurrent decode calls).
 *   path:           0 auto, 1 VALU fp32 kernel (fp32 and bf16 pools), 2 MFMA
 *                   bf16 kernel (bf16 and FP8 pools).
 *   units_per_head: number of split-K work units per kv head; 0 = automatic
 *                   (the device's resident workgroups divided by the kv
 *                   heads).  Values above what the device holds at once are
 *                   lowered to it.
 *   balance:        0 (default): every unit takes a fixed contiguous range
 *                   of the visible tiles, and results are bitwise the same
 *                   on every run.  1: each wave takes one tile and then
 *                   tiles from a per-kv-head counter, so units that HBM
 *                   serves faster take more tiles (the MFMA path, when
 *                   every visible block's rotated queries fit in LDS: at
 *                   most 6 visible blocks); results then vary in the last
 *                   bits from run to run, and the per-tile counter atomics
 *                   cost more than they balance (the 16K QwQ step's plan +
 *                   run call: 30.2 against 19.9 us).
 * Returns HW_EINVAL for values out of range.
 */
hw_status hw_set_tuning(int32_t path, int32_t units_per_head, int32_t balance);

#ifdef __cplusplus
}
#endif

#endif /* HOGWILD_ATTN_H */
