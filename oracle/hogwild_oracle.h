/*
 * hogwild_oracle.h — CPU reference ("oracle") for Hogwild! concurrent-attention
 * decode and the step-completion block append.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no source with the HIP library.
 *
 * Everything is plain, slow, single-threaded C++17 in fp64.  Arrays hold the
 * stored values exactly (bf16 / fp32 inputs widened to double by the caller).
 *
 * Sources (the pages this follows):
 *  - Hogwild! Inference (NeurIPS 2025 notes), "Key designs" 1: concurrent
 *    attention by rotating the query, the identity
 *      rho(q,i_q)[rho(A,i_A) (+) rho(B,i_B) (+) rho(C,i_C)]
 *        = rho(q,i_q-i_A)A (+) rho(q,i_q-i_B)B (+) rho(q,i_q-i_C)C.
 *  - same page, "Key designs" 2: the combined layout (common cache, other
 *    workers' unfinished steps in worker order, the current worker last) and
 *    the step completion that rotates a finished step's KV into the shared
 *    history.
 *  - same page, "Training strategy" list: every block keeps its KV at local
 *    positions 0..len-1; real positions are handled by rotating the query.
 *  - omica.com.cn news 1114328, section 2.1 (rotate_query sketch: rotate-half
 *    RoPE pairing, inverse frequencies base^(-2i/dim)) and section 3.2
 *    (hogwild_attention sketch: per-block scores scaled by 1/sqrt(dim), one
 *    softmax over the concatenation of all blocks' scores, weighted sum of V).
 *
 * Readings where the pages are silent (each listed with its reason in the
 * design notes of the repository):
 *  - i_q, the query position, is the last visible position of the worker's
 *    view: max over non-empty entries of (view_offset + len) - 1.
 *  - RoPE pairs element i with element i + D/2 (rotate-half), frequency
 *    theta^(-2i/D), theta a parameter.
 *  - kv head of q-head h is h / (Hq / Hkv).
 *  - append: dst receives the src keys re-encoded at local positions
 *    len_dst + j, rounded to the storage type; V is copied; dst.len grows by
 *    src.len and src.len becomes 0.
 */
#ifndef HOGWILD_ORACLE_H
#define HOGWILD_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define HWO_OK 0
#define HWO_EINVAL 1    /* bad id, duplicate block, bad shape               */
#define HWO_ENOTOKENS 2 /* a worker sees no token: softmax undefined         */
#define HWO_ECAPACITY 3 /* append would overflow dst capacity                */

/* Storage types for rounding the appended keys. */
#define HWO_F32 0
#define HWO_BF16 1
#define HWO_FP8 2 /* OCP FP8 E4M3 codes times a per-(layer, kv head) scale */

/* Round a double to the nearest bf16 value (ties to even), returned as double. */
double hwo_round_bf16(double x);
/* Round a double to the nearest fp32 value (ties to even), returned as double. */
double hwo_round_f32(double x);

/*
 * OCP FP8 E4M3 (the "e4m3fn" variant): 1 sign bit, 4 exponent bits with bias
 * 7, 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; codes
 * 0x7f and 0xff are NaN and there are no infinities, so the largest finite
 * magnitude is 1.75 * 2^8 = 448.  The FP8 pool of the future-work note on
 * mixed precision (news 1114328 sec. 6) stores code * scale.
 */
/* The value of code & 0xff. */
double hwo_e4m3_value(int32_t code);
/* Round a double to the nearest E4M3 value (ties to even), saturating at +-448;
 * NaN stays NaN. */
double hwo_round_e4m3(double x);

/* RoPE, rotate-half pairing: y = rho(x, pos).  x, y: [D]; may alias. */
void hwo_rope(const double* x, int32_t D, double theta, double pos, double* y);

/*
 * Combined layout (a1).  For worker w the view is
 *   [common, worker_block[v] for v != w in increasing v, worker_block[w]]
 * with view_offset = running sum of block_len in that order.
 * Outputs: tbl_block/tbl_off [W][W+1] (row stride W+1), num_entries[W] = W+1.
 */
int32_t hwo_build_combined_tables(int32_t W, int32_t common_block, const int32_t* worker_block,
                                  int32_t num_blocks, const int32_t* block_len,
                                  int32_t* tbl_block, int32_t* tbl_off, int32_t* num_entries);

/*
 * Interleaved layout (the Hogwild! notes' layout ablation: step-level
 * synchronization only): worker w sees the common history of finished steps
 * and its own block, [common @ 0, worker_block[w] @ len(common)]; the other
 * workers' current blocks are not visible.  Same arguments, checks and table
 * shape as hwo_build_combined_tables (entries past num_entries[w] = 2 are 0).
 */
int32_t hwo_build_interleaved_tables(int32_t W, int32_t common_block, const int32_t* worker_block,
                                     int32_t num_blocks, const int32_t* block_len,
                                     int32_t* tbl_block, int32_t* tbl_off, int32_t* num_entries);

/* i_q of one worker's view: max over entries with len > 0 of (off + len) - 1; -1 if none. */
int64_t hwo_query_position(int32_t n_entries, const int32_t* tbl_block, const int32_t* tbl_off,
                           const int32_t* block_len);

/*
 * Attention for ONE (worker, q-head) pair over one kv-head plane.
 *   form 0: definition — every visible key is first brought back to its raw
 *           (position-free) value and re-encoded at its absolute view
 *           position off + j; the query is encoded at i_q; plain softmax
 *           attention over all visible tokens.
 *   form 1: method — the stored keys are used as they are; the query is
 *           rotated by i_q - off for each block.
 * q: [D]; K_plane, V_plane: [num_slots][D] for the kv head; block b's token j
 * lives in slot block_start[b] + j.  out: [D].
 */
int32_t hwo_attn_one(int32_t form, int32_t D, double theta, int32_t n_entries,
                     const int32_t* tbl_block, const int32_t* tbl_off, int32_t num_blocks,
                     const int32_t* block_len, const int64_t* block_start, const double* q,
                     const double* K_plane, const double* V_plane, double* out);

/*
 * Whole decode call: every worker w < W, every q-head h < Hq.
 *   q: [W][Hq][D]; K, V: [Hkv][num_slots][D]; tables [W][E]; out: [W][Hq][D].
 * Returns the first error met (outputs of a failing pair are zero).
 */
int32_t hwo_attn_decode(int32_t form, int32_t W, int32_t Hq, int32_t Hkv, int32_t D, double theta,
                        int32_t E, const int32_t* tbl_block, const int32_t* tbl_off,
                        const int32_t* num_entries, int32_t num_blocks, const int32_t* block_len,
                        const int64_t* block_start, int64_t num_slots, const double* q,
                        const double* K, const double* V, double* out);

/*
 * Multi-token query chunk: every worker attends with its last n tokens at
 * once (a prompt injected into, or a header prefilled in, its own block).
 * q, out: [W][n][Hq][D].  Query j of worker w sits at view position
 * i_q[w] - (n - 1 - j) and sees the view's tokens at positions up to its own
 * (a causal mask over the view); n = 1 is hwo_attn_decode.  A row that sees
 * no token is zero and the call returns HWO_ENOTOKENS.
 */
int32_t hwo_attn_chunk(int32_t form, int32_t W, int32_t n, int32_t Hq, int32_t Hkv, int32_t D,
                       double theta, int32_t E, const int32_t* tbl_block, const int32_t* tbl_off,
                       const int32_t* num_entries, int32_t num_blocks, const int32_t* block_len,
                       const int64_t* block_start, int64_t num_slots, const double* q,
                       const double* K, const double* V, double* out);

/*
 * Step completion (a5) over all layers.  K, V: [L][Hkv][num_slots][D].
 * For j < len_src: dst token len_dst + j gets the src key re-encoded at that
 * local position (rounded to dtype) and the src value; then
 * len_dst += len_src, len_src = 0.  src data is left as it was.
 * dtype HWO_FP8: K, V hold code * scale; a key is stored as s * e4m3(x / s)
 * with s = k_scale[l * Hkv + g] (k_scale [L][Hkv], required, > 0); values
 * move unchanged.  k_scale is ignored for the other types (may be NULL).
 */
int32_t hwo_block_append(int32_t L, int32_t Hkv, int32_t D, int64_t num_slots, double* K, double* V,
                         int32_t num_blocks, const int64_t* block_start, const int32_t* block_cap,
                         int32_t* block_len, int32_t src, int32_t dst, double theta, int32_t dtype,
                         const double* k_scale);

/*
 * Token write for one layer (the new token of a decode step, stored at its
 * local position, Hogwild! notes key design 1).  K, V: [Hkv][num_slots][D].
 * For each listed block b with p = block_len[b] - 1: key slot p of kv head h
 * receives k_new[i][h] encoded at position p (rounded to dtype) and value slot
 * p receives v_new[i][h] (rounded to dtype).  Lengths are not changed.
 * k_new, v_new: [n][Hkv][D].  Returns HWO_EINVAL for a block id out of range,
 * HWO_ENOTOKENS when a listed block has length 0 (nothing is written then).
 * dtype HWO_FP8: key s_k * e4m3(x / s_k), value s_v * e4m3(v / s_v) with
 * s_k = k_scale[g], s_v = v_scale[g] (this layer's scales, required, > 0).
 */
int32_t hwo_block_write(int32_t Hkv, int32_t D, int64_t num_slots, double* K, double* V,
                        int32_t num_blocks, const int64_t* block_start, const int32_t* block_len,
                        int32_t n, const int32_t* blocks, const double* k_new,
                        const double* v_new, double theta, int32_t dtype, const double* k_scale,
                        const double* v_scale);

#ifdef __cplusplus
}
#endif

#endif /* HOGWILD_ORACLE_H */
