/*
 * kvq.h -- C ABI of libkvq.so: KV-cache compress -> quantise -> paged store on MI355X
 * (gfx950), plus the matching page dequant and the once-per-step full -> SWA slot
 * translation.
 *
 * Sources (web pages the operations follow):
 *  [P1] "sglang, DeepSeek V4.1 Paged KV Cache: V41 and FP4 formats" (sglang PR #39123
 *       analysis): section 1 (V41 / V41_FP4 layouts, PagedKV page/row/scale-row
 *       addressing, store_row with the ue8m0 exponent taken from the amax bits),
 *       section 2 (c1 / c2 compressor writes templated on the layout, FP4 quantised
 *       once), section 4 (dequant of pages into a bf16 workspace), section 5 (the pool
 *       reports bytes per token and bytes per page instead of a hard-coded 584).
 *  [P2] "SGLang: DeepSeek-v4 SWA index translation hoisting" (sglang PR #34890
 *       analysis): sections 1-2 (translate out_cache_loc once per step into a
 *       preallocated int32 buffer; zero the tail; refuse when the batch is larger).
 *  [P3] "DeepSeek V4 Sparse FP8 Compressor kernel optimisation with CuteDSL" (vLLM PR
 *       #44161 analysis): sections 1-3 (per-channel online-softmax pooling of each
 *       ratio-r window of fp32 rows, RoPE, per-32 absmax fp8 scale).
 *
 * Common rules for every entry point
 *  - All array arguments are DEVICE pointers owned by the caller; the library keeps no
 *    reference after the call returns.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously on it; no call allocates, frees or synchronises, so every call can
 *    be captured into a hipGraph.
 *  - Calls keep no state (apart from the per-thread request of kvq_profile_next_launch)
 *    and are thread-safe.  Two calls that write the same pool slots or output rows
 *    concurrently race (the caller orders them with streams/events).
 *  - Host-side validation only: arguments are checked before any launch and an error
 *    returns without enqueuing anything.  Device data is not validated, except that a
 *    row whose slot is outside [0, num_pages*64) or whose position is outside
 *    [0, max_pos) is skipped (nothing is written for it).  Duplicate slots within one
 *    call are a caller error (which row wins is unspecified).
 *  - n == 0 (or R == 0, P == 0) returns KVQ_OK without launching, except
 *    kv_translate_slots, which still zeroes out[0:cap].
 *  - Sizes above what one launch covers are refused with KVQ_EINVAL before anything is
 *    enqueued: rows n (or R) <= KVQ_MAX_ROWS, except R <= KVQ_MAX_LONG_ROWS for
 *    compressor ratios of 64 and more; pages P <= KVQ_MAX_PAGES; cap <= 2^31 - 1.
 *  - Inputs must be finite, no larger in magnitude than the largest finite bf16 (about
 *    3.39e38), and no larger than 2^127 (about 1.7e38) in the last 64 channels, which are
 *    rotated (a rotated pair can grow by up to a factor sqrt(2)), so that no pooled or
 *    rotated value overflows; values outside that domain give unspecified codes.  fp32
 *    denormals are handled.
 *
 * Pool layout (PagedKV, page size 64 tokens, [P1] section 1): the pool is num_pages
 * pages of kvq_page_bytes(layout) bytes each, contiguous from `pool`.  Slot s lives in
 * page s >> 6, row s & 63.  A page holds 64 code rows followed by 64 scale rows:
 *   code row  at pool + page*PB + row*CR          (CR = kvq_code_row_bytes)
 *   scale row at pool + page*PB + 64*CR + row*SR  (SR = kvq_scale_row_bytes)
 * V41:     CR = 512 (e4m3 code of channel c at byte c), SR = 16 (ue8m0 byte b scales
 *          channels 32b..32b+31): 528 B/token, PB = 33792.
 * V41_FP4: CR = 256 (channel 2j in the low nibble of byte j, 2j+1 in the high nibble),
 *          SR = 32 (16 e4m3 scale bytes, then 16 zero pad bytes): 288 B/token,
 *          PB = 18432.
 *
 * Row encoding (per 32-channel block of bf16 values v, amax = max |v|):
 *  V41:     k = smallest integer >= -127 with amax <= 448 * 2^k; scale byte k + 127;
 *           code = e4m3fn(v * 2^-k), round to nearest even, sign kept.
 *  V41_FP4: s = e4m3fn(fl32(amax / 6)) rounded to nearest even, held at 448;
 *           code = e2m1(fl32(v / s)), round to nearest even, magnitudes above 6 held at
 *           6, sign kept; all codes 0 when s == 0.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------------- */
#define KVQ_OK 0
#define KVQ_EINVAL (-1)    /* null pointer with work to do, ld < 512, misaligned
                              pointer or stride, negative size, max_pos <= 0,
                              num_pages > 2^32                                     */
#define KVQ_ELAYOUT (-2)   /* layout id is not KVQ_LAYOUT_V41 / KVQ_LAYOUT_V41_FP4 */
#define KVQ_ERATIO (-3)    /* ratio not built (supported: 1, 2, 4, 8, 16, 32, 64, 128) */
#define KVQ_ECAPACITY (-4) /* more slots than the translation buffer holds (n > cap
                              or R > cap); nothing enqueued                        */
#define KVQ_ELAUNCH (-5)   /* the HIP runtime rejected the kernel launch          */

/* ---- size limits of one call (larger requests return KVQ_EINVAL) --------------- */
#define KVQ_MAX_ROWS 33554432      /* 2^25 rows of a store / gather / short-window call */
#define KVQ_MAX_LONG_ROWS 4194304  /* 2^22 output rows of a compressor call, ratio >= 64 */
#define KVQ_MAX_PAGES 524288       /* 2^19 page ids of one kv_dequant call              */

/* ---- layout ids ---------------------------------------------------------------- */
#define KVQ_LAYOUT_V41 1     /* fp8 e4m3 codes + ue8m0 scale per 32: 528 B/token     */
#define KVQ_LAYOUT_V41_FP4 2 /* e2m1 codes + e4m3 scale per 32 (+pad): 288 B/token  */

/* Profiling aid: the next kernel launched by an entry point called on this thread records
 * start_event when the kernel begins executing and stop_event when it has finished, as
 * part of its own dispatch (hipExtLaunchKernel), so their elapsed time is the kernel's
 * duration without the gaps between commands.  Either event may be NULL.  The request is
 * consumed by that launch; a call that launches nothing (an error, or nothing to do)
 * leaves it pending.  The events (hipEvent_t, created with timing enabled, on the device
 * of the launch) stay owned by the caller.  Results are unaffected.  Meant for eager
 * timing: do not arm a launch that is being captured into a graph.  Returns KVQ_OK. */
int kvq_profile_next_launch(void* start_event, void* stop_event);

/* Human-readable name of a status code (static string, never NULL). */
const char* kvq_status_string(int status);

/* Identity of the build: the SHA-256 (hex) of the kernel sources this library was
 * compiled from (static string).  Loaders compare it with the sources next to them to
 * refuse a stale library. */
const char* kvq_build_id(void);

/* Layout queries ([P1] sections 1 and 5).  Each returns the byte count, or
 * KVQ_ELAYOUT for an unknown layout. */
int64_t kvq_bytes_per_token(int32_t layout);  /* 528 | 288                     */
int64_t kvq_page_bytes(int32_t layout);       /* 64 * bytes per token         */
int64_t kvq_code_row_bytes(int32_t layout);   /* 512 | 256                     */
int64_t kvq_scale_row_bytes(int32_t layout);  /* 16 | 32                       */

/* kv_store -- quantise n bf16 K rows and write them at their slots ([P1] section 1,
 * store_row; the plain "store" kernel of the latency table).
 *   pool       device, num_pages * kvq_page_bytes(layout) bytes, 16-byte aligned
 *   k          device bf16 bits, row i at k + i*ld, 512 channels used; 16-byte aligned
 *   ld         row stride in elements, >= 512 and a multiple of 8
 *   slots      device int32[n]
 * Returns KVQ_OK or KVQ_EINVAL / KVQ_ELAYOUT / KVQ_ELAUNCH. */
int kv_store(int32_t layout, void* pool, int64_t num_pages, const uint16_t* k, int64_t ld,
             const int32_t* slots, int64_t n, void* stream);

/* kv_store_rope -- as kv_store, but first rotates the last 64 channels of each row by
 * its position (NeoX half rotation: channel 448+i pairs with 480+i, i < 32) and rounds
 * the rotated values to bf16 ([P1] latency table "store + RoPE"; [P3] section 3).
 *   pos        device int32[n], positions; rows with pos outside [0, max_pos) skipped
 *   cos_sin    device fp32[max_pos][64]: cos of the 32 angles of a position, then their
 *              sin; 16-byte aligned.  Built by the caller (a RoPE table is model data).
 *   max_pos    rows in cos_sin, > 0
 * The rotation is o1 = x1*c - x2*s, o2 = x2*c + x1*s with every product and sum
 * rounded to fp32 separately (no fused multiply-add), so results are deterministic. */
int kv_store_rope(int32_t layout, void* pool, int64_t num_pages, const uint16_t* k,
                  int64_t ld, const int32_t* pos, const float* cos_sin, int64_t max_pos,
                  const int32_t* slots, int64_t n, void* stream);

/* kv_store_rope_layers -- kv_store_rope for L layers at once, for the hoisted per-step
 * slot translation of [P2] (sections 1-2, "why this is a good optimisation" items 1-2:
 * translate out_cache_loc once per step, then every layer's store reuses the result).
 * For every layer l < L and row i < n: row i of that layer's K (k_layers[l] + i*ld) is
 * rotated at pos[i] and stored at slots[i] of that layer's pool (pools[l]), exactly as
 * kv_store_rope does.  One kernel launch covers up to KVQ_MAX_LAYERS layers (more layers
 * take further launches on the same stream); the positions, slots and cos/sin rows are
 * shared by all layers.
 *   pools      HOST array of L device pool pointers, each num_pages pages of `layout`,
 *              16-byte aligned; read during the call only (the pointers travel as
 *              kernel arguments, so a graph capture keeps them)
 *   k_layers   HOST array of L device bf16 K pointers (same ld for every layer), 16-byte
 *              aligned
 *   L          number of layers, >= 1; n * L <= KVQ_MAX_ROWS
 * Other arguments, skipping rules and errors as kv_store_rope.  Distinct layers must not
 * share a pool (rows of different layers would race). */
#define KVQ_MAX_LAYERS 64
int kv_store_rope_layers(int32_t layout, void* const* pools, int64_t num_pages,
                         const uint16_t* const* k_layers, int64_t ld, int32_t L, const int32_t* pos,
                         const float* cos_sin, int64_t max_pos, const int32_t* slots, int64_t n,
                         void* stream);

/* kv_store_norm_rope -- the fused "K norm + RoPE" store of [P1]'s latency table.  The
 * page gives no formula; this library reads it as RMS normalisation of the whole row with
 * a per-channel weight, y_c = bf16((x_c * w_c) / sqrt(mean_c(x_c^2) + eps)), evaluated in
 * float64 (x_c * w_c and the squares exact, the mean a float64 sum, IEEE sqrt and
 * division) and rounded once to bf16, followed by kv_store_rope on y.
 *   weight     device bf16 bits [512], 16-byte aligned
 *   eps        >= 0 and finite (else KVQ_EINVAL)
 * Other arguments as kv_store_rope.  y equals the correctly rounded value unless the
 * exact quotient lies within a few float64 ulps of a bf16 rounding midpoint.  With eps == 0
 * an all-zero row has no defined value (0 / 0) and its codes are unspecified. */
int kv_store_norm_rope(int32_t layout, void* pool, int64_t num_pages, const uint16_t* k,
                       int64_t ld, const uint16_t* weight, float eps, const int32_t* pos,
                       const float* cos_sin, int64_t max_pos, const int32_t* slots, int64_t n,
                       void* stream);

/* kv_compress_store -- the c1 / C4A / C128A compressors ([P3] sections 1-3; [P1]
 * section 2).  Output row i pools input rows [i*ratio, i*ratio + ratio) channel by
 * channel: weights are the softmax over the window of score[.][c], the pooled value is
 * the weighted sum of kv[.][c], evaluated in float64 (weights exp(s - ref) against a
 * reference score of the window, online over the window) and rounded once to bf16; then
 * RoPE at pos[i] as in kv_store_rope; then quantise and store at slots[i].  ratio 1 is
 * the identity (score is not read).
 *   kv, score  device fp32, row j at base + j*ld, R*ratio rows; 16-byte aligned
 *   ld         row stride in elements, >= 512 and a multiple of 4
 *   ratio      1, 2, 4, 8, 16, 32, 64 or 128 (others: KVQ_ERATIO)
 *   pos, slots device int32[R]
 * The pooled bf16 equals the correctly rounded exact value unless that value lies within
 * about 1e-15 (relative to the window's |kv|) of a bf16 rounding midpoint; every later
 * step is exact, so the stored bytes are then those of the exact evaluation. */
int kv_compress_store(int32_t layout, void* pool, int64_t num_pages, const float* kv,
                      const float* score, int64_t ld, int32_t ratio, const int32_t* pos,
                      const float* cos_sin, int64_t max_pos, const int32_t* slots,
                      int64_t R, void* stream);

/* kv_compress_store_translate -- kv_compress_store with the step's full -> SWA slot
 * translation fused in ([P2] section 1: the translation is computed once per step; here
 * the first compressor of the step computes it and leaves it in out_loc for the later
 * consumers).  The result is that of
 *   kv_translate_slots(table, table_len, full_loc, R, out_loc, cap, stream);
 *   kv_compress_store(..., slots = out_loc, R, stream);
 * (out_loc[i] = table[full_loc[i]] for i < R, -1 for a full slot outside [0, table_len),
 * out_loc[R:cap] = 0; row i is stored at out_loc[i]), in one launch: each row looks its
 * slot up in the table itself.  When the zero tail is long against the grid (more than
 * 16 chunks of 64 entries per wavefront) the translation runs as its own launch first.
 * Errors: those of kv_compress_store; cap < 0, cap > 2^31 - 1 or table_len < 0 give
 * KVQ_EINVAL; R > cap gives KVQ_ECAPACITY and enqueues nothing.  R == 0 only zeroes
 * out_loc[0:cap].  out_loc must not overlap table or full_loc.
 *   table      device int32[table_len]
 *   full_loc   device int32[R]: full-pool slots of the output rows
 *   out_loc    device int32[cap]: the translated slots */
int kv_compress_store_translate(int32_t layout, void* pool, int64_t num_pages, const float* kv,
                                const float* score, int64_t ld, int32_t ratio, const int32_t* pos,
                                const float* cos_sin, int64_t max_pos, const int32_t* table,
                                int64_t table_len, const int32_t* full_loc, int32_t* out_loc,
                                int64_t cap, int64_t R, void* stream);

/* Bytes of one sequence's decode-step compressor state (kv_compress_state_update). */
int64_t kvq_compress_state_bytes(void);  /* 10240 */

/* kv_compress_state_update -- the compressor across decode steps: windows that fill one
 * row per step are folded into a per-sequence online-softmax state instead of keeping
 * their raw rows (the decode side of the mixed decode/prefill batches of [P3]'s
 * introduction).  For each j < n, row j (kv[j], score[j]) is folded into state
 * state_ids[j] and counted; when the count reaches `ratio` the window is finalised
 * exactly as kv_compress_store finalises a window (pooled value rounded to bf16, RoPE at
 * pos[j], quantise, store at slots[j]; an out-of-pool slot or out-of-range position
 * stores nothing) and the state becomes empty again.  Rows of one window must arrive in
 * order, at most one row per state per call (state_ids distinct within a call; repeats
 * race).  A state id outside [0, num_states) skips the row.
 *   state      device, num_states * kvq_compress_state_bytes() bytes, contents opaque
 *              (a float64 online-softmax state per sequence); 16-byte aligned
 *   count      device int32 [num_states]: rows folded so far; 0 = empty.  A zeroed
 *              state + count is a valid starting point.
 *   ratio      window length, 1 .. 2^20
 *   pos, slots device int32[n]: used for the row that completes its window
 *   kv, score  device fp32 rows, row j at base + j*ld; 16-byte aligned, ld >= 512, % 4
 * The fold is float64 like kv_compress_store's, so a finalised row carries the same
 * bytes as kv_compress_store on the same window (up to the float64 evaluation order,
 * which matters only within about 1e-15 of a bf16 rounding midpoint). */
int kv_compress_state_update(int32_t layout, void* pool, int64_t num_pages, void* state,
                             int32_t* count, int64_t num_states, int32_t ratio,
                             const int32_t* state_ids, const float* kv, const float* score,
                             int64_t ld, const int32_t* pos, const float* cos_sin,
                             int64_t max_pos, const int32_t* slots, int64_t n, void* stream);

/* kv_dequant -- turn whole pages back into a bf16 workspace ([P1] section 4).
 * For p < P and each of the 64 rows r of page page_ids[p]:
 *   out[(p*64 + r)*512 + c] = bf16_rne(fp32(decode(code) * decode(scale)))
 * A NaN code or scale gives 0x7FC0.  A page id outside [0, num_pages) leaves its 64
 * output rows untouched.
 *   page_ids   device int32[P]
 *   out        device bf16 bits, [P*64][512], 16-byte aligned */
int kv_dequant(int32_t layout, const void* pool, int64_t num_pages, const int32_t* page_ids,
               int64_t P, uint16_t* out, void* stream);

/* kv_dequant_slots -- the per-token form of kv_dequant: out[i*512 + c] is the
 * dequantised value of channel c of the row at slots[i] (same arithmetic and NaN rule as
 * kv_dequant); rows whose slot is outside [0, num_pages*64) are left untouched.  For a
 * consumer that needs a gathered set of tokens rather than whole pages.
 *   slots      device int32[n]
 *   out        device bf16 bits, [n][512], 16-byte aligned */
int kv_dequant_slots(int32_t layout, const void* pool, int64_t num_pages, const int32_t* slots,
                     int64_t n, uint16_t* out, void* stream);

/* kv_translate_slots -- full-pool -> SWA-pool slot translation, done once per step into
 * a preallocated buffer ([P2] sections 1-2):
 *   out[i] = table[full_loc[i]] for i < n (-1 when full_loc[i] is outside
 *            [0, table_len)), out[i] = 0 for n <= i < cap.
 * n > cap returns KVQ_ECAPACITY and enqueues nothing; the caller then translates into a
 * buffer of its own of n entries (the eager, still once-per-step, fallback).  out must
 * not overlap table or full_loc.
 *   table      device int32[table_len]
 *   full_loc   device int32[n]
 *   out        device int32[cap] */
int kv_translate_slots(const int32_t* table, int64_t table_len, const int32_t* full_loc,
                       int64_t n, int32_t* out, int64_t cap, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */
