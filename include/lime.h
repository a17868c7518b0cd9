/*
 * lime.h — C ABI of the LIME inference hot path on AMD Instinct MI355X
 * (gfx950).
 *
 * Three operations, following the LIME pages (plus the int8, uncached and
 * user-side variant forms and a combined user-side + scoring call declared
 * further down):
 *
 *   lime_xor_fwd        user side: stacked LIME-XOR layers over the context
 *                       links L^C and the user history E, giving the
 *                       personalised links L^P (LIME notes on papernotes.org,
 *                       "Key design 2", XORA equation; framework flowchart,
 *                       online user-side stage).
 *   lime_qk_cache_build offline: the QK cache phi(scale * K_L[h] . T_m) over
 *                       an item catalogue (LIME notes, "Key design 1" and the
 *                       offline stage of the framework; LIME summary page,
 *                       Table 12: per item, per head, ell weights).
 *   lime_cand_score     online: O_i = phi(T_i L^T) L^P_b, a gather of cached
 *                       weight rows by candidate id plus an ell-wide weighted
 *                       sum per head (LIME notes, "complete example", step 3).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor argument is a DEVICE pointer to memory OWNED BY THE CALLER,
 *   contiguous, row-major, 16-byte aligned.  Host pointers are named as such.
 *   The library allocates no device memory; lime_xor_fwd takes a caller
 *   workspace sized by lime_xor_fwd_workspace_size.  The library keeps no
 *   state between calls except a per-thread error message.
 * - Element type: LIME_F32 (float) or LIME_BF16 (bfloat16 bit patterns).
 *   Arithmetic accumulates in float32; bf16 results are stored rounded to
 *   nearest-even.  Candidate ids and offsets are int64.  Inside the bf16
 *   user side, the XOR attention's matrix products take their operands
 *   (queries, keys, values and attention weights) as float16, rounded to
 *   nearest-even: the same matrix-core rate, three more mantissa bits.
 *   Their magnitudes stay far inside float16's range (+-65504) for any
 *   weights whose rows have norm below about 65504 / sqrt(d); the
 *   projections' and the gated MLP's operands stay bf16.
 * - Each call enqueues its kernels on `stream` (a hipStream_t; NULL is the
 *   default stream) and returns without waiting.  Outputs are valid once the
 *   stream has reached that point.  Calls that share output or workspace
 *   memory must be ordered by the caller.
 * - Errors: problems visible on the host (null pointers, bad sizes, bad
 *   enums, misalignment, too small a workspace, unsupported shapes) return
 *   synchronously, BEFORE anything is enqueued, leaving outputs untouched.
 *   A failed launch returns LIME_ERR_HIP.  lime_last_error() gives details.
 *   Data errors only the device can see have defined results (see each call).
 *
 * Attention nonlinearity phi (LIME notes, "Key design 1"; training strategy:
 * scaled softmax for single-layer attention, SiLU for deep stacks):
 *   LIME_PHI_SOFTMAX   softmax over the keys a row may attend;
 *   LIME_PHI_SILU_MEAN SiLU(s) / (number of keys the row may attend):
 *                      ell for history rows and the cache, N_b for link rows.
 * `scale` multiplies every logit (usually 1/sqrt(d_h)).
 * A row with no keys to attend (a user with empty history) outputs 0.
 */
#ifndef LIME_H_
#define LIME_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LIME_OK = 0,
  LIME_ERR_INVALID_ARG = 1,  /* null pointer, negative/inconsistent size, bad enum, misalignment */
  LIME_ERR_UNSUPPORTED = 2,  /* valid but outside the supported shape limits */
  LIME_ERR_WORKSPACE = 3,    /* workspace null or smaller than required */
  LIME_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} lime_status_t;

typedef enum { LIME_F32 = 0, LIME_BF16 = 1 } lime_dtype_t;

typedef enum { LIME_PHI_SOFTMAX = 0, LIME_PHI_SILU_MEAN = 1 } lime_phi_t;

/* User-side variants (see lime_xor_fwd_variant). */
typedef enum {
  LIME_VARIANT_XOR = 0,        /* LIME-XOR: both cross attentions          */
  LIME_VARIANT_MHA = 1,        /* LIME-MHA: links -> history only          */
  LIME_VARIANT_XOR_WINDOW = 2  /* LIME-XOR+Window: XOR plus a local window */
} lime_variant_t;

/* Weights of one LIME-XOR layer, device pointers, all in [out, in] row-major
 * layout (y = x . W^T), element type = the call's dtype:
 *   w_qkv  [3d, d]   rows 0..d-1 give Q, d..2d-1 give K, 2d..3d-1 give V
 *                    (one projection shared by both XOR branches, as in the
 *                    XORA equation's single parameter set)
 *   w_o    [d, d]    output projection, added to the residual stream
 *   w_gate [d_ff, d], w_up [d_ff, d], w_down [d, d_ff]
 *                    gated MLP: x += (SiLU(G w_gate^T) * (G w_up^T)) w_down^T
 *                    with G = LayerNorm(x)  (LIME notes, "Key design 2":
 *                    residual + GatedMLP)                                     */
typedef struct {
  const void* w_qkv;
  const void* w_o;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
} lime_layer_weights_t;

/* Bytes of workspace lime_xor_fwd needs for these sizes (0 on invalid
 * sizes).  The same arguments must be passed to lime_xor_fwd.               */
size_t lime_xor_fwd_workspace_size(lime_dtype_t dtype, int32_t B, int32_t ell, int32_t d,
                                   int32_t heads, int32_t d_ff, int64_t total_N, int32_t max_N);

/* User-side encoder: `layers` LIME-XOR layers over X_b = [L^C_b ; E_b].
 *
 * Per layer (LIME notes, "Key design 2" and training strategy; the layer
 * internals beyond the XORA equation are this library's reading):
 *   H = LayerNorm(X) (no affine, eps 1e-5);  [Q|K|V] = H w_qkv^T
 *   history rows attend to their user's ell link rows only, link rows attend
 *   to their user's N_b history rows only (no history<->history and no
 *   link<->link terms), per head on column slices of width d/heads;
 *   X += Y w_o^T;  X += SwiGLU-MLP(LayerNorm(X)).
 *
 *   links_ctx    [B, ell, d]          context links L^C (device)
 *   hist         [total_N, d]         packed histories E (device); users
 *                                     stay independent even when one
 *                                     user's rows hold inf or nan
 *   hist_offsets [B+1] int64 (device) exclusive prefix sum of history
 *                                     lengths: user b owns rows
 *                                     [off[b], off[b+1]); off[0] = 0 and
 *                                     off[B] = total_N are required (other
 *                                     values give unspecified outputs but no
 *                                     access outside the buffers).
 *   total_N      host, rows of hist, at most 2^34 (LIME_ERR_UNSUPPORTED
 *                above).
 *   max_N        host, an upper bound of every N_b (it sizes the on-chip
 *                buffers).  A user with N_b > max_N gets unspecified
 *                outputs, but no access falls outside the passed buffers.
 *   w            HOST array of `layers` weight structs (device pointers).
 *   links_pers   [B, ell, d] out: L^P, the link rows after the last layer.
 *   hist_out     [total_N, d] out or NULL: the history rows after the last
 *                layer.  With NULL the last layer's history-row work that
 *                cannot reach L^P is skipped.
 *   workspace    device, >= lime_xor_fwd_workspace_size(...) bytes, 256-byte
 *                aligned; contents on entry are ignored.
 * Limits: d % heads == 0, d_h = d/heads in {16, 32, 64, 128}, d % 8 == 0,
 * d <= 1024, d_ff % 8 == 0, 1 <= ell <= 256, B >= 1, layers >= 1.           */
lime_status_t lime_xor_fwd(lime_dtype_t dtype, lime_phi_t phi, float scale,
                           int32_t B, int32_t ell, int32_t d, int32_t heads, int32_t layers,
                           int32_t d_ff, const void* links_ctx, const void* hist,
                           const int64_t* hist_offsets, int64_t total_N, int32_t max_N,
                           const lime_layer_weights_t* w, void* links_pers, void* hist_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* The user-side encoder in one of the pages' variants.  Arguments,
 * layouts, workspace (lime_xor_fwd_workspace_size) and errors as
 * lime_xor_fwd, plus:
 *   variant  LIME_VARIANT_XOR: exactly lime_xor_fwd.  `window` must be 0.
 *            LIME_VARIANT_MHA: LIME-MHA (LIME summary page, Fig. 2 and the
 *              scaling paragraph of the LIME notes' experiments; the
 *              notes' results table calls it single-layer decoupled): only
 *              the links -> history cross attention runs.  History rows
 *              are never updated; every layer reads the input E, and the
 *              link rows go through W_o, residual and gated MLP as in
 *              lime_xor_fwd.  `window` must be 0 and hist_out NULL.
 *            LIME_VARIANT_XOR_WINDOW: LIME-XOR+Window (LIME notes, "Key
 *              design 3"; Table 13): history row p of a user attends its
 *              ell links AND the history rows q of the same user with
 *              1 <= |p - q| <= window (neighbours before and after, itself
 *              excluded), under one phi over the union; with silu_mean the
 *              normaliser counts the union.  Link rows are unchanged.
 *   window   neighbours on each side, 1 <= window <= 4096 for
 *            LIME_VARIANT_XOR_WINDOW (window = ell / 2 gives each history
 *            row 2*ell keys, the context size the notes state).
 * Windows up to 16 (ell = 32) or 32 (ell = 64) run on the matrix-core
 * kernels; larger ones on the generic kernels.                             */
lime_status_t lime_xor_fwd_variant(lime_variant_t variant, int32_t window, lime_dtype_t dtype,
                                   lime_phi_t phi, float scale, int32_t B, int32_t ell, int32_t d,
                                   int32_t heads, int32_t layers, int32_t d_ff,
                                   const void* links_ctx, const void* hist,
                                   const int64_t* hist_offsets, int64_t total_N, int32_t max_N,
                                   const lime_layer_weights_t* w, void* links_pers,
                                   void* hist_out, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Size of the scratch array lime_xor_fwd_noalloc uses as its workspace. */
#define LIME_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* lime_xor_fwd with no workspace argument and no allocation of any kind, for
 * callers that cannot allocate device memory: code being captured into a
 * HIP graph, tight serving loops, harnesses that forbid hipMalloc.  The
 * workspace is a fixed device array inside the library of
 * LIME_NOALLOC_SCRATCH_BYTES (64 MiB), one per GPU, held from the library's
 * load until the process ends; its device address is looked up once per
 * device, on the first call made with that device current.
 * Arguments, results and errors are those of lime_xor_fwd (same kernels,
 * bit-identical outputs), without workspace/workspace_bytes.  A call whose
 * lime_xor_fwd_workspace_size(...) exceeds LIME_NOALLOC_SCRATCH_BYTES
 * returns LIME_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU shares that GPU's array, and the array keeps what
 * the last call left in it (no call depends on its contents on entry).
 * Calls that may overlap on one GPU (different streams, or different host
 * threads without ordering) race on it: the caller must order them.       */
lime_status_t lime_xor_fwd_noalloc(lime_dtype_t dtype, lime_phi_t phi, float scale, int32_t B,
                                   int32_t ell, int32_t d, int32_t heads, int32_t layers, int32_t d_ff,
                                   const void* links_ctx, const void* hist, const int64_t* hist_offsets,
                                   int64_t total_N, int32_t max_N, const lime_layer_weights_t* w,
                                   void* links_pers, void* hist_out, void* stream);

/* Launch plan lime_xor_fwd would use for these sizes (host only, no GPU
 * work): returns the number of kernel launches of one call (0 on invalid
 * sizes) and, if buf is not NULL, writes a one-line description (path name,
 * splits, rows per split) of at most buf_len bytes including the NUL.
 * with_hist says whether hist_out will be passed.  An introspection aid for
 * profiling and tuning; lime_xor_fwd does not need it.                     */
int32_t lime_xor_fwd_plan(lime_dtype_t dtype, int32_t B, int32_t ell, int32_t d, int32_t heads,
                          int32_t layers, int32_t d_ff, int64_t total_N, int32_t max_N,
                          int32_t with_hist, char* buf, size_t buf_len);

/* Offline QK cache over items [n_items, d] and per-head link keys
 * link_keys [heads, ell, d] (the global links with the candidate-side
 * query/key projections folded in; heads = 1 and link_keys = L is the
 * pages' literal formula):
 *   cache[m, h, k] = phi_k( scale * sum_c items[m, c] * link_keys[h, k, c] )
 * phi taken over the ell links of head h.  cache is [n_items, heads, ell],
 * same dtype.  Items are independent, so a partial refresh of rows
 * [r0, r1) is a call with items + r0*d, cache + r0*heads*ell and
 * n_items = r1 - r0.  n_items = 0 is a no-op.
 * Limits: 1 <= ell <= 256, d % 8 == 0, d <= 1024, heads >= 1.               */
lime_status_t lime_qk_cache_build(lime_dtype_t dtype, lime_phi_t phi, float scale,
                                  int64_t n_items, int32_t d, int32_t heads, int32_t ell,
                                  const void* items, const void* link_keys, void* cache,
                                  void* stream);

/* Candidate scoring: for candidate i of user b (cand_offsets[b] <= i <
 * cand_offsets[b+1]) and head h,
 *   out[i, h*d_h + c] = sum_k cache[cand_ids[i], h, k] * links_pers[b, k, h*d_h + c]
 *   cache       [n_items, heads, ell]   (from lime_qk_cache_build)
 *   links_pers  [B, ell, d]             (from lime_xor_fwd)
 *   cand_ids    [total_M] int64, cand_offsets [B+1] int64 (device), the
 *               exclusive prefix sum of per-user candidate counts with
 *               cand_offsets[0] = 0, cand_offsets[B] = total_M.
 *   out         [total_M, d]
 *   bad_id_count device int32 or NULL: an id outside [0, n_items) gives a
 *               zero output row and adds 1 here (the caller zeroes it).
 * Each output row depends only on its own id and user.
 * Limits: d % heads == 0, d_h in {16, 32, 64, 128}, 1 <= ell <= 256.        */
lime_status_t lime_cand_score(lime_dtype_t dtype, int32_t B, int32_t ell, int32_t d,
                              int32_t heads, const void* cache, int64_t n_items,
                              const void* links_pers, const int64_t* cand_ids,
                              const int64_t* cand_offsets, int64_t total_M, void* out,
                              int32_t* bad_id_count, void* stream);

/* User side and candidate scoring in one call: the online stage run for a
 * batch of requests, each user's personalised links followed at once by the
 * scoring of that user's candidates (LIME notes, framework flowchart, online
 * stage; "complete example", steps 2 and 3).  Arguments, results, errors and
 * limits are those of lime_xor_fwd followed by lime_cand_score on the same
 * stream (links_pers is written as there and is the scoring's input); for
 * offsets that meet their preconditions the outputs and bad_id_count are
 * bit-identical to that pair of calls.  On the user-resident
 * path (short histories, bf16) each user's workgroup scores its own
 * candidates from the links it holds on chip, so the pair costs one launch;
 * elsewhere the call enqueues lime_xor_fwd's kernels and then the scoring
 * kernel.  Every argument of both halves is checked before anything is
 * enqueued.                                                                */
lime_status_t lime_xor_fwd_score(lime_dtype_t dtype, lime_phi_t phi, float scale, int32_t B,
                                 int32_t ell, int32_t d, int32_t heads, int32_t layers, int32_t d_ff,
                                 const void* links_ctx, const void* hist, const int64_t* hist_offsets,
                                 int64_t total_N, int32_t max_N, const lime_layer_weights_t* w,
                                 void* links_pers, void* hist_out, void* workspace,
                                 size_t workspace_bytes, const void* cache, int64_t n_items,
                                 const int64_t* cand_ids, const int64_t* cand_offsets, int64_t total_M,
                                 void* out, int32_t* bad_id_count, void* stream);

/* Int8 QK cache (LIME summary page, Tables 10 and 12: int8 lookup with
 * dequantisation, int8 cache sizes; the scheme is not given there).  Same
 * weights as lime_qk_cache_build, stored per (item, head) as symmetric
 * codes with one float32 scale:
 *   qscale[m, h] = max_k |w_k| / 127,  codes[m, h, k] = round-half-even(w_k * 127 / max_k |w_k|)
 * (an all-zero row gets scale 0 and codes 0).  codes [n_items, heads, ell]
 * int8 and qscale [n_items, heads] float32 are device buffers owned by the
 * caller; dtype is the element type of items and link_keys.  Errors and
 * limits as lime_qk_cache_build; qscale must be 4-byte aligned.            */
lime_status_t lime_qk_cache_build_i8(lime_dtype_t dtype, lime_phi_t phi, float scale,
                                     int64_t n_items, int32_t d, int32_t heads, int32_t ell,
                                     const void* items, const void* link_keys, int8_t* codes,
                                     float* qscale, void* stream);

/* Candidate scoring from the int8 cache: as lime_cand_score with the cached
 * row dequantised, out[i, h-cols] = qscale[id,h] * sum_k codes[id,h,k] *
 * links_pers[b, k, h-cols].  dtype is the element type of links_pers and
 * out.  Out-of-range ids: zero rows, counted in bad_id_count.              */
lime_status_t lime_cand_score_i8(lime_dtype_t dtype, int32_t B, int32_t ell, int32_t d,
                                 int32_t heads, const int8_t* codes, const float* qscale,
                                 int64_t n_items, const void* links_pers, const int64_t* cand_ids,
                                 const int64_t* cand_offsets, int64_t total_M, void* out,
                                 int32_t* bad_id_count, void* stream);

/* Uncached (cold-start) scoring: the cache formula evaluated per candidate
 * from the item rows, then the weighted sum (LIME summary page, Table 10,
 * "Uncached global"; LIME notes, limitations: items without cached weights
 * fall back to online computation).
 *   out[i, h-cols] = sum_k phi_k(scale * link_keys[h,k,:] . items[id_i,:])
 *                          * links_pers[b, k, h-cols]
 * items [n_items, d], link_keys [heads, ell, d], links_pers [B, ell, d],
 * out [total_M, d], all of element type dtype.  Out-of-range ids give zero
 * rows and are counted in bad_id_count.  Limits as lime_qk_cache_build and
 * lime_cand_score.                                                        */
lime_status_t lime_cand_score_uncached(lime_dtype_t dtype, lime_phi_t phi, float scale, int32_t B,
                                       int32_t ell, int32_t d, int32_t heads, const void* items,
                                       int64_t n_items, const void* link_keys, const void* links_pers,
                                       const int64_t* cand_ids, const int64_t* cand_offsets,
                                       int64_t total_M, void* out, int32_t* bad_id_count, void* stream);

/* Kernel timing for measurement tools (profiling of the calls above; the
 * pages time their stages the same way, per stage, LIME summary page,
 * Table 10).  lime_trace_begin opens a trace: until lime_trace_end, every
 * kernel the library launches, from any thread and on any stream, carries a
 * pair of HIP events that the runtime stamps with that dispatch's own start
 * and end, for up to `capacity` launches (later ones run untraced and are
 * counted as dropped).  No device memory is allocated; the events are
 * created here and destroyed by lime_trace_end.  Tracing changes no result.
 * Do not open a trace while a stream that calls the library is being
 * captured into a graph.
 * Errors: LIME_ERR_INVALID_ARG if capacity < 1 or a trace is already open;
 * LIME_ERR_HIP if an event cannot be created (no trace is then open).      */
lime_status_t lime_trace_begin(int32_t capacity);

/* Closes the open trace: waits for every traced launch to finish, then
 * writes, for the first min(count, cap) traced launches in launch order,
 * names[i] = the kernel's name (a static string: "qk_cache", "cand_score",
 * "xor_attn", "post_block_stream", ...) and ms[i] = its duration in
 * milliseconds (names and ms are HOST arrays of `cap` entries, either may be
 * NULL).  *dropped (host, nullable) receives the launches past the capacity.
 * Returns the number of traced launches, or -1 if no trace is open or a wait
 * failed (lime_last_error tells which).                                    */
int32_t lime_trace_end(const char** names, float* ms, int32_t cap, int32_t* dropped);

/* Static string naming a status code. */
const char* lime_status_string(lime_status_t status);

/* Message describing the last failure on the calling thread ("" if none). */
const char* lime_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIME_H_ */
