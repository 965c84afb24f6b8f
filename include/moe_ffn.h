/*
 * moe_ffn.h -- C ABI of the routed mixture-of-experts FFN layer with RMSNorm
 * for AMD Instinct MI355X (gfx950), library libmoeffn.so.
 *
 * The layer is the one `forward_ffn_rows` encodes on the docs.rs source page
 * "hf2q 0.1.3 -- src/inference/models/deepseek4/ffn_forward.rs": RMSNorm of
 * the FFN input, router matmul ("MoE gate"), score route (sigmoid score +
 * selection bias) or hash route (token-id -> expert table), index
 * sanitising, routed and shared gate/up projections, SwiGLU, down
 * projections and the weighted reduce of routed plus shared outputs.  The
 * hyper-connection prelude and post-mix that wrap it on that page are not
 * part of this ABI: `x` here is the page's `ffn_input`, `out` its
 * `ffn_output`.
 *
 * Conventions shared by every entry point:
 *   - Return value: 0 (MOE_OK) or a positive moe_status code; moe_strerror()
 *     names it.  Argument errors are detected on the host BEFORE any HIP
 *     call, so they never leave work on the stream.
 *   - Pointers documented "device" are HIP device (or managed) memory owned
 *     by the caller; the library neither allocates nor frees on the call
 *     path and keeps no reference after the call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work; they do not synchronise (except moe_ffn_status and
 *     moe_ffn_stage_timing_end, which say so).
 *   - All matrices are row-major; weight matrices are [out][in].
 *   - Thread safety: the library is stateless apart from the optional stage
 *     timer.  Concurrent calls on different streams must use different
 *     workspaces; calls that share a workspace race.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = 1,       /* bad argument: rows <= 0, NULL pointer, unknown
                           layer kind, missing bias (score) or table (hash) */
  MOE_EUNSUPPORTED = 2, /* dims with no compiled kernels (see moe_dims_t)    */
  MOE_EOVERFLOW = 3,    /* rows * top_k (or a buffer size) overflows         */
  MOE_EWORKSPACE = 4,   /* workspace NULL, misaligned or too small           */
  MOE_EHIP = 5,         /* a HIP launch or runtime call failed               */
  MOE_EOVERLAP = 6,     /* x and out overlap                                 */
  MOE_ESCRATCH = 7      /* moe_ffn_forward_noalloc: the call needs more
                           intermediate memory than its built-in scratch of
                           MOE_NOALLOC_SCRATCH_BYTES holds                 */
};

/* Size of the device array that holds moe_ffn_forward_noalloc's
 * intermediates, one per GPU the library runs on (64 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* ---- layer kinds (ffn_forward.rs: the hash table is bound for layers below
 * hash_layer_count, the selection bias for the layers after them) -------- */
enum { MOE_LAYER_SCORE = 0, MOE_LAYER_HASH = 1 };

/* ---- device status bits, read with moe_ffn_status ----------------------- */
enum {
  MOE_FLAG_BAD_TOKEN = 1u,      /* a hash-layer token id outside [0, table_rows):
                                   all of that row's slots were masked      */
  MOE_FLAG_BAD_TABLE_ENTRY = 2u, /* a table entry outside [0, experts): that
                                    slot was masked                         */
  MOE_FLAG_SYNC_TIMEOUT = 4u,    /* reserved, never set: no workgroup of
                                    any call waits for another (kept so the
                                    bit values stay stable)                 */
  MOE_FLAG_F16_RANGE = 8u,       /* calls of more than 4 rows only (the
                                    matrix-core path, whose operands are
                                    fp16): a router logit, SwiGLU output,
                                    routed down output or layer output was
                                    not finite -- an activation or weight
                                    beyond fp16's range (|v| > 65504), or a
                                    non-finite input; the output is not
                                    valid.  Calls of 1 to 4 rows compute in
                                    f32 and never set it                    */
  MOE_FLAG_CHECK = 16u           /* checked build (libmoeffn_checked.so)
                                    only: an index that an earlier step of
                                    the call produced (a row list, a routing
                                    plan entry, a slot position) failed its
                                    bounds test where it was used; the access
                                    was clamped, the output is not valid.
                                    The default build never sets it         */
};

/* Layer dimensions.  ffn_forward.rs guards the native path with fixed
 * constants (hidden 4096, 256 experts, top-6, inter 2048); this library
 * compiles kernels for exactly two shapes and rejects others with
 * MOE_EUNSUPPORTED:
 *     hidden 4096, experts 256, top_k 6, inter 2048, n_shared 1   (full)
 *     hidden  512, experts  32, top_k 6, inter  256, n_shared 1   (tiny)
 * table_rows is the number of tid2eid rows (the token-id range of a hash
 * layer; ignored for score layers).  eps is the RMSNorm epsilon (> 0 or 0). */
typedef struct moe_dims {
  int32_t hidden;
  int32_t experts;
  int32_t top_k;
  int32_t inter;
  int32_t n_shared;
  int32_t reserved0;  /* must be 0 */
  int64_t table_rows;
  float eps;
  int32_t reserved1;  /* must be 0 */
} moe_dims_t;

/* One layer's parameters, all DEVICE pointers, caller-owned, read-only.
 * Names follow the GGUF tensors ffn_forward.rs binds for block L:
 *   norm_w    blk.L.ffn_norm.weight        f32  [hidden]
 *   router    blk.L.ffn_gate_inp.weight    bf16 [experts][hidden]
 *   sel_bias  blk.L.exp_probs_b.bias       f32  [experts]        (score layers)
 *   tid2eid   blk.L.ffn_gate_tid2eid       i32  [table_rows][top_k] (hash layers)
 *   gate_exps blk.L.ffn_gate_exps.weight   bf16 [experts][inter][hidden]
 *   up_exps   blk.L.ffn_up_exps.weight     bf16 [experts][inter][hidden]
 *   down_exps blk.L.ffn_down_exps.weight   bf16 [experts][hidden][inter]
 *   gate_sh   blk.L.ffn_gate_shexp.weight  bf16 [inter][hidden]
 *   up_sh     blk.L.ffn_up_shexp.weight    bf16 [inter][hidden]
 *   down_sh   blk.L.ffn_down_shexp.weight  bf16 [hidden][inter]
 * bf16 values are passed as their 16-bit patterns.  Every pointer must be
 * 16-byte aligned.  sel_bias may be NULL for hash layers, tid2eid for score
 * layers. */
typedef struct moe_weights {
  const float* norm_w;
  const uint16_t* router;
  const float* sel_bias;
  const int32_t* tid2eid;
  const uint16_t* gate_exps;
  const uint16_t* up_exps;
  const uint16_t* down_exps;
  const uint16_t* gate_sh;
  const uint16_t* up_sh;
  const uint16_t* down_sh;
} moe_weights_t;

/* Workspace size in bytes that moe_ffn_forward needs for `rows` rows of a
 * layer with dims *d (the page allocates the same intermediates per call:
 * logits, indices, safe indices, weights, routed and shared gate/up/
 * activation/down buffers; here the caller provides one block for them).
 * Host-only, no HIP call.  Errors: MOE_EINVAL, MOE_EUNSUPPORTED,
 * MOE_EOVERFLOW. */
int moe_ffn_workspace_bytes(const moe_dims_t* d, int64_t rows, size_t* bytes);

/* The whole layer for `rows` rows (ffn_forward.rs, forward_ffn_rows from
 * the FFN RMSNorm through the weighted reduce):
 *   x          device f32 [rows][hidden]  FFN input (the page's ffn_input)
 *   token_ids  device i32 [rows]          token id per row; required for
 *                                          MOE_LAYER_HASH, may be NULL for
 *                                          MOE_LAYER_SCORE
 *   layer_kind MOE_LAYER_SCORE or MOE_LAYER_HASH
 *   w          the layer's parameters (see moe_weights_t)
 *   out        device f32 [rows][hidden]  fully overwritten; must not
 *                                          overlap x
 *   workspace  device, >= moe_ffn_workspace_bytes(d, rows), 256-byte
 *              aligned, zero-filled before its first use (e.g. by
 *              hipMemset); after that every call leaves it valid for the
 *              next, whatever the row count, in any order of eager calls
 *              and graph replays.  (Calls of 2 to 4 rows keep an arrival
 *              count of their router workgroups in it, which must read 0
 *              when a call starts; the workgroup that completes the count
 *              routes the batch and sets it back to 0.)  After the call the
 *              workspace holds the routing (see moe_ffn_routing_view) and
 *              the status word (see moe_ffn_status) until the next call
 *              that uses it.
 * Token ids and table entries are device data, so a bad one is not a host
 * error: the affected slots are masked (they contribute nothing and the
 * row's other weights are renormalised over its valid slots) and a status
 * bit is set.  The result is bitwise reproducible for equal inputs.
 * Precision (the page keeps every activation in F32):
 *   rows <= 4  f32 activations, bf16 weights widened exactly, f32 FMA
 *              accumulation; no range limit beyond f32's.
 *   rows > 4   the normalised input and the SwiGLU output are rounded to
 *              fp16 (the router also adds the input's fp16 rounding
 *              remainder, about 22 significant bits in all), weights
 *              converted bf16 -> fp16, f32 accumulation on the matrix
 *              cores; routed down outputs are kept in fp16 until the
 *              f32 weighted reduce.  Domain: every such operand must stay
 *              within fp16's range (|v| <= 65504), else the output is not
 *              finite and MOE_FLAG_F16_RANGE is set; values below 2^-14
 *              are fp16 subnormals, carried within 2^-25 absolute, so a
 *              layer whose SwiGLU outputs are mostly that small (weights
 *              ~100x smaller than the N(0, 0.02) the accuracy is stated
 *              for) loses relative accuracy on this path. 
 * Errors (host-checked): MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EOVERFLOW,
 * MOE_EWORKSPACE, MOE_EOVERLAP; MOE_EHIP if a launch fails. */
int moe_ffn_forward(const moe_dims_t* d, const float* x, const int32_t* token_ids, int64_t rows,
                    int layer_kind, const moe_weights_t* w, float* out, void* workspace,
                    size_t workspace_bytes, void* stream);

/* ---- block-scaled 8-bit expert weights (OCP Microscaling MXFP8) --------
 * ffn_forward.rs binds the expert matrices (ffn_{gate,up,down}_exps,
 * ffn_{gate,up,down}_shexp) as GGML-typed raw matrices, i.e. in whatever
 * quantised type the model file holds; the library's second weight format
 * is OCP MXFP8: one FP8 E4M3 code per weight and one E8M0 power-of-two
 * scale per MOE_MX_BLOCK consecutive weights of a row (along the input
 * dimension), value = e4m3(code) * 2^(scale - 127).  (The pages' only MXFP8
 * step, the attention page's fake quantisation of activations, uses blocks
 * of 64; these are weights, in the OCP block of 32.)  The router stays
 * bf16. */
#define MOE_MX_BLOCK 32

typedef struct moe_mx_matrix {
  const uint8_t* codes;   /* E4M3 codes, [out][in] (routed: [experts][out][in]) */
  const uint8_t* scales;  /* E8M0 codes, [out][in / 32] (routed: [experts][out][in / 32]) */
} moe_mx_matrix_t;

/* The parameters of moe_weights_t with the six expert matrices in MXFP8.
 * All DEVICE pointers, caller-owned, read-only, 16-byte aligned; shapes as
 * in moe_weights_t (gate/up [inter][hidden], down [hidden][inter]). */
typedef struct moe_mx_weights {
  const float* norm_w;
  const uint16_t* router;
  const float* sel_bias;
  const int32_t* tid2eid;
  moe_mx_matrix_t gate_exps, up_exps, down_exps;
  moe_mx_matrix_t gate_sh, up_sh, down_sh;
} moe_mx_weights_t;

/* moe_ffn_forward with MXFP8 expert weights: same arguments, workspace
 * (moe_ffn_workspace_bytes), routing, status and bitwise reproducibility.
 * Reads about half the expert bytes of the bf16 layer.  Precision:
 *   rows <= 4  each weight is its decoded value exactly (E4M3 and E8M0
 *              values are exact in f32), f32 accumulation.
 *   rows > 4   each weight is its decoded value rounded to nearest even
 *              fp16 (exact for 2^-14 <= |w| <= 65504, within 2^-25
 *              below, infinite beyond), then as moe_ffn_forward's fp16
 *              path, with its domain and MOE_FLAG_F16_RANGE.
 * Errors: as moe_ffn_forward; MOE_EINVAL also for a missing or misaligned
 * code or scale array. */
int moe_ffn_forward_mxfp8(const moe_dims_t* d, const float* x, const int32_t* token_ids, int64_t rows,
                          int layer_kind, const moe_mx_weights_t* w, float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* moe_ffn_forward with MXFP4 expert weights (OCP Microscaling MXFP4): the
 * same moe_mx_weights_t, whose code arrays now hold FP4 E2M1 codes packed
 * two per byte -- [out][in / 2] (routed: [experts][out][in / 2]), the
 * element of the lower input index in the low nibble -- with the same E8M0
 * scales, value = e2m1(code) * 2^(scale - 127) (E2M1: sign, 2 exponent bits
 * of bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).  Same
 * arguments, workspace, routing, status and reproducibility.  Reads about a
 * quarter of the expert bytes of the bf16 layer.  Precision as
 * moe_ffn_forward_mxfp8: rows <= 4 each weight exactly, f32 accumulation;
 * rows > 4 each weight rounded to nearest even fp16 (exact for decoded
 * magnitudes 2^-14 .. 65504), then the fp16 path.
 * Errors: as moe_ffn_forward_mxfp8. */
int moe_ffn_forward_mxfp4(const moe_dims_t* d, const float* x, const int32_t* token_ids, int64_t rows,
                          int layer_kind, const moe_mx_weights_t* w, float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* moe_ffn_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, kernels and
 * results as moe_ffn_forward (bitwise), except that the intermediates live
 * in a library-owned device array of MOE_NOALLOC_SCRATCH_BYTES per GPU
 * (a file-scope device variable, held until the process ends), so the
 * call allocates and frees nothing.
 *   Limit: a call whose moe_ffn_workspace_bytes exceeds the array is
 *   rejected with MOE_ESCRATCH before any HIP call -- at the full shape
 *   (hidden 4096, 256 experts, inter 2048) that is more than 696 rows, at
 *   the tiny shape more than 5540 rows; decode calls (1 to 4 rows) always
 *   fit.
 *   Sharing: every call on one GPU uses that GPU's array, which keeps the
 *   last call's contents.  Calls on one stream (or otherwise ordered) are
 *   fine in any mix with moe_ffn_forward; calls that overlap in time on one
 *   GPU race and give wrong results.
 *   Set-up: the first call on each GPU looks up the array's device address
 *   (hipGetSymbolAddress, with that GPU current); until one call has run
 *   outside stream capture, a call also enqueues a small kernel that zeroes
 *   the array's handoff words before the forward (inside a capture it
 *   becomes part of the graph, harmless on every replay).
 *   The status word and routing of these calls are not exposed (there is no
 *   workspace pointer to read them from).
 * Errors: those of moe_ffn_forward except MOE_EWORKSPACE, plus
 * MOE_ESCRATCH; MOE_EHIP if the set-up or a launch fails. */
int moe_ffn_forward_noalloc(const moe_dims_t* d, const float* x, const int32_t* token_ids, int64_t rows,
                            int layer_kind, const moe_weights_t* w, float* out, void* stream);

/* ---- hyper-connection wrapper -------------------------------------------
 * forward_ffn_rows on the ffn_forward.rs page takes the residual state as
 * F32 [rows][hc][hidden] (hc = the model's hyper_connection_count) and
 * returns a new state of that shape.  Before the FFN it normalises each
 * row's flattened state without a scale (rms_norm_no_scale_f32 with
 * rms_norm_eps), multiplies it by hc_ffn_fn into (2 + hc) * hc "mixes"
 * (the "HC FFN function" matmul), splits those with hc_ffn_scale and
 * hc_ffn_base into pre [hc], post [hc] and comb [hc][hc]
 * (dispatch_hc_split_sinkhorn) and mixes the streams into the FFN input
 * with pre (dispatch_hc_pre); after the weighted reduce, dispatch_hc_post
 * combines the FFN output and the old state with post and comb.  The page
 * prints no formula for the split, pre and post steps; this library
 * computes (the published manifold-constrained hyper-connection maps, which
 * match those names and shapes):
 *   mixes  = state_flat * (mean(state_flat^2) + eps)^(-1/2) @ hc_fn^T,
 *            columns: pre (hc) | post (hc) | comb (hc * hc, row-major
 *            (output stream j, input stream i))
 *   pre_i  = sigmoid(hc_scale[0] * mix_pre_i + hc_base[i])
 *   post_j = 2 * sigmoid(hc_scale[1] * mix_post_j + hc_base[hc + j])
 *   comb   = exp(hc_scale[2] * mix_comb + hc_base[2hc ..]) after
 *            sinkhorn_iters rounds of dividing each row by its sum, then
 *            each column by its sum
 *   x      = sum_i pre_i * state_i            (the FFN input, moe_ffn_forward)
 *   new_j  = post_j * ffn(x) + sum_i comb[j][i] * state_i */
#define MOE_HC_MAX 4
#define MOE_HC_MAX_ITERS 1000

typedef struct moe_hc_weights {
  const uint16_t* hc_fn;   /* device bf16 [(2+hc)*hc][hc*hidden] (hc_ffn_fn), 16-byte aligned */
  const float* hc_scale;   /* device f32 [3]: pre, post, comb (hc_ffn_scale) */
  const float* hc_base;    /* device f32 [(2+hc)*hc] (hc_ffn_base) */
  int32_t hc;              /* streams, 1..MOE_HC_MAX */
  int32_t sinkhorn_iters;  /* Sinkhorn rounds, 1..MOE_HC_MAX_ITERS */
} moe_hc_weights_t;

/* Workspace bytes of moe_ffn_forward_hc: moe_ffn_workspace_bytes' layout at
 * offset 0 (so moe_ffn_routing_view and moe_ffn_status read the inner FFN
 * call's routing and status from it), then the wrapper's intermediates.
 * Host-only.  Errors: MOE_EINVAL, MOE_EUNSUPPORTED (also hc outside
 * 1..MOE_HC_MAX), MOE_EOVERFLOW. */
int moe_ffn_hc_workspace_bytes(const moe_dims_t* d, int32_t hc, int64_t rows, size_t* bytes);

/* The wrapped layer:
 *   state_in   device f32 [rows][hc][hidden], 16-byte aligned
 *   state_out  device f32 [rows][hc][hidden], 16-byte aligned, overlapping
 *              neither state_in nor the workspace
 *   token_ids, layer_kind, w   as moe_ffn_forward
 *   hw         the wrapper's parameters (struct read on the host)
 *   workspace  moe_ffn_hc_workspace_bytes of device memory, 256-byte
 *              aligned, zero-filled before its first use (as for
 *              moe_ffn_forward, whose intermediates it holds)
 * Launches on `stream`: the mixes' partial sums, the split with the FFN
 * input, moe_ffn_forward on it (same precision, routing and status), the
 * new state; with 1 to 4 rows the split, the FFN input and the new state
 * are formed inside moe_ffn_forward's own launches.  The wrapper's arithmetic is f32, sums in a fixed order; the
 * result is bitwise reproducible.
 * Errors: those of moe_ffn_forward; MOE_EINVAL also for a missing or
 * misaligned hc array or a round count outside 1..MOE_HC_MAX_ITERS,
 * MOE_EUNSUPPORTED for hc outside 1..MOE_HC_MAX. */
int moe_ffn_forward_hc(const moe_dims_t* d, const float* state_in, const int32_t* token_ids, int64_t rows,
                       int layer_kind, const moe_weights_t* w, const moe_hc_weights_t* hw, float* state_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Device pointers, inside a moe_ffn_forward_hc workspace, to the last
 * call's mixes and maps (f32 [rows][(2+hc)*hc]; maps: pre | post | comb as
 * above), FFN input and FFN output (f32 [rows][hidden]).  Any output
 * pointer may be NULL.  Host-only arithmetic, no HIP call.
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EOVERFLOW, MOE_EWORKSPACE. */
int moe_ffn_hc_view(const moe_dims_t* d, int32_t hc, int64_t rows, void* workspace, size_t workspace_bytes,
                    const float** mixes, const float** maps, const float** ffn_in, const float** ffn_out);

/* Routing alone, from caller-given logits (ffn_forward.rs: the score-route
 * and hash-route dispatches that turn the F32 logits into I32 indices and
 * F32 weights), using the same device routine as moe_ffn_forward:
 *   logits     device f32 [rows][experts]
 *   token_ids  device i32 [rows] (hash layers; NULL ok for score layers)
 *   w          only sel_bias (score) or tid2eid (hash) is read
 *   idx        device i32 [rows][top_k]  score: experts by key
 *              sigmoid(logit)+bias descending, equal keys to the lower
 *              index, key evaluated in float64; hash: the table row in
 *              column order, -1 for every slot of a bad token id and the
 *              raw entry for a bad table entry
 *   wout       device f32 [rows][top_k]  unbiased sigmoid scores of the
 *              chosen experts over their sum (0 for masked slots)
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EOVERFLOW, MOE_EHIP. */
int moe_route(const moe_dims_t* d, const float* logits, const int32_t* token_ids, int64_t rows,
              int layer_kind, const moe_weights_t* w, int32_t* idx, float* wout, void* stream);

/* Device pointers, inside `workspace`, to the last moe_ffn_forward's router
 * logits (f32 [rows][experts]), indices (i32 [rows][top_k]) and routing
 * weights (f32 [rows][top_k]) for a call with the same dims and rows.  Any
 * output pointer may be NULL.  Host-only arithmetic, no HIP call.
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EOVERFLOW, MOE_EWORKSPACE. */
int moe_ffn_routing_view(const moe_dims_t* d, int64_t rows, void* workspace, size_t workspace_bytes,
                         const float** logits, const int32_t** idx, const float** wout);

/* Synchronises `stream`, then copies the status word of the last
 * moe_ffn_forward that used `workspace` (OR of MOE_FLAG_* bits) to *flags.
 * ffn_forward.rs runs deepseek_moe_sanitize_indices between the route and
 * the expert matmuls, turning the I32 indices into U32 safe indices while
 * the weighted reduce still receives the raw ones; what that step found
 * (a token id outside the table, a table entry outside [0, experts)) is
 * device data the host cannot see at call time, so it is reported here
 * after the fact instead of as an error return.
 * Errors: MOE_EINVAL, MOE_EHIP. */
int moe_ffn_status(const void* workspace, void* stream, uint32_t* flags);

/* Static English text for a status code.  forward_ffn_rows on the
 * ffn_forward.rs page reports its argument failures as anyhow errors from
 * bail! checks (layer and rows range, routed-row overflow, the fixed MoE
 * shape, state dtype and shape, a layer with neither a tid2eid table nor a
 * selection bias); here each becomes a moe_status code checked on the host,
 * and this gives its text. */
const char* moe_strerror(int code);

/* ---- stage timing (replaces the page's env-flagged profile_stage_boundary
 * markers between the router, gate/up, activation and down stages) ------
 * moe_ffn_stage_timing_begin() makes every following moe_ffn_forward launch
 * its kernels with HIP start/stop events taken at the kernels' own start
 * and end.  moe_ffn_stage_timing_end() synchronises those events, writes up
 * to `max` per-kernel totals (name, summed milliseconds, launch count) and
 * stops timing.  *n gets the number of distinct kernels seen.  Not for use
 * under HIP graph capture.  Errors: MOE_EINVAL, MOE_EHIP. */
int moe_ffn_stage_timing_begin(void);
int moe_ffn_stage_timing_end(int max, const char** names, double* total_ms, int64_t* launches, int* n);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
