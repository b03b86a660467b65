/*
 * nrc.h - C ABI of libnrc, the MI355X (gfx950) context K/V chain of the
 * DSpark draft: hidden RMSNorm -> per-layer input RMSNorm, stacked -> batched
 * K/V projection -> weightless 64-wide K-norm -> GPT-J RoPE -> paged-cache
 * insert.
 *
 * Sources: the vLLM API pages of the Muse Spark specialized decode,
 *   "...cutedsl.draft.context"       (ContextNorms, ContextKvStore and their kernels),
 *   "...runtime.draft"               (ContextKV: _project, store),
 *   "...cutedsl.common.draft_boundary" (boundary_fragments: the row-norm arithmetic).
 *
 * Conventions for every call:
 *   - bf16 tensors are passed as uint16_t storage of the bf16 bit patterns.
 *   - Every data pointer is caller-owned DEVICE memory unless stated otherwise.
 *     The library never allocates, frees or reads device memory on the host.
 *     Host pointer arrays (slots, caches) are read during the call only.
 *   - `stream` is a hipStream_t (NULL: the null stream). Calls enqueue their
 *     kernels on it and return without synchronising; nothing is kept after
 *     the return. The current device (hipSetDevice) must be the GPU that
 *     holds the operands and the stream: launch shapes follow its compute
 *     unit count, and nrc_context_kv_project_noalloc uses its scratch.
 *   - Return value: NRC_OK (0) or a negative errno-style code. All argument
 *     checks finish before the first launch, so an error means nothing was
 *     enqueued. nrc_last_error() then describes it.
 *   - Results are deterministic: a call with the same inputs writes the same
 *     bits.
 *   - Outputs must not alias inputs.
 */
#ifndef NRC_H
#define NRC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NRC_OK 0
#define NRC_EIO (-5)       /* a HIP launch or runtime error */
#define NRC_EINVAL (-22)   /* NULL where required, bad shape, stride or alignment */
#define NRC_ENOTSUP (-95)  /* a shape the kernels do not take (hidden width, head dim, ...) */

#define NRC_HIDDEN 8192               /* the norms' row width (one tile of the row norm) */
#define NRC_HEAD_DIM 64               /* K/V head width */
#define NRC_MAX_LAYERS_PER_LAUNCH 8   /* layers per store launch; more are split */

/*
 * nrc_context_norms - stack([pre_norm_l(hidden_norm(x)) for l]).
 * Page "...cutedsl.draft.context", sections ContextNorms and
 * _ContextNormsKernel; arithmetic of one norm per "...draft_boundary",
 * boundary_fragments.
 *
 *   x          [T, D] bf16, contiguous, 16-byte aligned. D must be 8192.
 *   hidden_w   [D] bf16, 16-byte aligned, or NULL for a weightless hidden norm.
 *   pre_w      [L, D] bf16, contiguous, 16-byte aligned, or NULL (weightless
 *              layer norms). Every layer norm shares pre_eps and pre_center.
 *   hidden_eps, pre_eps        FP32 epsilons.
 *   hidden_center, pre_center  gain centers: the weight used is w + center
 *              (0.0 for a plain RMSNorm weight).
 *   out        [L, T, D] bf16, contiguous, 16-byte aligned; element (l, t, c)
 *              at (l * T + t) * D + c.
 * Per row: S = sum of squares in the library's fixed order, r = 1/sqrt(S/D +
 * eps) (one FMA, correctly rounded sqrt and divide), y = (x * r) * gamma,
 * rounded to bf16. The hidden norm's bf16 output feeds the layer norms.
 * T == 0 returns NRC_OK with nothing launched. Errors: NRC_EINVAL (NULL x or
 * out with T > 0, T < 0, L < 1, misalignment), NRC_ENOTSUP (D != 8192).
 */
int32_t nrc_context_norms(const uint16_t* x, int64_t T, int64_t D, const uint16_t* hidden_w,
                          const uint16_t* pre_w, int32_t L, float hidden_eps, float pre_eps,
                          float hidden_center, float pre_center, uint16_t* out, void* stream);

/* Weight kinds and flags of nrc_context_norms_ex. */
#define NRC_WEIGHT_NONE 0
#define NRC_WEIGHT_BF16 1
#define NRC_WEIGHT_F32 2
#define NRC_WEIGHT_F16 3 /* nrc_draft_boundary only */
#define NRC_HIDDEN_INPUT_SCALE 1u
#define NRC_PRE_INPUT_SCALE 2u

/*
 * nrc_context_norms_ex - nrc_context_norms with every weight form the norms
 * accept. Page "...cutedsl.draft.context", ContextNorms and
 * ContextNormConstants (each norm's weight absent, BF16 or FP32; whether the
 * weight scales the norm's input instead of its output); arithmetic of both
 * forms per "...draft_boundary", boundary_fragments.
 *
 *   hidden_w, hidden_kind  NRC_WEIGHT_NONE with NULL, NRC_WEIGHT_BF16 with
 *              [D] bf16, or NRC_WEIGHT_F32 with [D] float; 16-byte aligned.
 *   pre_w, pre_kind        the same for [L, D] layer weights.
 *   flags      NRC_HIDDEN_INPUT_SCALE / NRC_PRE_INPUT_SCALE: that norm's
 *              weight scales its input. Ignored for a weightless norm.
 *   Other arguments as nrc_context_norms.
 * gamma = w + center (FP32 add). Output-scaled: r = 1/sqrt(S(x)/D + eps),
 * y = (x * r) * gamma. Input-scaled: v = gamma * x, r = 1/sqrt(S(v)/D +
 * eps), y = v * r (input-scaled layer norms: one sum per layer). S in the
 * library's fixed order; y rounded to bf16 (nearest even, NaN -> 0x7FC0).
 * With no FP32 weight and no flag the result is nrc_context_norms'.
 * T == 0 returns NRC_OK. Errors: NRC_EINVAL (kind out of range, a pointer
 * NULL or not NULL against its kind, unknown flags, NULL x or out with
 * T > 0, T < 0, L < 1, misalignment), NRC_ENOTSUP (D != 8192).
 */
int32_t nrc_context_norms_ex(const uint16_t* x, int64_t T, int64_t D, const void* hidden_w, int32_t hidden_kind,
                             const void* pre_w, int32_t pre_kind, int32_t L, float hidden_eps, float pre_eps,
                             float hidden_center, float pre_center, uint32_t flags, uint16_t* out, void* stream);

/* Stream kinds and flags of nrc_draft_boundary. */
#define NRC_STREAM_F32 0
#define NRC_STREAM_BF16 1
#define NRC_POST_INPUT_SCALE 1u
#define NRC_PRE_INPUT_SCALE 2u

/*
 * nrc_draft_boundary - one residual boundary of the DSpark draft: post norm
 * of the bf16 branch, the gated FP32 residual, then the next pre norm.
 * Page "...cutedsl.common.draft_boundary": module summary,
 * boundary_fragments, DraftBoundary.run, DraftBoundaryConstants.
 *
 *   branch     [m, D] bf16, contiguous, 16-byte aligned; D must be 8192.
 *   stream_in  [m, D] FP32 (stream_kind NRC_STREAM_F32) or bf16
 *              (NRC_STREAM_BF16), contiguous, 16-byte aligned.
 *   alpha, beta  [D] FP32 gates, 16-byte aligned.
 *   post_w, pre_w  [D] weights of kind NRC_WEIGHT_NONE (NULL), _BF16, _F32
 *              or _F16; the gain is w + center (FP32 add).
 *   flags      NRC_POST_INPUT_SCALE / NRC_PRE_INPUT_SCALE: that norm's
 *              weight scales its input (else its output).
 *   stream_out [m, D] FP32 new stream, or NULL (not stored).
 *   out        [m, D] bf16.
 * Per row: post norm u = x (or gamma_post * x), r1 = 1/sqrt(S(u)/D +
 * post_eps), y = u * r1 (* gamma_post); res = alpha * stream + beta *
 * bf16(y) (each product rounded, then the sum), stream_out = res; pre norm of
 * z = bf16(res) the same way with gamma_pre and pre_eps, rounded to bf16.
 * Sums in the library's fixed order; bf16 rounding to nearest even, NaN ->
 * 0x7FC0. m == 0 returns NRC_OK. Errors: NRC_EINVAL (kinds out of range, a
 * weight pointer against its kind, unknown flags, NULL operands with
 * m > 0, m < 0, misalignment), NRC_ENOTSUP (D != 8192).
 */
int32_t nrc_draft_boundary(const uint16_t* branch, int64_t m, int64_t D, const void* stream_in, int32_t stream_kind,
                           const float* alpha, const float* beta, const void* post_w, int32_t post_kind,
                           const void* pre_w, int32_t pre_kind, float post_eps, float pre_eps, float post_center,
                           float pre_center, uint32_t flags, float* stream_out, uint16_t* out, void* stream);

/*
 * nrc_context_kv_project - the batched K/V projection C[l] = A[l] . B[l].
 * Page "...runtime.draft", ContextKV._project (the bmm of the stacked layer
 * norms against the stacked K/V weight).
 *
 *   normed  A: [L, T, D] bf16, contiguous, 16-byte aligned.
 *   w       B: [L, D, N] bf16, contiguous, 16-byte aligned (the bmm's logical
 *           right operand; N contiguous).
 *   kv      C: [L, T, N] bf16, contiguous, 16-byte aligned; per row the H K
 *           heads then the H V heads (N = 2 * H * 64).
 * FP32 accumulation on the bf16 matrix cores, rounded to bf16 (nearest even)
 * once. The summation order is the kernel's; results match an FP32 sum to
 * bf16 tolerance. T == 0 returns NRC_OK. Errors: NRC_EINVAL (NULLs, L < 1,
 * T < 0, misalignment), NRC_ENOTSUP (D not a positive multiple of 64, N not
 * a positive multiple of 128).
 */
int32_t nrc_context_kv_project(const uint16_t* normed, const uint16_t* w, uint16_t* kv, int32_t L, int64_t T,
                               int64_t D, int64_t N, void* stream);

/* Weight layouts of nrc_context_kv_project_ex. */
#define NRC_KV_WEIGHT_DN 0 /* [L, D, N], N contiguous (the bmm's logical right operand) */
#define NRC_KV_WEIGHT_ND 1 /* [L, N, D], D contiguous (the pages' stacked weight storage) */

/*
 * nrc_context_kv_project_ex - nrc_context_kv_project with the weight in
 * either layout. Page "...runtime.draft", ContextKV._project: the pages
 * stack the layers' K/V weights as [L, N, D] and multiply by its transpose.
 *
 *   w_layout  NRC_KV_WEIGHT_DN: w is [L, D, N]; NRC_KV_WEIGHT_ND: w is
 *             [L, N, D]; contiguous, 16-byte aligned.
 *   Other arguments and errors as nrc_context_kv_project, plus NRC_EINVAL
 *   for an unknown layout. Both layouts give the same bits.
 */
int32_t nrc_context_kv_project_ex(const uint16_t* normed, const uint16_t* w, int32_t w_layout, uint16_t* kv,
                                  int32_t L, int64_t T, int64_t D, int64_t N, void* stream);

/*
 * nrc_context_kv_project_workspace_bytes - bytes of workspace the split form
 * of the projection needs for this shape on the current device, or 0 when
 * the shape is not split. Shapes whose output tiles are too few to occupy
 * the device's compute units split the D (summation) axis into 2 to 16
 * slices, a power of two (the projection is a stock bmm, whose summation order is free).
 * Page "...runtime.draft", ContextKV._project. Returns a negative status
 * for shapes nrc_context_kv_project rejects.
 */
int64_t nrc_context_kv_project_workspace_bytes(int32_t L, int64_t T, int64_t D, int64_t N);

/*
 * nrc_context_kv_project_split - nrc_context_kv_project_ex that may split the
 * summation axis for shapes with few output tiles (small T). Each slice's
 * FP32 sums go to the workspace, then are added slice by slice in a fixed
 * order (deterministic) and rounded to bf16 once. Page "...runtime.draft",
 * ContextKV._project.
 *
 *   workspace        caller-owned device memory, 16-byte aligned, of at
 *                    least nrc_context_kv_project_workspace_bytes(L, T, D, N)
 *                    bytes; read and written by the call, contents on return
 *                    unspecified. Unused (may be NULL) when that size is 0.
 *   workspace_bytes  its size in bytes.
 *   Other arguments as nrc_context_kv_project_ex. Errors as there, plus
 *   NRC_EINVAL for a workspace that is NULL, too small or misaligned when
 *   the shape splits. Calls that share a workspace must not overlap.
 */
int32_t nrc_context_kv_project_split(const uint16_t* normed, const uint16_t* w, int32_t w_layout, uint16_t* kv,
                                     int32_t L, int64_t T, int64_t D, int64_t N, void* workspace,
                                     int64_t workspace_bytes, void* stream);

/* Bytes of device scratch behind nrc_context_kv_project_noalloc (one copy per GPU). */
#define NRC_PROJECT_SCRATCH_BYTES (64LL << 20)

/*
 * nrc_context_kv_project_noalloc - nrc_context_kv_project_split for callers
 * that cannot allocate device memory (code under graph capture, serving loops
 * and harnesses that forbid allocation): the split form's FP32 partial sums
 * go to a scratch array the library holds on each GPU (NRC_PROJECT_SCRATCH_BYTES,
 * taken when the library is first used on that GPU and held until the
 * process ends) instead of a caller workspace. Same kernels, split rule and
 * bits as nrc_context_kv_project_split; shapes that do not split run the
 * one-pass kernel and touch no scratch. The call allocates nothing.
 *
 *   Arguments as nrc_context_kv_project_ex; the caller owns every operand.
 *   Errors as nrc_context_kv_project_ex, plus NRC_EINVAL when the shape's
 *   split needs more than NRC_PROJECT_SCRATCH_BYTES (nothing is launched)
 *   and NRC_EIO when the scratch has no address on the current device.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap in
 *   time on one GPU (other streams, other threads) race and must be ordered
 *   by the caller. Each call writes every scratch element it reads, so no
 *   state carries over between calls.
 */
int32_t nrc_context_kv_project_noalloc(const uint16_t* normed, const uint16_t* w, int32_t w_layout, uint16_t* kv,
                                       int32_t L, int64_t T, int64_t D, int64_t N, void* stream);

/*
 * nrc_context_kv_project_timed - nrc_context_kv_project_ex (one pass, never
 * split) that also records, per workgroup, the shader clock counter
 * (s_memtime) and the constant-rate counter (s_memrealtime) when the
 * workgroup starts and when it ends. A diagnostic for callers that want the
 * clock the matrix cores ran at: (end - start) of the first counter over
 * that of the second, times the constant rate. Same operation and bits as
 * nrc_context_kv_project_ex (page "...runtime.draft", ContextKV._project).
 *
 *   stamps      caller-owned device memory, 8-byte aligned, uint64
 *               [stamps_len]; workgroup g writes stamps[4 g .. 4 g + 3] =
 *               shader clock at start, constant clock at start, shader
 *               clock at end, constant clock at end. Other entries untouched.
 *   stamps_len  its length in elements, at least nrc_context_kv_project_timed
 *               needs: 8 times the device's compute unit count.
 *   workgroups  host int32: receives the number of workgroups launched
 *               (each writes its 4 stamps).
 *   wall_khz    host int32: receives the constant counter's rate in kHz.
 *   Other arguments and errors as nrc_context_kv_project_ex, plus NRC_EINVAL
 *   for NULL or misaligned stamps, a short stamps_len, or NULL host outputs.
 *   T == 0: returns 0 with *workgroups = 0 and launches nothing.
 */
int32_t nrc_context_kv_project_timed(const uint16_t* normed, const uint16_t* w, int32_t w_layout, uint16_t* kv,
                                     int32_t L, int64_t T, int64_t D, int64_t N, uint64_t* stamps,
                                     int64_t stamps_len, int32_t* workgroups, int32_t* wall_khz, void* stream);

/*
 * nrc_context_hidden_norm - the pre-pass of the fused norms + projection: the
 * hidden norm and each row's layer-norm scale, the two quantities every
 * layer norm of a row shares. Page "...cutedsl.draft.context", ContextNorms
 * (the hidden norm's output is rounded to bf16 before the layer norms read
 * it; the layer norms share eps and center, page "...runtime.draft",
 * _context_norm_constants).
 *
 *   x, T, D, hidden_w, hidden_eps, hidden_center: as nrc_context_norms.
 *   pre_w [L, D] or NULL, pre_eps, pre_center: the layer norms' operands (the
 *          weights are only checked for finiteness here).
 *   h  [T, D] bf16, 16-byte aligned: the hidden norm's bf16 output.
 *   r  [T] float: 1/sqrt(S_p/8192 + pre_eps), S_p the row's sum of squares
 *      of h in the library's order. The sign bit is set on rows whose layer
 *      outputs may be NaN (non-finite S_p or scale, non-finite layer weights
 *      or center); |r| is the scale.
 * nrc_context_norms' output equals bf16((h * |r|) * (pre_w[l] + pre_center))
 * element by element. Errors as nrc_context_norms.
 */
int32_t nrc_context_hidden_norm(const uint16_t* x, int64_t T, int64_t D, const uint16_t* hidden_w,
                                const uint16_t* pre_w, int32_t L, float hidden_eps, float pre_eps,
                                float hidden_center, float pre_center, uint16_t* h, float* r, void* stream);

/*
 * nrc_context_kv_project_fused - the projection with the layer norms applied
 * on the fly: kv[l] = A_l . w[l], A_l = bf16((h * |r|) * (pre_w[l] +
 * pre_center)) (no weight: bf16(h * |r|)). Bit-identical to
 * nrc_context_norms followed by nrc_context_kv_project, without the
 * [L, T, D] intermediate. Page "...runtime.draft", ContextKV._project.
 *
 *   h [T, D] bf16 and r [T] from nrc_context_hidden_norm; pre_w [L, D] bf16
 *   or NULL; w [L, D, N]; kv [L, T, N] as nrc_context_kv_project. D = 8192.
 * Errors: NRC_EINVAL (NULLs, L < 1, T < 0, misalignment), NRC_ENOTSUP
 * (D != 8192, N not a positive multiple of 128).
 */
int32_t nrc_context_kv_project_fused(const uint16_t* h, const float* r, const uint16_t* pre_w, float pre_center,
                                     const uint16_t* w, uint16_t* kv, int32_t L, int64_t T, int64_t D, int64_t N,
                                     void* stream);

/*
 * nrc_context_kv_project_fused_split - nrc_context_kv_project_fused that
 * splits the summation axis for shapes with few output tiles (small T), as
 * nrc_context_kv_project_split does: the same slices, the same fixed-order
 * addition, so the same bits as nrc_context_kv_project_split on the stacked
 * layer norms. Page "...runtime.draft", ContextKV._project (a stock bmm,
 * summation order free) on the norms of "...cutedsl.draft.context",
 * _ContextNormsKernel.
 *
 *   workspace, workspace_bytes  as nrc_context_kv_project_split: caller-owned
 *                    device memory of nrc_context_kv_project_workspace_bytes(L,
 *                    T, D, N) bytes, 16-byte aligned; unused when that is 0.
 *   Other arguments and errors as nrc_context_kv_project_fused, plus
 *   NRC_EINVAL for a workspace that is NULL, too small or misaligned when
 *   the shape splits. Calls that share a workspace must not overlap.
 */
int32_t nrc_context_kv_project_fused_split(const uint16_t* h, const float* r, const uint16_t* pre_w, float pre_center,
                                           const uint16_t* w, uint16_t* kv, int32_t L, int64_t T, int64_t D,
                                           int64_t N, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * nrc_context_kv_store - weightless K-norm, GPT-J RoPE and paged-cache insert
 * of L layers. Page "...cutedsl.draft.context", sections ContextKvStore,
 * _ContextKvStoreKernel, _sum_squares_64 and _rope; operand checks per
 * "...runtime.draft", ContextKV.store.
 *
 *   k, v       bf16 [L, T, H, 64] views: unit stride in the last dim, 64 between
 *              heads; k_layer_stride, k_row_stride, v_layer_stride,
 *              v_row_stride in elements (multiples of 8: 16-byte rows).
 *              k and v 16-byte aligned. For the projection output [L, T, N]:
 *              k = kv, v = kv + H * 64, layer stride T * N, row stride N.
 *   positions  [>= rows] int64 device array; read only when cos_sin != NULL.
 *   slots      HOST array of L device pointers, each int64 [rows], contiguous.
 *              Row t of layer l goes to slot slots[l][t]; a negative slot skips
 *              the row. Only rows 0 .. rows-1 are inserted (rows <= T).
 *   cos_sin    [max_position, 64] bf16 (cos_0..31 then sin_0..31 per position),
 *              contiguous, 16-byte aligned; NULL: no RoPE.
 *   caches     HOST array of L device pointers, each a bf16 cache
 *              [num_blocks, H, block_size, 128], contiguous, 16-byte aligned:
 *              K of (slot, head h) at [slot / block_size, h, slot % block_size,
 *              0:64], V at [..., 64:128].
 *   eps        the K-norm's FP32 epsilon.
 * Per (layer, row, head): S = the 64 squares folded by halves (strides 32 ..
 * 1), r = 1/sqrt(S/64 + eps), n = bf16(k * r), then per pair (2j, 2j+1):
 * (n0 c - n1 s, n1 c + n0 s) with one FMA each, rounded to bf16; V is copied
 * bit for bit. No other cache cell is written.
 * Preconditions (not checked: they need device reads): 0 <= positions[t] <
 * max_position and 0 <= slot < num_blocks * block_size for inserted rows;
 * non-negative slots distinct within a layer. A row that breaks the range
 * preconditions is skipped by the kernel (never written out of bounds).
 * rows == 0 returns NRC_OK. Layers beyond 8 take further launches.
 * Errors: NRC_EINVAL (NULLs, rows > T, misaligned strides or pointers, H < 1),
 * NRC_ENOTSUP (H not a power of two, num_blocks * block_size >= 2^31).
 */
int32_t nrc_context_kv_store(const uint16_t* k, const uint16_t* v, int64_t k_layer_stride, int64_t k_row_stride,
                             int64_t v_layer_stride, int64_t v_row_stride, const int64_t* positions,
                             const int64_t* const* slots, int64_t rows, int64_t T, const uint16_t* cos_sin,
                             int64_t max_position, uint16_t* const* caches, int64_t num_blocks, int64_t block_size,
                             int32_t H, int32_t L, float eps, void* stream);

/*
 * nrc_context_kv_store_ex - nrc_context_kv_store with the pages' full
 * operand surface: page "...cutedsl.draft.context", ContextKvStore (strided
 * key-cache views: block, page and head strides, K then V in a 128-element
 * run), and page "...runtime.draft", _slot_groups (a per-layer slot list,
 * None for a layer that stores nothing, runs of layers with lists of their
 * own length).
 *
 *   slots    host array of L pointers: layer l's int64 slot list, 8-byte
 *            aligned, or NULL (the layer stores nothing; caches[l] unused).
 *   rows     host array of L counts: the first rows[l] rows of layer l are
 *            inserted, 0 <= rows[l] <= T (ignored where slots[l] is NULL).
 *   caches   host array of L pointers at K of (block 0, page 0, head 0) of
 *            each layer's cache, 16-byte aligned. (block, page, head) lives
 *            at block * block_stride + page * page_stride + head *
 *            head_stride elements: K in [0, 64), V in [64, 128). Strides are
 *            non-negative multiples of 8 elements; the runs must not overlap
 *            and must lie inside the caller's buffer for every slot below
 *            num_blocks * block_size (not checked: device memory).
 *   Other arguments as nrc_context_kv_store.
 * The contiguous [num_blocks, H, block_size, 128] cache of nrc_context_kv_store
 * is block_stride = H * block_size * 128, page_stride = 128, head_stride =
 * block_size * 128. Errors: as nrc_context_kv_store, plus NRC_EINVAL (NULL
 * rows array, rows[l] outside [0, T], negative stride) and NRC_ENOTSUP
 * (a cache stride not a multiple of 8 elements).
 */
int32_t nrc_context_kv_store_ex(const uint16_t* k, const uint16_t* v, int64_t k_layer_stride, int64_t k_row_stride,
                                int64_t v_layer_stride, int64_t v_row_stride, const int64_t* positions,
                                const int64_t* const* slots, const int64_t* rows, int64_t T,
                                const uint16_t* cos_sin, int64_t max_position, uint16_t* const* caches,
                                int64_t num_blocks, int64_t block_size, int64_t block_stride, int64_t page_stride,
                                int64_t head_stride, int32_t H, int32_t L, float eps, void* stream);

/*
 * nrc_context_kv_project_store - the projection and the store of
 * "...runtime.draft", ContextKV (_project, then store on the k/v views of the
 * projection's own output) in one call, with the same results as
 * nrc_context_kv_project_split followed by nrc_context_kv_store on
 * k = kv, v = kv + H 64 (layer stride T N, row stride N), H = N / 128: kv
 * and every cache cell bit for bit. Where the shape splits the summation,
 * the slices are added by the store's kernel (slice order, one rounding to
 * bf16, as nrc_context_kv_project_split adds them), which writes kv and
 * inserts each row in the same pass; otherwise the one-pass projection runs,
 * then the store.
 *
 *   normed, w, w_layout, kv, L, T, D, N, workspace, workspace_bytes
 *              as nrc_context_kv_project_split (kv [L, T, N] is written,
 *              every row).
 *   positions, slots, rows, cos_sin, max_position, caches, num_blocks,
 *   block_size, eps
 *              as nrc_context_kv_store (slots and caches: host arrays of L
 *              device pointers; rows <= T; caches contiguous
 *              [num_blocks, H, block_size, 128]).
 * Every operand is checked before anything is launched. Errors: those of
 * both calls (N / 128 must be a power of two). rows == 0: the projection
 * alone (slots, caches unused). T == 0: NRC_OK, nothing launched. Calls
 * that share a workspace must not overlap.
 */
int32_t nrc_context_kv_project_store(const uint16_t* normed, const uint16_t* w, int32_t w_layout, uint16_t* kv,
                                     int32_t L, int64_t T, int64_t D, int64_t N, void* workspace,
                                     int64_t workspace_bytes, const int64_t* positions, const int64_t* const* slots,
                                     int64_t rows, const uint16_t* cos_sin, int64_t max_position,
                                     uint16_t* const* caches, int64_t num_blocks, int64_t block_size, float eps,
                                     void* stream);

/*
 * nrc_check_scalars - diagnostic: the device primitives every kernel uses,
 * applied elementwise to n FP32 values (device arrays), so that they can be
 * compared with a reference over all 2^32 inputs:
 *   bf16_out[i]  = f32 -> bf16 rounding of in[i] (nearest even; NaN -> 0x7FC0)
 *   rsqrt_out[i] = 1 / sqrt(in[i]), both correctly rounded
 * Either output may be NULL. n <= 2^32. Errors: NRC_EINVAL.
 */
int32_t nrc_check_scalars(const float* in, uint16_t* bf16_out, float* rsqrt_out, int64_t n, void* stream);

/*
 * nrc_check_bf16_pair - diagnostic: the paired hardware f32 -> bf16
 * conversion (v_cvt_pk_bf16_f32) that nrc_context_norms uses on rows that
 * cannot produce NaN, applied to n device floats: out[i] for in[i]. For
 * every non-NaN input it must equal nrc_check_scalars' bf16 rounding.
 * n <= 2^32. Errors: NRC_EINVAL.
 */
int32_t nrc_check_bf16_pair(const float* in, uint16_t* out, int64_t n, void* stream);

/*
 * nrc_traffic_twin - diagnostic: the HBM traffic of nrc_context_norms
 * without its arithmetic, to measure the bandwidth ceiling of that traffic.
 * The same workgroups, grid, row walk and next-row prefetch as the norms
 * kernel; each 256-thread row slot reads its row of x [T, 8192] bf16 in the
 * norms' fragments (lane t: columns 2048 k + 8 t .. + 7, k < 4) and writes
 * it unchanged to that row of each of the L outputs out [L, T, 8192].
 *
 *   mode    0: the norms' stores (non-temporal, system scope, buffer form);
 *           1: plain stores; 2: reads only (out unused; each thread writes
 *           one uint32 to sink); 3: writes only (x unused; a pattern)
 *   per_cu  workgroups per CU at most: 1 as the norms with weights staged
 *           past 64 KiB of LDS (the long workload), 2 otherwise
 *   sink    mode 2: device uint32 array of at least per_cu * CUs * 1024
 *           entries; else unused
 * Errors: NRC_EINVAL (bad mode, per_cu, shape, NULL or misaligned operand).
 */
int32_t nrc_traffic_twin(const uint16_t* x, int64_t T, int32_t L, int32_t mode, int32_t per_cu, uint16_t* out,
                         uint32_t* sink, int64_t sink_len, void* stream);

/* Thread-local description of the last non-zero status of this thread. */
const char* nrc_last_error(void);

/* ABI version: 1. */
int32_t nrc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NRC_H */
