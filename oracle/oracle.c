/*
 * CPU oracle of the DSpark draft's context K/V chain.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the bench's
 * cpu_baseline leg use it. It shares no code, header, table or constant with
 * the HIP library; both sides are written separately from the same pages.
 *
 * Sources (vLLM API pages, docs builds of the Muse Spark specialized decode):
 *   [CTX]  page "vllm.models.muse_spark.nvidia.specialized_decode.cutedsl.draft.context"
 *          sections ContextKvStore, ContextNorms, _ContextNormsKernel,
 *          _ContextKvStoreKernel, _rope, _sum_squares_64.
 *   [RT]   page "vllm.models.muse_spark.nvidia.specialized_decode.runtime.draft"
 *          section ContextKV (_project, store).
 *   [BND]  page "vllm.models.muse_spark.nvidia.specialized_decode.cutedsl.common.draft_boundary"
 *          section boundary_fragments (the arithmetic of an 8192-wide row norm).
 *
 * Arithmetic: IEEE-754 binary32, round to nearest even, subnormals kept, no
 * contraction except where fmaf() is written. Build with
 *   gcc -O2 -ffp-contract=off -fno-fast-math
 * so that no a*b+c is fused behind our back.
 *
 * Readings where the pages leave a step open (each is listed in the design notes):
 *   - rsqrt: the pages use an approximate hardware reciprocal square root;
 *     here rs(v) = 1 / sqrt(v), both correctly rounded (no approximation).
 *   - the 8192-wide row's reduction order is not on the pages; the order in
 *     sumsq_row() below is this project's contract (256 lanes x 4 fragments x
 *     8 columns, two FMA accumulators per lane, a 64-lane fold per wave, then a
 *     fold of the 4 wave sums).
 *   - any NaN rounds to the bf16 quiet NaN 0x7FC0.
 *   - gain center: gamma = weight + center, center 0.0 unless given.
 *
 * Parity pins: every exported function is checked by the CPU tests against
 * closed forms, hand-derived instances, library routines or brute force.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_EINVAL (-22)

/* ---------------------------------------------------------------- scalars */

/* Exact bf16 -> f32: the bf16 bits are the top half of the f32. */
static float f_of(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* f32 -> bf16, round to nearest, ties to even, on the bit pattern. Overflow
 * reaches +-Inf by the carry into the exponent; subnormals and signed zeros
 * follow the same rule; every NaN becomes 0x7FC0. */
static uint16_t bf(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7FFFu + keep_lsb;
    return (uint16_t)(u >> 16);
}

/* Reciprocal square root as two correctly rounded IEEE operations. */
static float rs(float v) { return 1.0f / sqrtf(v); }

/* FOLD_n: pairwise fold by halves, v[i] + v[i + n/2] for i < n/2, repeated
 * until one value is left (in place; n a power of two). */
static float fold(float *v, int n) {
    while (n > 1) {
        n >>= 1;
        for (int i = 0; i < n; ++i) v[i] = v[i] + v[i + n];
    }
    return v[0];
}

/* ------------------------------------------------------- row norm (D=8192) */

#define ROW_D 8192
#define ROW_LANES 256
#define ROW_WAVE 64
#define ROW_FRAGS 4
#define ROW_VEC 8
#define ROW_CHUNK 2048 /* ROW_LANES * ROW_VEC */

/* Sum of squares of one 8192-wide row, in this project's fixed order:
 * lane t owns columns 2048 k + 8 t + i (k < 4, i < 8); it keeps one FMA
 * accumulator for the even and one for the odd columns of its fragments,
 * walking k then the pair index, and adds the two; each group of 64 lanes is
 * folded by halves (strides 32 .. 1); the four group sums are folded as
 * (W0 + W2) + (W1 + W3). */
static float sumsq_row(const float *u) {
    float lane_sum[ROW_LANES];
    for (int t = 0; t < ROW_LANES; ++t) {
        float even = 0.0f, odd = 0.0f;
        for (int k = 0; k < ROW_FRAGS; ++k) {
            const float *f = u + ROW_CHUNK * k + ROW_VEC * t;
            for (int p = 0; p < ROW_VEC / 2; ++p) {
                even = fmaf(f[2 * p], f[2 * p], even);
                odd = fmaf(f[2 * p + 1], f[2 * p + 1], odd);
            }
        }
        lane_sum[t] = even + odd;
    }
    float group[ROW_LANES / ROW_WAVE];
    for (int w = 0; w < ROW_LANES / ROW_WAVE; ++w) group[w] = fold(lane_sum + ROW_WAVE * w, ROW_WAVE);
    return fold(group, ROW_LANES / ROW_WAVE);
}

/* A norm's weight: none, bf16 bits or FP32 values ([CTX] ContextNormConstants:
 * a weight is absent, BF16 or FP32). gamma[c] = w[c] + center, one FP32 add
 * ([CTX] _ContextNormsKernel adds the gain center to every loaded weight). */
enum { W_NONE = 0, W_BF16 = 1, W_F32 = 2 };
typedef struct {
    int kind;
    const void *w;
    float center;
} weight_t;

static float gamma_of(const weight_t *g, int c) {
    float w = g->kind == W_BF16 ? f_of(((const uint16_t *)g->w)[c]) : ((const float *)g->w)[c];
    return w + g->center;
}

/* One RMSNorm of a row as the boundary page's row-norm arithmetic states it
 * ([BND] boundary_fragments): r = rs(fma(S, 1/D, eps)). Output-scaled (the
 * default): S sums the squares of x, y = x * r, then y * gamma. Input-scaled
 * (the weight scales the input): v = gamma * x first, S sums the squares of
 * v, y = v * r and no weight afterwards. out = bf16(y). 1/8192 = 2^-13. */
static void rms_norm_row_ex(const float *u, const weight_t *g, int input_scale, float eps, uint16_t *out) {
    float *v = malloc(sizeof(float) * ROW_D);
    if (!v) abort();
    const int scale_in = g->kind != W_NONE && input_scale;
    for (int c = 0; c < ROW_D; ++c) v[c] = scale_in ? gamma_of(g, c) * u[c] : u[c];
    float r = rs(fmaf(sumsq_row(v), 0x1p-13f, eps));
    for (int c = 0; c < ROW_D; ++c) {
        float y = v[c] * r;
        if (g->kind != W_NONE && !scale_in) y = y * gamma_of(g, c);
        out[c] = bf(y);
    }
    free(v);
}

/* The default form: bf16 weight (or none) applied to the norm's output. */
static void rms_norm_row(const float *u, const uint16_t *w, float eps, float center, uint16_t *out) {
    weight_t g = {w ? W_BF16 : W_NONE, w, center};
    rms_norm_row_ex(u, &g, 0, eps, out);
}

/* ----------------------------------------------------- 64-wide head K-norm */

#define HEAD 64

/* x.pow(2).sum over one 64-wide head in the order the context page gives for
 * the store: squares rounded, then folded by halves with strides 32,16,..,1. */
static float sumsq_head(const float *k) {
    float q[HEAD];
    for (int i = 0; i < HEAD; ++i) q[i] = k[i] * k[i];
    return fold(q, HEAD);
}

/* Weightless K-norm of one head, rounded to bf16, then GPT-J RoPE on the
 * pairs (2j, 2j+1) with cos_j, sin_j from the table row (cos 0..31 then sin
 * 0..31), each rotated value rounded to bf16. cs == NULL: no RoPE. */
static void knorm_rope_head(const uint16_t *k_in, const uint16_t *cs, float eps, uint16_t *out) {
    float k[HEAD];
    for (int i = 0; i < HEAD; ++i) k[i] = f_of(k_in[i]);
    float r = rs(fmaf(sumsq_head(k), 0x1p-6f, eps));
    uint16_t n[HEAD];
    for (int i = 0; i < HEAD; ++i) n[i] = bf(k[i] * r);
    if (!cs) {
        memcpy(out, n, sizeof n);
        return;
    }
    for (int j = 0; j < HEAD / 2; ++j) {
        float c = f_of(cs[j]), s = f_of(cs[HEAD / 2 + j]);
        float a = f_of(n[2 * j]), b = f_of(n[2 * j + 1]);
        out[2 * j] = bf(fmaf(a, c, -(b * s)));
        out[2 * j + 1] = bf(fmaf(b, c, a * s));
    }
}

/* =============================================================== exported */

uint16_t nrc_oracle_bf16(float x) { return bf(x); }
float nrc_oracle_rs(float v) { return rs(v); }

void nrc_oracle_bf16_array(const float *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf(in[i]);
}

void nrc_oracle_rs_array(const float *in, float *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = rs(in[i]);
}

float nrc_oracle_sumsq_row(const float *u) { return sumsq_row(u); }
float nrc_oracle_sumsq_head(const float *k) { return sumsq_head(k); }

/* stack([pre_norm_l(hidden_norm(x)) for l]): [CTX] ContextNorms and
 * _ContextNormsKernel. x [T, 8192] bf16; hidden_w [8192] or NULL; pre_w
 * [L, 8192] or NULL; out [L, T, 8192] bf16, element (l, t, c) at
 * (l * T + t) * 8192 + c. The hidden norm's output is rounded to bf16 before
 * the layer norms read it. */
int nrc_oracle_context_norms(const uint16_t *x, int64_t T, int64_t D, const uint16_t *hidden_w,
                             const uint16_t *pre_w, int32_t L, float hidden_eps, float pre_eps,
                             float hidden_center, float pre_center, uint16_t *out) {
    if (D != ROW_D || T < 0 || L < 1 || !x || !out) return ORACLE_EINVAL;
    float *u = malloc(sizeof(float) * ROW_D);
    uint16_t *h = malloc(sizeof(uint16_t) * ROW_D);
    if (!u || !h) {
        free(u);
        free(h);
        return ORACLE_EINVAL;
    }
    for (int64_t t = 0; t < T; ++t) {
        for (int c = 0; c < ROW_D; ++c) u[c] = f_of(x[t * ROW_D + c]);
        rms_norm_row(u, hidden_w, hidden_eps, hidden_center, h);
        for (int c = 0; c < ROW_D; ++c) u[c] = f_of(h[c]);
        for (int32_t l = 0; l < L; ++l)
            rms_norm_row(u, pre_w ? pre_w + (int64_t)l * ROW_D : NULL, pre_eps, pre_center,
                         out + ((int64_t)l * T + t) * ROW_D);
    }
    free(u);
    free(h);
    return 0;
}

/* The norms with every variant the context page's norms accept ([CTX]
 * ContextNorms, ContextNormConstants): each weight absent, bf16 or FP32
 * (hidden_kind / pre_kind: 0, 1, 2; pre_w is [L, 8192] of that type), gain
 * centers, and per norm whether the weight scales its input (flags bit 0:
 * hidden, bit 1: the layer norms) instead of its output. With the layer
 * norms input-scaled, each layer has its own sum of squares. */
int nrc_oracle_context_norms_ex(const uint16_t *x, int64_t T, int64_t D, const void *hidden_w, int32_t hidden_kind,
                                const void *pre_w, int32_t pre_kind, int32_t L, float hidden_eps, float pre_eps,
                                float hidden_center, float pre_center, int32_t flags, uint16_t *out) {
    if (D != ROW_D || T < 0 || L < 1 || !x || !out) return ORACLE_EINVAL;
    if (hidden_kind < W_NONE || hidden_kind > W_F32 || pre_kind < W_NONE || pre_kind > W_F32) return ORACLE_EINVAL;
    if ((hidden_kind == W_NONE) != (hidden_w == NULL) || (pre_kind == W_NONE) != (pre_w == NULL)) return ORACLE_EINVAL;
    float *u = malloc(sizeof(float) * ROW_D);
    uint16_t *h = malloc(sizeof(uint16_t) * ROW_D);
    if (!u || !h) {
        free(u);
        free(h);
        return ORACLE_EINVAL;
    }
    const weight_t gh = {hidden_kind, hidden_w, hidden_center};
    const size_t pre_elem = pre_kind == W_F32 ? sizeof(float) : sizeof(uint16_t);
    for (int64_t t = 0; t < T; ++t) {
        for (int c = 0; c < ROW_D; ++c) u[c] = f_of(x[t * ROW_D + c]);
        rms_norm_row_ex(u, &gh, flags & 1, hidden_eps, h);
        for (int c = 0; c < ROW_D; ++c) u[c] = f_of(h[c]);
        for (int32_t l = 0; l < L; ++l) {
            const weight_t gl = {pre_kind, pre_w ? (const char *)pre_w + (size_t)l * ROW_D * pre_elem : NULL,
                                 pre_center};
            rms_norm_row_ex(u, &gl, (flags >> 1) & 1, pre_eps, out + ((int64_t)l * T + t) * ROW_D);
        }
    }
    free(u);
    free(h);
    return 0;
}

/* The two per-row quantities the layer norms share, as a pre-pass of a
 * fused norms + projection computes them: h [T, 8192] bf16 (the hidden
 * norm's output) and r [T] = rs(fma(S_p, 1/8192, pre_eps)) with S_p the row
 * sum of squares of h. The layer outputs are bf16((h * r) * gamma_l). */
int nrc_oracle_hidden_norm(const uint16_t *x, int64_t T, int64_t D, const uint16_t *hidden_w, float hidden_eps,
                           float hidden_center, float pre_eps, uint16_t *h, float *r) {
    if (D != ROW_D || T < 0 || !x || !h || !r) return ORACLE_EINVAL;
    float *u = malloc(sizeof(float) * ROW_D);
    if (!u) return ORACLE_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        for (int c = 0; c < ROW_D; ++c) u[c] = f_of(x[t * ROW_D + c]);
        rms_norm_row(u, hidden_w, hidden_eps, hidden_center, h + t * ROW_D);
        for (int c = 0; c < ROW_D; ++c) u[c] = f_of(h[t * ROW_D + c]);
        r[t] = rs(fmaf(sumsq_row(u), 0x1p-13f, pre_eps));
    }
    free(u);
    return 0;
}

/* The batched projection of [RT] ContextKV._project: C[l] = A[l] B[l] with
 * A [L, T, D] bf16, B [L, D, N] bf16 (the logical operand of the bmm), C
 * [L, T, N] in FP32, each sum accumulated in FP32 in increasing d. The
 * products of two bf16 values are exact in FP32 (barring over/underflow). */
int nrc_oracle_kv_project(const uint16_t *A, const uint16_t *B, float *C, int32_t L, int64_t T, int64_t D,
                          int64_t N) {
    if (L < 1 || T < 0 || D < 1 || N < 1 || !A || !B || !C) return ORACLE_EINVAL;
    for (int32_t l = 0; l < L; ++l) {
        const uint16_t *Bl = B + (int64_t)l * D * N;
        for (int64_t t = 0; t < T; ++t) {
            const uint16_t *a = A + ((int64_t)l * T + t) * D;
            float *c = C + ((int64_t)l * T + t) * N;
            for (int64_t n = 0; n < N; ++n) c[n] = 0.0f;
            for (int64_t d = 0; d < D; ++d) {
                float ad = f_of(a[d]);
                const uint16_t *b = Bl + d * N;
                for (int64_t n = 0; n < N; ++n) c[n] = c[n] + ad * f_of(b[n]);
            }
        }
    }
    return 0;
}

/* The same projection with the weight stored as the pages keep it, [L, N, D]
 * (the bmm's right operand is its transpose, [RT] ContextKV._project):
 * C[l, t, n] = sum over d in increasing order of A[l, t, d] * B[l, n, d],
 * FP32. */
int nrc_oracle_kv_project_nd(const uint16_t *A, const uint16_t *B, float *C, int32_t L, int64_t T, int64_t D,
                             int64_t N) {
    if (L < 1 || T < 0 || D < 1 || N < 1 || !A || !B || !C) return ORACLE_EINVAL;
    for (int32_t l = 0; l < L; ++l)
        for (int64_t t = 0; t < T; ++t) {
            const uint16_t *a = A + ((int64_t)l * T + t) * D;
            for (int64_t n = 0; n < N; ++n) {
                const uint16_t *b = B + ((int64_t)l * N + n) * D;
                float c = 0.0f;
                for (int64_t d = 0; d < D; ++d) c = c + f_of(a[d]) * f_of(b[d]);
                C[((int64_t)l * T + t) * N + n] = c;
            }
        }
    return 0;
}

/* One head's K-norm (+ RoPE) as [CTX] _ContextKvStoreKernel computes it:
 * k_in [64] bf16, cs_row [64] bf16 (cos | sin) or NULL, out [64] bf16. */
void nrc_oracle_knorm_rope_head(const uint16_t *k_in, const uint16_t *cs_row, float eps, uint16_t *out) {
    knorm_rope_head(k_in, cs_row, eps, out);
}

/* Element offset of (slot, head h) inside one layer's cache
 * [num_blocks, H, block_size, 128]: block = slot / block_size and
 * page = slot % block_size in unsigned 32 bits ([CTX] _ContextKvStoreKernel),
 * K at [block, h, page, 0:64], V at +64. -1 for a negative slot. */
int64_t nrc_oracle_cache_offset(int64_t slot, int64_t block_size, int32_t H, int32_t h) {
    if (slot < 0) return -1;
    uint32_t page = (uint32_t)slot;
    uint32_t bs = (uint32_t)block_size;
    uint32_t block = page / bs;
    uint32_t in_block = page - block * bs;
    return (((int64_t)block * H + h) * block_size + in_block) * (2 * HEAD);
}

/* K-norm, RoPE and cache insert of every layer: [CTX] ContextKvStore.
 *   kv        [L, T, 2 H 64] bf16: per row the H K heads, then the H V heads
 *   positions [T] int64 (read only where a row is inserted and cos_sin != NULL)
 *   slots     [L, rows] int64, rows <= T; the first `rows` rows are inserted,
 *             a negative slot skips its row
 *   cos_sin   [max_position, 64] bf16 or NULL (RoPE off)
 *   caches    [L, num_blocks, H, block_size, 128] bf16, written in place
 * Preconditions checked here: slots in range and distinct per layer,
 * positions in range. */
int nrc_oracle_context_kv_store(const uint16_t *kv, int32_t L, int64_t T, int32_t H, const int64_t *positions,
                                const int64_t *slots, int64_t rows, const uint16_t *cos_sin,
                                int64_t max_position, uint16_t *caches, int64_t num_blocks, int64_t block_size,
                                float eps) {
    if (L < 1 || T < 0 || H < 1 || rows < 0 || rows > T || num_blocks < 1 || block_size < 1) return ORACLE_EINVAL;
    if (rows == 0) return 0;
    const int64_t n_slots = num_blocks * block_size;
    const int64_t N = 2 * (int64_t)H * HEAD;
    const int64_t layer_elems = n_slots * H * 2 * HEAD;
    unsigned char *seen = calloc((size_t)n_slots, 1);
    if (!seen) return ORACLE_EINVAL;
    int status = 0;
    for (int32_t l = 0; l < L && status == 0; ++l) {
        memset(seen, 0, (size_t)n_slots);
        for (int64_t t = 0; t < rows; ++t) {
            int64_t s = slots[(int64_t)l * rows + t];
            if (s < 0) continue;
            if (s >= n_slots || seen[s]) {
                status = ORACLE_EINVAL;
                break;
            }
            seen[s] = 1;
            const uint16_t *cs = NULL;
            if (cos_sin) {
                int64_t p = positions[t];
                if (p < 0 || p >= max_position) {
                    status = ORACLE_EINVAL;
                    break;
                }
                cs = cos_sin + p * 2 * (HEAD / 2);
            }
            const uint16_t *row = kv + ((int64_t)l * T + t) * N;
            uint16_t *cache = caches + (int64_t)l * layer_elems;
            for (int32_t h = 0; h < H; ++h) {
                uint16_t *dst = cache + nrc_oracle_cache_offset(s, block_size, H, h);
                knorm_rope_head(row + (int64_t)h * HEAD, cs, eps, dst);
                memcpy(dst + HEAD, row + (int64_t)(H + h) * HEAD, HEAD * sizeof(uint16_t));
            }
        }
    }
    free(seen);
    return status;
}

/* The store with the pages' full operand surface ([CTX] ContextKvStore,
 * [RT] ContextKV.store and _slot_groups): per layer l, slots[l] is NULL (the
 * layer stores nothing) or rows[l] int64 slots (the first rows[l] rows are
 * inserted); caches[l] points at K of (block 0, page 0, head 0) of a strided
 * view, element (b, o, h, c) at b * block_stride + o * page_stride +
 * h * head_stride + c, with K in c < 64 and V in 64 <= c < 128; cache_len[l]
 * is the number of elements the caller's buffer holds from caches[l] (every
 * write must fall inside). Other operands as nrc_oracle_context_kv_store. */
int nrc_oracle_context_kv_store_ex(const uint16_t *kv, int32_t L, int64_t T, int32_t H, const int64_t *positions,
                                   const int64_t *const *slots, const int64_t *rows, const uint16_t *cos_sin,
                                   int64_t max_position, uint16_t *const *caches, const int64_t *cache_len,
                                   int64_t num_blocks, int64_t block_size, int64_t block_stride,
                                   int64_t page_stride, int64_t head_stride, float eps) {
    if (L < 1 || T < 0 || H < 1 || num_blocks < 1 || block_size < 1) return ORACLE_EINVAL;
    const int64_t n_slots = num_blocks * block_size;
    const int64_t N = 2 * (int64_t)H * HEAD;
    unsigned char *seen = calloc((size_t)n_slots, 1);
    if (!seen) return ORACLE_EINVAL;
    int status = 0;
    for (int32_t l = 0; l < L && status == 0; ++l) {
        if (!slots[l]) continue;
        if (rows[l] < 0 || rows[l] > T) {
            status = ORACLE_EINVAL;
            break;
        }
        memset(seen, 0, (size_t)n_slots);
        for (int64_t t = 0; t < rows[l]; ++t) {
            int64_t s = slots[l][t];
            if (s < 0) continue;
            if (s >= n_slots || seen[s]) {
                status = ORACLE_EINVAL;
                break;
            }
            seen[s] = 1;
            const uint16_t *cs = NULL;
            if (cos_sin) {
                int64_t p = positions[t];
                if (p < 0 || p >= max_position) {
                    status = ORACLE_EINVAL;
                    break;
                }
                cs = cos_sin + p * 2 * (HEAD / 2);
            }
            const uint32_t page = (uint32_t)s, bs = (uint32_t)block_size;
            const int64_t b = page / bs, o = page - (uint32_t)b * bs;
            const uint16_t *row = kv + ((int64_t)l * T + t) * N;
            for (int32_t h = 0; h < H; ++h) {
                const int64_t off = b * block_stride + o * page_stride + (int64_t)h * head_stride;
                if (off < 0 || off + 2 * HEAD > cache_len[l]) {
                    status = ORACLE_EINVAL;
                    break;
                }
                uint16_t *dst = caches[l] + off;
                knorm_rope_head(row + (int64_t)h * HEAD, cs, eps, dst);
                memcpy(dst + HEAD, row + (int64_t)(H + h) * HEAD, HEAD * sizeof(uint16_t));
            }
        }
    }
    free(seen);
    return status;
}

/* ------------------------------------------------- the residual boundary */

/* Exact f16 -> f32 (every f16 is an f32): sign, then zero / subnormal
 * (mantissa * 2^-24) / normal (rebias the exponent by 112) / Inf / NaN. */
static float f_of_f16(uint16_t h) {
    const uint32_t sign = (uint32_t)(h >> 15) << 31;
    const uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
    float v;
    if (e == 0) {
        v = (float)m * 0x1p-24f; /* exact: m < 2^10 */
        uint32_t u;
        memcpy(&u, &v, sizeof u);
        u |= sign;
        memcpy(&v, &u, sizeof v);
        return v;
    }
    uint32_t u = sign | (e == 31 ? (0xFFu << 23) | (m << 13) : ((e + 112u) << 23) | (m << 13));
    memcpy(&v, &u, sizeof v);
    return v;
}

float nrc_oracle_f16_to_f32(uint16_t h) { return f_of_f16(h); }

enum { W_F16 = 3 };

static float boundary_gamma(const void *w, int kind, float center, int c) {
    float v = kind == W_BF16 ? f_of(((const uint16_t *)w)[c])
              : kind == W_F16 ? f_of_f16(((const uint16_t *)w)[c])
                              : ((const float *)w)[c];
    return v + center;
}

/* One residual boundary of the DSpark draft ([BND] module summary and
 * boundary_fragments): per row of the bf16 branch x,
 *   post norm: (input-scaled: u = gamma_post * x) S1 = sum of squares in the
 *     library's order, r1 = rs(fma(S1, 1/8192, post_eps)), y = u * r1, then
 *     * gamma_post when output-scaled;
 *   residual: res = alpha * stream + beta * bf16(y), each product rounded,
 *     then the sum (FP32); the new stream is res, z = bf16(res);
 *   pre norm of z, the same form with gamma_pre, rounded to bf16 -> out.
 * stream: FP32 (stream_kind 0) or bf16 bits (1), [m, 8192]; alpha, beta
 * FP32 [8192]; post_w / pre_w [8192] of kind 0 (none), 1 (bf16), 2 (FP32) or
 * 3 (FP16); flags bit 0: post input-scaled, bit 1: pre input-scaled;
 * stream_out [m, 8192] FP32 or NULL. */
int nrc_oracle_draft_boundary(const uint16_t *branch, int64_t m, const void *stream, int32_t stream_kind,
                              const float *alpha, const float *beta, const void *post_w, int32_t post_kind,
                              const void *pre_w, int32_t pre_kind, float post_eps, float pre_eps, float post_center,
                              float pre_center, int32_t flags, float *stream_out, uint16_t *out) {
    if (m < 0 || !branch || !stream || !alpha || !beta || !out || stream_kind < 0 || stream_kind > 1) return ORACLE_EINVAL;
    if (post_kind < 0 || post_kind > 3 || pre_kind < 0 || pre_kind > 3) return ORACLE_EINVAL;
    if ((post_kind == 0) != (post_w == NULL) || (pre_kind == 0) != (pre_w == NULL)) return ORACLE_EINVAL;
    const int post_in = post_kind != 0 && (flags & 1), pre_in = pre_kind != 0 && (flags & 2);
    float *u = malloc(sizeof(float) * ROW_D), *z = malloc(sizeof(float) * ROW_D);
    if (!u || !z) {
        free(u);
        free(z);
        return ORACLE_EINVAL;
    }
    for (int64_t t = 0; t < m; ++t) {
        for (int c = 0; c < ROW_D; ++c) {
            float x = f_of(branch[t * ROW_D + c]);
            u[c] = post_in ? boundary_gamma(post_w, post_kind, post_center, c) * x : x;
        }
        const float r1 = rs(fmaf(sumsq_row(u), 0x1p-13f, post_eps));
        for (int c = 0; c < ROW_D; ++c) {
            float y = u[c] * r1;
            if (post_kind != 0 && !post_in) y = y * boundary_gamma(post_w, post_kind, post_center, c);
            const float s = stream_kind == 0 ? ((const float *)stream)[t * ROW_D + c]
                                             : f_of(((const uint16_t *)stream)[t * ROW_D + c]);
            const float a = alpha[c] * s;
            const float b = beta[c] * f_of(bf(y));
            const float res = a + b;
            if (stream_out) stream_out[t * ROW_D + c] = res;
            const float zc = f_of(bf(res));
            z[c] = pre_in ? boundary_gamma(pre_w, pre_kind, pre_center, c) * zc : zc;
        }
        const float r2 = rs(fmaf(sumsq_row(z), 0x1p-13f, pre_eps));
        for (int c = 0; c < ROW_D; ++c) {
            float o = z[c] * r2;
            if (pre_kind != 0 && !pre_in) o = o * boundary_gamma(pre_w, pre_kind, pre_center, c);
            out[t * ROW_D + c] = bf(o);
        }
    }
    free(u);
    free(z);
    return 0;
}

/* The whole chain: norms, projection (rounded to bf16), store. normed
 * [L, T, 8192] and kv [L, T, N] are caller-provided scratch that receive the
 * intermediate results. */
int nrc_oracle_chain(const uint16_t *x, int64_t T, const uint16_t *hidden_w, const uint16_t *pre_w, int32_t L,
                     float hidden_eps, float pre_eps, const uint16_t *w_kv, int32_t H, const int64_t *positions,
                     const int64_t *slots, int64_t rows, const uint16_t *cos_sin, int64_t max_position,
                     uint16_t *caches, int64_t num_blocks, int64_t block_size, float k_eps, uint16_t *normed,
                     uint16_t *kv) {
    const int64_t N = 2 * (int64_t)H * HEAD;
    int st = nrc_oracle_context_norms(x, T, ROW_D, hidden_w, pre_w, L, hidden_eps, pre_eps, 0.0f, 0.0f, normed);
    if (st) return st;
    float *c = malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
    if (!c) return ORACLE_EINVAL;
    for (int32_t l = 0; l < L && st == 0; ++l)
        for (int64_t t = 0; t < T && st == 0; ++t) {
            st = nrc_oracle_kv_project(normed + ((int64_t)l * T + t) * ROW_D, w_kv + (int64_t)l * ROW_D * N, c, 1,
                                       1, ROW_D, N);
            for (int64_t n = 0; n < N; ++n) kv[((int64_t)l * T + t) * N + n] = bf(c[n]);
        }
    free(c);
    if (st) return st;
    return nrc_oracle_context_kv_store(kv, L, T, H, positions, slots, rows, cos_sin, max_position, caches,
                                       num_blocks, block_size, k_eps);
}
