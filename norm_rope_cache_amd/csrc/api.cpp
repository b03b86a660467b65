// The C ABI of libnrc (include/nrc.h): argument checks, then launches.
//
// Every check runs on the host before the first launch, so a non-zero status
// means nothing was enqueued; nrc_last_error() describes it. The operand
// rules follow the vLLM pages: ContextNorms (8192-wide rows, T >= 1 rows;
// zero rows are a no-op here), ContextKV.store (bf16 caches with 64-wide
// heads, even strides, 4-byte alignment, fewer than 2^31 slots, slot
// mappings of one length), ContextKvStore (rows == 0 is a no-op; at most 8
// layers per launch) and the runtime page's eligibility rules (head dim 64,
// KV heads a power of two).
#include <errno.h>
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <vector>

#include "../../include/nrc.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// CUs of the current device, looked up once per device (relaxed atomics:
// concurrent first calls store the same value).
int num_cus() {
    static std::atomic<int> cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    int n = dev < 64 ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

int launch_status(int rc, const char* what) {
    if (rc != 0) {
        hipError_t e = hipGetLastError();
        return fail(NRC_EIO, "%s: launch failed (%s)", what, hipGetErrorString(e));
    }
    return NRC_OK;
}

}  // namespace

extern "C" {

const char* nrc_last_error(void) { return g_err; }

int32_t nrc_abi_version(void) { return 1; }

int32_t nrc_context_norms(const uint16_t* x, int64_t T, int64_t D, const uint16_t* hidden_w, const uint16_t* pre_w,
                          int32_t L, float hidden_eps, float pre_eps, float hidden_center, float pre_center,
                          uint16_t* out, void* stream) {
    if (D != NRC_HIDDEN) return fail(NRC_ENOTSUP, "context_norms: rows of %lld, not %d", (long long)D, NRC_HIDDEN);
    if (T < 0) return fail(NRC_EINVAL, "context_norms: T = %lld < 0", (long long)T);
    if (L < 1) return fail(NRC_EINVAL, "context_norms: L = %d < 1", L);
    if (T > ((int64_t)1 << 40) / ((int64_t)L * D))
        return fail(NRC_EINVAL, "context_norms: output of %lld x %d rows too large", (long long)T, L);
    if (T == 0) return NRC_OK;
    if (!x || !out) return fail(NRC_EINVAL, "context_norms: NULL x or out");
    if (!aligned(x, 16) || !aligned(out, 16) || (hidden_w && !aligned(hidden_w, 16)) ||
        (pre_w && !aligned(pre_w, 16)))
        return fail(NRC_EINVAL, "context_norms: operands must be 16-byte aligned");
    nrc::NormsArgs a{x, T, hidden_w, pre_w, L, hidden_eps, pre_eps, hidden_center, pre_center, out, num_cus()};
    return launch_status(nrc::launch_context_norms(a, (hipStream_t)stream), "context_norms");
}

int32_t nrc_context_norms_ex(const uint16_t* x, int64_t T, int64_t D, const void* hidden_w, int32_t hidden_kind,
                             const void* pre_w, int32_t pre_kind, int32_t L, float hidden_eps, float pre_eps,
                             float hidden_center, float pre_center, uint32_t flags, uint16_t* out, void* stream) {
    if (D != NRC_HIDDEN) return fail(NRC_ENOTSUP, "context_norms_ex: rows of %lld, not %d", (long long)D, NRC_HIDDEN);
    if (T < 0) return fail(NRC_EINVAL, "context_norms_ex: T = %lld < 0", (long long)T);
    if (L < 1) return fail(NRC_EINVAL, "context_norms_ex: L = %d < 1", L);
    if (hidden_kind < NRC_WEIGHT_NONE || hidden_kind > NRC_WEIGHT_F32 || pre_kind < NRC_WEIGHT_NONE ||
        pre_kind > NRC_WEIGHT_F32)
        return fail(NRC_EINVAL, "context_norms_ex: weight kinds %d, %d (0 none, 1 bf16, 2 FP32)", hidden_kind,
                    pre_kind);
    if ((hidden_kind == NRC_WEIGHT_NONE) != (hidden_w == nullptr) || (pre_kind == NRC_WEIGHT_NONE) != (pre_w == nullptr))
        return fail(NRC_EINVAL, "context_norms_ex: a weight pointer must be NULL exactly when its kind is none");
    if (flags & ~(uint32_t)(NRC_HIDDEN_INPUT_SCALE | NRC_PRE_INPUT_SCALE))
        return fail(NRC_EINVAL, "context_norms_ex: unknown flags 0x%x", flags);
    if (T > ((int64_t)1 << 40) / ((int64_t)L * D))
        return fail(NRC_EINVAL, "context_norms_ex: output of %lld x %d rows too large", (long long)T, L);
    if (T == 0) return NRC_OK;
    if (!x || !out) return fail(NRC_EINVAL, "context_norms_ex: NULL x or out");
    if (!aligned(x, 16) || !aligned(out, 16) || (hidden_w && !aligned(hidden_w, 16)) ||
        (pre_w && !aligned(pre_w, 16)))
        return fail(NRC_EINVAL, "context_norms_ex: operands must be 16-byte aligned");
    const bool plain = hidden_kind != NRC_WEIGHT_F32 && pre_kind != NRC_WEIGHT_F32 && flags == 0;
    if (plain) {
        nrc::NormsArgs a{x, T, (const uint16_t*)hidden_w, (const uint16_t*)pre_w, L, hidden_eps, pre_eps,
                         hidden_center, pre_center, out, num_cus()};
        return launch_status(nrc::launch_context_norms(a, (hipStream_t)stream), "context_norms_ex");
    }
    nrc::NormsExArgs a{x, T, hidden_w, hidden_kind, pre_w, pre_kind, L, hidden_eps, pre_eps, hidden_center,
                       pre_center, (flags & NRC_HIDDEN_INPUT_SCALE) != 0, (flags & NRC_PRE_INPUT_SCALE) != 0, out,
                       num_cus()};
    return launch_status(nrc::launch_norms_ex(a, (hipStream_t)stream), "context_norms_ex");
}

int32_t nrc_draft_boundary(const uint16_t* branch, int64_t m, int64_t D, const void* stream_in, int32_t stream_kind,
                           const float* alpha, const float* beta, const void* post_w, int32_t post_kind,
                           const void* pre_w, int32_t pre_kind, float post_eps, float pre_eps, float post_center,
                           float pre_center, uint32_t flags, float* stream_out, uint16_t* out, void* stream) {
    if (D != NRC_HIDDEN) return fail(NRC_ENOTSUP, "draft_boundary: rows of %lld, not %d", (long long)D, NRC_HIDDEN);
    if (m < 0) return fail(NRC_EINVAL, "draft_boundary: m = %lld < 0", (long long)m);
    if (stream_kind != NRC_STREAM_F32 && stream_kind != NRC_STREAM_BF16)
        return fail(NRC_EINVAL, "draft_boundary: stream kind %d (0 FP32, 1 bf16)", stream_kind);
    if (post_kind < NRC_WEIGHT_NONE || post_kind > NRC_WEIGHT_F16 || pre_kind < NRC_WEIGHT_NONE ||
        pre_kind > NRC_WEIGHT_F16)
        return fail(NRC_EINVAL, "draft_boundary: weight kinds %d, %d (0 none, 1 bf16, 2 FP32, 3 FP16)", post_kind,
                    pre_kind);
    if ((post_kind == NRC_WEIGHT_NONE) != (post_w == nullptr) || (pre_kind == NRC_WEIGHT_NONE) != (pre_w == nullptr))
        return fail(NRC_EINVAL, "draft_boundary: a weight pointer must be NULL exactly when its kind is none");
    if (flags & ~(uint32_t)(NRC_POST_INPUT_SCALE | NRC_PRE_INPUT_SCALE))
        return fail(NRC_EINVAL, "draft_boundary: unknown flags 0x%x", flags);
    if (m > ((int64_t)1 << 40) / D) return fail(NRC_EINVAL, "draft_boundary: m too large");
    if (m == 0) return NRC_OK;
    if (!branch || !stream_in || !alpha || !beta || !out)
        return fail(NRC_EINVAL, "draft_boundary: NULL branch, stream, alpha, beta or out");
    if (!aligned(branch, 16) || !aligned(stream_in, 16) || !aligned(alpha, 16) || !aligned(beta, 16) ||
        !aligned(out, 16) || (stream_out && !aligned(stream_out, 16)) || (post_w && !aligned(post_w, 16)) ||
        (pre_w && !aligned(pre_w, 16)))
        return fail(NRC_EINVAL, "draft_boundary: operands must be 16-byte aligned");
    nrc::BoundaryArgs a{branch, m, stream_in, stream_kind == NRC_STREAM_BF16, alpha, beta, post_w, post_kind,
                        pre_w, pre_kind, post_eps, pre_eps, post_center, pre_center,
                        (flags & NRC_POST_INPUT_SCALE) != 0, (flags & NRC_PRE_INPUT_SCALE) != 0, stream_out, out,
                        num_cus()};
    return launch_status(nrc::launch_draft_boundary(a, (hipStream_t)stream), "draft_boundary");
}

int32_t nrc_context_hidden_norm(const uint16_t* x, int64_t T, int64_t D, const uint16_t* hidden_w,
                                const uint16_t* pre_w, int32_t L, float hidden_eps, float pre_eps,
                                float hidden_center, float pre_center, uint16_t* h, float* r, void* stream) {
    if (D != NRC_HIDDEN) return fail(NRC_ENOTSUP, "context_hidden_norm: rows of %lld, not %d", (long long)D, NRC_HIDDEN);
    if (T < 0) return fail(NRC_EINVAL, "context_hidden_norm: T = %lld < 0", (long long)T);
    if (L < 1) return fail(NRC_EINVAL, "context_hidden_norm: L = %d < 1", L);
    if (T > ((int64_t)1 << 40) / D) return fail(NRC_EINVAL, "context_hidden_norm: T too large");
    if (T == 0) return NRC_OK;
    if (!x || !h || !r) return fail(NRC_EINVAL, "context_hidden_norm: NULL x, h or r");
    if (!aligned(x, 16) || !aligned(h, 16) || !aligned(r, 4) || (hidden_w && !aligned(hidden_w, 16)) ||
        (pre_w && !aligned(pre_w, 16)))
        return fail(NRC_EINVAL, "context_hidden_norm: operands must be 16-byte aligned (r 4-byte)");
    nrc::NormsArgs a{x, T, hidden_w, pre_w, L, hidden_eps, pre_eps, hidden_center, pre_center, nullptr, num_cus()};
    return launch_status(nrc::launch_hidden_norm(a, h, r, (hipStream_t)stream), "context_hidden_norm");
}

}  // extern "C"

namespace {

// Checks of the fused projection's operands (both entry points).
int32_t fused_checks(const uint16_t* h, const float* r, const uint16_t* pre_w, const uint16_t* w, const uint16_t* kv,
                     int32_t L, int64_t T, int64_t D, int64_t N) {
    if (L < 1) return fail(NRC_EINVAL, "context_kv_project_fused: L = %d < 1", L);
    if (T < 0) return fail(NRC_EINVAL, "context_kv_project_fused: T = %lld < 0", (long long)T);
    if (D != NRC_HIDDEN)
        return fail(NRC_ENOTSUP, "context_kv_project_fused: rows of %lld, not %d", (long long)D, NRC_HIDDEN);
    if (N <= 0 || N % 128)
        return fail(NRC_ENOTSUP, "context_kv_project_fused: N = %lld is not a positive multiple of 128 (2 H 64)",
                    (long long)N);
    if (T > ((int64_t)1 << 31) || N > ((int64_t)1 << 20) || (int64_t)L * ((T + 127) / 128) * (N / 128) > ((int64_t)1 << 30))
        return fail(NRC_EINVAL, "context_kv_project_fused: shape too large");
    if (T == 0) return NRC_OK;
    if (!h || !r || !w || !kv) return fail(NRC_EINVAL, "context_kv_project_fused: NULL operand");
    if (!aligned(h, 16) || !aligned(w, 16) || !aligned(kv, 16) || !aligned(r, 4) || (pre_w && !aligned(pre_w, 16)))
        return fail(NRC_EINVAL, "context_kv_project_fused: operands must be 16-byte aligned (r 4-byte)");
    return NRC_OK;
}

}  // namespace

extern "C" {

int32_t nrc_context_kv_project_fused(const uint16_t* h, const float* r, const uint16_t* pre_w, float pre_center,
                                     const uint16_t* w, uint16_t* kv, int32_t L, int64_t T, int64_t D, int64_t N,
                                     void* stream) {
    if (int32_t rc = fused_checks(h, r, pre_w, w, kv, L, T, D, N)) return rc;
    if (T == 0) return NRC_OK;
    nrc::ProjectArgs a{h, w, kv, L, T, D, N, num_cus()};
    return launch_status(nrc::launch_kv_project_fused(a, r, pre_w, pre_center, (hipStream_t)stream),
                         "context_kv_project_fused");
}

}  // extern "C"

namespace {

// Shape checks shared by the projection entry points (no pointers).
int32_t project_shape_ok(int32_t L, int64_t T, int64_t D, int64_t N) {
    if (L < 1) return fail(NRC_EINVAL, "context_kv_project: L = %d < 1", L);
    if (T < 0) return fail(NRC_EINVAL, "context_kv_project: T = %lld < 0", (long long)T);
    if (D <= 0 || D % 64) return fail(NRC_ENOTSUP, "context_kv_project: D = %lld is not a positive multiple of 64",
                                      (long long)D);
    if (N <= 0 || N % 128)
        return fail(NRC_ENOTSUP, "context_kv_project: N = %lld is not a positive multiple of 128 (2 H 64)",
                    (long long)N);
    if (T > ((int64_t)1 << 31) || D > ((int64_t)1 << 20) || N > ((int64_t)1 << 20) ||
        (int64_t)L * ((T + 127) / 128) * (N / 128) > ((int64_t)1 << 30))
        return fail(NRC_EINVAL, "context_kv_project: shape too large");
    return NRC_OK;
}

int64_t project_workspace_bytes(int32_t L, int64_t T, int64_t D, int64_t N) {
    const int32_t s = nrc::kv_project_k_split(L, T, D, N, num_cus());
    return s > 1 ? (int64_t)s * L * T * N * 4 : 0;
}

// The projection behind the entry points; workspace NULL: never split.
int32_t project_impl(const uint16_t* normed, const uint16_t* w, int32_t w_layout, uint16_t* kv, int32_t L,
                     int64_t T, int64_t D, int64_t N, void* workspace, int64_t workspace_bytes, bool may_split,
                     void* stream) {
    if (w_layout != NRC_KV_WEIGHT_DN && w_layout != NRC_KV_WEIGHT_ND)
        return fail(NRC_EINVAL, "context_kv_project: weight layout %d (0 [L, D, N], 1 [L, N, D])", w_layout);
    if (int32_t rc = project_shape_ok(L, T, D, N)) return rc;
    if (T == 0) return NRC_OK;
    if (!normed || !w || !kv) return fail(NRC_EINVAL, "context_kv_project: NULL operand");
    if (!aligned(normed, 16) || !aligned(w, 16) || !aligned(kv, 16))
        return fail(NRC_EINVAL, "context_kv_project: operands must be 16-byte aligned");
    nrc::ProjectArgs a{normed, w, kv, L, T, D, N, num_cus()};
    a.b_nd = w_layout == NRC_KV_WEIGHT_ND;
    if (may_split) {
        const int64_t need = project_workspace_bytes(L, T, D, N);
        if (need > 0) {
            if (!workspace || workspace_bytes < need || !aligned(workspace, 16))
                return fail(NRC_EINVAL, "context_kv_project_split: needs a 16-byte aligned workspace of %lld bytes",
                            (long long)need);
            a.ws = static_cast<float*>(workspace);
            a.k_split = nrc::kv_project_k_split(L, T, D, N, a.num_cus);
        }
    }
    return launch_status(nrc::launch_kv_project(a, (hipStream_t)stream), "context_kv_project");
}

}  // namespace

extern "C" {

int32_t nrc_context_kv_project_ex(const uint16_t* normed, const uint16_t* w, int32_t w_layout, uint16_t* kv,
                                  int32_t L, int64_t T, int64_t D, int64_t N, void* stream) {
    return project_impl(normed, w, w_layout, kv, L, T, D, N, nullptr, 0, false, stream);
}

int64_t nrc_context_kv_project_workspace_bytes(int32_t L, int64_t T, int64_t D, int64_t N) {
    if (int32_t rc = project_shape_ok(L, T, D, N)) return rc;
    return T == 0 ? 0 : project_workspace_bytes(L, T, D, N);
}

int32_t nrc_context_kv_project_split(const uint16_t* normed, const uint16_t* w, int32_t w_layout, uint16_t* kv,
                                     int32_t L, int64_t T, int64_t D, int64_t N, void* workspace,
                                     int64_t workspace_bytes, void* stream) {
    return project_impl(normed, w, w_layout, kv, L, T, D, N, workspace, workspace_bytes, true, stream);
}

int32_t nrc_context_kv_project_fused_split(const uint16_t* h, const float* r, const uint16_t* pre_w, float pre_center,
                                           const uint16_t* w, uint16_t* kv, int32_t L, int64_t T, int64_t D,
                                           int64_t N, void* workspace, int64_t workspace_bytes, void* stream) {
    if (int32_t rc = fused_checks(h, r, pre_w, w, kv, L, T, D, N)) return rc;
    if (T == 0) return NRC_OK;
    nrc::ProjectArgs a{h, w, kv, L, T, D, N, num_cus()};
    const int64_t need = project_workspace_bytes(L, T, D, N);
    if (need > 0) {
        if (!workspace || workspace_bytes < need || !aligned(workspace, 16))
            return fail(NRC_EINVAL, "context_kv_project_fused_split: needs a 16-byte aligned workspace of %lld bytes",
                        (long long)need);
        a.ws = static_cast<float*>(workspace);
        a.k_split = nrc::kv_project_k_split(L, T, D, N, a.num_cus);
    }
    return launch_status(nrc::launch_kv_project_fused(a, r, pre_w, pre_center, (hipStream_t)stream),
                         "context_kv_project_fused_split");
}

static_assert(NRC_PROJECT_SCRATCH_BYTES == nrc::kProjectScratchBytes, "header and library scratch sizes differ");

int32_t nrc_context_kv_project_noalloc(const uint16_t* normed, const uint16_t* w, int32_t w_layout, uint16_t* kv,
                                       int32_t L, int64_t T, int64_t D, int64_t N, void* stream) {
    if (int32_t rc = project_shape_ok(L, T, D, N)) return rc;
    const int64_t need = T == 0 ? 0 : project_workspace_bytes(L, T, D, N);
    if (need > nrc::kProjectScratchBytes)
        return fail(NRC_EINVAL,
                    "context_kv_project_noalloc: this shape's split needs %lld bytes of scratch, more than the %lld "
                    "the library holds (use nrc_context_kv_project_split with a workspace)",
                    (long long)need, (long long)nrc::kProjectScratchBytes);
    void* ws = nullptr;
    if (need > 0 && nrc::project_scratch(&ws) != 0)
        return fail(NRC_EIO, "context_kv_project_noalloc: no address for the device scratch on the current device");
    return project_impl(normed, w, w_layout, kv, L, T, D, N, ws, need, true, stream);
}

int32_t nrc_context_kv_project_timed(const uint16_t* normed, const uint16_t* w, int32_t w_layout, uint16_t* kv,
                                     int32_t L, int64_t T, int64_t D, int64_t N, uint64_t* stamps,
                                     int64_t stamps_len, int32_t* workgroups, int32_t* wall_khz, void* stream) {
    if (!workgroups || !wall_khz) return fail(NRC_EINVAL, "context_kv_project_timed: NULL host output");
    *workgroups = 0;
    if (w_layout != NRC_KV_WEIGHT_DN && w_layout != NRC_KV_WEIGHT_ND)
        return fail(NRC_EINVAL, "context_kv_project: weight layout %d (0 [L, D, N], 1 [L, N, D])", w_layout);
    if (int32_t rc = project_shape_ok(L, T, D, N)) return rc;
    const int cus = num_cus();
    // At most two workgroups per CU (the 128 x 128 tiles' LDS ring), 4 stamps each.
    if (!stamps || !aligned(stamps, 8) || stamps_len < 8 * (int64_t)cus)
        return fail(NRC_EINVAL, "context_kv_project_timed: stamps must be 8-byte aligned with at least %lld entries",
                    (long long)(8 * (int64_t)cus));
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
        return fail(NRC_EIO, "context_kv_project_timed: no constant clock rate for the current device");
    *wall_khz = khz;
    if (T == 0) return NRC_OK;
    if (!normed || !w || !kv) return fail(NRC_EINVAL, "context_kv_project: NULL operand");
    if (!aligned(normed, 16) || !aligned(w, 16) || !aligned(kv, 16))
        return fail(NRC_EINVAL, "context_kv_project: operands must be 16-byte aligned");
    nrc::ProjectArgs a{normed, w, kv, L, T, D, N, cus};
    a.b_nd = w_layout == NRC_KV_WEIGHT_ND;
    a.stamps = stamps;
    a.stamps_len = stamps_len;
    a.workgroups = workgroups;
    return launch_status(nrc::launch_kv_project(a, (hipStream_t)stream), "context_kv_project_timed");
}

int32_t nrc_context_kv_project(const uint16_t* normed, const uint16_t* w, uint16_t* kv, int32_t L, int64_t T,
                               int64_t D, int64_t N, void* stream) {
    return nrc_context_kv_project_ex(normed, w, NRC_KV_WEIGHT_DN, kv, L, T, D, N, stream);
}

}  // extern "C"

namespace {

// The store behind both entry points: per-layer slot lists (NULL: the layer
// stores nothing) of rows[l] entries, and a strided cache view.
//
// Sum mode (sum != NULL, the tail of nrc_context_kv_project_store): k and v
// are the halves of the projection output kv [L, T, 2 H 64], which the
// launches write, every row, from the split projection's partial sums
// before inserting; launches happen even when no row is inserted.
// check_only: validate the operands and launch nothing.
struct SumSource {
    const float* ws;  // [k_split, L, T, N] FP32 partial sums
    int32_t k_split;
    uint16_t* kv;     // [L, T, N]
};

int32_t store_impl(const char* what, const uint16_t* k, const uint16_t* v, int64_t k_layer_stride,
                   int64_t k_row_stride, int64_t v_layer_stride, int64_t v_row_stride, const int64_t* positions,
                   const int64_t* const* slots, const int64_t* rows, int64_t T, const uint16_t* cos_sin,
                   int64_t max_position, uint16_t* const* caches, int64_t num_blocks, int64_t block_size,
                   int64_t block_stride, int64_t page_stride, int64_t head_stride, int32_t H, int32_t L, float eps,
                   void* stream, const SumSource* sum = nullptr, bool check_only = false) {
    if (L < 1) return fail(NRC_EINVAL, "%s: L = %d < 1", what, L);
    if (H < 1) return fail(NRC_EINVAL, "%s: H = %d < 1", what, H);
    if (H & (H - 1)) return fail(NRC_ENOTSUP, "%s: %d KV heads, not a power of two", what, H);
    if (T < 0) return fail(NRC_EINVAL, "%s: T = %lld < 0", what, (long long)T);
    if (num_blocks < 1 || block_size < 1) return fail(NRC_EINVAL, "%s: num_blocks and block_size must be >= 1", what);
    if (num_blocks > (((int64_t)1 << 31) - 1) / block_size)
        return fail(NRC_ENOTSUP, "%s: %lld x %lld slots do not fit 31 bits", what, (long long)num_blocks,
                    (long long)block_size);
    if (!slots || !caches || !rows) return fail(NRC_EINVAL, "%s: NULL slots, rows or caches array", what);
    int64_t max_rows = 0;
    for (int32_t l = 0; l < L; ++l) {
        if (!slots[l]) continue;
        if (rows[l] < 0 || rows[l] > T)
            return fail(NRC_EINVAL, "%s: layer %d: rows = %lld must lie in [0, T = %lld]", what, l, (long long)rows[l],
                        (long long)T);
        if (rows[l] > max_rows) max_rows = rows[l];
    }
    if (max_rows * H > ((int64_t)1 << 25))
        return fail(NRC_ENOTSUP, "%s: rows x heads = %lld too large for one call", what, (long long)(max_rows * H));
    // sum mode: 8 lanes per (layer, row, 64 columns), up to 8 layers a launch,
    // thread ids in 32 bits
    if (sum && T * H > ((int64_t)1 << 24))
        return fail(NRC_ENOTSUP, "%s: T x heads = %lld too large for one call", what, (long long)(T * H));
    if (max_rows == 0 && (!sum || T == 0)) return NRC_OK;
    if (!k || !v) return fail(NRC_EINVAL, "%s: NULL k or v", what);
    if (!aligned(k, 16) || !aligned(v, 16)) return fail(NRC_EINVAL, "%s: k and v must be 16-byte aligned", what);
    if ((k_layer_stride | k_row_stride | v_layer_stride | v_row_stride) & 7)
        return fail(NRC_EINVAL, "%s: k/v strides must be multiples of 8 elements", what);
    if (k_layer_stride < 0 || k_row_stride < 0 || v_layer_stride < 0 || v_row_stride < 0)
        return fail(NRC_EINVAL, "%s: negative stride", what);
    if (block_stride < 0 || page_stride < 0 || head_stride < 0)
        return fail(NRC_EINVAL, "%s: negative cache stride", what);
    if ((block_stride | page_stride | head_stride) & 7)
        return fail(NRC_ENOTSUP, "%s: cache strides must be multiples of 8 elements (16-byte accesses)", what);
    if (cos_sin) {
        if (!positions) return fail(NRC_EINVAL, "%s: RoPE needs positions", what);
        if (max_position < 1) return fail(NRC_EINVAL, "%s: max_position < 1", what);
        if (!aligned(cos_sin, 16) || !aligned(positions, 8))
            return fail(NRC_EINVAL, "%s: cos_sin must be 16-byte, positions 8-byte aligned", what);
    }
    for (int32_t l = 0; l < L; ++l) {
        if (!slots[l]) continue;
        if (!caches[l]) return fail(NRC_EINVAL, "%s: NULL cache of layer %d", what, l);
        if (!aligned(slots[l], 8) || !aligned(caches[l], 16))
            return fail(NRC_EINVAL, "%s: layer %d: slots must be 8-byte, cache 16-byte aligned", what, l);
    }

    if (check_only) return NRC_OK;

    const uint32_t bs = (uint32_t)block_size;
    int32_t bs_shift = -1;
    if ((bs & (bs - 1)) == 0) {
        bs_shift = 0;
        while ((1u << bs_shift) != bs) ++bs_shift;
    }
    uint32_t log2H = 0;
    while ((1u << log2H) != (uint32_t)H) ++log2H;

    for (int32_t first = 0; first < L; first += NRC_MAX_LAYERS_PER_LAUNCH) {
        const int32_t n = L - first < NRC_MAX_LAYERS_PER_LAUNCH ? L - first : NRC_MAX_LAYERS_PER_LAUNCH;
        nrc::KvStoreArgs a{};
        a.k = k + first * k_layer_stride;
        a.v = v + first * v_layer_stride;
        a.k_ls = k_layer_stride;
        a.k_rs = k_row_stride;
        a.v_ls = v_layer_stride;
        a.v_rs = v_row_stride;
        a.positions = positions;
        a.cos_sin = cos_sin;
        a.max_position = cos_sin ? max_position : 0;
        uint32_t launch_rows = 0;
        for (int32_t i = 0; i < nrc::kMaxLayersPerLaunch; ++i) {
            const int32_t l = first + i;
            const bool live = i < n && slots[l] != nullptr;
            // a layer that stores nothing keeps 0 rows (its pointers are never read)
            a.layers.cache[i] = live ? caches[l] : nullptr;
            a.layers.slots[i] = live ? slots[l] : nullptr;
            a.layers.rows[i] = live ? (uint32_t)rows[l] : 0u;
            if (a.layers.rows[i] > launch_rows) launch_rows = a.layers.rows[i];
        }
        if (launch_rows == 0 && !sum) continue;
        if (sum) {
            const int64_t layer_elems = T * 2 * H * NRC_HEAD_DIM;
            a.ws = sum->ws + first * layer_elems;
            a.ws_slice = (int64_t)L * layer_elems;
            a.k_split = sum->k_split;
            a.kv = sum->kv + first * layer_elems;
            a.T = (uint32_t)T;
        }
        a.layers_in_launch = (uint32_t)n;
        a.rows = launch_rows;
        a.H = (uint32_t)H;
        a.log2H = log2H;
        a.block_size = bs;
        a.bs_shift = bs_shift;
        a.n_slots = (uint32_t)(num_blocks * block_size);
        a.block_stride = block_stride;
        a.page_stride = page_stride;
        a.head_stride = head_stride;
        a.eps = eps;
        const int st = launch_status(nrc::launch_kv_store(a, (hipStream_t)stream), what);
        if (st) return st;
    }
    return NRC_OK;
}

}  // namespace

extern "C" {

int32_t nrc_context_kv_store(const uint16_t* k, const uint16_t* v, int64_t k_layer_stride, int64_t k_row_stride,
                             int64_t v_layer_stride, int64_t v_row_stride, const int64_t* positions,
                             const int64_t* const* slots, int64_t rows, int64_t T, const uint16_t* cos_sin,
                             int64_t max_position, uint16_t* const* caches, int64_t num_blocks, int64_t block_size,
                             int32_t H, int32_t L, float eps, void* stream) {
    if (L < 1) return fail(NRC_EINVAL, "context_kv_store: L = %d < 1", L);
    if (T < 0 || rows < 0 || rows > T)
        return fail(NRC_EINVAL, "context_kv_store: rows = %lld must lie in [0, T = %lld]", (long long)rows,
                    (long long)T);
    if (rows > 0 && (!slots || !caches)) return fail(NRC_EINVAL, "context_kv_store: NULL operand");
    if (rows > 0)
        for (int32_t l = 0; l < L; ++l)
            if (!slots[l] || !caches[l])
                return fail(NRC_EINVAL, "context_kv_store: NULL slots or cache of layer %d", l);
    // contiguous [num_blocks, H, block_size, 128] caches, one row count for every layer
    const int64_t hs = block_size * 2 * NRC_HEAD_DIM;
    std::vector<int64_t> per_layer((size_t)L, rows);
    static const int64_t* const none[1] = {nullptr};
    return store_impl("context_kv_store", k, v, k_layer_stride, k_row_stride, v_layer_stride, v_row_stride, positions,
                      rows > 0 ? slots : none, per_layer.data(), T, cos_sin, max_position, caches, num_blocks, block_size,
                      (int64_t)H * hs, 2 * NRC_HEAD_DIM, hs, H, rows > 0 ? L : 1, eps, stream);
}

int32_t nrc_context_kv_project_store(const uint16_t* normed, const uint16_t* w, int32_t w_layout, uint16_t* kv,
                                     int32_t L, int64_t T, int64_t D, int64_t N, void* workspace,
                                     int64_t workspace_bytes, const int64_t* positions, const int64_t* const* slots,
                                     int64_t rows, const uint16_t* cos_sin, int64_t max_position,
                                     uint16_t* const* caches, int64_t num_blocks, int64_t block_size, float eps,
                                     void* stream) {
    const char* what = "context_kv_project_store";
    if (w_layout != NRC_KV_WEIGHT_DN && w_layout != NRC_KV_WEIGHT_ND)
        return fail(NRC_EINVAL, "%s: weight layout %d (0 [L, D, N], 1 [L, N, D])", what, w_layout);
    if (int32_t rc = project_shape_ok(L, T, D, N)) return rc;
    if (T < 0 || rows < 0 || rows > T)
        return fail(NRC_EINVAL, "%s: rows = %lld must lie in [0, T = %lld]", what, (long long)rows, (long long)T);
    if (T == 0) return NRC_OK;
    if (!normed || !w || !kv) return fail(NRC_EINVAL, "%s: NULL operand", what);
    if (!aligned(normed, 16) || !aligned(w, 16) || !aligned(kv, 16))
        return fail(NRC_EINVAL, "%s: operands must be 16-byte aligned", what);
    const int64_t need = project_workspace_bytes(L, T, D, N);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return fail(NRC_EINVAL, "%s: needs a 16-byte aligned workspace of %lld bytes", what, (long long)need);
    // no row inserted: the projection alone
    if (rows == 0) return project_impl(normed, w, w_layout, kv, L, T, D, N, workspace, workspace_bytes, true, stream);

    if (!slots || !caches) return fail(NRC_EINVAL, "%s: NULL slots or caches array", what);
    for (int32_t l = 0; l < L; ++l)
        if (!slots[l] || !caches[l]) return fail(NRC_EINVAL, "%s: NULL slots or cache of layer %d", what, l);
    const int32_t H = (int32_t)(N / (2 * NRC_HEAD_DIM));
    const int64_t hs = block_size * 2 * NRC_HEAD_DIM;
    std::vector<int64_t> per_layer((size_t)L, rows);
    nrc::ProjectArgs a{normed, w, kv, L, T, D, N, num_cus()};
    a.b_nd = w_layout == NRC_KV_WEIGHT_ND;
    SumSource sum{nullptr, 1, kv};
    if (need > 0) {
        a.ws = static_cast<float*>(workspace);
        a.k_split = nrc::kv_project_k_split(L, T, D, N, a.num_cus);
        a.leave_partials = true;
        sum.ws = a.ws;
        sum.k_split = a.k_split;
    }
    // every operand checked before anything is launched
    auto store = [&](bool check_only) {
        return store_impl(what, kv, kv + (int64_t)H * NRC_HEAD_DIM, T * N, N, T * N, N, positions, slots,
                          per_layer.data(), T, cos_sin, max_position, caches, num_blocks, block_size,
                          (int64_t)H * hs, 2 * NRC_HEAD_DIM, hs, H, L, eps, stream, need > 0 ? &sum : nullptr,
                          check_only);
    };
    if (int32_t rc = store(true)) return rc;
    if (int32_t rc = launch_status(nrc::launch_kv_project(a, (hipStream_t)stream), what)) return rc;
    return store(false);
}

int32_t nrc_context_kv_store_ex(const uint16_t* k, const uint16_t* v, int64_t k_layer_stride, int64_t k_row_stride,
                                int64_t v_layer_stride, int64_t v_row_stride, const int64_t* positions,
                                const int64_t* const* slots, const int64_t* rows, int64_t T,
                                const uint16_t* cos_sin, int64_t max_position, uint16_t* const* caches,
                                int64_t num_blocks, int64_t block_size, int64_t block_stride, int64_t page_stride,
                                int64_t head_stride, int32_t H, int32_t L, float eps, void* stream) {
    return store_impl("context_kv_store_ex", k, v, k_layer_stride, k_row_stride, v_layer_stride, v_row_stride,
                      positions, slots, rows, T, cos_sin, max_position, caches, num_blocks, block_size, block_stride,
                      page_stride, head_stride, H, L, eps, stream);
}

int32_t nrc_check_scalars(const float* in, uint16_t* bf16_out, float* rsqrt_out, int64_t n, void* stream) {
    if (n < 0) return fail(NRC_EINVAL, "check_scalars: n < 0");
    if (n > ((int64_t)1 << 32)) return fail(NRC_EINVAL, "check_scalars: n > 2^32");
    if (n == 0) return NRC_OK;
    if (!in || (!bf16_out && !rsqrt_out)) return fail(NRC_EINVAL, "check_scalars: NULL operand");
    return launch_status(nrc::launch_scalars(in, bf16_out, rsqrt_out, n, (hipStream_t)stream), "check_scalars");
}

int32_t nrc_check_bf16_pair(const float* in, uint16_t* out, int64_t n, void* stream) {
    if (n < 0 || n > ((int64_t)1 << 32)) return fail(NRC_EINVAL, "check_bf16_pair: n out of range");
    if (n == 0) return NRC_OK;
    if (!in || !out) return fail(NRC_EINVAL, "check_bf16_pair: NULL operand");
    return launch_status(nrc::launch_bf16_pair(in, out, n, (hipStream_t)stream), "check_bf16_pair");
}


int32_t nrc_traffic_twin(const uint16_t* x, int64_t T, int32_t L, int32_t mode, int32_t per_cu, uint16_t* out,
                         uint32_t* sink, int64_t sink_len, void* stream) {
    if (mode < 0 || mode > 3) return fail(NRC_EINVAL, "traffic_twin: mode %d (0..3)", mode);
    if (per_cu != 1 && per_cu != 2) return fail(NRC_EINVAL, "traffic_twin: per_cu %d (1 or 2)", per_cu);
    if (T < 0 || L < 1 || T > ((int64_t)1 << 31)) return fail(NRC_EINVAL, "traffic_twin: T = %lld, L = %d", (long long)T, L);
    if (T == 0) return NRC_OK;
    if ((mode != 3 && !x) || (mode != 2 && !out)) return fail(NRC_EINVAL, "traffic_twin: NULL operand");
    const int cus = num_cus();
    if (mode == 2 && (!sink || sink_len < (int64_t)per_cu * cus * 1024))
        return fail(NRC_EINVAL, "traffic_twin: the reads-only mode needs a sink of %lld uint32",
                    (long long)((int64_t)per_cu * cus * 1024));
    if ((x && !aligned(x, 16)) || (out && !aligned(out, 16)))
        return fail(NRC_EINVAL, "traffic_twin: operands must be 16-byte aligned");
    return launch_status(nrc::launch_traffic_twin(x, T, L, mode, per_cu, out, sink, cus, (hipStream_t)stream),
                         "traffic_twin");
}

}  // extern "C"
