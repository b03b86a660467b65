// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Arguments reach these functions already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace nrc {

// Raise a kernel's dynamic-LDS limit to `bytes` on the current device (the
// opt-in above 64 KiB is per kernel and device). `done` caches per device
// the largest limit set so far; setting it twice from racing threads is
// harmless. Returns 0, or -1 when the runtime refuses.
template <int DEVICES>
inline int raise_lds_limit(const void* kernel, int bytes, std::atomic<int> (&done)[DEVICES]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    if (dev < DEVICES && done[dev].load(std::memory_order_relaxed) >= bytes) return 0;
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) return -1;
    if (dev < DEVICES) done[dev].store(bytes, std::memory_order_relaxed);
    return 0;
}

constexpr int kMaxLayersPerLaunch = 8;

struct StoreLayers {
    uint16_t* cache[kMaxLayersPerLaunch];
    const int64_t* slots[kMaxLayersPerLaunch];
    uint32_t rows[kMaxLayersPerLaunch];  // rows inserted per layer (0: the layer stores nothing)
};

struct KvStoreArgs {
    const uint16_t* k;
    const uint16_t* v;
    int64_t k_ls, k_rs, v_ls, v_rs;
    const int64_t* positions;
    const uint16_t* cos_sin;  // nullptr: RoPE off
    int64_t max_position;
    StoreLayers layers;
    uint32_t layers_in_launch;
    uint32_t rows;
    uint32_t H;
    uint32_t log2H;
    uint32_t block_size;
    int32_t bs_shift;  // log2(block_size), or -1 when not a power of two
    int64_t block_stride, page_stride, head_stride;  // cache view strides, elements
    uint32_t n_slots;
    float eps;
    // Non-null: the launch also finishes a split projection - K and V come
    // from the FP32 partial sums ws [k_split, L, T, N] (at this launch's first
    // layer; ws_slice elements between slices), added in slice order and
    // rounded into kv [L, T, N] (every row), instead of from k and v.
    const float* ws = nullptr;
    int64_t ws_slice = 0;
    int32_t k_split = 0;
    uint16_t* kv = nullptr;
    uint32_t T = 0;
};

int launch_kv_store(const KvStoreArgs& a, hipStream_t stream);

struct NormsArgs {
    const uint16_t* x;
    int64_t T;
    const uint16_t* hidden_w;  // nullptr: weightless
    const uint16_t* pre_w;     // nullptr: weightless
    int32_t L;
    float hidden_eps, pre_eps, hidden_center, pre_center;
    uint16_t* out;
    int32_t num_cus;
};

// The norms with FP32 weights and/or input-scaled weights (norms_ex.hip).
struct NormsExArgs {
    const uint16_t* x;
    int64_t T;
    const void* hidden_w;  // kind 0: nullptr; 1: bf16 [8192]; 2: float [8192]
    int32_t hidden_kind;
    const void* pre_w;     // [L, 8192] of pre_kind's type, or nullptr
    int32_t pre_kind;
    int32_t L;
    float hidden_eps, pre_eps, hidden_center, pre_center;
    bool hidden_input_scale, pre_input_scale;
    uint16_t* out;
    int num_cus;
};

int launch_norms_ex(const NormsExArgs& a, hipStream_t stream);

// The residual boundary (draft_boundary.hip).
struct BoundaryArgs {
    const uint16_t* branch;  // [m, 8192] bf16
    int64_t m;
    const void* stream_in;   // [m, 8192] FP32, or bf16 when stream_bf16
    bool stream_bf16;
    const float* alpha;      // [8192]
    const float* beta;       // [8192]
    const void* post_w;      // [8192] of post_kind (0 none, 1 bf16, 2 FP32, 3 FP16)
    int32_t post_kind;
    const void* pre_w;
    int32_t pre_kind;
    float post_eps, pre_eps, post_center, pre_center;
    bool post_input_scale, pre_input_scale;
    float* stream_out;       // [m, 8192] FP32, or nullptr
    uint16_t* out;           // [m, 8192] bf16
    int num_cus;
};

int launch_draft_boundary(const BoundaryArgs& a, hipStream_t stream);

int launch_context_norms(const NormsArgs& a, hipStream_t stream);
// h_out [T, 8192] bf16 and r_out [T]: the pre-pass of the fused projection (a.out unused).
int launch_hidden_norm(const NormsArgs& a, uint16_t* h_out, float* r_out, hipStream_t stream);

struct ProjectArgs {
    const uint16_t* A;  // [L, M, K]
    const uint16_t* B;  // [L, K, N], or [L, N, K] when b_nd
    uint16_t* C;        // [L, M, N]
    int32_t L;
    int64_t M, K, N;
    int32_t num_cus;
    bool b_nd = false;
    float* ws = nullptr;  // split K: FP32 partial sums [k_split, L, M, N]
    int32_t k_split = 1;
    bool leave_partials = false;  // split K: stop after the sums (the store adds them)
    // Diagnostic clock stamps, 4 per workgroup (shader clock and constant-rate
    // clock at the start, then at the end), written when non-null; unfused,
    // unsplit form only. *workgroups receives the grid size when non-null.
    uint64_t* stamps = nullptr;
    int64_t stamps_len = 0;
    int32_t* workgroups = nullptr;
};

int launch_kv_project(const ProjectArgs& a, hipStream_t stream);
// Bytes of the device-resident scratch behind the no-allocation projection.
constexpr int64_t kProjectScratchBytes = (int64_t)64 << 20;
// This GPU's (the current device's) address of that scratch; looked up once
// per device. 0 on success.
int project_scratch(void** ptr);
// Number of K slices the projection of this shape is split into (1: none):
// only shapes with too few output tiles to fill the CUs are split.
int32_t kv_project_k_split(int32_t L, int64_t M, int64_t K, int64_t N, int num_cus);
// A = bf16((h * |r[m]|) * (gamma_l + center)) built in the kernel; a.A is h [M, K].
int launch_kv_project_fused(const ProjectArgs& a, const float* r, const uint16_t* gamma, float center,
                            hipStream_t stream);

int launch_bf16_pair(const float* in, uint16_t* out, int64_t n, hipStream_t stream);
// The norms' traffic without their arithmetic (selftest.hip): mode 0 the
// norms' stores, 1 plain stores, 2 reads only (one dword per thread to sink),
// 3 writes only; per_cu workgroups per CU at most.
int launch_traffic_twin(const uint16_t* x, int64_t T, int32_t L, int32_t mode, int32_t per_cu, uint16_t* out,
                        uint32_t* sink, int32_t num_cus, hipStream_t stream);
int launch_scalars(const float* in, uint16_t* bf, float* rs, int64_t n, hipStream_t stream);

}  // namespace nrc
