// stack([pre_norm_l(hidden_norm(x)) for l]) for 8192-wide bf16 rows.
//
// Follows the vLLM page "...cutedsl.draft.context" (ContextNorms,
// _ContextNormsKernel: the hidden norm's output is rounded to bf16 before the
// layer norms read it; the output is [L, T, 8192]) with the per-norm
// arithmetic of "...cutedsl.common.draft_boundary", boundary_fragments:
// r = 1/sqrt(S * 2^-13 + eps) with one FMA, y = x * r, then y * (w + center).
//
// The row sum of squares uses the library's fixed order, which the CPU oracle
// defines independently: thread t of 256 owns columns 2048k + 8t + i
// (k < 4, i < 8) as four 16-byte loads, accumulates the even and the odd
// columns in two FMA chains (k, then the pair index), adds them, folds the 64
// lanes of its wave by halves, and the four wave sums combine as
// (W0 + W2) + (W1 + W3).
//
// Differences from the pages' kernel (one CTA per (row, layer), recomputing
// the hidden norm and the layer-norm sum for every layer): one 256-thread
// workgroup walks rows with a grid stride, normalises each row once and
// writes all L layer outputs from the same registers. Every layer norm shares
// eps and center (the runtime page's ContextKV takes one set for all layers),
// and with the weight applied after the norm the layer-norm sum does not
// depend on the layer, so one sum per row serves all layers (identical bits).
// Weights stay in registers (packed bf16) for L <= 8; above that they are
// read per row from memory (L2-resident).
#include "device_common.h"
#include "kernels.h"

namespace nrc {

namespace {

constexpr int kThreads = 256;
constexpr int kFrags = 4;
constexpr int kChunk = 2048;  // kThreads * 8

__device__ __forceinline__ void unpack8(const U32x4& w, float* f) {
    f[0] = bf16_lo(w.x);
    f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y);
    f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z);
    f[5] = bf16_hi(w.z);
    f[6] = bf16_lo(w.w);
    f[7] = bf16_hi(w.w);
}

// This lane's share of the row sum: even and odd FMA chains over k then the
// pair index, then even + odd.
__device__ __forceinline__ float lane_sumsq(const float (&u)[kFrags][8]) {
    float even = 0.0f, odd = 0.0f;
#pragma unroll
    for (int k = 0; k < kFrags; ++k)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            even = __builtin_fmaf(u[k][2 * p], u[k][2 * p], even);
            odd = __builtin_fmaf(u[k][2 * p + 1], u[k][2 * p + 1], odd);
        }
    return even + odd;
}

// Row sum from the 4 wave sums in shared memory.
__device__ __forceinline__ float block_sum(float lane_part, float* slot) {
    const float w = wave_fold64(lane_part);
    if (__lane_id() == 0) slot[threadIdx.x >> 6] = w;
    __syncthreads();
    return (slot[0] + slot[2]) + (slot[1] + slot[3]);
}

template <int LREG, bool HW, bool PW>
__global__ __launch_bounds__(kThreads) void context_norms_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                                 const uint16_t* __restrict__ hidden_w,
                                                                 const uint16_t* __restrict__ pre_w, int32_t L,
                                                                 float hidden_eps, float pre_eps, float hidden_center,
                                                                 float pre_center, uint16_t* __restrict__ out) {
    __shared__ float sums[2][4];
    const int tid = threadIdx.x;
    const int col0 = 8 * tid;

    U32x4 gh[kFrags];
    if constexpr (HW) {
#pragma unroll
        for (int k = 0; k < kFrags; ++k) gh[k] = load16(hidden_w + col0 + k * kChunk);
    }
    constexpr int kRegLayers = LREG > 0 ? LREG : 1;
    U32x4 gp[kRegLayers][kFrags];
    if constexpr (PW && LREG > 0) {
#pragma unroll
        for (int l = 0; l < LREG; ++l)
#pragma unroll
            for (int k = 0; k < kFrags; ++k) gp[l][k] = load16(pre_w + (int64_t)l * kHidden + col0 + k * kChunk);
    }
    const int layers = LREG > 0 ? LREG : L;

    int64_t row = blockIdx.x;
    U32x4 xv[kFrags];
    if (row < T) {
#pragma unroll
        for (int k = 0; k < kFrags; ++k) xv[k] = load16_nt(x + row * kHidden + col0 + k * kChunk);
    }
    for (; row < T; row += gridDim.x) {
        float u[kFrags][8];
#pragma unroll
        for (int k = 0; k < kFrags; ++k) unpack8(xv[k], u[k]);
        // Prefetch the next row while this one is normalised and written.
        const int64_t next = row + gridDim.x;
        if (next < T) {
#pragma unroll
            for (int k = 0; k < kFrags; ++k) xv[k] = load16_nt(x + next * kHidden + col0 + k * kChunk);
        }

        // Hidden norm, rounded to bf16.
        const float Sh = block_sum(lane_sumsq(u), sums[0]);
        const float rh = rsqrt_rn(__builtin_fmaf(Sh, 0x1p-13f, hidden_eps));
#pragma unroll
        for (int k = 0; k < kFrags; ++k) {
            float g[8];
            if constexpr (HW) unpack8(gh[k], g);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float y = u[k][i] * rh;
                if constexpr (HW) y = y * (g[i] + hidden_center);
                u[k][i] = __uint_as_float(to_bf16(y) << 16);
            }
        }

        // One layer-norm sum for all layers.
        const float Sp = block_sum(lane_sumsq(u), sums[1]);
        const float rp = rsqrt_rn(__builtin_fmaf(Sp, 0x1p-13f, pre_eps));
#pragma unroll
        for (int k = 0; k < kFrags; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i) u[k][i] = u[k][i] * rp;

        for (int l = 0; l < layers; ++l) {
            uint16_t* o = out + ((int64_t)l * T + row) * kHidden + col0;
#pragma unroll
            for (int k = 0; k < kFrags; ++k) {
                uint32_t w[4];
                if constexpr (PW) {
                    U32x4 gw;
                    if constexpr (LREG > 0) {
                        gw = gp[l][k];
                    } else {
                        gw = load16(pre_w + (int64_t)l * kHidden + col0 + k * kChunk);
                    }
                    float g[8];
                    unpack8(gw, g);
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        w[p] = pack_bf16(u[k][2 * p] * (g[2 * p] + pre_center),
                                         u[k][2 * p + 1] * (g[2 * p + 1] + pre_center));
                } else {
#pragma unroll
                    for (int p = 0; p < 4; ++p) w[p] = pack_bf16(u[k][2 * p], u[k][2 * p + 1]);
                }
                store16_nt(o + k * kChunk, U32x4{w[0], w[1], w[2], w[3]});
            }
        }
    }
}

template <int LREG>
void launch_l(const NormsArgs& a, dim3 grid, hipStream_t stream) {
    const bool hw = a.hidden_w != nullptr, pw = a.pre_w != nullptr;
#define NRC_NORMS_LAUNCH(H, P)                                                                                     \
    hipLaunchKernelGGL((context_norms_kernel<LREG, H, P>), grid, dim3(kThreads), 0, stream, a.x, a.T, a.hidden_w, \
                       a.pre_w, a.L, a.hidden_eps, a.pre_eps, a.hidden_center, a.pre_center, a.out)
    if (hw && pw)
        NRC_NORMS_LAUNCH(true, true);
    else if (hw)
        NRC_NORMS_LAUNCH(true, false);
    else if (pw)
        NRC_NORMS_LAUNCH(false, true);
    else
        NRC_NORMS_LAUNCH(false, false);
#undef NRC_NORMS_LAUNCH
}

}  // namespace

int launch_context_norms(const NormsArgs& a, hipStream_t stream) {
    // Enough resident workgroups to keep every CU busy; rows beyond them are
    // walked with a grid stride.
    const int64_t per_cu = a.L <= 4 ? 4 : 2;
    const int64_t max_blocks = (int64_t)(a.num_cus > 0 ? a.num_cus : 256) * per_cu;
    const dim3 grid((unsigned)(a.T < max_blocks ? a.T : max_blocks));
    switch (a.L) {
        case 1: launch_l<1>(a, grid, stream); break;
        case 2: launch_l<2>(a, grid, stream); break;
        case 3: launch_l<3>(a, grid, stream); break;
        case 4: launch_l<4>(a, grid, stream); break;
        case 5: launch_l<5>(a, grid, stream); break;
        case 6: launch_l<6>(a, grid, stream); break;
        case 7: launch_l<7>(a, grid, stream); break;
        case 8: launch_l<8>(a, grid, stream); break;
        default: launch_l<0>(a, grid, stream); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nrc
