// stack([pre_norm_l(hidden_norm(x)) for l]) with every weight form the
// context page's norms accept (vLLM page "...cutedsl.draft.context",
// ContextNorms and ContextNormConstants): each norm's weight absent, bf16 or
// FP32, a gain center added to it, and the weight scaling either the norm's
// output (y = (x * r) * gamma) or its input (v = gamma * x, the sum of
// squares over v, y = v * r), as page "...cutedsl.common.draft_boundary",
// boundary_fragments, states both forms. With input-scaled layer norms each
// layer has its own sum of squares.
//
// The row sum keeps the library's fixed order (the one context_norms.hip
// states: thread t of 256 owns columns 2048k + 8t + i, two FMA chains, a
// 64-lane fold per wave, then (W0 + W2) + (W1 + W3)). One 256-thread
// workgroup normalises one row at a time (grid stride); weights are read
// from memory for every row (they stay in L2). Every conversion to bf16 is
// the exact bit-pattern rounding. The plain form (bf16 or no weights on the
// outputs) takes the faster kernel of context_norms.hip instead.
#include "device_common.h"
#include "kernels.h"

namespace nrc {

namespace {

constexpr int kThreads = 256;
constexpr int kFrags = 4;
constexpr int kChunk = 2048;  // kThreads * 8

// Eight gamma values (w + center) of a weight row at column c (a multiple
// of 8). KIND 1: bf16 bits, KIND 2: FP32.
template <int KIND>
__device__ __forceinline__ void load_gamma8(const void* w, int64_t c, float center, float* g) {
    if constexpr (KIND == 1) {
        const U32x4 v = load16(static_cast<const uint16_t*>(w) + c);
        const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            g[2 * i] = bf16_lo(p[i]) + center;
            g[2 * i + 1] = bf16_hi(p[i]) + center;
        }
    } else {
        const float* f = static_cast<const float*>(w) + c;
        const U32x4 a = load16(f), b = load16(f + 4);
        const uint32_t p[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = __uint_as_float(p[i]) + center;
    }
}

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

// HK / PK: hidden / layer weight kind (0 none, 1 bf16, 2 FP32).
template <int HK, int PK>
__global__ __launch_bounds__(kThreads) void norms_ex_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                            const void* __restrict__ hidden_w,
                                                            const void* __restrict__ pre_w, int32_t L,
                                                            float hidden_eps, float pre_eps, float hidden_center,
                                                            float pre_center, bool hidden_in, bool pre_in,
                                                            uint16_t* __restrict__ out) {
    __shared__ float sums[2][4];
    const int t = threadIdx.x;
    const int col0 = 8 * t;
    const size_t pre_elem = PK == 2 ? 4 : 2;
    int buf = 0;
    // Row sum: each wave folds its lanes, lane 0 posts the wave sum, and the
    // four combine as (W0 + W2) + (W1 + W3). Two alternating buffers: a
    // buffer is rewritten only after the barrier of the next sum, which
    // every thread passes after reading it.
    auto row_sum = [&](float lane_part) {
        const float w = wave_fold64(lane_part);
        if (__lane_id() == 0) sums[buf][t >> 6] = w;
        __syncthreads();
        const float s = (sums[buf][0] + sums[buf][2]) + (sums[buf][1] + sums[buf][3]);
        buf ^= 1;
        return s;
    };
    for (int64_t row = blockIdx.x; row < T; row += gridDim.x) {
        float u[kFrags][8];
#pragma unroll
        for (int k = 0; k < kFrags; ++k) {
            const U32x4 v = load16(x + row * kHidden + col0 + k * kChunk);
            const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u[k][2 * i] = bf16_lo(p[i]);
                u[k][2 * i + 1] = bf16_hi(p[i]);
            }
        }
        // hidden norm, rounded to bf16
        float g[kFrags][8];
        if constexpr (HK != 0) {
#pragma unroll
            for (int k = 0; k < kFrags; ++k) load_gamma8<HK>(hidden_w, col0 + k * kChunk, hidden_center, g[k]);
            if (hidden_in) {
#pragma unroll
                for (int k = 0; k < kFrags; ++k)
#pragma unroll
                    for (int i = 0; i < 8; ++i) u[k][i] = g[k][i] * u[k][i];
            }
        }
        const float rh = rsqrt_rn(__builtin_fmaf(row_sum(lane_sumsq(u)), 0x1p-13f, hidden_eps));
#pragma unroll
        for (int k = 0; k < kFrags; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float y = u[k][i] * rh;
                if (HK != 0 && !hidden_in) y = y * g[k][i];
                u[k][i] = bf16_lo(to_bf16(y));
            }
        // layer norms
        float rp = 0.0f;
        const bool per_layer = PK != 0 && pre_in;
        if (!per_layer) rp = rsqrt_rn(__builtin_fmaf(row_sum(lane_sumsq(u)), 0x1p-13f, pre_eps));
        for (int l = 0; l < L; ++l) {
            float v[kFrags][8];
            if constexpr (PK != 0) {
                const void* wl = static_cast<const char*>(pre_w) + (size_t)l * kHidden * pre_elem;
#pragma unroll
                for (int k = 0; k < kFrags; ++k) load_gamma8<PK>(wl, col0 + k * kChunk, pre_center, g[k]);
            }
            if (per_layer) {
#pragma unroll
                for (int k = 0; k < kFrags; ++k)
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[k][i] = g[k][i] * u[k][i];
                rp = rsqrt_rn(__builtin_fmaf(row_sum(lane_sumsq(v)), 0x1p-13f, pre_eps));
            }
            uint16_t* o = out + ((int64_t)l * T + row) * kHidden + col0;
#pragma unroll
            for (int k = 0; k < kFrags; ++k) {
                float y[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (per_layer) {
                        y[i] = v[k][i] * rp;
                    } else {
                        y[i] = u[k][i] * rp;
                        if constexpr (PK != 0) y[i] = y[i] * g[k][i];
                    }
                }
                store16_nt(o + k * kChunk, U32x4{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]),
                                                 pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])});
            }
        }
    }
}

template <int HK, int PK>
void launch_k(const NormsExArgs& a, hipStream_t stream) {
    const int64_t cap = (int64_t)(a.num_cus > 0 ? a.num_cus : 256) * 8;
    const unsigned grid = (unsigned)(a.T < cap ? a.T : cap);
    hipLaunchKernelGGL((norms_ex_kernel<HK, PK>), dim3(grid), dim3(kThreads), 0, stream, a.x, a.T, a.hidden_w,
                       a.pre_w, a.L, a.hidden_eps, a.pre_eps, a.hidden_center, a.pre_center, a.hidden_input_scale,
                       a.pre_input_scale, a.out);
}

template <int HK>
void launch_h(const NormsExArgs& a, hipStream_t stream) {
    if (a.pre_kind == 0)
        launch_k<HK, 0>(a, stream);
    else if (a.pre_kind == 1)
        launch_k<HK, 1>(a, stream);
    else
        launch_k<HK, 2>(a, stream);
}

}  // namespace

int launch_norms_ex(const NormsExArgs& a, hipStream_t stream) {
    if (a.hidden_kind == 0)
        launch_h<0>(a, stream);
    else if (a.hidden_kind == 1)
        launch_h<1>(a, stream);
    else
        launch_h<2>(a, stream);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nrc
