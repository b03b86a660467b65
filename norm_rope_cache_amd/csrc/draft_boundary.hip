// The DSpark draft's residual boundary: post norm -> gated FP32 residual ->
// pre norm, over 8192-wide rows. Follows the vLLM page
// "...cutedsl.common.draft_boundary" (module summary, boundary_fragments,
// DraftBoundary, DraftBoundaryConstants): per row of the bf16 branch x
//   post norm: u = x, or gamma_post * x when the weight scales the input;
//              r1 = 1/sqrt(S(u)/8192 + post_eps); y = u * r1, times
//              gamma_post when the weight scales the output;
//   residual:  res = alpha * stream + beta * bf16(y), each product rounded,
//              then the FP32 sum (optionally stored as the new stream);
//   pre norm:  of z = bf16(res), the same form with gamma_pre, rounded to
//              bf16.
// gamma = w + center (FP32 add); weights bf16, FP16 or FP32 (or none);
// the stream FP32 or bf16; alpha and beta FP32.
//
// The row sums keep the library's fixed order (thread t of 256 owns columns
// 2048k + 8t + i; two FMA chains; a 64-lane fold per wave; then
// (W0 + W2) + (W1 + W3)). One 256-thread workgroup per row (grid stride);
// the gates and gains of the thread's 32 columns stay in registers for all
// its rows. Every bf16 rounding is the exact bit-pattern rounding.
#include "device_common.h"
#include "kernels.h"

namespace nrc {

namespace {

constexpr int kThreads = 256;
constexpr int kFrags = 4;
constexpr int kChunk = 2048;  // kThreads * 8

__device__ __forceinline__ void load_f32x8(const float* p, float* f) {
    const U32x4 a = load16(p), b = load16(p + 4);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = __uint_as_float(w[i]);
}

__device__ __forceinline__ void load_bf16x8(const uint16_t* p, float* f) {
    const U32x4 v = load16(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(w[i]);
        f[2 * i + 1] = bf16_hi(w[i]);
    }
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);  // exact (v_cvt_f32_f16)
}

// Eight gains (w + center) of a weight of `kind` at column c: 1 bf16, 2 FP32,
// 3 FP16 (0: none, left untouched).
__device__ __forceinline__ void load_gain8(const void* w, int kind, int c, float center, float* g) {
    if (kind == 1) {
        load_bf16x8(static_cast<const uint16_t*>(w) + c, g);
    } else if (kind == 2) {
        load_f32x8(static_cast<const float*>(w) + c, g);
    } else if (kind == 3) {
        const U32x4 v = load16(static_cast<const uint16_t*>(w) + c);
        const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            g[2 * i] = f16_bits_to_f32(p[i] & 0xFFFFu);
            g[2 * i + 1] = f16_bits_to_f32(p[i] >> 16);
        }
    } else {
        return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) g[i] = g[i] + center;
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

template <bool STREAM_BF16, bool STORE>
__global__ __launch_bounds__(kThreads) void draft_boundary_kernel(
    const uint16_t* __restrict__ branch, int64_t m, const void* __restrict__ stream_in,
    const float* __restrict__ alpha, const float* __restrict__ beta, const void* __restrict__ post_w, int32_t post_kind,
    const void* __restrict__ pre_w, int32_t pre_kind, float post_eps, float pre_eps, float post_center,
    float pre_center, bool post_in, bool pre_in, float* __restrict__ stream_out, uint16_t* __restrict__ out) {
    __shared__ float sums[2][4];
    const int t = threadIdx.x;
    const int col0 = 8 * t;
    int buf = 0;
    auto row_sum = [&](float lane_part) {
        const float w = wave_fold64(lane_part);
        if (__lane_id() == 0) sums[buf][t >> 6] = w;
        __syncthreads();
        const float s = (sums[buf][0] + sums[buf][2]) + (sums[buf][1] + sums[buf][3]);
        buf ^= 1;
        return s;
    };
    const bool post_w_on = post_kind != 0, pre_w_on = pre_kind != 0;
    const bool scale_post_in = post_w_on && post_in, scale_pre_in = pre_w_on && pre_in;
    float al[kFrags][8], be[kFrags][8], gp[kFrags][8], gq[kFrags][8];
#pragma unroll
    for (int k = 0; k < kFrags; ++k) {
        const int c = col0 + k * kChunk;
        load_f32x8(alpha + c, al[k]);
        load_f32x8(beta + c, be[k]);
        load_gain8(post_w, post_kind, c, post_center, gp[k]);
        load_gain8(pre_w, pre_kind, c, pre_center, gq[k]);
    }
    for (int64_t row = blockIdx.x; row < m; row += gridDim.x) {
        const int64_t base = row * kHidden + col0;
        float u[kFrags][8], s[kFrags][8];
        // the stream's loads go out with the branch's, before the first row sum
#pragma unroll
        for (int k = 0; k < kFrags; ++k) {
            if constexpr (STREAM_BF16)
                load_bf16x8(static_cast<const uint16_t*>(stream_in) + base + k * kChunk, s[k]);
            else
                load_f32x8(static_cast<const float*>(stream_in) + base + k * kChunk, s[k]);
        }
#pragma unroll
        for (int k = 0; k < kFrags; ++k) {
            load_bf16x8(branch + base + k * kChunk, u[k]);
            if (scale_post_in) {
#pragma unroll
                for (int i = 0; i < 8; ++i) u[k][i] = gp[k][i] * u[k][i];
            }
        }
        const float r1 = rsqrt_rn(__builtin_fmaf(row_sum(lane_sumsq(u)), 0x1p-13f, post_eps));
#pragma unroll
        for (int k = 0; k < kFrags; ++k) {
            float res[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float y = u[k][i] * r1;
                if (post_w_on && !post_in) y = y * gp[k][i];
                const float a = al[k][i] * s[k][i];
                const float b = be[k][i] * bf16_lo(to_bf16(y));
                res[i] = a + b;
                float z = bf16_lo(to_bf16(res[i]));
                if (scale_pre_in) z = gq[k][i] * z;
                u[k][i] = z;
            }
            if constexpr (STORE) {
                float* so = stream_out + base + k * kChunk;
                store16_nt(so, U32x4{__float_as_uint(res[0]), __float_as_uint(res[1]), __float_as_uint(res[2]),
                                     __float_as_uint(res[3])});
                store16_nt(so + 4, U32x4{__float_as_uint(res[4]), __float_as_uint(res[5]), __float_as_uint(res[6]),
                                         __float_as_uint(res[7])});
            }
        }
        const float r2 = rsqrt_rn(__builtin_fmaf(row_sum(lane_sumsq(u)), 0x1p-13f, pre_eps));
#pragma unroll
        for (int k = 0; k < kFrags; ++k) {
            float o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                o[i] = u[k][i] * r2;
                if (pre_w_on && !pre_in) o[i] = o[i] * gq[k][i];
            }
            store16_nt(out + base + k * kChunk, U32x4{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]),
                                                      pack_bf16(o[4], o[5]), pack_bf16(o[6], o[7])});
        }
    }
}

template <bool STREAM_BF16, bool STORE>
void launch_b(const BoundaryArgs& a, hipStream_t stream) {
    const int64_t cap = (int64_t)(a.num_cus > 0 ? a.num_cus : 256) * 8;
    const unsigned grid = (unsigned)(a.m < cap ? a.m : cap);
    hipLaunchKernelGGL((draft_boundary_kernel<STREAM_BF16, STORE>), dim3(grid), dim3(kThreads), 0, stream, a.branch,
                       a.m, a.stream_in, a.alpha, a.beta, a.post_w, a.post_kind, a.pre_w, a.pre_kind, a.post_eps,
                       a.pre_eps, a.post_center, a.pre_center, a.post_input_scale, a.pre_input_scale, a.stream_out,
                       a.out);
}

}  // namespace

int launch_draft_boundary(const BoundaryArgs& a, hipStream_t stream) {
    if (a.stream_bf16) {
        if (a.stream_out)
            launch_b<true, true>(a, stream);
        else
            launch_b<true, false>(a, stream);
    } else {
        if (a.stream_out)
            launch_b<false, true>(a, stream);
        else
            launch_b<false, false>(a, stream);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nrc
