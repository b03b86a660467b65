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
// (W0 + W2) + (W1 + W3)). Every bf16 rounding is the exact bit-pattern
// rounding.
//
// Layout: 512-thread workgroups of two 256-thread row slots (rows
// 2b + slot, then + 2 gridDim), each slot prefetching its next row while it
// works on the current one. Wave w of a slot owns the 512-column segments
// 2048k + 512w (k < 4). For the two norms lane l holds columns 8l .. 8l + 7
// of each segment (the row-sum order); the residual is elementwise and runs
// with lane l on columns 4l .. 4l + 3 and 256 + 4l .. 256 + 4l + 3, so that
// the FP32 stream is read and written as contiguous 1 KiB per wave
// instruction (8 consecutive FP32 per lane would take two half-strided
// accesses, measured about a quarter slower on this traffic). bf16(y) and
// bf16(res) move between the two layouts through 1 KiB of LDS private to
// each wave. The gains w + center (FP32) are staged once per workgroup in
// LDS as two 16-byte planes (a wave's 32-byte-per-lane reads then cover all
// banks); alpha and beta in plain column order for the residual's layout.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace nrc {

namespace {

constexpr int kThreads = 256;
constexpr int kFrags = 4;
constexpr int kChunk = 2048;  // kThreads * 8
constexpr int kSlots = 2;
constexpr int kBlockThreads = kSlots * kThreads;
constexpr int kGate = kHidden / 4;  // 16-byte entries per staged gate (32 KiB)

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);  // exact (v_cvt_f32_f16)
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

// Four values of a gate source at columns 4j .. 4j + 3: kind 1 bf16, 2 FP32,
// 3 FP16; alpha and beta are FP32 (kind 2).
__device__ __forceinline__ void load_gate4(const void* w, int kind, int j, float* g) {
    if (kind == 2) {
        const U32x4 v = static_cast<const U32x4*>(w)[j];
        g[0] = __uint_as_float(v.x);
        g[1] = __uint_as_float(v.y);
        g[2] = __uint_as_float(v.z);
        g[3] = __uint_as_float(v.w);
    } else {
        const uint2 v = static_cast<const uint2*>(w)[j];
        if (kind == 1) {
            g[0] = bf16_lo(v.x);
            g[1] = bf16_hi(v.x);
            g[2] = bf16_lo(v.y);
            g[3] = bf16_hi(v.y);
        } else {
            g[0] = f16_bits_to_f32(v.x & 0xFFFFu);
            g[1] = f16_bits_to_f32(v.x >> 16);
            g[2] = f16_bits_to_f32(v.y & 0xFFFFu);
            g[3] = f16_bits_to_f32(v.y >> 16);
        }
    }
}

constexpr int kExchange = 1024;  // bytes of LDS per wave for the layout exchange

template <bool STREAM_BF16, bool STORE>
__global__ __launch_bounds__(kBlockThreads) void draft_boundary_kernel(
    const uint16_t* __restrict__ branch, int64_t m, const void* __restrict__ stream_in,
    const float* __restrict__ alpha, const float* __restrict__ beta, const void* __restrict__ post_w, int32_t post_kind,
    const void* __restrict__ pre_w, int32_t pre_kind, float post_eps, float pre_eps, float post_center,
    float pre_center, bool post_in, bool pre_in, float* __restrict__ stream_out, uint16_t* __restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ float sums[kSlots][2][4];
    const int tid = threadIdx.x;
    const int slot = __builtin_amdgcn_readfirstlane(tid >> 8);  // a slot is four whole waves
    const int t = tid & (kThreads - 1);
    const int wv = t >> 6;
    const int lane = t & 63;
    const int col0 = 8 * t;            // norm layout: columns 2048k + col0 + i
    const int seg = 512 * wv;          // residual layout: columns 2048k + seg + 4 lane + 256 h + i
    const bool post_w_on = post_kind != 0, pre_w_on = pre_kind != 0;
    const bool scale_post_in = post_w_on && post_in, scale_pre_in = pre_w_on && pre_in;
    const int ngains = (post_w_on ? 1 : 0) + (pre_w_on ? 1 : 0);
    const int post_gain = 0, pre_gain = post_w_on ? 1 : 0;

    // ---- LDS: alpha, beta (FP32, column order), the gains present (FP32,
    // entry j of columns 4j .. 4j + 3 in plane j & 1 at index j >> 1), then
    // each wave's exchange buffer.
    U32x4* g_ab = reinterpret_cast<U32x4*>(smem);
    U32x4* g_gain = g_ab + 2 * kGate;
    unsigned char* xbuf = smem + (size_t)(2 + ngains) * kGate * 16 + (size_t)(tid >> 6) * kExchange;
    for (int e = tid; e < (2 + ngains) * kGate; e += kBlockThreads) {
        const int gi = e / kGate, j = e % kGate;
        float g[4];
        if (gi == 0) {
            load_gate4(alpha, 2, j, g);
        } else if (gi == 1) {
            load_gate4(beta, 2, j, g);
        } else if (gi - 2 == post_gain && post_w_on) {
            load_gate4(post_w, post_kind, j, g);
#pragma unroll
            for (int i = 0; i < 4; ++i) g[i] = g[i] + post_center;
        } else {
            load_gate4(pre_w, pre_kind, j, g);
#pragma unroll
            for (int i = 0; i < 4; ++i) g[i] = g[i] + pre_center;
        }
        const U32x4 v{__float_as_uint(g[0]), __float_as_uint(g[1]), __float_as_uint(g[2]), __float_as_uint(g[3])};
        if (gi < 2)
            g_ab[gi * kGate + j] = v;
        else
            g_gain[(gi - 2) * kGate + (j & 1) * (kGate / 2) + (j >> 1)] = v;
    }
    __syncthreads();
    // Gain gi's eight values at this lane's norm-layout fragment k.
    auto gain8 = [&](int gi, int k, float* g) {
        const U32x4* base = g_gain + gi * kGate + (col0 + k * kChunk) / 8;
        const U32x4 a = base[0], b = base[kGate / 2];
        const uint32_t p[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = __uint_as_float(p[i]);
    };
    // alpha or beta (gi 0 / 1) at the residual layout's four columns c .. c + 3
    auto ab4 = [&](int gi, int c, float* g) {
        const U32x4 a = g_ab[gi * kGate + c / 4];
        g[0] = __uint_as_float(a.x);
        g[1] = __uint_as_float(a.y);
        g[2] = __uint_as_float(a.z);
        g[3] = __uint_as_float(a.w);
    };
    auto post = [&](float lane_part, float* slot_sums) {
        const float w = wave_fold64(lane_part);
        if (__lane_id() == 0) slot_sums[wv] = w;
    };
    auto combine = [&](const float* s) { return (s[0] + s[2]) + (s[1] + s[3]); };

    // Residual-layout stream: per fragment k two pieces h of four columns.
    typedef typename std::conditional<STREAM_BF16, uint2, U32x4>::type SPiece;
    auto rcol = [&](int k, int h) { return k * kChunk + seg + 256 * h + 4 * lane; };
    auto load_row = [&](int64_t r, U32x4 (&bv)[kFrags], SPiece (&sv)[kFrags][2]) {
        const int64_t base = r * kHidden;
#pragma unroll
        for (int k = 0; k < kFrags; ++k)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (STREAM_BF16)
                    sv[k][h] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(stream_in) + base + rcol(k, h));
                else
                    sv[k][h] = load16(static_cast<const float*>(stream_in) + base + rcol(k, h));
            }
#pragma unroll
        for (int k = 0; k < kFrags; ++k) bv[k] = load16(branch + base + col0 + k * kChunk);
    };
    auto piece = [&](const SPiece& v, int i) {
        if constexpr (STREAM_BF16)
            return (i & 1) ? bf16_hi(i < 2 ? v.x : v.y) : bf16_lo(i < 2 ? v.x : v.y);
        else
            return __uint_as_float(i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w);
    };

    const int64_t stride = (int64_t)gridDim.x * kSlots;
    int64_t row = (int64_t)blockIdx.x * kSlots + slot;
    U32x4 bv[kFrags];
    SPiece sv[kFrags][2];
    if (row < m) load_row(row, bv, sv);
    for (int64_t first = (int64_t)blockIdx.x * kSlots; first < m; first += stride, row += stride) {
        const bool active = row < m;
        float u[kFrags][8];
        SPiece sc[kFrags][2];
#pragma unroll
        for (int k = 0; k < kFrags; ++k) {
            const uint32_t b[4] = {bv[k].x, bv[k].y, bv[k].z, bv[k].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u[k][2 * i] = active ? bf16_lo(b[i]) : 0.0f;
                u[k][2 * i + 1] = active ? bf16_hi(b[i]) : 0.0f;
            }
            sc[k][0] = sv[k][0];
            sc[k][1] = sv[k][1];
        }
        const int64_t next = row + stride;
        if (next < m) load_row(next, bv, sv);

        // post norm (norm layout)
        if (scale_post_in) {
#pragma unroll
            for (int k = 0; k < kFrags; ++k) {
                float gp[8];
                gain8(post_gain, k, gp);
#pragma unroll
                for (int i = 0; i < 8; ++i) u[k][i] = gp[i] * u[k][i];
            }
        }
        post(lane_sumsq(u), sums[slot][0]);
        __syncthreads();
        const float r1 = rsqrt_rn(__builtin_fmaf(combine(sums[slot][0]), 0x1p-13f, post_eps));

        const int64_t rbase = row * kHidden;
#pragma unroll
        for (int k = 0; k < kFrags; ++k) {
            // bf16(y) in the norm layout, to LDS
            {
                float gp[8];
                if (post_w_on && !post_in) gain8(post_gain, k, gp);
                uint32_t yw[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    float y0 = u[k][2 * p] * r1, y1 = u[k][2 * p + 1] * r1;
                    if (post_w_on && !post_in) {
                        y0 = y0 * gp[2 * p];
                        y1 = y1 * gp[2 * p + 1];
                    }
                    yw[p] = pack_bf16(y0, y1);
                }
                *reinterpret_cast<U32x4*>(xbuf + 16 * lane) = U32x4{yw[0], yw[1], yw[2], yw[3]};
            }
            // residual in the residual layout: res = alpha s + beta bf16(y)
            uint2 zw[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint2 y2 = *reinterpret_cast<const uint2*>(xbuf + 512 * h + 8 * lane);
                const int c = rcol(k, h);
                float al[4], be[4], res[4];
                ab4(0, c, al);
                ab4(1, c, be);
                const float yv[4] = {bf16_lo(y2.x), bf16_hi(y2.x), bf16_lo(y2.y), bf16_hi(y2.y)};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a = al[i] * piece(sc[k][h], i);
                    const float b = be[i] * yv[i];
                    res[i] = a + b;
                }
                if constexpr (STORE) {
                    if (active)
                        store16_stream(stream_out + rbase, kHidden * 4, (uint32_t)c * 4,
                                       U32x4{__float_as_uint(res[0]), __float_as_uint(res[1]),
                                             __float_as_uint(res[2]), __float_as_uint(res[3])});
                }
                zw[h] = make_uint2(pack_bf16(res[0], res[1]), pack_bf16(res[2], res[3]));
            }
            // bf16(res) back to the norm layout (after every lane's read of y)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                *reinterpret_cast<uint2*>(xbuf + 512 * h + 8 * lane) = zw[h];
            const U32x4 z4 = *reinterpret_cast<const U32x4*>(xbuf + 16 * lane);
            const uint32_t zp[4] = {z4.x, z4.y, z4.z, z4.w};
            float gq[8];
            if (scale_pre_in) gain8(pre_gain, k, gq);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float z0 = bf16_lo(zp[p]), z1 = bf16_hi(zp[p]);
                if (scale_pre_in) {
                    z0 = gq[2 * p] * z0;
                    z1 = gq[2 * p + 1] * z1;
                }
                u[k][2 * p] = z0;
                u[k][2 * p + 1] = z1;
            }
        }

        // pre norm (norm layout)
        post(lane_sumsq(u), sums[slot][1]);
        __syncthreads();
        const float r2 = rsqrt_rn(__builtin_fmaf(combine(sums[slot][1]), 0x1p-13f, pre_eps));
        if (active) {
#pragma unroll
            for (int k = 0; k < kFrags; ++k) {
                float gq[8], o[8];
                if (pre_w_on && !pre_in) gain8(pre_gain, k, gq);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    o[i] = u[k][i] * r2;
                    if (pre_w_on && !pre_in) o[i] = o[i] * gq[i];
                }
                store16_stream(out + rbase, kHidden * 2, (uint32_t)(col0 + k * kChunk) * 2,
                               U32x4{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]), pack_bf16(o[4], o[5]),
                                     pack_bf16(o[6], o[7])});
            }
        }
    }
}

template <bool STREAM_BF16, bool STORE>
int launch_b(const BoundaryArgs& a, hipStream_t stream) {
    const int gates = 2 + (a.post_kind ? 1 : 0) + (a.pre_kind ? 1 : 0);
    const size_t lds = (size_t)gates * kGate * 16 + (size_t)(kBlockThreads / 64) * kExchange;
    auto kernel = draft_boundary_kernel<STREAM_BF16, STORE>;
    if (lds > 65536) {
        static std::atomic<int> done[64] = {};
        if (raise_lds_limit((const void*)kernel, (int)lds, done)) return -1;
    }
    // Workgroups resident per CU: two when the gates take at most half the
    // LDS; rows beyond the grid are walked with a grid stride.
    const int64_t per_cu = lds <= 64 * 1024 ? 2 : 1;
    const int64_t groups = (a.m + kSlots - 1) / kSlots;
    const int64_t cap = (int64_t)(a.num_cus > 0 ? a.num_cus : 256) * per_cu;
    const unsigned grid = (unsigned)(groups < cap ? groups : cap);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kBlockThreads), lds, stream, a.branch, a.m, a.stream_in, a.alpha,
                       a.beta, a.post_w, a.post_kind, a.pre_w, a.pre_kind, a.post_eps, a.pre_eps, a.post_center,
                       a.pre_center, a.post_input_scale, a.pre_input_scale, a.stream_out, a.out);
    return 0;
}

}  // namespace

int launch_draft_boundary(const BoundaryArgs& a, hipStream_t stream) {
    int rc;
    if (a.stream_bf16)
        rc = a.stream_out ? launch_b<true, true>(a, stream) : launch_b<true, false>(a, stream);
    else
        rc = a.stream_out ? launch_b<false, true>(a, stream) : launch_b<false, false>(a, stream);
    if (rc) return rc;
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nrc
