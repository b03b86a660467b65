// Diagnostic kernels: the library's device scalar primitives applied to an
// array, so tests can compare them exhaustively with the CPU oracle; and a
// traffic twin of the norms, which moves exactly the norms' bytes in the
// norms' access pattern with no arithmetic, to measure the HBM ceiling of
// that traffic on this chip.
#include "device_common.h"
#include "kernels.h"

namespace nrc {

__global__ __launch_bounds__(256) void scalars_kernel(const float* __restrict__ in, uint16_t* __restrict__ bf,
                                                      float* __restrict__ rs, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float x = in[i];
    if (bf) bf[i] = (uint16_t)to_bf16(x);
    if (rs) rs[i] = rsqrt_rn(x);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The paired v_cvt_pk_bf16_f32 conversion the norms kernel uses on rows that
// cannot hold NaN; out[i] for in[i], two values per instruction.
__global__ __launch_bounds__(256) void bf16_pair_kernel(const float* __restrict__ in, uint16_t* __restrict__ out,
                                                        int64_t n) {
    const int64_t i = 2 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
    if (i >= n) return;
    const float a = in[i], b = i + 1 < n ? in[i + 1] : 0.0f;
    const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
    out[i] = (uint16_t)(w & 0xFFFFu);
    if (i + 1 < n) out[i + 1] = (uint16_t)(w >> 16);
}

// Traffic twin of context_norms: the same 1024-thread workgroups of four
// 256-thread row slots, the same grid, row walk and next-row prefetch, lane
// t reading its four 16-byte fragments at columns 2048 k + 8 t of the row
// and writing them to the row of each of the L outputs in the norms' store
// form (MODE 0: non-temporal system-scope buffer stores from the row's base;
// 1: plain stores; 2: no writes - the reads only, one dword per thread at the
// end keeps them live; 3: no reads - the writes only, of a per-thread
// pattern). No sums, barriers or conversions.
template <int MODE>
__global__ __launch_bounds__(1024) void traffic_twin_kernel(const uint16_t* __restrict__ x, int64_t T, int32_t L,
                                                           uint16_t* __restrict__ out, uint32_t* __restrict__ sink) {
    constexpr int kHiddenW = 8192, kChunk = 2048, kSlots = 4;
    const int tid = threadIdx.x;
    const int slot = __builtin_amdgcn_readfirstlane(tid >> 8);
    const int col0 = 8 * (tid & 255);
    const int64_t stride = (int64_t)gridDim.x * kSlots;
    int64_t row = (int64_t)blockIdx.x * kSlots + slot;
    U32x4 xv[4] = {};
    if (MODE != 3 && row < T) {
#pragma unroll
        for (int k = 0; k < 4; ++k) xv[k] = load16(x + row * kHiddenW + col0 + k * kChunk);
    }
    U32x4 acc = {0u, (uint32_t)tid, 0u, 0u};
    for (; row < T; row += stride) {
        U32x4 cur[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) cur[k] = MODE == 3 ? U32x4{acc.x + k, acc.y, (uint32_t)row, 0u} : xv[k];
        const int64_t next = row + stride;
        if (MODE != 3 && next < T) {
#pragma unroll
            for (int k = 0; k < 4; ++k) xv[k] = load16(x + next * kHiddenW + col0 + k * kChunk);
        }
        if constexpr (MODE == 2) {
#pragma unroll
            for (int k = 0; k < 4; ++k) acc = U32x4{acc.x ^ cur[k].x, acc.y ^ cur[k].y, acc.z ^ cur[k].z, acc.w ^ cur[k].w};
        } else {
            for (int l = 0; l < L; ++l) {
                uint16_t* orow = out + ((int64_t)l * T + row) * kHiddenW;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if constexpr (MODE == 1)
                        store16(orow + col0 + k * kChunk, cur[k]);
                    else
                        store16_stream(orow, kHiddenW * 2, (uint32_t)(col0 + k * kChunk) * 2, cur[k]);
                }
            }
        }
    }
    if (MODE == 2 && sink) sink[(int64_t)blockIdx.x * 1024 + tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

int launch_traffic_twin(const uint16_t* x, int64_t T, int32_t L, int32_t mode, int32_t per_cu, uint16_t* out,
                        uint32_t* sink, int32_t num_cus, hipStream_t stream) {
    // the norms' grid: one workgroup per four rows, at most per_cu (1 or 2,
    // as the norms' staged weights allow) per CU
    const int64_t groups = (T + 3) / 4, cap = (int64_t)per_cu * (num_cus > 0 ? num_cus : 256);
    const dim3 grid((unsigned)(groups < cap ? groups : cap));
    switch (mode) {
        case 0: hipLaunchKernelGGL(traffic_twin_kernel<0>, grid, dim3(1024), 0, stream, x, T, L, out, sink); break;
        case 1: hipLaunchKernelGGL(traffic_twin_kernel<1>, grid, dim3(1024), 0, stream, x, T, L, out, sink); break;
        case 2: hipLaunchKernelGGL(traffic_twin_kernel<2>, grid, dim3(1024), 0, stream, x, T, L, out, sink); break;
        case 3: hipLaunchKernelGGL(traffic_twin_kernel<3>, grid, dim3(1024), 0, stream, x, T, L, out, sink); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_bf16_pair(const float* in, uint16_t* out, int64_t n, hipStream_t stream) {
    const int64_t blocks = ((n + 1) / 2 + 255) / 256;
    hipLaunchKernelGGL(bf16_pair_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_scalars(const float* in, uint16_t* bf, float* rs, int64_t n, hipStream_t stream) {
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(scalars_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, bf, rs, n);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nrc
