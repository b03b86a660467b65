// Diagnostic kernel: the library's device scalar primitives applied to an
// array, so tests can compare them exhaustively with the CPU oracle.
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
