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

int launch_scalars(const float* in, uint16_t* bf, float* rs, int64_t n, hipStream_t stream) {
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(scalars_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, bf, rs, n);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nrc
