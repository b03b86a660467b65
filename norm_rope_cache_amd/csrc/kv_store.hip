// Weightless K-norm + GPT-J RoPE + paged-cache insert, all layers of a call
// in one launch (up to 8 layers; the host splits more).
//
// Follows the vLLM page "...cutedsl.draft.context": _ContextKvStoreKernel
// (operands, rounding points, slot addressing), _sum_squares_64 (the 64-wide
// fold by halves) and _rope (the GPT-J pair with one FMA per output). The
// pages' kernel gives one 32-lane warp per (row, layer) and a 4-byte pair per
// lane; here each 64-wide head is owned by 8 lanes holding 8 consecutive bf16
// (one 16-byte load of K and one of V per lane), so a wave64 covers 8 heads
// with fully coalesced 128-byte runs and the fold's three cross-lane strides
// are DPP / swizzle exchanges inside each 8-lane group.
//
// Work unit u = (layer, row, head) with the head fastest; lanes 8u .. 8u+7.
// Rows whose slot is negative (or out of range, or whose position is out of
// range), and rows past their layer's slot list, read nothing and write
// nothing. The cache is a strided view: (block, page, head) at block *
// block_stride + page * page_stride + head * head_stride, K in the first 64
// elements of the 128-element run and V in the next 64.
#include "device_common.h"
#include "kernels.h"

namespace nrc {

template <bool ROPE>
__global__ __launch_bounds__(256) void kv_store_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                       int64_t k_ls, int64_t k_rs, int64_t v_ls, int64_t v_rs,
                                                       const int64_t* __restrict__ positions,
                                                       const uint16_t* __restrict__ cos_sin, int64_t max_position,
                                                       StoreLayers layers, uint32_t rows, uint32_t H,
                                                       uint32_t log2H, uint32_t total_units, uint32_t block_size,
                                                       int32_t bs_shift, uint32_t n_slots, int64_t block_stride,
                                                       int64_t page_stride, int64_t head_stride, float eps) {
    const uint32_t unit = (blockIdx.x * blockDim.x + threadIdx.x) >> 3;
    const uint32_t g = threadIdx.x & 7u;  // this lane's 8 elements of the head: 8g .. 8g+7
    if (unit >= total_units) return;  // whole 8-lane groups leave together
    const uint32_t h = unit & (H - 1u);
    const uint32_t rt = unit >> log2H;
    const uint32_t l = rt / rows;
    const uint32_t t = rt - l * rows;

    if (t >= layers.rows[l]) return;  // past this layer's slot list (or a layer without one)
    const int64_t slot = layers.slots[l][t];
    if (slot < 0 || (uint64_t)slot >= (uint64_t)n_slots) return;
    const uint16_t* cs = nullptr;
    if constexpr (ROPE) {
        const int64_t p = positions[t];
        if (p < 0 || p >= max_position) return;
        cs = cos_sin + p * kHeadDim;
    }

    const U32x4 kw = load16(k + (int64_t)l * k_ls + (int64_t)t * k_rs + h * kHeadDim + 8 * g);
    const U32x4 vw = load16(v + (int64_t)l * v_ls + (int64_t)t * v_rs + h * kHeadDim + 8 * g);
    uint2 cw, sw;
    if constexpr (ROPE) {
        cw = *reinterpret_cast<const uint2*>(cs + 4 * g);                  // cos of pairs 4g .. 4g+3
        sw = *reinterpret_cast<const uint2*>(cs + kHeadDim / 2 + 4 * g);   // sin of the same pairs
    }

    float kf[8] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y),
                   bf16_lo(kw.z), bf16_hi(kw.z), bf16_lo(kw.w), bf16_hi(kw.w)};
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = kf[i] * kf[i];
    // Fold of the 64 squares by halves. Element e = 8g + i: strides 32, 16
    // and 8 pair lane g with g^4, g^2, g^1 (same i); strides 4, 2, 1 pair
    // i with i+4, i+2, i+1 inside the lane.
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = q[i] + lane_xor<4>(q[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = q[i] + lane_xor<2>(q[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = q[i] + lane_xor<1>(q[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = q[i] + q[i + 4];
    q[0] = q[0] + q[2];
    q[1] = q[1] + q[3];
    const float S = q[0] + q[1];
    const float r = rsqrt_rn(__builtin_fmaf(S, 0.015625f, eps));  // mean: 1/64 exact

    uint32_t nb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) nb[i] = to_bf16(kf[i] * r);

    U32x4 out;
    if constexpr (ROPE) {
        const float c[4] = {bf16_lo(cw.x), bf16_hi(cw.x), bf16_lo(cw.y), bf16_hi(cw.y)};
        const float s[4] = {bf16_lo(sw.x), bf16_hi(sw.x), bf16_lo(sw.y), bf16_hi(sw.y)};
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float a = __uint_as_float(nb[2 * p] << 16);
            const float b = __uint_as_float(nb[2 * p + 1] << 16);
            const float bs = b * s[p];
            const float as = a * s[p];
            o[p] = to_bf16(__builtin_fmaf(a, c[p], -bs)) | (to_bf16(__builtin_fmaf(b, c[p], as)) << 16);
        }
        out = U32x4{o[0], o[1], o[2], o[3]};
    } else {
        out = U32x4{nb[0] | (nb[1] << 16), nb[2] | (nb[3] << 16), nb[4] | (nb[5] << 16), nb[6] | (nb[7] << 16)};
    }

    // Slots fit 32 bits (checked on the host): block = s / block_size, page = s % block_size.
    const uint32_t s32 = (uint32_t)slot;
    uint32_t block, page;
    if (bs_shift >= 0) {
        block = s32 >> bs_shift;
        page = s32 & (block_size - 1u);
    } else {
        block = s32 / block_size;
        page = s32 - block * block_size;
    }
    uint16_t* dst = layers.cache[l] + (int64_t)block * block_stride + (int64_t)page * page_stride +
                    (int64_t)h * head_stride + 8 * g;
    // Non-temporal: the cache rows are scattered and not read back by this
    // chain, so they go out to HBM now instead of lingering dirty in the
    // caches until the next kernel's traffic evicts them.
    store16_nt(dst, out);
    store16_nt(dst + kHeadDim, vw);
}

int launch_kv_store(const KvStoreArgs& a, hipStream_t stream) {
    const uint32_t total_units = (uint32_t)a.layers_in_launch * a.rows * a.H;
    const uint32_t threads = 256;
    const uint32_t blocks = (uint32_t)(((uint64_t)total_units * 8 + threads - 1) / threads);
    if (a.cos_sin)
        hipLaunchKernelGGL(kv_store_kernel<true>, dim3(blocks), dim3(threads), 0, stream, a.k, a.v, a.k_ls, a.k_rs,
                           a.v_ls, a.v_rs, a.positions, a.cos_sin, a.max_position, a.layers, a.rows, a.H, a.log2H,
                           total_units, a.block_size, a.bs_shift, a.n_slots, a.block_stride, a.page_stride,
                           a.head_stride, a.eps);
    else
        hipLaunchKernelGGL(kv_store_kernel<false>, dim3(blocks), dim3(threads), 0, stream, a.k, a.v, a.k_ls, a.k_rs,
                           a.v_ls, a.v_rs, a.positions, a.cos_sin, a.max_position, a.layers, a.rows, a.H, a.log2H,
                           total_units, a.block_size, a.bs_shift, a.n_slots, a.block_stride, a.page_stride,
                           a.head_stride, a.eps);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nrc
