// Weightless K-norm + GPT-J RoPE + paged-cache insert, all layers of a call
// in one launch (up to 8 layers; the host splits more). A second kernel
// (kv_sum_store_kernel, below) also finishes a split projection: it adds the
// partial sums into kv and inserts the rows in the same pass.
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
// Work unit = (layer, row, head), taken by an 8-lane group; heads are
// fastest, then rows (then layers, in the H < 8 form's one-dimensional
// grid). Rows whose slot is negative (or out of range, or whose position is
// out of range), and rows past their layer's slot list, read nothing but
// their slot and position and write nothing.
// The cache is a strided view: (block, page, head) at block * block_stride +
// page * page_stride + head * head_stride, K in the first 64 elements of the
// 128-element run and V in the next 64.
#include "device_common.h"
#include "kernels.h"

namespace nrc {

typedef __attribute__((address_space(1))) const int64_t GlobalI64;
typedef __attribute__((address_space(1))) uint16_t GlobalU16;

// 16-byte non-temporal store through a global-memory pointer.
__device__ __forceinline__ void store16_nt_global(GlobalU16* p, U32x4 v) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, (__attribute__((address_space(1))) u32x4*)p);
}

// The K-norm, RoPE and packing of one lane's 8 elements of K (the fold's
// lane exchanges stay inside the lane's 8-lane group). Each rounding to bf16
// takes the paired hardware conversion when its inputs cannot be NaN (equal
// to the exact rounding for every other input), else the exact one.
template <bool ROPE>
__device__ __forceinline__ U32x4 k_out(U32x4 kw, uint2 cw, uint2 sw, float eps) {
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

    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = kf[i] * r;
    // A finite S means every k is finite; with r finite too, no k * r is NaN.
    uint32_t nb[4];
    if (__builtin_isfinite(S) && __builtin_isfinite(r)) {
#pragma unroll
        for (int p = 0; p < 4; ++p) nb[p] = pack_bf16_pair_hw(y[2 * p], y[2 * p + 1]);
    } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) nb[p] = pack_bf16(y[2 * p], y[2 * p + 1]);
    }
    if constexpr (!ROPE) {
        return U32x4{nb[0], nb[1], nb[2], nb[3]};
    } else {
        const float c[4] = {bf16_lo(cw.x), bf16_hi(cw.x), bf16_lo(cw.y), bf16_hi(cw.y)};
        const float s[4] = {bf16_lo(sw.x), bf16_hi(sw.x), bf16_lo(sw.y), bf16_hi(sw.y)};
        float z[8];
        bool nan = false;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float a = bf16_lo(nb[p]);
            const float b = bf16_hi(nb[p]);
            const float bs = b * s[p];
            const float as = a * s[p];
            z[2 * p] = __builtin_fmaf(a, c[p], -bs);
            z[2 * p + 1] = __builtin_fmaf(b, c[p], as);
            nan = nan || __builtin_isnan(z[2 * p]) || __builtin_isnan(z[2 * p + 1]);
        }
        uint32_t o[4];
        if (!nan) {
#pragma unroll
            for (int p = 0; p < 4; ++p) o[p] = pack_bf16_pair_hw(z[2 * p], z[2 * p + 1]);
        } else {
#pragma unroll
            for (int p = 0; p < 4; ++p) o[p] = pack_bf16(z[2 * p], z[2 * p + 1]);
        }
        return U32x4{o[0], o[1], o[2], o[3]};
    }
}

// One 8-lane group per work unit. ROW_WAVE (H >= 8): the grid is (waves of
// rows, layers) and a wave's 8 groups are 8 heads of one row, so the layer,
// the row, its slot and position and the K/V row bases are wave-uniform and
// computed once, in scalar registers; only the head offset is per lane.
// Otherwise (H < 8) a wave spans 8 / H rows, possibly of two layers, and
// each lane works them out itself.
template <bool ROPE, bool ROW_WAVE>
__global__ __launch_bounds__(256) void kv_store_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                       int64_t k_ls, int64_t k_rs, int64_t v_ls, int64_t v_rs,
                                                       const int64_t* __restrict__ positions,
                                                       const uint16_t* __restrict__ cos_sin, int64_t max_position,
                                                       StoreLayers layers, uint32_t rows, uint32_t H,
                                                       uint32_t log2H, uint32_t total_units, uint32_t block_size,
                                                       int32_t bs_shift, uint32_t n_slots, int64_t block_stride,
                                                       int64_t page_stride, int64_t head_stride, float eps,
                                                       uint32_t head_span) {
    const uint32_t g = threadIdx.x & 7u;  // this lane's 8 elements of the head: 8g .. 8g+7
    uint32_t l, t, h;
    uint32_t l_rows = 0;
    uint64_t l_slots_a = 0, l_cache_a = 0;
    if constexpr (ROW_WAVE) {
        // Grid (row waves, layers): the layer is the block's y. The wave's
        // first unit is a multiple of 8 and H a power of two >= 8, so its 8
        // units are 8 heads of one row. The layer's operands come from the
        // argument block at a uniform index (scalar loads).
        l = blockIdx.y;
        const uint32_t unit0 = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) >> 3 & ~7u);
        t = unit0 >> log2H;
        h = (unit0 & (H - 1u)) + ((threadIdx.x & 63u) >> 3);
        l_rows = layers.rows[l];
        l_slots_a = (uint64_t)(uintptr_t)layers.slots[l];
        l_cache_a = (uint64_t)(uintptr_t)layers.cache[l];
    } else {
        const uint32_t unit = (blockIdx.x * blockDim.x + threadIdx.x) >> 3;
        if (unit >= total_units) return;  // whole 8-lane groups leave together
        h = unit & (H - 1u);
        const uint32_t rt = unit >> log2H;
        l = rt / rows;
        t = rt - l * rows;
        // The layers' operands, held in scalar registers and picked by
        // compares: indexing the argument arrays by a per-lane l would be a
        // memory load, one more round trip ahead of the row's own loads. The
        // empty asm statements keep the compiler from folding the selection
        // back into such a load.
#pragma unroll
        for (uint32_t i = 0; i < (uint32_t)kMaxLayersPerLaunch; ++i) {
            uint32_t ri = layers.rows[i];
            uint64_t si = (uint64_t)(uintptr_t)layers.slots[i];
            uint64_t ci = (uint64_t)(uintptr_t)layers.cache[i];
            asm volatile("" : "+s"(ri), "+s"(si), "+s"(ci));
            if (l == i) {
                l_rows = ri;
                l_slots_a = si;
                l_cache_a = ci;
            }
        }
    }
    // Past this layer's slot list, a layer without one, or (row waves) past
    // the grid's last row: nothing to do.
    if (t >= l_rows) return;
    // The slot and the position (every row below rows has one) in one round
    // trip, tested together; K, V and the cos/sin row in a second.
    const int64_t slot = ((const GlobalI64*)l_slots_a)[t];  // a device allocation: global memory
    const int64_t pos = ROPE ? positions[t] : 0;
    // (bitwise &: both loads are needed before the one test)
    const bool slot_ok = (slot >= 0) & ((uint64_t)slot < (uint64_t)n_slots);
    const bool pos_ok = !ROPE || ((pos >= 0) & (pos < max_position));
    if (!(slot_ok & pos_ok)) return;

    const U32x4 kw = load16(k + (int64_t)l * k_ls + (int64_t)t * k_rs + h * kHeadDim + 8 * g);
    const U32x4 vw = load16(v + (int64_t)l * v_ls + (int64_t)t * v_rs + h * kHeadDim + 8 * g);
    uint2 cw = {0u, 0u}, sw = {0u, 0u};
    if constexpr (ROPE) {
        const uint16_t* cs = cos_sin + pos * kHeadDim;
        cw = *reinterpret_cast<const uint2*>(cs + 4 * g);                  // cos of pairs 4g .. 4g+3
        sw = *reinterpret_cast<const uint2*>(cs + kHeadDim / 2 + 4 * g);   // sin of the same pairs
    }
    const U32x4 out = k_out<ROPE>(kw, cw, sw, eps);

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
    // Non-temporal: the cache rows are scattered and not read back by this
    // chain, so they go out to HBM now instead of lingering dirty in the
    // caches until the next kernel's traffic evicts them. With one row per
    // wave the (block, page) base is wave-uniform and the heads lie within
    // head_span bytes of it (0: too far apart for a 32-bit offset), so the
    // stores take the buffer form at system scope, which streams faster.
    if (ROW_WAVE && head_span != 0) {
        const uint16_t* base = (const uint16_t*)l_cache_a + (int64_t)block * block_stride + (int64_t)page * page_stride;
        const uint32_t off = (uint32_t)((h * (uint64_t)head_stride + 8 * g) * 2);
        store16_stream(base, head_span, off, out);
        store16_stream(base, head_span, off + 2 * kHeadDim, vw);
    } else {
        GlobalU16* dst = (GlobalU16*)l_cache_a + (int64_t)block * block_stride + (int64_t)page * page_stride +
                         (int64_t)h * head_stride + 8 * g;
        store16_nt_global(dst, out);
        store16_nt_global(dst + kHeadDim, vw);
    }
}

// The split projection's last step and the store in one pass (page
// "...runtime.draft", ContextKV: the store reads the k/v views of the
// projection's own output, so it may take that output as it is formed): the FP32
// partial sums of the S slices [S, L, T, N] (slice stride ws_slice
// elements) are added in slice order and rounded to bf16 once - the same
// operations and order as the projection's adding kernel, so kv gets the
// same bits - and the result, written to kv [L, T, N], is at once the K or V
// row part that the store inserts. One 8-lane group per (layer, row,
// 64-wide column block c of the kv row): c < H is K head c, c >= H is V
// head c - H, so the groups of a wave cover contiguous kv columns. Every row
// of kv is written; rows at or past the layer's slot count, and rows whose
// slot or position is out of range, insert nothing.
template <int S, bool ROPE>
__global__ __launch_bounds__(256) void kv_sum_store_kernel(
    const float* __restrict__ ws, int64_t ws_slice, uint16_t* __restrict__ kv, uint32_t T, uint32_t H,
    uint32_t log2_cols, uint32_t total_units, const int64_t* __restrict__ positions,
    const uint16_t* __restrict__ cos_sin, int64_t max_position, StoreLayers layers, uint32_t block_size,
    int32_t bs_shift, uint32_t n_slots, int64_t block_stride, int64_t page_stride, int64_t head_stride, float eps) {
    const uint32_t unit = (blockIdx.x * blockDim.x + threadIdx.x) >> 3;
    if (unit >= total_units) return;  // whole 8-lane groups leave together
    const uint32_t g = threadIdx.x & 7u;
    const uint32_t c = unit & ((1u << log2_cols) - 1u);
    const uint32_t rt = unit >> log2_cols;  // l T + t
    const uint32_t l = rt / T, t = rt - l * T;
    uint32_t l_rows = 0;
    uint64_t l_slots_a = 0, l_cache_a = 0;
#pragma unroll
    for (uint32_t i = 0; i < (uint32_t)kMaxLayersPerLaunch; ++i) {
        uint32_t ri = layers.rows[i];
        uint64_t si = (uint64_t)(uintptr_t)layers.slots[i];
        uint64_t ci = (uint64_t)(uintptr_t)layers.cache[i];
        asm volatile("" : "+s"(ri), "+s"(si), "+s"(ci));
        if (l == i) {
            l_rows = ri;
            l_slots_a = si;
            l_cache_a = ci;
        }
    }
    const bool insert = t < l_rows;
    const bool is_k = c < H;
    int64_t slot = -1, pos = 0;
    if (insert) {
        slot = ((const GlobalI64*)l_slots_a)[t];
        if constexpr (ROPE) pos = positions[t];
    }
    const int64_t off = (int64_t)rt * ((int64_t)kHeadDim << log2_cols) + c * kHeadDim + 8 * g;
    U32x4 lo[S], hi[S];
#pragma unroll
    for (int k = 0; k < S; ++k) {
        lo[k] = load16(ws + (int64_t)k * ws_slice + off);
        hi[k] = load16(ws + (int64_t)k * ws_slice + off + 4);
    }
    const bool slot_ok = (slot >= 0) & ((uint64_t)slot < (uint64_t)n_slots);
    const bool pos_ok = !ROPE || ((pos >= 0) & (pos < max_position));
    const bool store_row = insert & slot_ok & pos_ok;
    // the cos/sin row of an inserted K head, fetched while the sums are in flight
    uint2 cw = {0u, 0u}, sw = {0u, 0u};
    if (ROPE && is_k && store_row) {
        const uint16_t* cs = cos_sin + pos * kHeadDim;
        cw = *reinterpret_cast<const uint2*>(cs + 4 * g);
        sw = *reinterpret_cast<const uint2*>(cs + kHeadDim / 2 + 4 * g);
    }
    float acc[8] = {__uint_as_float(lo[0].x), __uint_as_float(lo[0].y), __uint_as_float(lo[0].z),
                    __uint_as_float(lo[0].w), __uint_as_float(hi[0].x), __uint_as_float(hi[0].y),
                    __uint_as_float(hi[0].z), __uint_as_float(hi[0].w)};
#pragma unroll
    for (int k = 1; k < S; ++k) {
        const uint32_t p[8] = {lo[k].x, lo[k].y, lo[k].z, lo[k].w, hi[k].x, hi[k].y, hi[k].z, hi[k].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] + __uint_as_float(p[e]);
    }
    const U32x4 w{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]), pack_bf16(acc[4], acc[5]),
                  pack_bf16(acc[6], acc[7])};
    store16(kv + off, w);

    if (!store_row) return;
    const uint32_t s32 = (uint32_t)slot;
    uint32_t block, page;
    if (bs_shift >= 0) {
        block = s32 >> bs_shift;
        page = s32 & (block_size - 1u);
    } else {
        block = s32 / block_size;
        page = s32 - block * block_size;
    }
    const uint32_t h = is_k ? c : c - H;
    GlobalU16* dst = (GlobalU16*)l_cache_a + (int64_t)block * block_stride + (int64_t)page * page_stride +
                     (int64_t)h * head_stride + 8 * g;
    if (is_k) {
        store16_nt_global(dst, k_out<ROPE>(w, cw, sw, eps));
    } else {
        store16_nt_global(dst + kHeadDim, w);
    }
}

template <int S>
void launch_sum_store_s(const KvStoreArgs& a, hipStream_t stream) {
    uint32_t log2_cols = 0;
    while ((1u << log2_cols) != 2 * a.H) ++log2_cols;
    const uint32_t total_units = a.layers_in_launch * a.T * 2 * a.H;
    const dim3 grid((uint32_t)(((uint64_t)total_units * 8 + 255) / 256));
    auto kernel = a.cos_sin ? kv_sum_store_kernel<S, true> : kv_sum_store_kernel<S, false>;
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, a.ws, a.ws_slice, a.kv, a.T, a.H, log2_cols, total_units,
                       a.positions, a.cos_sin, a.max_position, a.layers, a.block_size, a.bs_shift, a.n_slots,
                       a.block_stride, a.page_stride, a.head_stride, a.eps);
}

template <bool ROPE>
void launch_rope(const KvStoreArgs& a, uint32_t total_units, hipStream_t stream) {
    const uint32_t threads = 256;
    dim3 grid;
    if (a.H >= 8) {
        // one wave per 8 heads of a row: rows * H / 8 waves per layer, 4 per block
        const uint64_t waves = (uint64_t)a.rows * a.H / 8;
        grid = dim3((uint32_t)((waves + 3) / 4), a.layers_in_launch);
    } else {
        grid = dim3((uint32_t)(((uint64_t)total_units * 8 + threads - 1) / threads));
    }
    auto kernel = a.H >= 8 ? kv_store_kernel<ROPE, true> : kv_store_kernel<ROPE, false>;
    // bytes from a row's (block, page) base to the end of its last head's run
    const uint64_t span = ((uint64_t)(a.H - 1) * (uint64_t)a.head_stride + 2 * kHeadDim) * 2;
    const uint32_t head_span = span < (1ull << 31) ? (uint32_t)span : 0u;
    hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, stream, a.k, a.v, a.k_ls, a.k_rs, a.v_ls, a.v_rs, a.positions,
                       a.cos_sin, a.max_position, a.layers, a.rows, a.H, a.log2H, total_units, a.block_size,
                       a.bs_shift, a.n_slots, a.block_stride, a.page_stride, a.head_stride, a.eps, head_span);
}

int launch_kv_store(const KvStoreArgs& a, hipStream_t stream) {
    if (a.ws) {
        switch (a.k_split) {
            case 2: launch_sum_store_s<2>(a, stream); break;
            case 4: launch_sum_store_s<4>(a, stream); break;
            case 8: launch_sum_store_s<8>(a, stream); break;
            case 16: launch_sum_store_s<16>(a, stream); break;
            default: return -1;
        }
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    const uint32_t total_units = (uint32_t)a.layers_in_launch * a.rows * a.H;
    if (a.cos_sin)
        launch_rope<true>(a, total_units, stream);
    else
        launch_rope<false>(a, total_units, stream);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nrc
