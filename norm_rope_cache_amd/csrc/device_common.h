// Device helpers shared by the libnrc kernels (gfx950 / CDNA4, wave64).
//
// Arithmetic contract (matches the chain as the vLLM context page's kernels
// state it, with correctly rounded operations in place of the approximate
// reciprocal square root):
//   - every FP32 op rounds to nearest even; FMA only where written
//     (__builtin_fmaf); the library builds with -ffp-contract=off;
//   - f32 subnormals are kept (no flush-to-zero);
//   - 1/sqrt(v) is a correctly rounded sqrt followed by a correctly rounded
//     divide;
//   - f32 -> bf16 rounds to nearest even on the bit pattern; every NaN
//     becomes 0x7FC0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nrc {

constexpr int kHidden = 8192;
constexpr int kHeadDim = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// f32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC0u : r;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) { return to_bf16(lo) | (to_bf16(hi) << 16); }

// 1/sqrt(v): llvm.sqrt.f32 and fdiv without fast-math flags lower to the
// correctly rounded gfx9 sequences (checked exhaustively by the GPU tests).
__device__ __forceinline__ float rsqrt_rn(float v) { return 1.0f / __builtin_sqrtf(v); }

// Cross-lane exchange inside a wave64 (value of lane ^ MASK). MASK 1 and 2
// use DPP quad permutes, MASK 4/8/16 a ds_swizzle xor pattern (within 32
// lanes), MASK 32 a bpermute.
template <int MASK>
__device__ __forceinline__ float lane_xor(float v) {
    int x = __float_as_int(v);
    if constexpr (MASK == 1) {
        x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
    } else if constexpr (MASK == 2) {
        x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
    } else if constexpr (MASK == 4 || MASK == 8 || MASK == 16) {
        x = __builtin_amdgcn_ds_swizzle(x, (MASK << 10) | 0x1F);  // bitmask mode: and 0x1F, xor MASK
    } else {
        static_assert(MASK == 32, "lane_xor: mask 1, 2, 4, 8, 16 or 32");
        x = __builtin_amdgcn_ds_bpermute((int)((__lane_id() ^ 32u) << 2), x);
    }
    return __int_as_float(x);
}

// Fold by halves over the 64 lanes of a wave (strides 32, 16, 8, 4, 2, 1);
// IEEE addition commutes, so both lanes of each pair hold the same sum and
// every lane ends with the fold's value.
__device__ __forceinline__ float wave_fold64(float v) {
    v = v + lane_xor<32>(v);
    v = v + lane_xor<16>(v);
    v = v + lane_xor<8>(v);
    v = v + lane_xor<4>(v);
    v = v + lane_xor<2>(v);
    v = v + lane_xor<1>(v);
    return v;
}

struct alignas(16) U32x4 {
    uint32_t x, y, z, w;
};

// Two f32 -> packed bf16 with one v_cvt_pk_bf16_f32 (round to nearest even,
// subnormals kept). Only for values that cannot be NaN: the hardware's NaN
// encoding is not 0x7FC0 (pack_bf16 handles those).
typedef float nrc_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 nrc_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16_pair_hw(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((nrc_f32x2){lo, hi}, nrc_bf16x2));
}

// (w + 0.0) on packed bf16 weights: a -0.0 weight becomes +0.0, all others
// are unchanged.
__device__ __forceinline__ uint32_t plus_zero_pair16(uint32_t w) {
    if ((w & 0xFFFFu) == 0x8000u) w &= 0xFFFF0000u;
    if ((w >> 16) == 0x8000u) w &= 0x0000FFFFu;
    return w;
}
__device__ __forceinline__ U32x4 plus_zero16(U32x4 w) {
    return U32x4{plus_zero_pair16(w.x), plus_zero_pair16(w.y), plus_zero_pair16(w.z), plus_zero_pair16(w.w)};
}

__device__ __forceinline__ U32x4 load16(const void* p) {
    return *reinterpret_cast<const U32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, U32x4 v) { *reinterpret_cast<U32x4*>(p) = v; }

__device__ __forceinline__ U32x4 load16_nt(const void* p) {
    const U32x4* q = reinterpret_cast<const U32x4*>(p);
    U32x4 v;
    v.x = __builtin_nontemporal_load(&q->x);
    v.y = __builtin_nontemporal_load(&q->y);
    v.z = __builtin_nontemporal_load(&q->z);
    v.w = __builtin_nontemporal_load(&q->w);
    return v;
}

// 16 bytes at byte offset `off` of a wave-uniform run of `bytes` bytes,
// written non-temporally at system scope (buffer store with nt sc1). On this
// chip that streams faster than a plain non-temporal store (61 against 56%
// of HBM peak, 1 GiB written) and, like it, leaves no dirty lines behind for
// the next kernel to write back (a plain store writes at 72% but slows the
// next 1 GiB read from 78 to 57%). `base` must be the same in every lane.
__device__ __forceinline__ void store16_stream(const void* base, uint32_t bytes, uint32_t off, U32x4 v) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                                                       0x00020000);
    const i32x4 t = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    __builtin_amdgcn_raw_buffer_store_b128(t, r, (int)off, 0, 18);  // cache policy: nt (2) | sc1 (16)
}

__device__ __forceinline__ void store16_nt(void* p, U32x4 v) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(p));
}

}  // namespace nrc
