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
// the hidden norm and the layer-norm sum for every layer): each 256-thread
// slot of a 1024-thread workgroup normalises a row once and writes all L
// layer outputs from the same registers. Every layer norm shares eps and
// center (the runtime page's ContextKV takes one set for all layers), and
// with the weight applied after the norm the layer-norm sum does not depend
// on the layer, so one sum per row serves all layers (identical bits). Rows
// whose sums, scales and weights are finite convert with the paired hardware
// instruction; others with the exact bit-pattern rounding.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace nrc {

namespace {

constexpr int kThreads = 256;
constexpr int kFrags = 4;
constexpr int kChunk = 2048;  // kThreads * 8

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

// Two f32 -> packed bf16 with one v_cvt_pk_bf16_f32 (round to nearest even;
// subnormals kept). Used only where neither value can be NaN: the hardware's
// NaN encoding is not the library's 0x7FC0, so rows that may hold NaN take
// pack_bf16 (exact bit-pattern rounding) instead.
__device__ __forceinline__ uint32_t pack_bf16_fast(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// -0.0 weights become +0.0: (w + 0.0) for a bf16 weight, kept as bf16 bits.
__device__ __forceinline__ uint32_t plus_zero_pair(uint32_t w) {
    if ((w & 0xFFFFu) == 0x8000u) w &= 0xFFFF0000u;
    if ((w >> 16) == 0x8000u) w &= 0x0000FFFFu;
    return w;
}
__device__ __forceinline__ U32x4 plus_zero(U32x4 w) {
    return U32x4{plus_zero_pair(w.x), plus_zero_pair(w.y), plus_zero_pair(w.z), plus_zero_pair(w.w)};
}

// Every bf16 weight of the fragment is finite.
__device__ __forceinline__ bool finite_pair(uint32_t w) {
    return (w & 0x7F80u) != 0x7F80u && (w & 0x7F800000u) != 0x7F800000u;
}
__device__ __forceinline__ bool finite8(const U32x4& w) {
    return finite_pair(w.x) && finite_pair(w.y) && finite_pair(w.z) && finite_pair(w.w);
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

__device__ __forceinline__ bool finite(float v) { return __builtin_fabsf(v) < __builtin_huge_valf(); }

// Every gain w + center (FP32 add) of the eight bf16 weights is finite.
__device__ __forceinline__ bool gains_finite8(const U32x4& w, float center) {
    const uint32_t p[4] = {w.x, w.y, w.z, w.w};
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) ok = ok && finite(bf16_lo(p[i]) + center) && finite(bf16_hi(p[i]) + center);
    return ok;
}

constexpr int kSlots = 4;                  // rows in flight per workgroup (one per 256 threads)
constexpr int kBlockThreads = kSlots * kThreads;
constexpr int kRowBytes = kHidden * 2;     // 16 KiB of bf16 weights per norm

// One workgroup = 4 row slots of 256 threads; every slot walks its own rows
// (row = 4 b + slot, then + 4 gridDim) and all slots take the same number
// of steps, so the workgroup barriers of the row sums line up (a slot past
// the last row idles through them). The norm weights are staged once per
// workgroup in LDS as packed bf16 (hidden first, then each layer), so the
// registers hold only the row in flight and its prefetched successor.
//
// WEIGHTS_IN_LDS: the layer weights are staged in LDS (up to 5 layers);
// otherwise they are read from memory per row (L2-resident).
// ADD_CENTER: gamma = w + center with an FP32 add per use; otherwise both
// centers are +-0.0 and the add is folded into the staged weights (a -0.0
// weight turns into +0.0 when its center is +0.0, the only case where
// w + center differs from w).
//
// PREPASS: instead of the L layer outputs, write the two per-row quantities
// the layer norms share - h_out [T, 8192], the hidden norm's bf16 output, and
// r_out [T], the layer-norm scale 1/sqrt(S_p/8192 + eps) - for a projection
// that applies the layer weights itself. r_out's sign bit marks a row whose
// layer outputs may be NaN (non-finite sum or scale, or a non-finite layer
// weight or center), which must take the exact bf16 rounding.
template <bool WEIGHTS_IN_LDS, bool HW, bool PW, bool ADD_CENTER, bool PREPASS>
__global__ __launch_bounds__(kBlockThreads) void context_norms_kernel(
    const uint16_t* __restrict__ x, int64_t T, const uint16_t* __restrict__ hidden_w,
    const uint16_t* __restrict__ pre_w, int32_t L, float hidden_eps, float pre_eps, float hidden_center,
    float pre_center, uint16_t* __restrict__ out, uint16_t* __restrict__ h_out, float* __restrict__ r_out) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ float sums[kSlots][2][4];
    const int tid = threadIdx.x;
    const int slot = __builtin_amdgcn_readfirstlane(tid >> 8);  // a slot is four whole waves
    const int t = tid & (kThreads - 1);
    const int col0 = 8 * t;
    const bool fix_h = !ADD_CENTER && !__builtin_signbit(hidden_center);
    const bool fix_p = !ADD_CENTER && !__builtin_signbit(pre_center);

    // ---- stage the weights (16-byte chunks, every thread a share) and check
    // that every gain is finite (the fast bf16 conversion relies on it; with
    // a center the check is on w + center, which can overflow).
    bool wfinite = true;
    U32x4* wl = reinterpret_cast<U32x4*>(smem);
    const int hw_chunks = HW ? kRowBytes / 16 : 0;
    const int pw_chunks = (PW && WEIGHTS_IN_LDS) ? L * (kRowBytes / 16) : 0;
    for (int c = tid; c < hw_chunks + pw_chunks; c += kBlockThreads) {
        U32x4 w;
        if (c < hw_chunks) {
            w = load16(hidden_w + 8 * c);
            if (fix_h) w = plus_zero(w);
        } else {
            w = load16(pre_w + 8 * (c - hw_chunks));
            if (fix_p) w = plus_zero(w);
        }
        wfinite = wfinite && (ADD_CENTER ? gains_finite8(w, c < hw_chunks ? hidden_center : pre_center) : finite8(w));
        wl[c] = w;
    }
    bool pfinite = true;  // layer gains finite
    if constexpr (PW && !WEIGHTS_IN_LDS) {
        for (int c = tid; c < L * (kRowBytes / 16); c += kBlockThreads) {
            const U32x4 w = load16(pre_w + 8 * c);
            pfinite = pfinite && (ADD_CENTER ? gains_finite8(w, pre_center) : finite8(w));
        }
    }
    if constexpr (PREPASS) {
        // the hidden conversion needs only the hidden weights finite
        wfinite = __syncthreads_and(wfinite) != 0;
        pfinite = __syncthreads_and(pfinite) != 0;
    } else {
        wfinite = __syncthreads_and(wfinite && pfinite) != 0;
    }
    const U32x4* gh = wl + (col0 >> 3);                    // chunk (col0 + 2048 k) / 8
    const U32x4* gp = wl + hw_chunks + (col0 >> 3);

    auto row_sum = [&](float lane_part, float* slot_sums) {
        const float w = wave_fold64(lane_part);
        if (__lane_id() == 0) slot_sums[(tid >> 6) & 3] = w;
        __syncthreads();
        return (slot_sums[0] + slot_sums[2]) + (slot_sums[1] + slot_sums[3]);
    };

    const int64_t stride = (int64_t)gridDim.x * kSlots;
    int64_t row = (int64_t)blockIdx.x * kSlots + slot;
    U32x4 xv[kFrags];
    if (row < T) {
#pragma unroll
        for (int k = 0; k < kFrags; ++k) xv[k] = load16(x + row * kHidden + col0 + k * kChunk);
    }
    for (int64_t base = (int64_t)blockIdx.x * kSlots; base < T; base += stride, row += stride) {
        const bool active = row < T;
        float u[kFrags][8];
#pragma unroll
        for (int k = 0; k < kFrags; ++k) unpack8(xv[k], u[k]);
        if (!active) {
#pragma unroll
            for (int k = 0; k < kFrags; ++k)
#pragma unroll
                for (int i = 0; i < 8; ++i) u[k][i] = 0.0f;
        }
        // Prefetch the next row while this one is normalised and written.
        const int64_t next = row + stride;
        if (next < T) {
#pragma unroll
            for (int k = 0; k < kFrags; ++k) xv[k] = load16(x + next * kHidden + col0 + k * kChunk);
        }

        // Hidden norm, rounded to bf16. With a finite sum, a finite r and
        // finite weights no product is NaN (|x r| <= sqrt(8192)), so the
        // paired hardware conversion gives the same bits.
        const float Sh = row_sum(lane_sumsq(u), sums[slot][0]);
        const float rh = rsqrt_rn(__builtin_fmaf(Sh, 0x1p-13f, hidden_eps));
        const bool fast_h = wfinite && finite(Sh) && finite(rh);
        auto hidden = [&](auto fast) {
#pragma unroll
            for (int k = 0; k < kFrags; ++k) {
                float g[8];
                if constexpr (HW) unpack8(gh[k * (kChunk / 8)], g);
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    float y0 = u[k][2 * p] * rh, y1 = u[k][2 * p + 1] * rh;
                    if constexpr (HW) {
                        y0 = y0 * (ADD_CENTER ? g[2 * p] + hidden_center : g[2 * p]);
                        y1 = y1 * (ADD_CENTER ? g[2 * p + 1] + hidden_center : g[2 * p + 1]);
                    }
                    const uint32_t w = decltype(fast)::value ? pack_bf16_fast(y0, y1) : pack_bf16(y0, y1);
                    u[k][2 * p] = bf16_lo(w);
                    u[k][2 * p + 1] = bf16_hi(w);
                }
            }
        };
        if (fast_h)
            hidden(std::true_type{});
        else
            hidden(std::false_type{});

        // One layer-norm sum for all layers (every layer norm shares eps and
        // center, and the weight applies after the norm).
        const float Sp = row_sum(lane_sumsq(u), sums[slot][1]);
        const float rp = rsqrt_rn(__builtin_fmaf(Sp, 0x1p-13f, pre_eps));
        if constexpr (PREPASS) {
            if (active) {
                uint16_t* o = h_out + row * kHidden + col0;
#pragma unroll
                for (int k = 0; k < kFrags; ++k) {
                    uint32_t w[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        w[p] = (__float_as_uint(u[k][2 * p]) >> 16) | (__float_as_uint(u[k][2 * p + 1]) & 0xFFFF0000u);
                    store16(o + k * kChunk, U32x4{w[0], w[1], w[2], w[3]});
                }
                if (t == 0) {
                    const bool ok = pfinite && finite(Sp) && finite(rp);
                    r_out[row] = ok ? rp : __uint_as_float(__float_as_uint(rp) | 0x80000000u);
                }
            }
            continue;
        }
        // The layer outputs take the paired conversion whenever Sp and rp are
        // finite, however the hidden norm was rounded: a NaN or infinite h
        // makes Sp NaN or infinite, so with a finite Sp every h is finite,
        // |h rp| stays within about sqrt(8192), and with finite gains no
        // product is NaN (a row whose hidden sum overflows has h = +-0 and
        // still takes this path for all L outputs).
        const bool fast_p = wfinite && finite(Sp) && finite(rp);
#pragma unroll
        for (int k = 0; k < kFrags; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i) u[k][i] = u[k][i] * rp;

        auto layer_out = [&](int l, auto fast) {
            const uint16_t* orow = out + ((int64_t)l * T + row) * kHidden;  // the same in every lane of the wave
#pragma unroll
            for (int k = 0; k < kFrags; ++k) {
                uint32_t w[4];
                float g[8];
                if constexpr (PW) {
                    U32x4 gw;
                    if constexpr (WEIGHTS_IN_LDS) {
                        gw = gp[l * (kRowBytes / 16) + k * (kChunk / 8)];
                    } else {
                        gw = load16(pre_w + (int64_t)l * kHidden + col0 + k * kChunk);
                        if (fix_p) gw = plus_zero(gw);
                    }
                    unpack8(gw, g);
                    if constexpr (ADD_CENTER) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) g[i] = g[i] + pre_center;
                    }
                }
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    float a = u[k][2 * p], b = u[k][2 * p + 1];
                    if constexpr (PW) {
                        a = a * g[2 * p];
                        b = b * g[2 * p + 1];
                    }
                    w[p] = decltype(fast)::value ? pack_bf16_fast(a, b) : pack_bf16(a, b);
                }
                store16_stream(orow, kRowBytes, (uint32_t)(col0 + k * kChunk) * 2, U32x4{w[0], w[1], w[2], w[3]});
            }
        };
        if (active) {
            if (fast_p) {
                for (int l = 0; l < L; ++l) layer_out(l, std::true_type{});
            } else {
                for (int l = 0; l < L; ++l) layer_out(l, std::false_type{});
            }
        }
    }
}

template <bool WEIGHTS_IN_LDS, bool ADD_CENTER, bool PREPASS>
void launch_w(const NormsArgs& a, dim3 grid, size_t lds, uint16_t* h_out, float* r_out, hipStream_t stream) {
    const bool hw = a.hidden_w != nullptr, pw = a.pre_w != nullptr;
#define NRC_NORMS_LAUNCH(H, P)                                                                                \
    hipLaunchKernelGGL((context_norms_kernel<WEIGHTS_IN_LDS, H, P, ADD_CENTER, PREPASS>), grid,                 \
                       dim3(kBlockThreads), lds, stream, a.x, a.T, a.hidden_w, a.pre_w, a.L, a.hidden_eps,      \
                       a.pre_eps, a.hidden_center, a.pre_center, a.out, h_out, r_out)
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

template <bool WEIGHTS_IN_LDS, bool ADD_CENTER, bool PREPASS>
int set_lds_limit() {
    static std::atomic<int> done[4][64] = {};
    const void* fns[4] = {(const void*)context_norms_kernel<WEIGHTS_IN_LDS, true, true, ADD_CENTER, PREPASS>,
                          (const void*)context_norms_kernel<WEIGHTS_IN_LDS, true, false, ADD_CENTER, PREPASS>,
                          (const void*)context_norms_kernel<WEIGHTS_IN_LDS, false, true, ADD_CENTER, PREPASS>,
                          (const void*)context_norms_kernel<WEIGHTS_IN_LDS, false, false, ADD_CENTER, PREPASS>};
    for (int i = 0; i < 4; ++i)
        if (raise_lds_limit(fns[i], 9 * kRowBytes, done[i])) return -1;
    return 0;
}

dim3 norms_grid(const NormsArgs& a, size_t lds) {
    // Workgroups resident per CU: LDS (160 KiB) and the 1024-thread size allow
    // one or two; rows beyond the grid are walked with a grid stride.
    const int64_t per_cu = lds <= 64 * 1024 ? 2 : 1;
    const int64_t groups = (a.T + kSlots - 1) / kSlots;
    const int64_t max_blocks = (int64_t)(a.num_cus > 0 ? a.num_cus : 256) * per_cu;
    return dim3((unsigned)(groups < max_blocks ? groups : max_blocks));
}

}  // namespace

int launch_context_norms(const NormsArgs& a, hipStream_t stream) {
    // Layer weights staged in LDS up to 5 layers; beyond, each row reads them
    // from L2 and the workgroup stages only the hidden weight, so two
    // workgroups share a CU instead of one (cold launches, same bits: edge
    // workload, L = 8, 1016 -> 922 us; the long workload's rows at L = 6 and
    // 8, 2% faster; at L = 5 1% slower, so 5 keeps LDS).
    const bool in_lds = a.L <= 5;
    const size_t lds = (size_t)((a.hidden_w ? 1 : 0) + (a.pre_w && in_lds ? a.L : 0)) * kRowBytes;
    const dim3 grid = norms_grid(a, lds);
    // A center of exactly +0.0 or -0.0 folds into the bf16 weights.
    const bool zero_centers = a.hidden_center == 0.0f && a.pre_center == 0.0f;
    int rc;
    if (in_lds) {
        if (zero_centers) {
            if ((rc = set_lds_limit<true, false, false>())) return rc;
            launch_w<true, false, false>(a, grid, lds, nullptr, nullptr, stream);
        } else {
            if ((rc = set_lds_limit<true, true, false>())) return rc;
            launch_w<true, true, false>(a, grid, lds, nullptr, nullptr, stream);
        }
    } else {
        if (zero_centers)
            launch_w<false, false, false>(a, grid, lds, nullptr, nullptr, stream);
        else
            launch_w<false, true, false>(a, grid, lds, nullptr, nullptr, stream);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_hidden_norm(const NormsArgs& a, uint16_t* h_out, float* r_out, hipStream_t stream) {
    const size_t lds = (size_t)(a.hidden_w ? 1 : 0) * kRowBytes;
    const dim3 grid = norms_grid(a, lds);
    const bool zero_centers = a.hidden_center == 0.0f && a.pre_center == 0.0f;
    if (zero_centers)
        launch_w<false, false, true>(a, grid, lds, h_out, r_out, stream);
    else
        launch_w<false, true, true>(a, grid, lds, h_out, r_out, stream);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nrc
