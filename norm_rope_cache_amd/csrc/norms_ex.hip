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
// 64-lane fold per wave, then (W0 + W2) + (W1 + W3)). Every conversion to
// bf16 gives the bits of the exact round-to-nearest-even rounding with NaN as
// 0x7FC0. The plain form (bf16 or no weights on the outputs) takes the
// kernel of context_norms.hip instead.
//
// Main kernel (layer weights up to 128 KiB): like context_norms.hip, row
// slots of 256 threads, each prefetching its next row - two per 512-thread
// workgroup, so that the hidden gain (w + center), held in each thread's
// registers for its 32 columns, fits without spilling. The layer weights are
// staged in LDS once per workgroup: as FP32 gains w + center when they fit
// (split into two 16-byte planes so that a wave's reads cover all banks),
// else as the stored bf16. Input-scaled layer norms post all L per-layer
// sums behind one barrier. Rows whose sums, scales and gains are finite
// convert with the paired hardware instruction (no product can be NaN
// there); others with the exact bit-pattern rounding.
// Fallback (FP32 layer weights beyond 4 layers): one 256-thread workgroup
// per row, weights read from memory (L2) for every row.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace nrc {

namespace {

constexpr int kThreads = 256;
constexpr int kFrags = 4;
constexpr uint32_t kRowBytesOut = 8192 * 2;  // one bf16 output row
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
            const uint16_t* orow = out + ((int64_t)l * T + row) * kHidden;  // one row per workgroup
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
                store16_stream(orow, kRowBytesOut, (uint32_t)(col0 + k * kChunk) * 2,
                               U32x4{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]),
                                     pack_bf16(y[6], y[7])});
            }
        }
    }
}

constexpr int kSlots = 2;
constexpr int kBlockThreads = kSlots * kThreads;
constexpr int kLayerLds = 128 * 1024;  // layer weights staged in LDS up to this size
constexpr int kMaxLdsLayers = kLayerLds / (kHidden * 2);

__device__ __forceinline__ bool finite(float v) { return __builtin_fabsf(v) < __builtin_huge_valf(); }

// HK: hidden weight kind (0 none, 1 bf16, 2 FP32). LF: layer weights in
// LDS as 0 - none; 1 - the stored bf16 (center added at use); 2 - FP32 gains
// w + center, computed once when staged from bf16 or FP32 (pre_kind).
template <int HK, int LF>
__global__ __launch_bounds__(kBlockThreads) void norms_ex_lds_kernel(
    const uint16_t* __restrict__ x, int64_t T, const void* __restrict__ hidden_w, const void* __restrict__ pre_w,
    int32_t pre_kind, int32_t L, float hidden_eps, float pre_eps, float hidden_center, float pre_center,
    bool hidden_in, bool pre_in, uint16_t* __restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ float sums[kSlots][1 + kMaxLdsLayers][4];
    const int tid = threadIdx.x;
    const int slot = __builtin_amdgcn_readfirstlane(tid >> 8);  // a slot is four whole waves
    const int t = tid & (kThreads - 1);
    const int wv = t >> 6;  // wave within the slot
    const int col0 = 8 * t;
    const bool scale_h_in = HK != 0 && hidden_in;
    const bool per_layer = LF != 0 && pre_in;

    // ---- hidden gains in registers, layer weights into LDS. The hardware
    // conversion needs every gain finite (a gain that overflows to infinity
    // times a zero is NaN), so finiteness is checked on w + center.
    bool wfinite = true;
    float gh[kFrags][8];
    if constexpr (HK != 0) {
#pragma unroll
        for (int k = 0; k < kFrags; ++k) {
            load_gamma8<HK>(hidden_w, col0 + k * kChunk, hidden_center, gh[k]);
#pragma unroll
            for (int i = 0; i < 8; ++i) wfinite = wfinite && finite(gh[k][i]);
        }
    }
    // LF 1: layer l's row at l * 16 KiB, chunk c (columns 8c .. 8c + 7) at
    // 16 c. LF 2: layer l at l * 32 KiB, gains of columns 8c .. 8c + 3 at
    // 16 c of the first 16 KiB plane, 8c + 4 .. 8c + 7 at 16 c of the second.
    if constexpr (LF == 1) {
        const U32x4* src = static_cast<const U32x4*>(pre_w);
        U32x4* dst = reinterpret_cast<U32x4*>(smem);
        for (int c = tid; c < L * (kHidden / 8); c += kBlockThreads) {
            const U32x4 w = src[c];
            const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wfinite = wfinite && finite(bf16_lo(p[i]) + pre_center) && finite(bf16_hi(p[i]) + pre_center);
            dst[c] = w;
        }
    } else if constexpr (LF == 2) {
        U32x4* dst = reinterpret_cast<U32x4*>(smem);
        for (int j = tid; j < L * (kHidden / 4); j += kBlockThreads) {
            float g[4];
            if (pre_kind == 2) {
                const U32x4 w = static_cast<const U32x4*>(pre_w)[j];
                g[0] = __uint_as_float(w.x);
                g[1] = __uint_as_float(w.y);
                g[2] = __uint_as_float(w.z);
                g[3] = __uint_as_float(w.w);
            } else {
                const uint2 w = static_cast<const uint2*>(pre_w)[j];
                g[0] = bf16_lo(w.x);
                g[1] = bf16_hi(w.x);
                g[2] = bf16_lo(w.y);
                g[3] = bf16_hi(w.y);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                g[i] = g[i] + pre_center;
                wfinite = wfinite && finite(g[i]);
            }
            const int l = j / (kHidden / 4), jj = j % (kHidden / 4);
            dst[l * (kHidden / 4) + (jj & 1) * (kHidden / 8) + (jj >> 1)] =
                U32x4{__float_as_uint(g[0]), __float_as_uint(g[1]), __float_as_uint(g[2]), __float_as_uint(g[3])};
        }
    }
    wfinite = __syncthreads_and(wfinite) != 0;

    // Layer l's eight gains (w + center) for this thread's fragment k.
    auto layer_gain = [&](int l, int k, float* g) {
        if constexpr (LF == 1) {
            const U32x4 w = reinterpret_cast<const U32x4*>(smem)[l * (kHidden / 8) + (col0 + k * kChunk) / 8];
            const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                g[2 * i] = bf16_lo(p[i]) + pre_center;
                g[2 * i + 1] = bf16_hi(p[i]) + pre_center;
            }
        } else if constexpr (LF == 2) {
            const U32x4* base = reinterpret_cast<const U32x4*>(smem) + l * (kHidden / 4) + (col0 + k * kChunk) / 8;
            const U32x4 a = base[0], b = base[kHidden / 8];
            const uint32_t p[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) g[i] = __uint_as_float(p[i]);
        }
    };
    auto post = [&](float lane_part, float* slot_sums) {
        const float w = wave_fold64(lane_part);
        if (__lane_id() == 0) slot_sums[wv] = w;
    };
    auto combine = [&](const float* s) { return (s[0] + s[2]) + (s[1] + s[3]); };

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
        for (int k = 0; k < kFrags; ++k) {
            const uint32_t p[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u[k][2 * i] = active ? bf16_lo(p[i]) : 0.0f;
                u[k][2 * i + 1] = active ? bf16_hi(p[i]) : 0.0f;
            }
        }
        const int64_t next = row + stride;
        if (next < T) {
#pragma unroll
            for (int k = 0; k < kFrags; ++k) xv[k] = load16(x + next * kHidden + col0 + k * kChunk);
        }

        // hidden norm, rounded to bf16
        if (HK != 0 && scale_h_in) {
#pragma unroll
            for (int k = 0; k < kFrags; ++k)
#pragma unroll
                for (int i = 0; i < 8; ++i) u[k][i] = gh[k][i] * u[k][i];
        }
        post(lane_sumsq(u), sums[slot][0]);
        __syncthreads();
        const float Sh = combine(sums[slot][0]);
        const float rh = rsqrt_rn(__builtin_fmaf(Sh, 0x1p-13f, hidden_eps));
        const bool fast_h = wfinite && finite(Sh) && finite(rh);
        // the hidden output is exact bf16: keep it packed through the layers
        uint32_t uh[kFrags][4];
        auto hidden_out = [&](auto fast) {
#pragma unroll
            for (int k = 0; k < kFrags; ++k)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    float y0 = u[k][2 * p] * rh, y1 = u[k][2 * p + 1] * rh;
                    if (HK != 0 && !scale_h_in) {
                        y0 = y0 * gh[k][2 * p];
                        y1 = y1 * gh[k][2 * p + 1];
                    }
                    uh[k][p] = decltype(fast)::value ? pack_bf16_pair_hw(y0, y1) : pack_bf16(y0, y1);
                }
        };
        if (fast_h)
            hidden_out(std::true_type{});
        else
            hidden_out(std::false_type{});
        auto hval = [&](int k, int i) { return (i & 1) ? bf16_hi(uh[k][i >> 1]) : bf16_lo(uh[k][i >> 1]); };

        // layer norms, one 8-column fragment at a time
        auto store_frag = [&](int l, int k, const float (&y)[8], auto fast) {
            uint32_t w[4];
#pragma unroll
            for (int p = 0; p < 4; ++p)
                w[p] = decltype(fast)::value ? pack_bf16_pair_hw(y[2 * p], y[2 * p + 1])
                                             : pack_bf16(y[2 * p], y[2 * p + 1]);
            store16_stream(out + ((int64_t)l * T + row) * kHidden, kRowBytesOut, (uint32_t)(col0 + k * kChunk) * 2,
                           U32x4{w[0], w[1], w[2], w[3]});
        };
        if (!per_layer) {
            // one layer-norm sum serves every layer: y = (u * rp) * gamma_l
            float even = 0.0f, odd = 0.0f;
#pragma unroll
            for (int k = 0; k < kFrags; ++k)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    even = __builtin_fmaf(hval(k, 2 * p), hval(k, 2 * p), even);
                    odd = __builtin_fmaf(hval(k, 2 * p + 1), hval(k, 2 * p + 1), odd);
                }
            post(even + odd, sums[slot][1]);
            __syncthreads();
            const float Sp = combine(sums[slot][1]);
            const float rp = rsqrt_rn(__builtin_fmaf(Sp, 0x1p-13f, pre_eps));
            // finite Sp: every h finite, whichever path rounded it (a NaN or
            // infinite h makes the sum NaN or infinite), so no product is NaN
            const bool fast_p = wfinite && finite(Sp) && finite(rp);
            auto layers_out = [&](auto fast) {
                for (int l = 0; l < L; ++l)
#pragma unroll
                    for (int k = 0; k < kFrags; ++k) {
                        float g[8], y[8];
                        layer_gain(l, k, g);
#pragma unroll
                        for (int i = 0; i < 8; ++i) y[i] = LF != 0 ? (hval(k, i) * rp) * g[i] : hval(k, i) * rp;
                        store_frag(l, k, y, fast);
                    }
            };
            if (active) {
                if (fast_p)
                    layers_out(std::true_type{});
                else
                    layers_out(std::false_type{});
            }
        } else {
            // v_l = gamma_l * u; every layer's sum posted before one barrier
            for (int l = 0; l < L; ++l) {
                float even = 0.0f, odd = 0.0f;
#pragma unroll
                for (int k = 0; k < kFrags; ++k) {
                    float g[8];
                    layer_gain(l, k, g);
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const float v0 = g[2 * p] * hval(k, 2 * p), v1 = g[2 * p + 1] * hval(k, 2 * p + 1);
                        even = __builtin_fmaf(v0, v0, even);
                        odd = __builtin_fmaf(v1, v1, odd);
                    }
                }
                post(even + odd, sums[slot][1 + l]);
            }
            __syncthreads();
            if (active) {
                for (int l = 0; l < L; ++l) {
                    const float Sl = combine(sums[slot][1 + l]);
                    const float rl = rsqrt_rn(__builtin_fmaf(Sl, 0x1p-13f, pre_eps));
                    auto layer_out = [&](auto fast) {
#pragma unroll
                        for (int k = 0; k < kFrags; ++k) {
                            float g[8], y[8];
                            layer_gain(l, k, g);
#pragma unroll
                            for (int i = 0; i < 8; ++i) y[i] = (g[i] * hval(k, i)) * rl;
                            store_frag(l, k, y, fast);
                        }
                    };
                    // finite Sl: every g h finite (one NaN or infinite
                    // product makes the sum NaN or infinite), whatever path
                    // rounded h
                    if (wfinite && finite(Sl) && finite(rl))
                        layer_out(std::true_type{});
                    else
                        layer_out(std::false_type{});
                }
            }
        }
    }
}

template <int HK, int LF>
int launch_lds(const NormsExArgs& a, hipStream_t stream) {
    const size_t lds = LF == 0 ? 0 : (size_t)a.L * kHidden * (LF == 2 ? 4 : 2);
    auto kernel = norms_ex_lds_kernel<HK, LF>;
    if (lds > 65536) {
        static std::atomic<int> done[64] = {};
        if (raise_lds_limit((const void*)kernel, (int)lds, done)) return -1;
    }
    // One workgroup per CU when the weights take more than half the LDS.
    const int64_t per_cu = lds <= 64 * 1024 ? 2 : 1;
    const int64_t groups = (a.T + kSlots - 1) / kSlots;
    const int64_t cap = (int64_t)(a.num_cus > 0 ? a.num_cus : 256) * per_cu;
    const unsigned grid = (unsigned)(groups < cap ? groups : cap);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kBlockThreads), lds, stream, a.x, a.T, a.hidden_w, a.pre_w,
                       a.pre_kind, a.L, a.hidden_eps, a.pre_eps, a.hidden_center, a.pre_center,
                       a.hidden_input_scale, a.pre_input_scale, a.out);
    return 0;
}

// Layer weights as FP32 gains when they fit (up to 4 layers), else stored bf16.
template <int HK>
int launch_lds_h(const NormsExArgs& a, hipStream_t stream) {
    if (a.pre_kind == 0) return launch_lds<HK, 0>(a, stream);
    if ((int64_t)a.L * kHidden * 4 <= kLayerLds) return launch_lds<HK, 2>(a, stream);
    return launch_lds<HK, 1>(a, stream);
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
    const int64_t layer_bytes = a.pre_kind == 0 ? 0 : (int64_t)a.L * kHidden * (a.pre_kind == 2 ? 4 : 2);
    if (layer_bytes <= kLayerLds) {
        int rc;
        if (a.hidden_kind == 0)
            rc = launch_lds_h<0>(a, stream);
        else if (a.hidden_kind == 1)
            rc = launch_lds_h<1>(a, stream);
        else
            rc = launch_lds_h<2>(a, stream);
        if (rc) return rc;
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    if (a.hidden_kind == 0)
        launch_h<0>(a, stream);
    else if (a.hidden_kind == 1)
        launch_h<1>(a, stream);
    else
        launch_h<2>(a, stream);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nrc
