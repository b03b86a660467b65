// Batched K/V projection C[l] = A[l] . B[l] on the gfx950 bf16 matrix cores.
//
// The vLLM page "...runtime.draft" (ContextKV._project) keeps this step a
// stock bmm of the stacked layer norms [L, T, D] against the stacked K/V
// weight; the logical right operand is [L, D, N] with N contiguous. Results
// are FP32 sums of exact bf16 products, rounded once to bf16.
//
// Kernel: one 256-thread workgroup (4 waves, 2 x 2) per BM x BN output tile
// of one layer, K walked in steps of 64 with double-buffered LDS.
//   - A tiles (K contiguous) go global -> registers -> LDS as 16-byte chunks.
//   - B tiles arrive N-contiguous; each thread loads an 8(k) x NPT(n) block
//     (one 8- or 16-byte load per k row), transposes it in registers and
//     writes NPT rows of 8 consecutive k, so both operands sit in LDS as
//     [row][k] with 16-byte k chunks, the layout v_mfma_f32_32x32x16_bf16
//     reads (8 consecutive k per lane).
//   - LDS rows are 128 bytes (64 k); chunk c of row r is stored at chunk
//     c ^ ((r ^ (r >> 3)) & 7), which keeps both the 16-byte writes and the
//     MFMA operand reads free of bank conflicts.
//   - Tiles are ordered layer, M tile, N tile (N fastest); consecutive tile
//     ids are assigned to the same XCD (workgroup ids are dealt round-robin
//     over the 8 XCDs), so the N tiles sharing an A panel meet in one L2.
#include "device_common.h"
#include "kernels.h"

namespace nrc {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBK = 64;       // K per LDS stage
constexpr int kRowChunks = 8; // 16-byte chunks per LDS row (64 bf16)

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// LDS address (in 16-byte units) of chunk c of row r.
__device__ __forceinline__ int lds_chunk(int r, int c) { return r * kRowChunks + (c ^ swz(r)); }

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

template <int BM, int BN>
struct Tile {
    static constexpr int MI = BM / 64;          // 32-row MFMA blocks per wave (wave tile BM/2 rows)
    static constexpr int NI = BN / 64;          // 32-col MFMA blocks per wave
    static constexpr int A_PER_THREAD = BM / 32;  // 16-byte A chunks per thread per stage
    static constexpr int NPT = BN / 32;         // B columns per thread (4 or 8)
    static constexpr int A_CHUNKS = BM * kRowChunks;
    static constexpr int B_CHUNKS = BN * kRowChunks;
    static constexpr int STAGE_CHUNKS = A_CHUNKS + B_CHUNKS;
};

template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void kv_project_kernel(const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ B,
                                                              uint16_t* __restrict__ C, int64_t M, int64_t K,
                                                              int64_t N, int32_t tiles_m, int32_t tiles_n,
                                                              int32_t total_tiles) {
    using TL = Tile<BM, BN>;
    extern __shared__ U32x4 lds[];  // 2 stages of [A rows | B rows]

    // XCD-aware tile id: workgroup b runs on XCD b % 8; give each XCD a
    // contiguous range of tiles.
    int tile = blockIdx.x;
    if ((total_tiles & 7) == 0) {
        const int per_xcd = total_tiles >> 3;
        tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    }
    const int tn = tile % tiles_n;
    const int tm = (tile / tiles_n) % tiles_m;
    const int layer = tile / (tiles_n * tiles_m);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;
    const uint16_t* Al = A + (int64_t)layer * M * K;
    const uint16_t* Bl = B + (int64_t)layer * K * N;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- global -> register staging assignments
    // A: chunk column a_c = tid % 8, rows tid / 8 + 32 i (rows past M clamp to M-1).
    const int a_c = tid & 7;
    const uint16_t* a_src[TL::A_PER_THREAD];
#pragma unroll
    for (int i = 0; i < TL::A_PER_THREAD; ++i) {
        int64_t r = m0 + (tid >> 3) + 32 * i;
        r = r < M ? r : M - 1;
        a_src[i] = Al + r * K + 8 * a_c;
    }
    // B: k rows 8 kb .. 8 kb + 7 of the stage, columns n0 + NPT nq .. + NPT.
    const int nq = tid & 31, kb = tid >> 5;
    const uint16_t* b_src = Bl + (int64_t)(8 * kb) * N + n0 + TL::NPT * nq;

    U32x4 a_reg[TL::A_PER_THREAD];
    U32x4 b_reg[8];  // NPT = 8: full 16 bytes; NPT = 4: x, y used

    auto load_stage = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < TL::A_PER_THREAD; ++i) a_reg[i] = load16(a_src[i] + k0);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const uint16_t* p = b_src + (k0 + r) * N;
            if constexpr (TL::NPT == 8) {
                b_reg[r] = load16(p);
            } else {
                const uint2 v = *reinterpret_cast<const uint2*>(p);
                b_reg[r] = U32x4{v.x, v.y, 0u, 0u};
            }
        }
    };

    auto store_stage = [&](int stage) {
        U32x4* sa = lds + stage * TL::STAGE_CHUNKS;
        U32x4* sb = sa + TL::A_CHUNKS;
#pragma unroll
        for (int i = 0; i < TL::A_PER_THREAD; ++i) sa[lds_chunk((tid >> 3) + 32 * i, a_c)] = a_reg[i];
        // Transpose the 8 x NPT block: column j collects k rows 0..7.
        const uint32_t* w[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) w[r] = &b_reg[r].x;
#pragma unroll
        for (int j = 0; j < TL::NPT; ++j) {
            U32x4 col;
            if ((j & 1) == 0) {
                col.x = lo_pair(w[0][j >> 1], w[1][j >> 1]);
                col.y = lo_pair(w[2][j >> 1], w[3][j >> 1]);
                col.z = lo_pair(w[4][j >> 1], w[5][j >> 1]);
                col.w = lo_pair(w[6][j >> 1], w[7][j >> 1]);
            } else {
                col.x = hi_pair(w[0][j >> 1], w[1][j >> 1]);
                col.y = hi_pair(w[2][j >> 1], w[3][j >> 1]);
                col.z = hi_pair(w[4][j >> 1], w[5][j >> 1]);
                col.w = hi_pair(w[6][j >> 1], w[7][j >> 1]);
            }
            sb[lds_chunk(TL::NPT * nq + j, kb)] = col;
        }
    };

    f32x16 acc[TL::MI][TL::NI];
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
#pragma unroll
        for (int j = 0; j < TL::NI; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int ksteps = (int)(K / kBK);
    load_stage(0);
    store_stage(0);
    __syncthreads();

    // MFMA operand rows of this lane.
    const int a_row0 = wm * (BM / 2) + (lane & 31);
    const int b_row0 = wn * (BN / 2) + (lane & 31);
    const int khalf = lane >> 5;  // lanes 32..63 hold k 8..15 of each 16-wide step

    for (int ks = 0; ks < ksteps; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < ksteps) load_stage((int64_t)(ks + 1) * kBK);
        const U32x4* sa = lds + cur * TL::STAGE_CHUNKS;
        const U32x4* sb = sa + TL::A_CHUNKS;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int chunk = 2 * kk + khalf;
            bf16x8 af[TL::MI], bfr[TL::NI];
#pragma unroll
            for (int i = 0; i < TL::MI; ++i) {
                const U32x4 t = sa[lds_chunk(a_row0 + 32 * i, chunk)];
                af[i] = __builtin_bit_cast(bf16x8, t);
            }
#pragma unroll
            for (int j = 0; j < TL::NI; ++j) {
                const U32x4 t = sb[lds_chunk(b_row0 + 32 * j, chunk)];
                bfr[j] = __builtin_bit_cast(bf16x8, t);
            }
#pragma unroll
            for (int i = 0; i < TL::MI; ++i)
#pragma unroll
                for (int j = 0; j < TL::NI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (ks + 1 < ksteps) store_stage(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: lane holds column (lane & 31) of each 32 x 32 block, rows
    // 8 (v / 4) + 4 (lane / 32) + (v % 4).
    uint16_t* Cl = C + (int64_t)layer * M * N;
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
#pragma unroll
        for (int j = 0; j < TL::NI; ++j) {
            const int64_t col = n0 + wn * (BN / 2) + 32 * j + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm * (BM / 2) + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < M) Cl[row * N + col] = (uint16_t)to_bf16(acc[i][j][v]);
            }
        }
}

template <int BM, int BN>
int launch_tiles(const ProjectArgs& a, hipStream_t stream) {
    using TL = Tile<BM, BN>;
    const int tiles_m = (int)((a.M + BM - 1) / BM);
    const int tiles_n = (int)(a.N / BN);
    const int total = a.L * tiles_m * tiles_n;
    const size_t lds_bytes = 2 * TL::STAGE_CHUNKS * sizeof(U32x4);
    if (lds_bytes > 65536) {
        // The opt-in above 64 KiB is per kernel and device; set it on each device once.
        static bool attr_set[64] = {};
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return -1;
        if (dev < 0 || dev >= 64) return -1;
        if (!attr_set[dev]) {
            if (hipFuncSetAttribute((const void*)kv_project_kernel<BM, BN>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes) != hipSuccess)
                return -1;
            attr_set[dev] = true;
        }
    }
    hipLaunchKernelGGL((kv_project_kernel<BM, BN>), dim3(total), dim3(kThreads), lds_bytes, stream, a.A, a.B, a.C,
                       a.M, a.K, a.N, tiles_m, tiles_n, total);
    return 0;
}

}  // namespace

int launch_kv_project(const ProjectArgs& a, hipStream_t stream) {
    // 256 x 256 tiles when they fill the chip, else 128 x 128.
    const int64_t big_tiles = (int64_t)a.L * ((a.M + 255) / 256) * (a.N / 256);
    const int cus = a.num_cus > 0 ? a.num_cus : 256;
    int rc;
    if (a.N % 256 == 0 && big_tiles >= cus)
        rc = launch_tiles<256, 256>(a, stream);
    else
        rc = launch_tiles<128, 128>(a, stream);
    if (rc) return rc;
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nrc
