// Batched K/V projection C[l] = A[l] . B[l] on the gfx950 bf16 matrix cores.
//
// The vLLM page "...runtime.draft" (ContextKV._project) keeps this step a
// stock bmm of the stacked layer norms [L, T, D] against the stacked K/V
// weight; the logical right operand is [L, D, N] with N contiguous. Results
// are FP32 sums of exact bf16 products, rounded once to bf16.
//
// Kernel: one workgroup per BM x BN output tile of one layer; waves split
// the tile WM x WN, each wave owning a (BM/WM) x (BN/WN) block of
// v_mfma_f32_16x16x32_bf16 accumulators (one MFMA per 16 x 16 block covers a
// whole 32-wide stage of K). On this chip the 16 x 16 x 32 form draws less
// power per flop than 32 x 32 x 16 (a loop of either on toggling operands
// holds 1.95 against 1.75 GHz) and accumulates in the same order (identical
// bits). K is walked in stages of 32 through a 4-deep LDS ring:
//   - both operands go global -> LDS with global_load_lds_dwordx4 (no
//     register staging); B k-rows are 2 BN bytes per stage; A moves in pairs
//     of stages (two 32 KiB buffers of 64 k, 128-byte rows: whole cache lines,
//     half the L2 requests of 64-byte rows; 1-3% faster on the long workload,
//     5% with the [L, N, D] weight), except in the fused form, which rebuilds
//     A stage by stage;
//   - A fragments are read with ds_read_b128 (8 consecutive k of one row),
//     B fragments with ds_read_b64_tr_b16, which transposes the N-contiguous
//     B tile into the k-contiguous operand layout on the fly;
//   - XOR swizzles on 16-byte chunks make every fragment read free of LDS
//     bank conflicts (the SQ_LDS_BANK_CONFLICT counter reads 0): B k-rows
//     XOR 2 (k & 3) and 8 ((k >> 3) & 1), so that the lanes of an 8-byte
//     transposing read hit distinct bank groups (the k-row group must not
//     touch chunk bit 0, which the column pair sets); A rows of a stage pair
//     XOR r & 7 (per-stage A rows, in the fused form, bits (r1 ^ r2, r2 ^
//     r3) of the row);
//   - the loop is scheduled by hand (reads and DMA between consecutive
//     MFMAs, sched_barrier fences): while stage st is multiplied, the
//     fragments of stage st + 1 are read and the DMA of stage st + 3 goes
//     out, one barrier per stage;
//   - consecutive tile ids go to one XCD (workgroup ids are dealt
//     round-robin over the 8 XCDs), so tiles sharing an A panel or a B panel
//     meet in one L2.
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace nrc {

// Scratch of the no-allocation projection: the split form's FP32 partial
// sums for callers that cannot allocate device memory. One copy per GPU,
// held from the library's first use on that GPU until the process ends; host
// code reaches it only through the address hipGetSymbolAddress returns for
// the current device (project_scratch), never through this name.
static __device__ __align__(256) float scratch[kProjectScratchBytes / sizeof(float)];

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4v lds_u32x4;

constexpr int kBK = 32;     // K per LDS stage
constexpr int kStages = 4;  // LDS ring depth

// 16-byte chunk swizzles of the LDS tiles (see the header). swz_a depends on
// bits 1..3 of the row only, so every A chunk a lane's DMA writes (rows 16
// apart) sits at the same k chunk.
__device__ __forceinline__ int swz_a(int row) { return (((row >> 1) ^ (row >> 2)) & 1) | ((((row >> 2) ^ (row >> 3)) & 1) << 1); }
__device__ __forceinline__ int swz_b(int krow) { return (2 * (krow & 3)) ^ (8 * ((krow >> 3) & 1)); }
// A rows of a stage pair (64 k, 128 bytes = 8 chunks): chunk ^ (r & 7).
// Chosen by the SQ_LDS_BANK_CONFLICT counter, which reads 0 with it; a
// swizzle that also XORed row bit 3 (conflict-free by a 64-bank, 16-lanes-
// per-cycle model of the reads) read 2 conflict cycles per LDS instruction.
__device__ __forceinline__ int swz_a2(int row) { return row & 7; }

template <int BM, int BN, int WM, int WN>
struct Cfg {
    static constexpr int WAVES = WM * WN;              // waves per workgroup, WM along M x WN along N
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int WTM = BM / WM, WTN = BN / WN; // wave tile
    static constexpr int MI = WTM / 16;                // 16-row MFMA blocks per wave
    static constexpr int NI = WTN / 16;                // 16-column MFMA blocks per wave
    static constexpr int A_BYTES = BM * kBK * 2;       // one stage of A: BM rows x 64 bytes
    static constexpr int B_BYTES = kBK * BN * 2;       // one stage of B: 32 k rows x 2 BN bytes
    static constexpr int B_ROW = BN * 2;
    static constexpr int A_LOADS = A_BYTES / 1024 / WAVES;  // 1 KiB DMA blocks per wave per stage
    static constexpr int A2_LOADS = 2 * A_LOADS;             // the same for a stage pair (64 k)
    static constexpr int B_LOADS = B_BYTES / 1024 / WAVES;
    static constexpr int LOADS = A_LOADS + B_LOADS;
    static constexpr int A_REGION = kStages * A_BYTES;
    static constexpr int LDS_BYTES = kStages * (A_BYTES + B_BYTES);
    static_assert(A_LOADS >= 1 && B_LOADS >= 1 && A_LOADS * WAVES * 1024 == A_BYTES &&
                      B_LOADS * WAVES * 1024 == B_BYTES,
                  "tile must split into whole 1 KiB DMA blocks per wave");
};

// s_waitcnt immediates (gfx9 encoding: vmcnt in [3:0] and [15:14], expcnt
// in [6:4], lgkmcnt in [11:8]); the counters not named are left at their
// maximum so they do not wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 *
// lane (global_load_lds_dwordx4, gfx950). Issued as inline assembly so the
// kernel alone accounts for these writes with explicit vmcnt waits and
// barriers (the pipeline below), instead of a conservative wait for every
// outstanding load before each LDS read. An LDS DMA that reads M0 right after
// a scalar write of M0 needs one wait state in between (the compiler puts an
// s_nop there for its own LDS DMA; nothing does inside an asm statement).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base)
                 : "memory", "m0");
}

// A operand of the fused form: the layer-norm output built on the fly from
// the hidden norm's bf16 output h [M, K], each row's scale r[m] (sign bit
// set: the row may produce NaN and takes the exact bf16 rounding) and the
// layer's weight gamma [L, K] (nullptr: weightless).
struct FusedA {
    const float* r;
    const uint16_t* gamma;
    float center;
};

// Tiles are ordered layer, M tile, N tile (N fastest), so each XCD's share
// of a round touches one layer's weight panels. FUSED: false - A is the
// stacked layer-norm output [L, M, K]; true - A is built from FusedA (each h
// panel is then read once per layer: ordering the layers of an h panel
// together instead re-read the weight panels of every layer in each round,
// 2.6 GB fetched per launch, and ran 2% slower).
// CMODE (fused, with weights): 0 - gamma = w; 1 - gamma = w with -0.0 turned
// into +0.0 (a +0.0 center); 2 - gamma = w + center in FP32.
// B_ND: the weight is stored [L, N, K] (K contiguous, the pages' storage)
// instead of [L, K, N]; its tile then takes A's path (64-byte rows per
// stage, A's swizzle, ds_read_b128 fragments).
// SPLIT: K is cut into k_split slices of K / k_split; tile ids run over
// (slice, layer, M tile, N tile), and each tile writes its FP32 sums to
// W [k_split, L, M, N] instead of rounding into C (the fused form rebuilds
// the slice's A chunks with the slice's part of the layer weight).
template <int BM, int BN, int WM, int WN, bool FUSED, bool PW, int CMODE, bool B_ND, bool SPLIT>
__global__ __launch_bounds__(64 * WM * WN) void kv_project_kernel(const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ B,
                                                              uint16_t* __restrict__ C, int64_t M, int64_t K,
                                                              int64_t N, int32_t L, int32_t tiles_m, int32_t tiles_n,
                                                              int32_t total_tiles, FusedA fa, float* __restrict__ W,
                                                              int32_t k_split, uint64_t* __restrict__ stamps,
                                                              int64_t stamps_len, bool layer_sync, bool layer_inner) {
    using CF = Cfg<BM, BN, WM, WN>;
    // Clock stamps (diagnostic, stamps non-null): the shader clock counter
    // and the constant-rate counter when the workgroup starts; the wait keeps
    // the scalar reads from staying outstanding into the loop.
    uint64_t clk_s0 = 0, clk_r0 = 0;
    if (stamps != nullptr) {
        clk_s0 = __builtin_amdgcn_s_memtime();
        clk_r0 = __builtin_amdgcn_s_memrealtime();
        wait_lgkmcnt0();
    }
    extern __shared__ __attribute__((aligned(1024))) char lds_raw[];
    lds_char* lds = (lds_char*)lds_raw;

    // Persistent workgroups: workgroup b takes the tiles tile_of(0),
    // tile_of(1), ... Workgroup b runs on XCD b % 8; when both the tile
    // count and the grid split evenly over the 8 XCDs, each XCD owns a
    // contiguous range of tile ids (N fastest), so tiles sharing an A panel
    // or a B panel run side by side under one L2.
    //
    // layer_sync (the stacked weight is too large for the 256 MB infinity
    // cache to hold every layer's at once): round `it` takes tiles it G ..
    // it G + G - 1 instead, the x-th eighth of them on XCD x, so that every
    // XCD works on the same layer at a time and the rounds' re-reads of that
    // layer's weight panels come from the infinity cache, not HBM.
    const int G = (int)gridDim.x;
    const bool xcd_split = (total_tiles & 7) == 0 && (G & 7) == 0;
    auto tile_of = [&](int it) -> int {
        if (layer_sync && (G & 7) == 0) {
            const int t = it * G + (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3);
            return t < total_tiles ? t : total_tiles;
        }
        if (xcd_split) {
            const int loc = (int)(blockIdx.x >> 3) + it * (G >> 3);
            return loc < (total_tiles >> 3) ? (int)(blockIdx.x & 7) * (total_tiles >> 3) + loc : total_tiles;
        }
        const int t = (int)blockIdx.x + it * G;
        return t < total_tiles ? t : total_tiles;
    };
    //
    // layer_inner (fused form, unsplit, N <= 256): tile ids run over (M tile,
    // layer, N tile) instead, so the layers of one h panel sit side by side
    // under one L2 and the panel comes from memory once rather than once per
    // layer (with N this narrow the layers' weights are small).
    int layer = 0, ks = 0;
    int64_t m0 = 0, n0 = 0;
    const int64_t k_len = SPLIT ? K / k_split : K;  // K walked per tile
    auto decode = [&](int tile) {
        const int tn = tile % tiles_n;
        if (!SPLIT && layer_inner) {
            layer = (tile / tiles_n) % L;
            m0 = (int64_t)(tile / (tiles_n * L)) * BM;
            n0 = (int64_t)tn * BN;
            return;
        }
        const int tm = (tile / tiles_n) % tiles_m;
        const int lt = tile / (tiles_n * tiles_m);
        layer = SPLIT ? lt % L : lt;
        ks = SPLIT ? lt / L : 0;
        m0 = (int64_t)tm * BM;
        n0 = (int64_t)tn * BN;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // ---- DMA assignments (global -> LDS, 16 bytes per lane, 1 KiB per wave
    // instruction written to consecutive LDS bytes). The global source of
    // each lane is chosen so that LDS holds the swizzled layouts below.
    //   A stage: row r (BM rows, 64 bytes = 4 chunks of 8 k), chunk c stored
    //            at chunk c ^ swz_a(r).
    //   B stage: k row r (32 rows, 2 BN bytes), 16-byte chunk c stored at
    //            chunk c ^ swz_b(r).
    // A2 (unfused): A moves in stage pairs of 64 k, 128-byte rows (whole
    // cache lines), into two buffers of two stages each; B per stage as
    // before. The fused form rebuilds A per stage and keeps 64-byte rows.
    constexpr bool A2 = !FUSED;
    constexpr int A_SRC = A2 ? CF::A2_LOADS : CF::A_LOADS;
    const uint16_t* a_src[A_SRC];
    const uint16_t* b_src[CF::B_LOADS];
    auto set_sources = [&]() {
        const int64_t k0 = (int64_t)ks * k_len;  // first k of this tile's slice
        const uint16_t* Al = (FUSED ? A : A + (int64_t)layer * M * K) + k0;
        const uint16_t* Bl = B + (int64_t)layer * K * N + (B_ND ? k0 : k0 * N);
#pragma unroll
        for (int t = 0; t < A_SRC; ++t) {
            const int off = (wave * A_SRC + t) * 1024 + lane * 16;
            const int r = A2 ? off >> 7 : off >> 6;
            const int pc = A2 ? (off >> 4) & 7 : (off >> 4) & 3;
            const int c = A2 ? pc ^ swz_a2(r) : pc ^ swz_a(r);
            int64_t row = m0 + r;
            row = row < M ? row : M - 1;
            a_src[t] = Al + row * K + 8 * c;
        }
#pragma unroll
        for (int t = 0; t < CF::B_LOADS; ++t) {
            const int off = (wave * CF::B_LOADS + t) * 1024 + lane * 16;
            if constexpr (B_ND) {
                const int r = off >> 6, pc = (off >> 4) & 3;
                const int c = pc ^ swz_a(r);
                b_src[t] = Bl + (n0 + r) * K + 8 * c;
            } else {
                const int r = off / CF::B_ROW, pc = (off % CF::B_ROW) >> 4;
                const int c = pc ^ swz_b(r);
                b_src[t] = Bl + (int64_t)r * N + n0 + 8 * c;
            }
        }
    };

    // ---- fused form: the layer weights of this tile sit in LDS past the
    // ring; each lane rebuilds, in place, the A chunks its own DMA wrote:
    // a = bf16((h * |r|) * gamma) per element with the paired hardware
    // conversion (round to nearest even; a NaN stays a NaN, and any NaN
    // operand makes the FP32 sum NaN, which the epilogue writes as 0x7FC0,
    // so the C tile matches the one computed from the exactly rounded
    // norms). All of a lane's chunks sit at the same k chunk, so one weight
    // read serves them all. The work is split into pieces (reads, one
    // element pair, a write) that the loop places between MFMAs.
    constexpr int G_OFF = CF::LDS_BYTES;
    float a_r[CF::A_LOADS];
    const int a_kc = 8 * ((lane & 3) ^ swz_a(lane >> 2));  // k chunk of every A chunk this lane owns
    int staged_layer = -1;
    // Per-tile fused state: each owned row's scale, and (when the layer
    // changes) the layer weight staged in LDS. Called only when no wave
    // still reads the weights of the previous tile.
    auto set_fused = [&]() {
        if constexpr (FUSED) {
#pragma unroll
            for (int t = 0; t < CF::A_LOADS; ++t) {
                const int off = (wave * CF::A_LOADS + t) * 1024 + lane * 16;
                int64_t row = m0 + (off >> 6);
                row = row < M ? row : M - 1;
                a_r[t] = __builtin_fabsf(fa.r[row]);
            }
            if constexpr (PW) {
                if (layer != staged_layer) {
                    const uint16_t* g = fa.gamma + (int64_t)layer * K;
                    for (int c = tid; c < (int)(K / 8); c += CF::THREADS) {
                        U32x4 w = load16(g + 8 * c);
                        if constexpr (CMODE == 1) w = plus_zero16(w);
                        *(lds_u32x4*)(lds + G_OFF + 16 * c) = u32x4v{w.x, w.y, w.z, w.w};
                    }
                    staged_layer = layer;
                }
            }
        }
    };
    u32x4v t_h[CF::A_LOADS], t_g;
    uint32_t t_o[CF::A_LOADS][4];
    auto t_chunk = [&](int buf, int t) {
        return (lds_u32x4*)(lds + buf * CF::A_BYTES + (wave * CF::A_LOADS + t) * 1024 + lane * 16);
    };
    auto t_read = [&](int st, int buf) {
        const int nks = (int)(k_len / kBK);  // stages of this tile's slice
        const int sk = st < nks ? st : nks - 1;
#pragma unroll
        for (int t = 0; t < CF::A_LOADS; ++t) t_h[t] = *t_chunk(buf, t);
        if constexpr (PW) t_g = *(const lds_u32x4*)(lds + G_OFF + 2 * ((int)(ks * k_len) + sk * kBK + a_kc));
    };
    auto t_pair = [&](int t, int q) {
        float y0 = bf16_lo(t_h[t][q]) * a_r[t];
        float y1 = bf16_hi(t_h[t][q]) * a_r[t];
        if constexpr (PW) {
            const float g0 = bf16_lo(t_g[q]), g1 = bf16_hi(t_g[q]);
            y0 = y0 * (CMODE == 2 ? g0 + fa.center : g0);
            y1 = y1 * (CMODE == 2 ? g1 + fa.center : g1);
        }
        t_o[t][q] = pack_bf16_pair_hw(y0, y1);
    };
    auto t_write = [&](int buf, int t) { *t_chunk(buf, t) = u32x4v{t_o[t][0], t_o[t][1], t_o[t][2], t_o[t][3]}; };
    auto transform = [&](int st, int buf) {
        t_read(st, buf);
#pragma unroll
        for (int t = 0; t < CF::A_LOADS; ++t) {
#pragma unroll
            for (int q = 0; q < 4; ++q) t_pair(t, q);
            t_write(buf, t);
        }
    };

    // ---- MFMA operand reads (v_mfma_f32_16x16x32_bf16: lane l supplies row
    // (or column) l % 16 of its 16-block and the 8 k values 8 (l / 16) ..
    // 8 (l / 16) + 7 of the 32-wide stage; one MFMA covers a whole stage).
    // A (ds_read_b128): lane reads row wm WTM + 16 i + (lane & 15), k chunk
    // lane >> 4; block i adds 16 rows (1 KiB; the swizzle repeats every 4 rows).
    const int kq = lane >> 4;
    int a_off, a2_off[2];  // a2_off[p]: stage parity p within a pair
    {
        const int r = wm * CF::WTM + (lane & 15);
        a_off = r * 64 + 16 * (kq ^ swz_a(r));
        a2_off[0] = r * 128 + 16 * (kq ^ swz_a2(r));
        a2_off[1] = r * 128 + 16 * ((4 + kq) ^ swz_a2(r));
    }
    // B (ds_read_b64_tr_b16): within each 16-lane group g = lane >> 4, lane
    // c = 4 jj + q points at 4 bf16 of k row 8 g + 4 h + jj, columns 4 q ..
    // 4 q + 3 of the block's 16 columns; the transposing read hands lane i of
    // the group the 4 k values 8 g + 4 h .. 8 g + 4 h + 3 of column i, which
    // are elements 4 h .. 4 h + 3 of its operand. Half h = 1 is 4 k rows on.
    int b_off[CF::NI];
    {
        const int c = lane & 15, jj = c >> 2, q = c & 3;
        const int krow = 8 * kq + jj;
#pragma unroll
        for (int j = 0; j < CF::NI; ++j) {
            const int n = wn * CF::WTN + 16 * j + 4 * q;
            const int pc = (n >> 3) ^ swz_b(krow);
            b_off[j] = CF::A_REGION + krow * CF::B_ROW + pc * 16 + ((n >> 2) & 1) * 8;
        }
    }
    // B stored [L, N, K]: lane reads column row wn WTN + 16 j + (lane & 15),
    // k chunk lane >> 4, as for A.
    int bnd_off;
    {
        const int r = wn * CF::WTN + (lane & 15);
        bnd_off = CF::A_REGION + r * 64 + 16 * (kq ^ swz_a(r));
    }

    f32x4 acc[CF::MI][CF::NI];

    // ---- one-instruction building blocks of the scheduled loop.
    // af[i] holds the wave's 16-row block i of a stage; bfr[f][j] its
    // 16-column block j, in two sets (f = stage parity): the next stage's B
    // blocks are read while the current ones are still in use, and each A
    // block of the next stage is read into af[i] once block i's last MFMA
    // has issued.
    bf16x8 af[CF::MI], bfr[2][CF::NI];
    constexpr int NM = CF::MI * CF::NI;                 // MFMAs per stage
    constexpr int NB = (B_ND ? 1 : 2) * CF::NI;          // B reads per stage
    // read_a(stage buffer, block): per-stage layout; read_a2(stage, block):
    // the stage-pair layout (pair buffer (st >> 1) & 1, half st & 1).
    auto read_a = [&](int buf, int i) {
        af[i] = *(const __attribute__((address_space(3))) bf16x8*)(lds + buf * CF::A_BYTES + a_off + i * 16 * 64);
    };
    auto read_a2 = [&](int st, int i) {
        af[i] = *(const __attribute__((address_space(3))) bf16x8*)(lds + ((st >> 1) & 1) * 2 * CF::A_BYTES +
                                                                   a2_off[st & 1] + i * 16 * 128);
    };
    // B read r (0 .. NB - 1) of stage buffer buf into set f.
    auto read_b = [&](int buf, int f, int r) {
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const lds_char* sb = lds + buf * CF::B_BYTES;
        if constexpr (B_ND) {
            bfr[f][r] = *(const __attribute__((address_space(3))) bf16x8*)(sb + bnd_off + r * 16 * 64);
        } else {
            const int j = r >> 1, hi = r & 1;
            const lds_char* p = sb + b_off[j] + hi * 4 * CF::B_ROW;
            const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
            const i16x8 v8 = __builtin_shufflevector(v, v, 0, 1, 2, 3, 0, 1, 2, 3);
            const i16x8 cur = __builtin_bit_cast(i16x8, bfr[f][j]);
            const i16x8 nxt = hi ? __builtin_shufflevector(cur, v8, 0, 1, 2, 3, 8, 9, 10, 11)
                                 : __builtin_shufflevector(v8, cur, 0, 1, 2, 3, 12, 13, 14, 15);
            bfr[f][j] = __builtin_bit_cast(bf16x8, nxt);
        }
    };
    // The weight fragment goes in as the MFMA's first operand: the block is
    // computed transposed, so that each lane ends with four consecutive
    // columns of one row (16 x 16 block: lane l holds row l % 16, columns
    // 4 (l / 16) .. 4 (l / 16) + 3) and the epilogue stores them together.
    auto mfma_one = [&](int f, int idx) {
        const int i = idx / CF::NI, j = idx % CF::NI;
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[f][j], af[i], acc[i][j], 0, 0, 0);
    };
    const int nk = (int)(k_len / kBK);
    // DMA d (0 .. LOADS-1: A blocks, then B blocks) of stage st into buffer
    // st mod 4. Past the last stage the source is clamped to stage nk - 1 and
    // lands in a buffer nobody reads again, so every iteration issues the
    // same number of loads and the vmcnt arithmetic is the same everywhere.
    // A pair j (stages 2 j, 2 j + 1), block d of A2_LOADS, into pair buffer
    // j & 1; past the last pair the source is clamped to the last one.
    auto dma_a2 = [&](int j, int d) {
        const int s = j < nk / 2 ? j : nk / 2 - 1;
        const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
        dma16(a_src[d] + (int64_t)s * 2 * kBK,
              __builtin_amdgcn_readfirstlane(base + (j & 1) * 2 * CF::A_BYTES + (wave * CF::A2_LOADS + d) * 1024));
    };
    auto dma_b = [&](int st, int t) {
        const int s = st < nk ? st : nk - 1;
        const int buf = st & (kStages - 1);
        const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
        dma16(b_src[t] + (B_ND ? (int64_t)s * kBK : (int64_t)s * kBK * N),
              __builtin_amdgcn_readfirstlane(base + CF::A_REGION + buf * CF::B_BYTES + (wave * CF::B_LOADS + t) * 1024));
    };
    auto dma_one = [&](int st, int d) {
        const int s = st < nk ? st : nk - 1;
        const int buf = st & (kStages - 1);
        const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
        if (d < CF::A_LOADS) {
            dma16(a_src[d] + (int64_t)s * kBK,
                  __builtin_amdgcn_readfirstlane(base + buf * CF::A_BYTES + (wave * CF::A_LOADS + d) * 1024));
        } else {
            const int t = d - CF::A_LOADS;
            dma16(b_src[t] + (B_ND ? (int64_t)s * kBK : (int64_t)s * kBK * N),
                  __builtin_amdgcn_readfirstlane(base + CF::A_REGION + buf * CF::B_BYTES +
                                                 (wave * CF::B_LOADS + t) * 1024));
        }
    };

    // ---- pipeline. Stage st is computed from fragments read during stage
    // st - 1. Iteration st:
    //   wait until this wave's DMAs of stage st + 1 have landed (vmcnt <= the
    //   loads of stage st + 2, the only later ones issued), barrier: stage
    //   st + 1 visible to all;
    //   the NM MFMAs of stage st (A block by A block); between them the DMA
    //   of stage st + 3 into buffer (st + 3) mod 4 = (st - 1) mod 4, whose
    //   fragments were read during stage st - 2 and used before this
    //   iteration's barrier, and the reads of stage st + 1: its B blocks into
    //   the other B set, and each A block into af[i] after block i's last
    //   MFMA. The fused form first rebuilds this lane's A chunks of stage
    //   st + 1 between the first half's MFMAs and takes a second barrier
    //   before any read of that stage; its reads go in the second half.
    // ---- tiles. The first tile's setup and prologue DMA (stages 0-2) go out
    // before the loop; each later tile's go out as soon as the previous
    // tile's K loop has finished, before that tile's results are stored, so
    // the store burst and the first loads of the next tile overlap.
    // A2: pair 0, B 0, B 1, pair 1, B 2 (stage 0 needs the first two).
    auto issue_prologue = [&]() {
        if constexpr (A2) {
#pragma unroll
            for (int d = 0; d < CF::A2_LOADS; ++d) dma_a2(0, d);
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int t = 0; t < CF::B_LOADS; ++t) dma_b(st, t);
#pragma unroll
            for (int d = 0; d < CF::A2_LOADS; ++d) dma_a2(1, d);
#pragma unroll
            for (int t = 0; t < CF::B_LOADS; ++t) dma_b(2, t);
        } else {
#pragma unroll
            for (int st = 0; st < kStages - 1; ++st)
#pragma unroll
                for (int d = 0; d < CF::LOADS; ++d) dma_one(st, d);
        }
    };
    int it = 0;
    int tile = tile_of(0);
    if (tile >= total_tiles) return;
    decode(tile);
    set_sources();
    set_fused();
    issue_prologue();
    // Epilogue: lane holds row (lane & 15) of each 16 x 16 block, columns
    // 4 (lane / 16) + v, v < 4: one 8-byte store of bf16 (16 bytes of FP32
    // partial sums) per block. Rounding: the paired hardware conversion
    // (nearest even, the library's rounding for every non-NaN value) when no
    // sum of the wave's tile is NaN, else the exact bit-pattern rounding
    // (NaN -> 0x7FC0).
    auto epilogue = [&](int e_layer, int64_t e_m0, int64_t e_n0, int e_ks) {
    uint16_t* Cl = C + (int64_t)e_layer * M * N;
    float* Wl = W + ((int64_t)e_ks * L + e_layer) * M * N;
    bool nan = false;
    if constexpr (!SPLIT) {
#pragma unroll
        for (int i = 0; i < CF::MI; ++i)
#pragma unroll
            for (int j = 0; j < CF::NI; ++j)
                nan = nan || __builtin_isunordered(acc[i][j][0], acc[i][j][1]) ||
                      __builtin_isunordered(acc[i][j][2], acc[i][j][3]);
    }
    auto store_tile = [&](auto checked, auto exact) {
#pragma unroll
        for (int i = 0; i < CF::MI; ++i) {
            const int64_t row = e_m0 + wm * CF::WTM + 16 * i + (lane & 15);
            if (decltype(checked)::value && row >= M) continue;
#pragma unroll
            for (int j = 0; j < CF::NI; ++j) {
                const int64_t col = e_n0 + wn * CF::WTN + 16 * j + 4 * (lane >> 4);
                const f32x4 c = acc[i][j];
                if constexpr (SPLIT) {
                    *reinterpret_cast<f32x4*>(Wl + row * N + col) = c;
                } else if constexpr (decltype(exact)::value) {
                    *reinterpret_cast<uint2*>(Cl + row * N + col) = uint2{pack_bf16(c[0], c[1]), pack_bf16(c[2], c[3])};
                } else {
                    *reinterpret_cast<uint2*>(Cl + row * N + col) =
                        uint2{pack_bf16_pair_hw(c[0], c[1]), pack_bf16_pair_hw(c[2], c[3])};
                }
            }
        }
    };
    const bool full = e_m0 + BM <= M;
    if (__builtin_amdgcn_ballot_w64(nan) != 0) {
        if (full)
            store_tile(std::false_type{}, std::true_type{});
        else
            store_tile(std::true_type{}, std::true_type{});
    } else {
        if (full)
            store_tile(std::false_type{}, std::false_type{});
        else
            store_tile(std::true_type{}, std::false_type{});
    }
    };

    // Slots of the schedule (MFMA index after which a piece is issued).
    constexpr int HALFM = NM / 2;
    auto dma_slot = [](int d) { return (d * NM) / CF::LOADS + 1 < NM ? (d * NM) / CF::LOADS + 1 : NM - 1; };
    // unfused: B reads spread over the first NB slots; fused: over the second half
    auto b_slot = [](int r) { return FUSED ? HALFM + (r * HALFM) / NB : (r * NM) / (2 * NB); };
    // A block i of the next stage: after its last MFMA (fused: not before the half)
    auto a_slot = [](int i) {
        const int last = i * CF::NI + CF::NI - 1;
        return FUSED && last < HALFM ? HALFM + i : last;
    };
    constexpr int NP = 4 * CF::A_LOADS;  // fused: element pairs per lane per stage
    auto pair_slot = [](int p) { return HALFM > 1 ? 1 + (p * (HALFM - 1)) / NP : 0; };

    while (true) {
#pragma unroll
        for (int i = 0; i < CF::MI; ++i)
#pragma unroll
            for (int j = 0; j < CF::NI; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0f;
        // Stage 0 landed. On the first tile: vmcnt <= stages 1-2; later tiles
        // also have the previous tile's stores in flight, issued after these
        // loads, so wait for everything.
        if (it != 0)
            wait_vmcnt<0>();
        else if constexpr (A2)
            wait_vmcnt<2 * CF::B_LOADS + CF::A2_LOADS>();  // B 1, pair 1, B 2 may be in flight
        else
            wait_vmcnt<(kStages - 2) * CF::LOADS>();
        if constexpr (FUSED) {
            __syncthreads();  // staged weights visible to every wave
            transform(0, 0);
            wait_lgkmcnt0();
        }
        barrier();
#pragma unroll
        for (int i = 0; i < CF::MI; ++i) {
            if constexpr (A2)
                read_a2(0, i);
            else
                read_a(0, i);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < NB; ++r) {
            read_b(0, 0, r);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Two iterations per loop trip (nk is even): B sets 0 then 1.
        auto iteration = [&](int st, auto fset) {
            constexpr int f = decltype(fset)::value;
            const int b1 = (st + 1) & (kStages - 1);
            // A2: an odd iteration issues B and an A pair, an even one B only;
            // the stage read next landed once at most the previous
            // iteration's loads are in flight.
            if constexpr (A2)
                wait_vmcnt<f == 0 ? CF::B_LOADS + CF::A2_LOADS : CF::B_LOADS>();
            else
                wait_vmcnt<CF::LOADS>();
            // The fused form's only barrier is the mid-stage one: its rebuilt
            // chunks are read only after it, and no wave can issue the DMA
            // into buffer (st - 1) mod 4 before every wave has passed the
            // previous stage's mid barrier, by which point their reads of
            // that buffer (stage st - 1, read during stage st - 2) were
            // consumed.
            // A2, odd iteration: this iteration's DMA refills the pair buffer
            // that holds stage st, whose fragments every wave read during the
            // previous iteration; those reads complete before the barrier, so
            // no DMA write can land on data a wave has yet to read (nothing
            // else orders a wave's LDS reads against another wave's LDS DMA;
            // measured cost within noise).
            if constexpr (A2 && f == 1) wait_lgkmcnt0();
            if constexpr (!FUSED) barrier();
            if constexpr (FUSED) t_read(st + 1, b1);
#pragma unroll
            for (int idx = 0; idx < NM; ++idx) {
                mfma_one(f, idx);
                if constexpr (FUSED) {
#pragma unroll
                    for (int p = 0; p < NP; ++p)
                        if (idx < HALFM && pair_slot(p) == idx) {
                            t_pair(p >> 2, p & 3);
                            if ((p & 3) == 3) t_write(b1, p >> 2);
                        }
                    if (idx == HALFM - 1) {
                        wait_lgkmcnt0();
                        barrier();  // every wave's rebuilt chunks of stage st + 1 visible
                    }
                }
                if constexpr (A2) {
                    // B of stage st + 3; odd iterations also A pair (st + 3) / 2
                    constexpr int NL = f == 1 ? CF::B_LOADS + CF::A2_LOADS : CF::B_LOADS;
#pragma unroll
                    for (int d = 0; d < NL; ++d)
                        if ((d * NM) / NL + 1 == idx || (idx == NM - 1 && (d * NM) / NL + 1 >= NM)) {
                            if (d < CF::B_LOADS)
                                dma_b(st + kStages - 1, d);
                            else
                                dma_a2((st + 3) >> 1, d - CF::B_LOADS);
                        }
                } else {
#pragma unroll
                    for (int d = 0; d < CF::LOADS; ++d)
                        if (dma_slot(d) == idx) dma_one(st + kStages - 1, d);
                }
#pragma unroll
                for (int r = 0; r < NB; ++r)
                    if (b_slot(r) == idx) read_b(b1, f ^ 1, r);
#pragma unroll
                for (int i = 0; i < CF::MI; ++i)
                    if (a_slot(i) == idx) {
                        if constexpr (A2)
                            read_a2(st + 1, i);
                        else
                            read_a(b1, i);
                    }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for (int st = 0; st < nk; st += 2) {
            iteration(st, std::integral_constant<int, 0>{});
            iteration(st + 1, std::integral_constant<int, 1>{});
        }
        wait_vmcnt<0>();  // the clamped loads past the last stage have landed
        barrier();         // every wave is done with the ring and the weights
        const int e_layer = layer, e_ks = ks;
        const int64_t e_m0 = m0, e_n0 = n0;
        const int next = tile_of(++it);
        if (next < total_tiles) {
            decode(next);
            set_sources();
            set_fused();
            issue_prologue();
        }
        epilogue(e_layer, e_m0, e_n0, e_ks);
        if (next >= total_tiles) break;
    }
    wait_vmcnt<0>();  // no DMA may still target this workgroup's LDS at exit
    if (stamps != nullptr && threadIdx.x == 0 && 4 * (int64_t)blockIdx.x + 3 < stamps_len) {
        const uint64_t clk_s1 = __builtin_amdgcn_s_memtime(), clk_r1 = __builtin_amdgcn_s_memrealtime();
        uint64_t* p = stamps + 4 * (int64_t)blockIdx.x;
        p[0] = clk_s0;
        p[1] = clk_r0;
        p[2] = clk_s1;
        p[3] = clk_r1;
    }
}

template <int BM, int BN, int WM, int WN, bool FUSED, bool PW, int CMODE, bool B_ND, bool SPLIT>
int launch_tiles(const ProjectArgs& a, const FusedA& fa, hipStream_t stream) {
    using CF = Cfg<BM, BN, WM, WN>;
    const int tiles_m = (int)((a.M + BM - 1) / BM);
    const int tiles_n = (int)(a.N / BN);
    const int total = a.L * tiles_m * tiles_n * (SPLIT ? a.k_split : 1);
    // The K loop takes two 32-wide stages per trip: every workgroup's share
    // of K must be a multiple of 64 (the callers' shapes and the split rule
    // guarantee it; anything else is refused rather than summed wrong).
    if ((a.K / (SPLIT ? a.k_split : 1)) % (2 * kBK) != 0 || (SPLIT && a.K % a.k_split != 0)) return -1;
    const size_t lds_bytes = CF::LDS_BYTES + ((FUSED && PW) ? (size_t)a.K * 2 : 0);
    auto kernel = kv_project_kernel<BM, BN, WM, WN, FUSED, PW, CMODE, B_ND, SPLIT>;
    if (lds_bytes > 65536) {
        static std::atomic<int> done[64] = {};
        if (raise_lds_limit((const void*)kernel, (int)lds_bytes, done)) return -1;
    }
    // One persistent workgroup per LDS-resident slot (the ring and weights
    // take most of a CU's 160 KiB), never more than there are tiles.
    const int per_cu = (int)(163840 / lds_bytes) < 1 ? 1 : (int)(163840 / lds_bytes);
    const int cus = a.num_cus > 0 ? a.num_cus : 256;
    const int grid = total < per_cu * cus ? total : per_cu * cus;
    // Weights beyond half the infinity cache: the layer-synchronous tile order
    // (edge workload, 268 MB: projection 6.22 -> 5.55 ms; the long
    // workload's 67 MB run 3.5% faster in the per-XCD layer order).
    const bool layer_sync = (int64_t)a.L * a.K * a.N * 2 > ((int64_t)128 << 20);
    // H = 2 (N = 256): fused projection 0.301 -> 0.270 ms on the long
    // workload's rows; neutral at N = 128.
    const bool layer_inner = FUSED && !SPLIT && !layer_sync && a.N <= 256;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(CF::THREADS), lds_bytes, stream, a.A, a.B, a.C, a.M, a.K, a.N, a.L,
                       tiles_m, tiles_n, total, fa, a.ws, SPLIT ? a.k_split : 1, a.stamps, a.stamps_len, layer_sync,
                       layer_inner);
    if (a.workgroups) *a.workgroups = grid;
    return 0;
}

// C = bf16(W[0] + W[1] + ... + W[S - 1]) element by element, the slices added
// in order (deterministic); eight elements per thread, grid stride. S is a
// template argument so that every slice's loads are issued before the first
// add (one memory round trip per eight elements, not S).
template <int S>
__global__ __launch_bounds__(256) void kv_project_reduce_kernel(const float* __restrict__ W, uint16_t* __restrict__ C,
                                                                int64_t count) {
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < count; i += (int64_t)gridDim.x * 256 * 8) {
        U32x4 lo[S], hi[S];
#pragma unroll
        for (int k = 0; k < S; ++k) {
            lo[k] = load16(W + (int64_t)k * count + i);
            hi[k] = load16(W + (int64_t)k * count + i + 4);
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
        store16(C + i, U32x4{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]), pack_bf16(acc[4], acc[5]),
                             pack_bf16(acc[6], acc[7])});
    }
}

int launch_reduce(const ProjectArgs& a, int cus, hipStream_t stream) {
    const int64_t count = (int64_t)a.L * a.M * a.N;
    const int64_t blocks = (count / 8 + 255) / 256, cap = (int64_t)cus * 8;
    const dim3 grid((unsigned)(blocks < cap ? blocks : cap));
    switch (a.k_split) {
        case 2: hipLaunchKernelGGL(kv_project_reduce_kernel<2>, grid, dim3(256), 0, stream, a.ws, a.C, count); break;
        case 4: hipLaunchKernelGGL(kv_project_reduce_kernel<4>, grid, dim3(256), 0, stream, a.ws, a.C, count); break;
        case 8: hipLaunchKernelGGL(kv_project_reduce_kernel<8>, grid, dim3(256), 0, stream, a.ws, a.C, count); break;
        case 16: hipLaunchKernelGGL(kv_project_reduce_kernel<16>, grid, dim3(256), 0, stream, a.ws, a.C, count); break;
        default: return -1;
    }
    return 0;
}

template <bool FUSED, bool PW, int CMODE, bool B_ND>
int launch_shape(const ProjectArgs& a, const FusedA& fa, hipStream_t stream) {
    // 256 x 256 tiles when they fill the chip, else 128 x 128, with K split
    // when even those are too few (k_split > 1). The fused form takes
    // 256 x 128 tiles (eight waves of 64 x 64) where those fill the chip and
    // 256 x 256 ones do not (N = 128, a KV head per GPU: 0.234 -> 0.198 ms on
    // the long workload's rows; the unfused form ran slower with them, 0.247
    // against 0.210 ms).
    const int64_t big_tiles = (int64_t)a.L * ((a.M + 255) / 256) * (a.N / 256);
    const int cus = a.num_cus > 0 ? a.num_cus : 256;
    if (a.N % 256 == 0 && big_tiles >= cus)
        return launch_tiles<256, 256, 2, 4, FUSED, PW, CMODE, B_ND, false>(a, fa, stream);
    if constexpr (FUSED) {
        const int64_t wide_tiles = (int64_t)a.L * ((a.M + 255) / 256) * (a.N / 128);
        if (a.k_split <= 1 && a.N % 128 == 0 && wide_tiles >= cus)
            return launch_tiles<256, 128, 4, 2, FUSED, PW, CMODE, B_ND, false>(a, fa, stream);
    }
    if (a.k_split > 1) {
        // 256 x 256 slices when the tile is not mostly empty rows (half
        // the operand traffic per flop of 128 x 128), else 128 x 128
        const int rc = a.N % 256 == 0 && a.M >= 256
                           ? launch_tiles<256, 256, 2, 4, FUSED, PW, CMODE, B_ND, true>(a, fa, stream)
                           : launch_tiles<128, 128, 2, 2, FUSED, PW, CMODE, B_ND, true>(a, fa, stream);
        if (rc) return rc;
        return a.leave_partials ? 0 : launch_reduce(a, cus, stream);
    }
    return launch_tiles<128, 128, 2, 2, FUSED, PW, CMODE, B_ND, false>(a, fa, stream);
}

}  // namespace

int32_t kv_project_k_split(int32_t L, int64_t M, int64_t K, int64_t N, int num_cus) {
    const int cus = num_cus > 0 ? num_cus : 256;
    const int64_t big_tiles = (int64_t)L * ((M + 255) / 256) * (N / 256);
    if (N % 256 == 0 && big_tiles >= cus) return 1;
    // Slices of 256 x 256 tiles (N a multiple of 256, at least 256 rows) up
    // to one per CU, else of 128 x 128 tiles up to two per CU (their LDS ring
    // lets two share a CU); each slice an even number (the loop takes two
    // stages per trip) of at least 4 stages, at most 8 slices of 256 x 256
    // tiles and 16 of 128 x 128 (measured: a 16-slice 256 x 256 split, whose
    // partial sums double, ran 3% slower at 256 rows; the 128 x 128 splits
    // gained 15-30% from 8 to 16 slices).
    const bool big = N % 256 == 0 && M >= 256;
    const int64_t tiles = big ? big_tiles : (int64_t)L * ((M + 127) / 128) * (N / 128);
    const int64_t target = big ? (int64_t)cus : 2 * (int64_t)cus;
    const int64_t nk = K / kBK;
    int32_t s = 1;
    const int32_t max_s = big ? 8 : 16;
    while (tiles * s < target && s < max_s && nk % (4 * s) == 0 && nk / (2 * s) >= 4) s *= 2;
    return s;
}

int project_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return -1;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return 0;
}

int launch_kv_project(const ProjectArgs& a, hipStream_t stream) {
    const int rc = a.b_nd ? launch_shape<false, false, 0, true>(a, FusedA{nullptr, nullptr, 0.0f}, stream)
                          : launch_shape<false, false, 0, false>(a, FusedA{nullptr, nullptr, 0.0f}, stream);
    if (rc) return rc;
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_kv_project_fused(const ProjectArgs& a, const float* r, const uint16_t* gamma, float center,
                            hipStream_t stream) {
    const FusedA fa{r, gamma, center};
    int rc;
    if (!gamma)
        rc = launch_shape<true, false, 0, false>(a, fa, stream);
    else if (center == 0.0f)
        rc = __builtin_signbit(center) ? launch_shape<true, true, 0, false>(a, fa, stream)
                                       : launch_shape<true, true, 1, false>(a, fa, stream);
    else
        rc = launch_shape<true, true, 2, false>(a, fa, stream);
    if (rc) return rc;
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace nrc
