// k_ffn2d.hip -- the FFN block one chip holds under 2D weight-stationary
// partitioning, on bf16 MFMA: H = silu(X W_gate^T) * (X W_in^T) (bf16), then
// Y = H W_out^T (fp32).
//
// Pages: CS349E lecture 4, 03_pope_partitioning.py, demo 1 (PaLM-540B FFN,
// E = 18432, F = 73728, 2D weight-stationary: each chip holds an E-slice x
// F-slice block, so an 8 x 8 grid gives 2304 x 9216 blocks) and demo 2 (the
// same layout serves decode batches and prefill token counts); aiterms.tw
// "Tensor Parallelism", 核心概念 item 3 (2D split). The cross-chip
// reduce-scatter / all-gather of the block's activations is not part of one
// chip's computation.
//
// Both products are "NT": C[m][n] = sum_k A[m][k] B[n][k] with A and B stored
// K-contiguous, which is the operand layout of v_mfma_f32_16x16x32_bf16
// (each lane holds 8 consecutive k of one row of A and of one row of B).
//  - workgroup tile BM x 288 (BM = 64 up to 256 rows, 128 up to 4095, else
//    256); 288 divides the PaLM block's 2F = 18432 and E = 2304. Waves form a
//    kWM x 2 grid over the tile (wave tile BM/kWM x 144, MFMA tiles of 16 x
//    16): 16 waves of 32 x 144 for 256 rows, 8 of 32 x 144 for 128 rows with
//    64-K stages, 4 of 64 x 144 (two waves a SIMD by occupancy) for 128 rows
//    with 32-K stages, and for 64 rows two k-groups of 8 waves of 16 x 144.
//    Smaller wave tiles read more LDS bytes per MFMA, but the extra waves
//    hide each other's LDS, barrier and load waits: measured, 256 rows 8 ->
//    16 waves 0.849 -> 0.830 ms per 8192-token block, 128 rows 4 -> 8 waves
//    92.2 -> 86.1 us per 512-token block (16 waves: 87.7), and one wave a
//    SIMD with 128 x 128 or 112 x 128 wave tiles was slower still. The
//    256-row tiles fetch each operand tile from L2 for half as many partner
//    tiles as 128-row tiles, and give the 8192-token down-projection exactly
//    one workgroup per CU (8 N-tiles x 32 M-tiles): 8192-token block 1.133 ->
//    1.080 ms;
//  - an LDS ring filled by direct global->LDS loads (global_load_lds_dwordx4),
//    one barrier per stage, waits by vmcnt and no register staging. Up to
//    1024 rows: 3 stages (loads two stages ahead) of 64 K values (128 bytes
//    of every row, occupancy 1): each 1 KiB wave load is 8 full 128-byte
//    lines, where 64-byte rows made it 16 half-used lines and the L2
//    delivered about half the bytes per request (512 tokens: 124.6 -> 118.4
//    us per block). Below 4096 rows: 3 stages of 32 K values at occupancy 2,
//    which hides more latency there. 256-row tiles: 2 stages (loads one
//    stage ahead) of 64 K values, so the eight waves meet at half as many
//    barriers per MFMA (8192-token block 0.944 -> 0.879 ms; 3 stages of 32,
//    or 4, were level, and a raised wave priority over the MFMAs slower).
//    16-byte chunks are XOR-swizzled per row against bank conflicts;
//  - tile order puts the M-tiles of one N-tile on the same XCD (linear
//    workgroup id % 8), so a weight tile is fetched into one L2 once;
//  - up-projection epilogue: the packed W_gate/W_in rows interleave in
//    groups of 8 inside each 16-row MFMA tile, so lanes n and n ^ 8 hold the
//    gate and the up value of the same feature; the pair trades two values
//    so each lane finishes two of the four rows (with half the lanes idle the
//    epilogue's vector instructions outnumbered the MFMAs 2 : 1), and silu
//    uses the hardware exp2 / reciprocal ahead of the bf16 rounding of h
//    (512-token up-projection 64.8 -> 52.4 us, 8192 tokens 725 -> 637 us);
//  - down-projection at small M: deterministic split-K, fp32 partials summed
//    in split order by a reduce kernel.
#include "common.h"

namespace tps {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBN = 288;                                        // N tile
constexpr int kNT = 9;                                          // MFMA tiles per wave in N (144)
constexpr int kWN = kNT * 16;                                   // wave tile width

enum { FFN_UP = 0, FFN_DOWN = 1 };

struct GemmArgs {
    const uint16_t *A; // [M][K]
    const uint16_t *B; // [N][K]
    uint16_t *H;       // FFN_UP: [M][N/2] bf16
    float *C;          // FFN_DOWN: [splits][M][N] fp32
    int M, N, K, ksteps_per_split;
    // Which tiles share an XCD (consecutive linear workgroup ids go to the 8
    // XCDs in turn, so the tiles with the same id % 8 share one L2).
    // 0: grid order, x = N-tile fastest: the M-tiles of an N-tile share an XCD
    //    (the weight tile is fetched into one L2; every XCD fetches all of A).
    // 1: split-K, S dividing 8: an XCD takes one split's K range and 8/S of
    //    the N-tiles with every M-tile, so each weight tile is fetched once
    //    and each A slice by 8/S XCDs instead of all the N-tiles' XCDs.
    // 2: one split: the XCDs form gm groups of M-tiles x 8/gm groups of
    //    N-tiles, an XCD taking every tile of its pair of groups (gm = 8: A
    //    fetched once, the weights by every XCD).
    int map, gm;
};

// An LDS row holds the stage's KB values of a matrix row (2 KB bytes); its
// 16-byte chunk c sits at chunk c ^ ((r >> 1) & (chunks - 1)), so that the 16
// rows of a fragment read (same logical chunk) spread over the LDS banks.
template <int KB>
__device__ __forceinline__ int swx(int row) { return (row >> 1) & (KB / 8 - 1); }
template <int KB>
__device__ __forceinline__ int swz(int row, int c) { return row * (KB * 2) + ((c ^ swx<KB>(row)) << 4); }

// silu(z) = z / (1 + e^-z) with the hardware exp2 and reciprocal (about 1 ulp
// each); the product is rounded to bf16 right after, 2^8 times coarser.
__device__ __forceinline__ float silu_fast(float z)
{
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// s_waitcnt vmcnt(N), other counters unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// BM = 64, 128 or 256 rows of A per workgroup; KB = 32 or 64 K values per
// stage; NST stages in the LDS ring. KB = 64 (occupancy 1) makes every wave
// load 8 full 128-byte lines and suits decode-sized M, where the L2 delivery
// of the weights is the limit; KB = 32 (64-byte rows, occupancy 2) hides more
// latency for 128-row tiles of a larger M.
// KS = 2 (64-row tiles): two groups of NWV / 2 waves share the tile and the
// LDS ring, group g taking MFMA k-step g of every 64-K stage; group 1 hands
// its sums to group 0 through LDS at the end. The waves then hide each
// other's LDS and barrier waits (512-token split-K down-projection with two
// groups of four: 45.6 -> 43.4 us; of eight: 43.9 -> 42.7 us). 64-row tiles
// for the 512-token up-projection were slower (58 -> 71 us: each weight tile
// fetched for twice as many M-tiles).
template <int EPI, int BM, int KB, int NWV = 4, int NST = 3, int KS = 1>
__global__ __launch_bounds__(64 * NWV, (KB == 32 && NWV == 4) ? 2 : 1) void k_gemm_nt(GemmArgs a)
{
    constexpr int kBK = KB;
    constexpr int kStages = NST;                       // LDS ring of NST stages
    static_assert(NST >= 2, "a stage is loaded while another is read");
    constexpr int kGW = NWV / KS;                      // waves of a k-group
    constexpr int kWM = kGW / 2;                       // waves in M (2 in N)
    static_assert(KS == 1 || (KS == 2 && KB == 64), "a k-group takes one MFMA k-step of a 64-K stage");
    constexpr int kRowB = KB * 2;                      // bytes of a row per stage
    constexpr int kRowsSeg = 1024 / kRowB;             // rows per 1 KiB wave load
    constexpr int kChunks = kRowB / 16;                // 16-byte chunks per row
    constexpr int kMT = BM / (16 * kWM);               // MFMA tiles per wave in M (BM/kWM rows)
    constexpr int kStageB = (BM + kBN) * kRowB;        // bytes per stage
    constexpr int kSegs = kStageB / 1024;              // 1 KiB wave loads per stage
    constexpr int kSegsA = BM * kRowB / 1024;          // of which A
    constexpr int kMaxSegs = (kSegs + NWV - 1) / NWV;  // per wave
    constexpr int kMinSegs = kSegs / NWV;
    static_assert((BM * kRowB) % 1024 == 0 && kStageB % 1024 == 0, "whole wave loads");
    static_assert(kMaxSegs - kMinSegs <= 1, "waves issue kMaxSegs or kMaxSegs - 1 segments");
    __shared__ __attribute__((aligned(1024))) char lds[kStages * kStageB];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int kg = wv / kGW, wl = wv % kGW; // k-group, wave in the group
    const int wm = wl >> 1, wn = wl & 1;    // wave grid kWM x 2
    // grid: x = N-tile, y = M-tile, z = split; the tile this workgroup takes
    // depends on a.map (see GemmArgs)
    int tn = blockIdx.x, tm = blockIdx.y, tz = blockIdx.z;
    if (a.map != 0) {
        const int NT = gridDim.x, MT = gridDim.y, SZ = gridDim.z;
        const int L = blockIdx.x + NT * (blockIdx.y + MT * blockIdx.z), x = L & 7, j = L >> 3;
        if (a.map == 1) {
            const int g = 8 / SZ, per = NT / g;
            tz = x / g;
            tm = j / per;
            tn = (x % g) * per + j % per;
        } else {
            const int gn = 8 / a.gm, mtg = MT / a.gm, ntg = NT / gn;
            tz = 0;
            tm = (x / gn) * mtg + j / ntg;
            tn = (x % gn) * ntg + j % ntg;
        }
    }
    const int n0 = tn * kBN, m0 = tm * BM;
    const int ks0 = tz * a.ksteps_per_split;
    const int nks = min(a.ksteps_per_split, a.K / kBK - ks0);

    f32x4 acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; i++)
#pragma unroll
        for (int j = 0; j < kNT; j++)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Stage loads go straight from global memory to LDS (global_load_lds_dwordx4:
    // lane i's 16 bytes land at base + 16 i), each wave instruction a segment of
    // 8 rows x 128 bytes (full cache lines). Wave w issues segments w, w+4, ...;
    // lane i of segment t fills LDS slot 64 t + i = (row, physical chunk), so it
    // loads the row's logical chunk physical ^ swx(row). A rows past M read row
    // M-1 (their outputs are never stored).
    const int nseg = (kSegs - wv + NWV - 1) / NWV; // kMaxSegs or kMaxSegs - 1
    const uint16_t *src[kMaxSegs];
#pragma unroll
    for (int u = 0; u < kMaxSegs; u++) {
        const int t = wv + NWV * u;
        const int p = lane, rs = p / kChunks, phys = p % kChunks;
        if (t < kSegsA) {
            const int row = t * kRowsSeg + rs;
            const int m = min(m0 + row, a.M - 1);
            src[u] = a.A + (size_t)m * a.K + 8 * (phys ^ swx<KB>(row));
        } else {
            const int row = (t - kSegsA) * kRowsSeg + rs;
            src[u] = a.B + (size_t)(n0 + row) * a.K + 8 * (phys ^ swx<KB>(row));
        }
    }
    auto issue = [&](int ks) {
        const int kbase = (ks0 + ks) * kBK;
        char *base = lds + (ks % kStages) * kStageB;
#pragma unroll
        for (int u = 0; u < kMaxSegs; u++)
            if (u < nseg)
                __builtin_amdgcn_global_load_lds((const void *)(src[u] + kbase),
                                                 (__attribute__((address_space(3))) void *)(base + (wv + NWV * u) * 1024),
                                                 16, 0, 0);
    };

    for (int s = 0; s < kStages - 1 && s < nks; s++)
        issue(s);
    const int q = lane >> 4;
    for (int ks = 0; ks < nks; ks++) {
        // this wave's loads of stage ks are done once at most the later stages'
        // remain (kStages - 2 of them in the steady state; drain at the tail)
        if (ks + kStages - 2 <= nks - 1) {
            if (nseg == kMaxSegs)
                wait_vmcnt<kMaxSegs * (kStages - 2)>();
            else
                wait_vmcnt<(kMaxSegs - 1) * (kStages - 2)>();
        } else {
            wait_vmcnt<0>();
        }
        // every wave's stage ks is in LDS and stage ks-1's buffer is free; a bare
        // barrier (no fence: a fence would also wait for the later stages' loads),
        // with compiler-only memory clobbers on both sides so that no LDS read or
        // load issue can be moved across it
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (ks + kStages - 1 < nks)
            issue(ks + kStages - 1);
        const char *As = lds + (ks % kStages) * kStageB, *Bs = As + BM * kRowB;
        // MFMA k-steps of 32 (a k-group takes every KS-th): lane quarter q takes
        // chunk 4 kk + q
#pragma unroll
        for (int k2 = 0; k2 < kBK / 32 / KS; k2++) {
            const int kk = k2 * KS + kg;
            bf16x8 af[kMT], bfr[kNT];
#pragma unroll
            for (int i = 0; i < kMT; i++)
                af[i] = *(const bf16x8 *)(As + swz<KB>(wm * (BM / kWM) + i * 16 + (lane & 15), 4 * kk + q));
#pragma unroll
            for (int j = 0; j < kNT; j++)
                bfr[j] = *(const bf16x8 *)(Bs + swz<KB>(wn * kWN + j * 16 + (lane & 15), 4 * kk + q));
#pragma unroll
            for (int j = 0; j < kNT; j++)
#pragma unroll
                for (int i = 0; i < kMT; i++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            // scheduling: the A reads and three B reads, then one B read per column of
            // MFMAs, so the MFMAs of column j start while later columns' reads are in
            // flight (8192-token FFN block 1.015 -> 0.992 ms)
            __builtin_amdgcn_sched_group_barrier(0x100, kMT + 3, 0);
#pragma unroll
            for (int j = 0; j < kNT; j++) {
                if (j + 3 < kNT)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, kMT, 0);
            }
        }
    }

    if constexpr (KS == 2) {
        // every wave is past its last LDS read of the ring (and no load is in
        // flight: the last iteration waited for all), so the ring holds group
        // 1's sums, lane-major per (wave, tile)
        static_assert(kGW * kMT * kNT * 64 * 16 <= kStages * kStageB, "the sums fit the ring");
        f32x4 *red = (f32x4 *)lds;
        __syncthreads();
        if (kg == 1) {
#pragma unroll
            for (int i = 0; i < kMT; i++)
#pragma unroll
                for (int j = 0; j < kNT; j++)
                    red[((wl * kMT + i) * kNT + j) * 64 + lane] = acc[i][j];
        }
        __syncthreads();
        if (kg == 1)
            return;
#pragma unroll
        for (int i = 0; i < kMT; i++)
#pragma unroll
            for (int j = 0; j < kNT; j++)
                acc[i][j] += red[((wl * kMT + i) * kNT + j) * 64 + lane];
    }

    // lane holds C[m0 + wm*BM/kWM + i*16 + 4*(lane/16) + r][n0 + wn*kWN + j*16 + lane%16]
    const int col = lane & 15, rq = (lane >> 4) * 4;
    if constexpr (EPI == FFN_UP) {
        // lanes col < 8 hold the gate and lanes col ^ 8 the up value of
        // feature tile*8 + col % 8, rows rq .. rq + 3: the pair trades two
        // values so that the low lane finishes rows rq, rq + 1 and the high
        // lane rows rq + 2, rq + 3 (every lane two outputs, none idle)
        const int F = a.N / 2;
        const bool hi = col >= 8;
#pragma unroll
        for (int i = 0; i < kMT; i++)
#pragma unroll
            for (int j = 0; j < kNT; j++) {
                const f32x4 c = acc[i][j];
                const float r0 = __shfl_xor(hi ? c[0] : c[2], 8, 64);
                const float r1 = __shfl_xor(hi ? c[1] : c[3], 8, 64);
                const float g0 = hi ? r0 : c[0], u0 = hi ? c[2] : r0;
                const float g1 = hi ? r1 : c[1], u1 = hi ? c[3] : r1;
                const int tile = (n0 + wn * kWN + j * 16) / 16;
                const int f = tile * 8 + (col & 7);
                const int m = m0 + wm * (BM / kWM) + i * 16 + rq + (hi ? 2 : 0);
                if (m < a.M)
                    a.H[(size_t)m * F + f] = f32_to_bf16(silu_fast(g0) * u0);
                if (m + 1 < a.M)
                    a.H[(size_t)(m + 1) * F + f] = f32_to_bf16(silu_fast(g1) * u1);
            }
    } else {
        float *C = a.C + (size_t)tz * a.M * a.N;
#pragma unroll
        for (int i = 0; i < kMT; i++)
#pragma unroll
            for (int j = 0; j < kNT; j++) {
                const int n = n0 + wn * kWN + j * 16 + col;
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int m = m0 + wm * (BM / kWM) + i * 16 + rq + r;
                    if (m < a.M)
                        C[(size_t)m * a.N + n] = acc[i][j][r];
                }
            }
    }
}

// Y[i] = sum_s P[s][i] in split order, 4 elements per thread.
__global__ __launch_bounds__(256) void k_split_reduce(const float *P, float *Y, size_t n, int splits)
{
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n)
        return;
    float4 acc = *(const float4 *)(P + i);
    for (int s = 1; s < splits; s++) {
        const float4 v = *(const float4 *)(P + (size_t)s * n + i);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    *(float4 *)(Y + i) = acc;
}

// Tile rows and K values per stage for a batch of B rows (see k_gemm_nt; the
// wave count and stage count follow from these in launch_gemm_cfg).
struct Ffn2dCfg {
    int bm, kb;
};
static Ffn2dCfg ffn2d_cfg(int B)
{
    if (B <= 256)
        return {64, 64};
    if (B <= 1024)
        return {128, 64};
    if (B < 4096)
        return {128, 32};
    // 256 x 288 tiles: each operand tile is fetched from L2 for half as many
    // partner tiles in M as with 128-row tiles; 64 K values a stage, two stages
    return {256, 64};
}

// The down-projection's tiles: 64 rows up to 1024 (twice the output tiles of
// 128-row tiles, so half the K splits and half the fp32 partials written and
// read back), else those of the up-projection.
static Ffn2dCfg ffn2d_cfg_down(int B)
{
    if (B <= 1024)
        return {64, 64};
    return ffn2d_cfg(B);
}

// Number of K splits of the down-projection for a batch of B rows: enough
// workgroups for the 256 CUs when the output has few tiles.
int ffn2d_splits(int B, int E, int F)
{
    const Ffn2dCfg c = ffn2d_cfg_down(B);
    const int tiles = ((B + c.bm - 1) / c.bm) * (E / kBN);
    int s = 256 / (tiles > 0 ? tiles : 1);
    s = s < 1 ? 1 : s > 8 ? 8 : s;
    const int ksteps = F / c.kb;
    return s > ksteps ? ksteps : s;
}

template <int EPI, int BM, int KB, int NWV = 4, int NST = 3, int KS = 1>
static void launch_gemm(const GemmArgs &g, dim3 grid, hipStream_t st)
{
    hipLaunchKernelGGL((k_gemm_nt<EPI, BM, KB, NWV, NST, KS>), grid, dim3(64 * NWV), 0, st, g);
}

// 256 rows: 16 waves, two stages; 64 rows: two k-groups of 8 waves; 128 rows:
// 8 waves with 64-K stages, 4 (occupancy 2) with 32-K stages.
template <int EPI>
static void launch_gemm_cfg(const Ffn2dCfg &c, const GemmArgs &g, dim3 grid, hipStream_t st)
{
    if (c.bm == 256)
        launch_gemm<EPI, 256, 64, 16, 2>(g, grid, st);
    else if (c.bm == 64)
        launch_gemm<EPI, 64, 64, 16, 3, 2>(g, grid, st);
    else if (c.kb == 64)
        launch_gemm<EPI, 128, 64, 8>(g, grid, st);
    else
        launch_gemm<EPI, 128, 32>(g, grid, st);
}

// which = 0: up-projection + SwiGLU into a.h; which = 1: down-projection
// into a.y (through the split partials in a.part when splitting).
// Host-checked: E % 288 == 0, (2F) % 288 == 0, E and F multiples of 64.
hipError_t launch_ffn2d(const Ffn2dArgs &f, hipStream_t st, int which)
{
    const Ffn2dCfg c = ffn2d_cfg(f.B);
    const int mt = (f.B + c.bm - 1) / c.bm;
    if (which == 0) {
        GemmArgs g{f.x, f.w13, f.h, nullptr, f.B, 2 * f.F, f.E, f.E / c.kb, 0, 1};
        launch_gemm_cfg<FFN_UP>(c, g, dim3(2 * f.F / kBN, mt, 1), st);
        return hipGetLastError();
    }
    const Ffn2dCfg cd = ffn2d_cfg_down(f.B);
    const int mtd = (f.B + cd.bm - 1) / cd.bm;
    const int S = ffn2d_splits(f.B, f.E, f.F);
    const int ksteps = f.F / cd.kb;
    const int per = (ksteps + S - 1) / S;
    const int splits = (ksteps + per - 1) / per;
    GemmArgs g{f.h, f.w2, nullptr, splits > 1 ? f.part : f.y, f.B, f.E, f.F, per, 0, 1};
    const int ntd = f.E / kBN;
    if (splits > 1 && 8 % splits == 0 && ntd % (8 / splits) == 0) {
        g.map = 1;
    } else if (splits == 1 && mtd % 8 == 0 && f.B >= 2 * f.E) {
        // an XCD then fetches 1/8 of H and all of W_out instead of all of H
        // and 1/8 of W_out: fewer bytes when H has at least twice the rows
        // (8192 tokens: 339 -> 307 us; at E = F' = B = 18432, where the two
        // are equal, grid order was faster: 11.2 against 12.5 ms)
        g.map = 2;
        g.gm = 8;
    }
    launch_gemm_cfg<FFN_DOWN>(cd, g, dim3(ntd, mtd, splits), st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1)
        return e;
    const size_t n = (size_t)f.B * f.E;
    hipLaunchKernelGGL(k_split_reduce, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st,
                       (const float *)f.part, f.y, n, splits);
    return hipGetLastError();
}

} // namespace tps
