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
//  - workgroup tile 128 x 256, four waves as 2 x 2, wave tile 64 x 128
//    (4 x 8 MFMA tiles, 128 fp32 accumulators per lane), K step 64;
//  - the next K step's tiles are loaded into registers (16-byte global
//    loads) while the current one is multiplied from LDS; LDS rows are 128
//    bytes with the 16-byte chunk index XOR-swizzled by (row & 7), so the
//    fragment reads (16 rows x 16 bytes per 8-lane phase) are conflict-free;
//  - tile order puts the M-tiles of one N-tile on the same XCD (linear
//    workgroup id % 8), so a weight tile is fetched into one L2 once;
//  - up-projection epilogue: the packed W_gate/W_in rows interleave in
//    groups of 8 inside each 16-row MFMA tile, so lanes n and n ^ 8 hold the
//    gate and the up value of the same feature: h = silu(g) * u, stored bf16;
//  - down-projection at small M: deterministic split-K, fp32 partials summed
//    in split order by a reduce kernel.
#include "common.h"

namespace tps {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 256, kBK = 64;
constexpr int kMT = 4, kNT = 8;                                // MFMA tiles per wave (64 x 128)
constexpr int kChunksA = kBM * kBK / 8, kChunksB = kBN * kBK / 8; // 16-byte chunks per K step
constexpr int kLoads = (kChunksA + kChunksB) / 256;            // per thread (12)

enum { FFN_UP = 0, FFN_DOWN = 1 };

struct GemmArgs {
    const uint16_t *A; // [M][K]
    const uint16_t *B; // [N][K]
    uint16_t *H;       // FFN_UP: [M][N/2] bf16
    float *C;          // FFN_DOWN: [splits][M][N] fp32
    int M, N, K, ksteps_per_split;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK * 2 + ((chunk ^ (row & 7)) << 4); }

template <int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm_nt(GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) char As[kBM * kBK * 2];
    __shared__ __attribute__((aligned(16))) char Bs[kBN * kBK * 2];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    // grid: x = N-tile (fastest, so the M-tiles of one N-tile share id % 8), y = M-tile, z = split
    const int n0 = blockIdx.x * kBN, m0 = blockIdx.y * kBM;
    const int ks0 = blockIdx.z * a.ksteps_per_split;
    const int nks = min(a.ksteps_per_split, a.K / kBK - ks0);

    f32x4 acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; i++)
#pragma unroll
        for (int j = 0; j < kNT; j++)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // global chunk ids of this thread: id < kChunksA are A chunks, the rest B
    u32x4 pre[kLoads];
    auto load_step = [&](int ks) {
        const int kbase = (ks0 + ks) * kBK;
#pragma unroll
        for (int i = 0; i < kLoads; i++) {
            const int id = tid + 256 * i;
            if (id < kChunksA) {
                const int row = id >> 3, ch = id & 7;
                const int m = m0 + row;
                if (m < a.M)
                    pre[i] = *(const u32x4 *)(a.A + (size_t)m * a.K + kbase + ch * 8);
                else
                    pre[i] = u32x4{0u, 0u, 0u, 0u};
            } else {
                const int idb = id - kChunksA;
                const int row = idb >> 3, ch = idb & 7;
                pre[i] = __builtin_nontemporal_load(
                    (const u32x4 *)(a.B + (size_t)(n0 + row) * a.K + kbase + ch * 8));
            }
        }
    };
    auto store_step = [&]() {
#pragma unroll
        for (int i = 0; i < kLoads; i++) {
            const int id = tid + 256 * i;
            if (id < kChunksA)
                *(u32x4 *)(As + swz(id >> 3, id & 7)) = pre[i];
            else
                *(u32x4 *)(Bs + swz((id - kChunksA) >> 3, (id - kChunksA) & 7)) = pre[i];
        }
    };

    if (nks > 0)
        load_step(0);
    for (int ks = 0; ks < nks; ks++) {
        __syncthreads(); // the previous step's fragment reads are done
        store_step();
        __syncthreads();
        if (ks + 1 < nks)
            load_step(ks + 1);
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
            const int ch = kk * 4 + (lane >> 4);
            bf16x8 af[kMT], bfr[kNT];
#pragma unroll
            for (int i = 0; i < kMT; i++) {
                const int row = wm * 64 + i * 16 + (lane & 15);
                af[i] = *(const bf16x8 *)(As + swz(row, ch));
            }
#pragma unroll
            for (int j = 0; j < kNT; j++) {
                const int row = wn * 128 + j * 16 + (lane & 15);
                bfr[j] = *(const bf16x8 *)(Bs + swz(row, ch));
            }
#pragma unroll
            for (int i = 0; i < kMT; i++)
#pragma unroll
                for (int j = 0; j < kNT; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }

    // lane holds C[m0 + wm*64 + i*16 + 4*(lane/16) + r][n0 + wn*128 + j*16 + lane%16]
    const int col = lane & 15, rq = (lane >> 4) * 4;
    if constexpr (EPI == FFN_UP) {
        const int F = a.N / 2;
#pragma unroll
        for (int i = 0; i < kMT; i++)
#pragma unroll
            for (int j = 0; j < kNT; j++) {
                const int tile = (n0 + wn * 128 + j * 16) / 16;
                const int f = tile * 8 + (col & 7);
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const float mine = acc[i][j][r];
                    const float other = __shfl_xor(mine, 8, 64); // lanes col and col ^ 8
                    const int m = m0 + wm * 64 + i * 16 + rq + r;
                    if (col < 8 && m < a.M)
                        a.H[(size_t)m * F + f] = f32_to_bf16(silu(mine) * other);
                }
            }
    } else {
        float *C = a.C + (size_t)blockIdx.z * a.M * a.N;
#pragma unroll
        for (int i = 0; i < kMT; i++)
#pragma unroll
            for (int j = 0; j < kNT; j++) {
                const int n = n0 + wn * 128 + j * 16 + col;
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int m = m0 + wm * 64 + i * 16 + rq + r;
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

// Number of K splits of the down-projection for a batch of B rows: enough
// workgroups for the 256 CUs when the output has few tiles.
int ffn2d_splits(int B, int E, int F)
{
    const int tiles = ((B + kBM - 1) / kBM) * (E / kBN);
    int s = 256 / (tiles > 0 ? tiles : 1);
    s = s < 1 ? 1 : s > 8 ? 8 : s;
    const int ksteps = F / kBK;
    return s > ksteps ? ksteps : s;
}

// which = 0: up-projection + SwiGLU into a.h; which = 1: down-projection
// into a.y (through the split partials in a.part when splitting).
// Host-checked: E % 256 == 0, F % 128 == 0, E and F multiples of 64.
hipError_t launch_ffn2d(const Ffn2dArgs &f, hipStream_t st, int which)
{
    const int mt = (f.B + kBM - 1) / kBM;
    if (which == 0) {
        GemmArgs g{f.x, f.w13, f.h, nullptr, f.B, 2 * f.F, f.E, f.E / kBK};
        hipLaunchKernelGGL(k_gemm_nt<FFN_UP>, dim3(2 * f.F / kBN, mt, 1), dim3(256), 0, st, g);
        return hipGetLastError();
    }
    const int S = ffn2d_splits(f.B, f.E, f.F);
    const int ksteps = f.F / kBK;
    const int per = (ksteps + S - 1) / S;
    const int splits = (ksteps + per - 1) / per;
    GemmArgs g{f.h, f.w2, nullptr, splits > 1 ? f.part : f.y, f.B, f.E, f.F, per};
    hipLaunchKernelGGL(k_gemm_nt<FFN_DOWN>, dim3(f.E / kBN, mt, splits), dim3(256), 0, st, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1)
        return e;
    const size_t n = (size_t)f.B * f.E;
    hipLaunchKernelGGL(k_split_reduce, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st,
                       (const float *)f.part, f.y, n, splits);
    return hipGetLastError();
}

} // namespace tps
