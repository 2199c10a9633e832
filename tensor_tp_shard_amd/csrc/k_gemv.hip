// k_gemv.hip -- weight-streaming matrix-vector products of the shard step
// (small batch, B <= 16): y[b][n] = sum_k W[n][k] x[b][k].
//
// Pages: aiterms.tw "Tensor Parallelism", 核心概念 items 1-2 (a column-split
// shard owns whole output rows of Wq/Wk/Wv/W1/W3; a row-split shard owns a
// column block of Wo/W2 and produces a full-size partial) and 運作原理 (the
// FFN: column-split Linear1, elementwise activation, row-split Linear2);
// distributed-llama issue "[Feature Suggest] Tensor Parallellism for
// Accelerating LLM", buildLlama2Arch tasks llamaQkv, llamaAttOutput, llamaFfn
// ("Compute SwiGLU activation"), llamaFfn2.
//
// Design (HBM-bound; one weight byte is used B times):
//  - one wave per group of RPW consecutive rows; the 64 lanes stride the row
//    in 16-byte vectors, so one wave instruction reads 1 KiB of contiguous
//    weights (nontemporal: every weight is read once per step);
//  - U chunk-iterations of loads are issued before any arithmetic, keeping
//    U*RPW*1 KiB in flight per wave;
//  - the activation rows x[b] (fp32, a few KiB, L1/L2 resident) are read
//    with 16-byte loads matching the weight chunk;
//  - fp32 accumulation, then a 64-lane butterfly per output;
//  - SwiGLU epilogue: the packed up-projection interleaves W1 row f and W3
//    row f, so a wave with RPW = 2 holds both and writes silu(g) * u.
#include "common.h"

namespace tps {

template <bool BF16>
__device__ __forceinline__ void load_x(const float *xrow, int c, float (&xv)[BF16 ? 8 : 4])
{
    const float4 *p = (const float4 *)xrow + c * (BF16 ? 2 : 1);
    const float4 a = p[0];
    xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
    if constexpr (BF16) {
        const float4 b = p[1];
        xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
    }
}

template <bool BF16>
__device__ __forceinline__ float dot16(const u32x4 &w, const float (&xv)[BF16 ? 8 : 4], float acc)
{
    if constexpr (BF16) {
        acc += bf16_lo(w.x) * xv[0];
        acc += bf16_hi(w.x) * xv[1];
        acc += bf16_lo(w.y) * xv[2];
        acc += bf16_hi(w.y) * xv[3];
        acc += bf16_lo(w.z) * xv[4];
        acc += bf16_hi(w.z) * xv[5];
        acc += bf16_lo(w.w) * xv[6];
        acc += bf16_hi(w.w) * xv[7];
    } else {
        acc += __uint_as_float(w.x) * xv[0];
        acc += __uint_as_float(w.y) * xv[1];
        acc += __uint_as_float(w.z) * xv[2];
        acc += __uint_as_float(w.w) * xv[3];
    }
    return acc;
}

template <bool BF16, int NB, int RPW, int EPI>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a)
{
    constexpr int V = BF16 ? 8 : 4; // elements per 16-byte chunk
    constexpr int U = 4;            // chunk iterations loaded ahead
    const int lane = threadIdx.x & 63;
    const int row0 = ((blockIdx.x * 256 + threadIdx.x) >> 6) * RPW;
    if (row0 >= a.N)
        return;
    const int nchunk = a.K / V;
    const u32x4 *Wr[RPW];
#pragma unroll
    for (int r = 0; r < RPW; r++)
        Wr[r] = (const u32x4 *)((const char *)a.W + (size_t)(row0 + r) * a.K * (BF16 ? 2 : 4));

    float acc[RPW][NB];
#pragma unroll
    for (int r = 0; r < RPW; r++)
#pragma unroll
        for (int b = 0; b < NB; b++)
            acc[r][b] = 0.f;

    int c = lane;
    for (; c + 64 * (U - 1) < nchunk; c += 64 * U) {
        u32x4 w[U][RPW];
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
            for (int r = 0; r < RPW; r++)
                w[u][r] = __builtin_nontemporal_load(Wr[r] + c + 64 * u);
#pragma unroll
        for (int u = 0; u < U; u++) {
#pragma unroll
            for (int b = 0; b < NB; b++) {
                if (b < a.B) {
                    float xv[V];
                    load_x<BF16>(a.x + (size_t)b * a.ldx, c + 64 * u, xv);
#pragma unroll
                    for (int r = 0; r < RPW; r++)
                        acc[r][b] = dot16<BF16>(w[u][r], xv, acc[r][b]);
                }
            }
        }
    }
    for (; c < nchunk; c += 64) {
        u32x4 w[RPW];
#pragma unroll
        for (int r = 0; r < RPW; r++)
            w[r] = __builtin_nontemporal_load(Wr[r] + c);
#pragma unroll
        for (int b = 0; b < NB; b++) {
            if (b < a.B) {
                float xv[V];
                load_x<BF16>(a.x + (size_t)b * a.ldx, c, xv);
#pragma unroll
                for (int r = 0; r < RPW; r++)
                    acc[r][b] = dot16<BF16>(w[r], xv, acc[r][b]);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < RPW; r++)
#pragma unroll
        for (int b = 0; b < NB; b++)
            acc[r][b] = group_sum<64>(acc[r][b]);

    if constexpr (EPI == EPI_SWIGLU) {
        static_assert(RPW == 2, "SwiGLU pairs rows (W1_f, W3_f)");
        const int f = row0 / 2;
#pragma unroll
        for (int b = 0; b < NB; b++) {
            if (lane == b && b < a.B) {
                const float v = silu(acc[0][b]) * acc[1][b];
                a.y[(size_t)b * a.ldy + f] = v;
                if (a.tap)
                    a.tap[(size_t)b * a.ldy + f] = v;
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < RPW; r++)
#pragma unroll
            for (int b = 0; b < NB; b++) {
                if (lane == r * NB + b && b < a.B) {
                    a.y[(size_t)b * a.ldy + row0 + r] = acc[r][b];
                    if (a.tap)
                        a.tap[(size_t)b * a.ldy + row0 + r] = acc[r][b];
                }
            }
    }
}

template <bool BF16, int NB>
static hipError_t launch_nb(const GemvArgs &a, int epi, hipStream_t st)
{
    constexpr int RPW = 2;
    const int waves = (a.N + RPW - 1) / RPW;
    const dim3 grid((waves + 3) / 4), block(256);
    if (epi == EPI_SWIGLU)
        hipLaunchKernelGGL((k_gemv<BF16, NB, RPW, EPI_SWIGLU>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((k_gemv<BF16, NB, RPW, EPI_STORE>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_t(const GemvArgs &a, int epi, hipStream_t st)
{
    if (a.B <= 1)
        return launch_nb<BF16, 1>(a, epi, st);
    if (a.B <= 2)
        return launch_nb<BF16, 2>(a, epi, st);
    if (a.B <= 4)
        return launch_nb<BF16, 4>(a, epi, st);
    if (a.B <= 8)
        return launch_nb<BF16, 8>(a, epi, st);
    return launch_nb<BF16, 16>(a, epi, st);
}

// Host-checked preconditions: N even, K a multiple of the 16-byte vector,
// rows 16-byte aligned, 1 <= B <= 16.
hipError_t launch_gemv(const GemvArgs &a, int w_bf16, int epi, hipStream_t st)
{
    return w_bf16 ? launch_t<true>(a, epi, st) : launch_t<false>(a, epi, st);
}

} // namespace tps
