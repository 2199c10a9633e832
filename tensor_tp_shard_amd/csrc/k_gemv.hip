// k_gemv.hip -- weight-streaming matrix-vector products of the shard step
// (decode batch B <= 16): y[b][n] = sum_k W[n][k] x[b][k].
//
// Pages: aiterms.tw "Tensor Parallelism", 核心概念 items 1-2 (a column-split
// shard owns whole output rows of Wq/Wk/Wv/W1/W3; a row-split shard owns a
// column block of Wo/W2 and produces a full-size partial) and 運作原理 (the
// FFN: column-split Linear1, elementwise activation, row-split Linear2);
// distributed-llama issue "[Feature Suggest] Tensor Parallellism for
// Accelerating LLM", buildLlama2Arch tasks llamaRmsAttNorm / llamaRmfFfnNorm
// (fused here as the prologue of the projection that consumes the normalised
// row), llamaQuantizeRmsAtt / llamaQuantizeRmfFfn (int8 round trip of that
// row), llamaQkv, llamaAttOutput, llamaFfn (the SwiGLU activation),
// llamaFfn2.
//
// Design (HBM-bound: every weight byte is read once and used B times):
//  - one wave per RPW consecutive rows (1, or 2 for SwiGLU); the 64 lanes
//    stride a row in 16-byte vectors, so one wave instruction reads 1 KiB of
//    contiguous weights (nontemporal: read once per step);
//  - all of a wave's weight vectors for up to KC x 1 KiB of each row are
//    issued before anything waits on them, unconditionally, through a
//    buffer resource per row (a lane past the row end reads zeros without a
//    memory access): with no branch around them the compiler counts them
//    exactly, so staging the activations waits only for the activation
//    loads issued ahead of the weights, not for every weight as it did with
//    predicated loads (7B shard step 41.2 -> 39.9 us);
//  - the activation rows are staged once per workgroup in LDS (fp32) while
//    the weights are in flight; with the fused RMSNorm every workgroup
//    recomputes the row's sum of squares from L2 (B*K*4 bytes), which is
//    cheaper than a separate launch;
//  - fp32 accumulation, one 64-lane butterfly per output;
//  - SwiGLU epilogue: the packed up-projection interleaves W1 row f and W3
//    row f, so a wave with RPW = 2 holds both and writes silu(g) * u;
#include "gemv_lds.h"

namespace tps {

// NW waves per workgroup, one (RPW rows) per wave
template <int WT, int NB, int RPW, int EPI, bool MO, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemv_lds(GemvArgs a)
{
    extern __shared__ __attribute__((aligned(16))) float xs[]; // [B][K]
    gemv_lds_body<WT, NB, RPW, EPI, MO, NW>(a, blockIdx.x, xs, nullptr, 0u);
}

// ---------------------------------------------------------------- general-batch path
// Activations read from global memory (L1/L2 resident), no fused prologue /
// epilogue: used when the batch's activation rows do not fit in LDS.

template <int WT, int NB, int RPW, int EPI, bool MO>
__global__ __launch_bounds__(256) void k_gemv_gx(GemvArgs a)
{
    constexpr int V = wt_per_chunk(WT);
    constexpr int U = 4;
    const int lane = threadIdx.x & 63;
    const int row0 = ((blockIdx.x * 256 + threadIdx.x) >> 6) * RPW;
    if (a.epoch && blockIdx.x == 0 && threadIdx.x == 0)
        a.epoch[0] = (a.epoch[0] + 1u) & 0x7fffffffu;
    if (row0 >= a.N)
        return;
    float mres = 0.f;
    uint2 mpre[kMO];
    if constexpr (MO) {
        const int mr = lane / NB, mb = lane % NB;
        if (lane < RPW * NB && mb < a.B)
            merge_preload1<false>(a.mo, (size_t)mb * a.ldy + row0 + mr, mres, mpre);
    }
    const int nchunk = a.K / V;
    const u32x4 *Wr[RPW];
#pragma unroll
    for (int r = 0; r < RPW; r++)
        Wr[r] = (const u32x4 *)((const char *)a.W + (size_t)(row0 + r) * a.K * 16 / V);
    float acc[RPW][NB];
#pragma unroll
    for (int r = 0; r < RPW; r++)
#pragma unroll
        for (int b = 0; b < NB; b++)
            acc[r][b] = 0.f;
    for (int c0 = lane; c0 < nchunk; c0 += 64 * U) {
        u32x4 w[U][RPW];
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
            for (int r = 0; r < RPW; r++)
                if (c0 + 64 * u < nchunk)
                    w[u][r] = __builtin_nontemporal_load(Wr[r] + c0 + 64 * u);
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int c = c0 + 64 * u;
            if (c < nchunk) {
#pragma unroll
                for (int b = 0; b < NB; b++) {
                    if (b < a.B) {
                        const float4 *xp = (const float4 *)(a.x + (size_t)b * a.ldx) + c * (V / 4);
#pragma unroll
                        for (int r = 0; r < RPW; r++)
                            acc[r][b] = dot_chunk<WT>(w[u][r], xp,
                                                      WT == WT_I8 ? a.ws[(size_t)(row0 + r) * (a.K / 32) + (c >> 1)] : 1.f,
                                                      acc[r][b]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RPW; r++)
#pragma unroll
        for (int b = 0; b < NB; b++)
            acc[r][b] = group_sum<64>(acc[r][b]);
    if constexpr (EPI == EPI_SWIGLU) {
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
                    if constexpr (MO)
                        merge_finish1<false>(a.mo, (size_t)b * a.ldy + row0 + r, acc[r][b], mres, mpre);
                }
            }
    }
}

// ---------------------------------------------------------------- launchers

constexpr int kRPW = 2;

size_t gemv_lds_bytes(int B, int K) { return (size_t)B * K * sizeof(float); }

bool gemv_fused_ok(int B, int K) { return B <= 4 && K <= 4 * 256 * kXV && gemv_lds_bytes(B, K) <= 64 * 1024; }

// One row per wave for the plain-store projections (QKV, W_O, W2): twice the
// waves of two rows per wave, each with a whole row of loads in flight
// (7B shard step 42.2 -> 41.1 us); the SwiGLU projection pairs W1_f / W3_f
// rows in one wave. Four waves a workgroup; eight for a plain store of at
// least 6144 rows (the 7B shard's 8000 classifier rows: 14.5 -> 14.1 us, the
// activations staged by half as many workgroups), where the grid still has
// three workgroups a CU: with eight waves the W1/W3 projection (344
// workgroups) went 11.2 -> 11.9 us and the QKV one 8.0 -> 8.1 us; two waves
// were slower everywhere (W1/W3 15.6 us).
template <int WT, int NB>
static hipError_t launch_lds(const GemvArgs &a, int epi, hipStream_t st)
{
    const size_t sm = gemv_lds_bytes(a.B, a.K);
    if (epi == EPI_Q8) { // 32-row workgroups: eight waves of four rows (sixteen waves of two
                         // rows were slower: 7B int8-wire step 45.8 -> 49.4 us)
        if (a.mo.n_wires)
            hipLaunchKernelGGL((k_gemv_lds<WT, NB, 4, EPI_Q8, true, 8>), dim3((a.N + 31) / 32), dim3(512), sm,
                               st, a);
        else
            hipLaunchKernelGGL((k_gemv_lds<WT, NB, 4, EPI_Q8, false, 8>), dim3((a.N + 31) / 32), dim3(512), sm,
                               st, a);
    } else if (epi == EPI_SWIGLU) {
        const dim3 grid((a.N + 4 * kRPW - 1) / (4 * kRPW));
        hipLaunchKernelGGL((k_gemv_lds<WT, NB, kRPW, EPI_SWIGLU, false, 4>), grid, dim3(256), sm, st, a);
    } else if (a.mo.n_wires) {
        hipLaunchKernelGGL((k_gemv_lds<WT, NB, 1, EPI_STORE, true, 4>), dim3((a.N + 3) / 4), dim3(256), sm,
                           st, a);
    } else if (a.N >= 6144) {
        hipLaunchKernelGGL((k_gemv_lds<WT, NB, 1, EPI_STORE, false, 8>), dim3((a.N + 7) / 8), dim3(512), sm,
                           st, a);
    } else {
        hipLaunchKernelGGL((k_gemv_lds<WT, NB, 1, EPI_STORE, false, 4>), dim3((a.N + 3) / 4), dim3(256), sm,
                           st, a);
    }
    return hipGetLastError();
}

template <int WT, int NB>
static hipError_t launch_gx(const GemvArgs &a, int epi, hipStream_t st)
{
    const int waves = (a.N + kRPW - 1) / kRPW;
    const dim3 grid((waves + 3) / 4), block(256);
    if (epi == EPI_SWIGLU)
        hipLaunchKernelGGL((k_gemv_gx<WT, NB, kRPW, EPI_SWIGLU, false>), grid, block, 0, st, a);
    else if (a.mo.n_wires)
        hipLaunchKernelGGL((k_gemv_gx<WT, NB, kRPW, EPI_STORE, true>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((k_gemv_gx<WT, NB, kRPW, EPI_STORE, false>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int WT>
static hipError_t launch_t(const GemvArgs &a, int epi, hipStream_t st)
{
    if (gemv_fused_ok(a.B, a.K)) {
        if (a.B <= 1)
            return launch_lds<WT, 1>(a, epi, st);
        if (a.B <= 2)
            return launch_lds<WT, 2>(a, epi, st);
        return launch_lds<WT, 4>(a, epi, st);
    }
    if (a.g || epi == EPI_Q8)
        return hipErrorInvalidValue; // the fused norm and the int8 epilogue need the LDS path
    if (a.B <= 8)
        return launch_gx<WT, 8>(a, epi, st);
    return launch_gx<WT, 16>(a, epi, st);
}

// Host-checked preconditions: N a multiple of 8, K a
// multiple of the 16-byte vector (of 32 with qin), rows 16-byte aligned,
// 1 <= B <= 16; a fused merge (mo.n_wires > 0) only with EPI_STORE and fp32
// wires.
hipError_t launch_gemv(const GemvArgs &a, int wt, int epi, hipStream_t st)
{
    if (wt == WT_I8)
        return launch_t<WT_I8>(a, epi, st);
    return wt == WT_BF16 ? launch_t<WT_BF16>(a, epi, st) : launch_t<WT_F32>(a, epi, st);
}

} // namespace tps
