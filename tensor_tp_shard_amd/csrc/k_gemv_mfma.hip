// k_gemv_mfma.hip -- the shard's projections for a decode batch of 5..16
// sequences on bf16 MFMA: y[b][n] = sum_k W[n][k] x[b][k].
//
// Pages: aiterms.tw "Tensor Parallelism", 核心概念 items 1-2 and 運作原理
// (column- and row-split projections of one shard); distributed-llama issue
// "[Feature Suggest] Tensor Parallellism for Accelerating LLM",
// buildLlama2Arch tasks llamaQkv, llamaAttOutput, llamaFfn (SwiGLU),
// llamaFfn2.
//
// Why MFMA here: with 16 sequences every weight feeds 16 multiply-adds, and
// at the HBM rate (2.8 T bf16 weights/s at 70% of 8 TB/s) that is 45 T FMA/s,
// more than the chip's non-packed fp32 vector rate (39 T FMA/s). A batch of
// 16 times a weight block is a dense 16-row contraction, the shape of
// v_mfma_f32_16x16x32_bf16. Weights are the A operand (16 rows per tile),
// the 16 batch rows the B operand. The fp32 activations enter as bf16 hi and
// lo parts (two MFMAs per step), so the product carries ~16 mantissa bits of
// every activation with fp32 accumulation -- fp32-class accuracy. The
// activations are written in the fragment layout once by their producer
// (RMSNorm, attention combine, SwiGLU).
//
// Work split: one workgroup per T 16-row tiles (T = 2 for the large
// projections, sharing each activation fragment between two tiles), its wk
// waves split K in 128-wide blocks (about 8 per wave); a wave keeps two
// blocks of weights (16-byte nontemporal loads; per load instruction the 4
// lanes of a row read 64 contiguous bytes of it) and their activation
// fragments in flight, then the waves' 16x16 accumulators are summed in wave
// order through LDS. Epilogues: store, or SwiGLU of the interleaved
// (W1_f, W3_f) rows (accumulator rows 4q..4q+3 of a lane are two pairs).
#include "common.h"

namespace tps {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxWk = 16;

// Eight int8 codes -> the bf16 MFMA operand, biased: u = code + 128 (the
// sign bit flipped, one xor per four codes) as exact bf16 integers in
// [1, 255], one unsigned-byte conversion to fp32 per code and one packed
// fp32 -> bf16 conversion per two. The product then carries 128 times the
// block's activation sum too, taken out by starting the accumulator at
// x . (-128) (kNeg128, an MFMA per activation half shared by the step's tiles).
__device__ __forceinline__ bf16x8 i8x8_to_bf16_biased(u32x2 v)
{
    const uint32_t lo = v.x ^ 0x80808080u, hi = v.y ^ 0x80808080u;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; e++)
        o[e] = (__bf16)(float)(((e < 4 ? lo : hi) >> (8 * (e & 3))) & 0xffu);
    return o;
}

// -128 in every element of a bf16 MFMA operand
__device__ __forceinline__ bf16x8 neg128_bf16x8()
{
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; e++)
        o[e] = (__bf16)(-128.f);
    return o;
}

// T = 16-row weight tiles per wave sharing each activation fragment (1 or
// 2): two tiles halve the activation bytes the waves pull from L2 per weight
// byte; the register cost limits such workgroups to 8 waves.
// W8: int8 codes with a scale per 32 k of a row. MFMA step s of 128-block j
// then covers exactly the 32-block 4j + s (lane q holds its codes 8q..8q+7,
// 8 contiguous bytes), so each step's product goes through an accumulator
// of its own (started at the step's -128 x correction of the biased codes,
// shared by the step's tiles) and is added times the scale. The operands swap roles
// (activations A, weights B): lane (q, r) then holds batches 4q..4q+3 of the
// single weight row r, whose scale is one value per step; the partial sums
// go to the reduction buffer in the usual (row 4q + i, batch r) places.
// (At most 8 waves for W8: its conversions need more than the 128 registers
// a 16-wave workgroup leaves.)
constexpr int mfma_max_waves(int T, bool W8) { return T == 1 && !W8 ? kMaxWk : 8; }

template <int EPI, int T, bool W8>
__global__ __launch_bounds__(64 * mfma_max_waves(T, W8)) void k_gemv_mfma(MfmaGemvArgs a)
{
    constexpr int P = 2; // 128-wide K blocks in flight per wave
    __shared__ f32x4 red[mfma_max_waves(T, W8)][T][64];
    const int n0 = blockIdx.x * 16 * T;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4, r = lane & 15;
    const int nb = a.K >> 7;
    const int per = (nb + a.wk - 1) / a.wk;
    const int j0 = wv * per, j1 = min(nb, j0 + per);
    const u32x4 *wrow[T];
    const u32x2 *w8row[T];
    const float *srow[T]; // W8: scales of the lane's weight row r of tile t
#pragma unroll
    for (int t = 0; t < T; t++) {
        wrow[t] = (const u32x4 *)(a.W + (size_t)(n0 + 16 * t + r) * a.K + 8 * q);
        w8row[t] = (const u32x2 *)((const int8_t *)a.W + (size_t)(n0 + 16 * t + r) * a.K + 8 * q);
        srow[t] = W8 ? a.ws + (size_t)(n0 + 16 * t + r) * (a.K / 32) : nullptr;
    }
    const u32x4 *xf = (const u32x4 *)a.xf; // 16-byte units: [j][hl][s][q][b]
    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; t++)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = j0; j < j1; j += P) {
        u32x4 w[P][T][4], xh[P][4], xl[P][4];
        u32x2 w8[P][T][4];
        float4 sc[P][T]; // W8: row r's scales of the block's four 32-blocks
#pragma unroll
        for (int p = 0; p < P; p++)
            if (j + p < j1)
#pragma unroll
                for (int t = 0; t < T; t++)
#pragma unroll
                    for (int s = 0; s < 4; s++) {
                        if constexpr (W8) {
                            w8[p][t][s] = __builtin_nontemporal_load(w8row[t] + (size_t)(j + p) * 16 + 4 * s);
                            if (s == 0)
                                sc[p][t] = *(const float4 *)(srow[t] + 4 * (j + p));
                        } else {
                            w[p][t][s] = __builtin_nontemporal_load(wrow[t] + (size_t)(j + p) * 16 + 4 * s);
                        }
                    }
#pragma unroll
        for (int p = 0; p < P; p++)
            if (j + p < j1)
#pragma unroll
                for (int s = 0; s < 4; s++) {
                    xh[p][s] = xf[(((size_t)(j + p) * 2 + 0) * 4 + s) * 64 + lane];
                    xl[p][s] = xf[(((size_t)(j + p) * 2 + 1) * 4 + s) * 64 + lane];
                }
#pragma unroll
        for (int p = 0; p < P; p++)
            if (j + p < j1)
#pragma unroll
                for (int s = 0; s < 4; s++)
                {
                    f32x4 c0 = f32x4{0.f, 0.f, 0.f, 0.f};
                    if constexpr (W8) {
                        // c0[i] = -128 x (batch 4q + i) summed over the 32-block
                        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xh[p][s]), neg128_bf16x8(), c0, 0, 0, 0);
                        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xl[p][s]), neg128_bf16x8(), c0, 0, 0, 0);
                    }
#pragma unroll
                    for (int t = 0; t < T; t++) {
                        if constexpr (W8) {
                            const bf16x8 wb = i8x8_to_bf16_biased(w8[p][t][s]);
                            // d[i] = batch 4q + i of weight row r over 32-block 4 (j + p) + s
                            f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xh[p][s]), wb,
                                                                              c0, 0, 0, 0);
                            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xl[p][s]), wb, d, 0, 0, 0);
                            const float scv = sc[p][t][s];
                            acc[t][0] += scv * d[0];
                            acc[t][1] += scv * d[1];
                            acc[t][2] += scv * d[2];
                            acc[t][3] += scv * d[3];
                        } else {
                            const bf16x8 wa = __builtin_bit_cast(bf16x8, w[p][t][s]);
                            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, __builtin_bit_cast(bf16x8, xh[p][s]), acc[t], 0, 0, 0);
                            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, __builtin_bit_cast(bf16x8, xl[p][s]), acc[t], 0, 0, 0);
                        }
                    }
                }
    }
    // lane holds rows n0 + 16 t + 4q + i (i < 4) of batch column b = r
    const int b = r;
    // fused merge (EPI_STORE, fp32 wires): wave 0 requests the residual and
    // the other wires' elements of its outputs before the reduction
    constexpr int kM = EPI == EPI_STORE ? kMO : 1;
    const bool mlane = EPI == EPI_STORE && a.mo.n_wires && wv == 0 && b < a.B;
    float4 mres[T], mpre[T][kM];
    if (mlane) {
#pragma unroll
        for (int t = 0; t < T; t++) {
            const size_t mi = (size_t)b * a.ldy + n0 + 16 * t + 4 * q;
            mres[t] = *(const float4 *)(a.mo.residual + mi);
#pragma unroll
            for (int k = 0; k < kM; k++)
                if (k < a.mo.n_wires && k != a.mo.own)
                    mpre[t][k] = *(const float4 *)((const float *)a.mo.wires[k] + mi);
        }
    }
    if constexpr (W8) {
        // acc[t][i] = (row r, batch 4q + i) -> the place of lane (r / 4, b), element r % 4
#pragma unroll
        for (int t = 0; t < T; t++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                ((float *)&red[wv][t][(r >> 2) * 16 + 4 * q + i])[r & 3] = acc[t][i];
    } else {
#pragma unroll
        for (int t = 0; t < T; t++)
            red[wv][t][lane] = acc[t];
    }
    __syncthreads();
    if (wv != 0 || b >= a.B)
        return;
#pragma unroll
    for (int t = 0; t < T; t++) {
        const int nt = n0 + 16 * t;
        const size_t mi = (size_t)b * a.ldy + nt + 4 * q;
        f32x4 c = red[0][t][lane];
        for (int w = 1; w < a.wk; w++) {
            const f32x4 v = red[w][t][lane];
            c = f32x4{c[0] + v[0], c[1] + v[1], c[2] + v[2], c[3] + v[3]};
        }
        if constexpr (EPI == EPI_SWIGLU) {
            const int f = (nt >> 1) + 2 * q; // rows (4q, 4q+1) and (4q+2, 4q+3) are features f, f+1
            const float h0 = silu(c[0]) * c[1], h1 = silu(c[2]) * c[3];
            *(float2 *)(a.y + (size_t)b * a.ldy + f) = make_float2(h0, h1);
            if (a.tap)
                *(float2 *)(a.tap + (size_t)b * a.ldy + f) = make_float2(h0, h1);
            if (a.yf) {
                xf_store(a.yf, b, f, h0);
                xf_store(a.yf, b, f + 1, h1);
            }
        } else {
            const int n = nt + 4 * q;
            const float4 v = make_float4(c[0], c[1], c[2], c[3]);
            *(float4 *)(a.y + (size_t)b * a.ldy + n) = v;
            if (a.tap)
                *(float4 *)(a.tap + (size_t)b * a.ldy + n) = v;
            if (mlane) {
                float4 m = mres[t];
#pragma unroll
                for (int k = 0; k < kM; k++)
                    if (k < a.mo.n_wires) {
                        const float4 d = k == a.mo.own ? v : mpre[t][k];
                        m.x = m.x + d.x;
                        m.y = m.y + d.y;
                        m.z = m.z + d.z;
                        m.w = m.w + d.w;
                    }
                for (int k = kM; k < a.mo.n_wires; k++) {
                    const float4 d = k == a.mo.own ? v : *(const float4 *)((const float *)a.mo.wires[k] + mi);
                    m.x = m.x + d.x;
                    m.y = m.y + d.y;
                    m.z = m.z + d.z;
                    m.w = m.w + d.w;
                }
                *(float4 *)(a.mo.x_out + mi) = m;
            }
        }
    }
}

// ---------------------------------------------------------------- split K
// The batch-16 projections with many rows and a long K: a workgroup of 8
// waves takes 8 x T 16-row tiles and one K slice of nbs 128-blocks. The
// slice's activation fragments (nbs x 8 KiB) go to LDS once per workgroup
// (direct global->LDS loads, issued before the weights) and every wave reads
// its MFMA B operands there, so each activation byte leaves L2 once per
// workgroup instead of once per tile; the weights stream from HBM into
// registers as in k_gemv_mfma. Each slice's fp32 partial goes to a.part
// [S][B][N]; k_gemv_sk_epi sums the slices in order and applies the
// epilogue. (In a probe on the 70B up-projection shape the activations in
// LDS took the stream from 38 to 26 us.)
//
// RMSNorm folded in (the up-projections, xs set): RMSNorm is a per-row
// scale of x g, so W (g x / rms(x)) = (W (g x)) / rms(x). Each workgroup
// builds its slice's fragments of x g from the raw fp32 input (same bytes
// as the ready fragments), the workgroups of tile column 0 also store each
// row's sum of squares over their slice, and the reduce scales row b by
// 1 / sqrt(sum / K + eps). This drops the RMSNorm launch that had to finish
// before the projection (70B step 97.4 -> 88.9 us with the reduce below).
constexpr int kSkMaxNbs = 8;

// s_waitcnt vmcnt(N), other counters unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// NORM: the fragments are built here from the raw fp32 input (RMSNorm
// folded in, see MfmaGemvArgs::xs): thread u of the slice takes the 8
// consecutive k = 128 (jb + jl) + 32 s + 8 q of row b, where u = ((jl * 4 +
// s) * 4 + q) * 16 + b is also its 16-byte unit in the fragment layout;
// the workgroups of tile column 0 add up each row's squares over the slice.
template <int NW>
constexpr int sk_units() { return (kSkMaxNbs * 256 + 64 * NW - 1) / (64 * NW); } // 8-element units per thread

// W8: int8 weights as in k_gemv_mfma (each MFMA step one 32-block, operands
// swapped, the step's product times the row's scale); the lane's partials
// (row r, batches 4q..4q+3) are stored one by one.
// NW waves a workgroup (8, or 7 where that makes the tile columns times the
// slices fill the 256 CUs: 70B W1/W3, 224 -> 256 workgroups).
template <int T, int NW, bool NORM, bool W8>
__global__ __launch_bounds__(64 * NW) void k_gemv_sk(MfmaGemvArgs a)
{
    constexpr int kSkUnits = sk_units<NW>();
    constexpr int P = W8 ? 4 : 2; // 128-wide K blocks in flight per wave (the same bytes)
    __shared__ __attribute__((aligned(1024))) char lds[kSkMaxNbs * 8192];
    __shared__ float ssr[NORM ? 64 * NW : 1];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4, r = lane & 15;
    const int ks = blockIdx.y, jb = ks * a.nbs;
    const int nbl = min(a.nbs, (a.K >> 7) - jb); // blocks in this slice
    // every load below is unconditional (buffer loads, kOob past the data):
    // the compiler then counts outstanding loads exactly, so a wait for the
    // activations never also waits for weights issued after them
    u32x4 xv[NORM ? kSkUnits : 1][2], gv[NORM ? kSkUnits : 1][2];
    if constexpr (NORM) {
        const int b = threadIdx.x & 15;
        const __amdgpu_buffer_rsrc_t xr = buf_rsrc(a.xs, (uint32_t)a.B * a.K * 4);
        const __amdgpu_buffer_rsrc_t gr = buf_rsrc(a.g, (uint32_t)a.K * 4);
#pragma unroll
        for (int i = 0; i < kSkUnits; i++) {
            const int u = threadIdx.x + 64 * NW * i;
            const uint32_t k = (uint32_t)(jb << 7) + (u >> 4) * 8;
            const bool in = u < 256 * nbl;
            const uint32_t xo = in && b < a.B ? ((uint32_t)b * a.K + k) * 4 : kOob;
            xv[i][0] = buf_load16(xr, xo);
            xv[i][1] = buf_load16(xr, xo + 16);
            gv[i][0] = buf_load16(gr, in ? k * 4 : kOob);
            gv[i][1] = buf_load16(gr, in ? k * 4 + 16 : kOob);
        }
        __builtin_amdgcn_sched_barrier(0); // the activation loads stay ahead of the weights
    } else {
        // the slice's fragments: nbl x 8 KiB = 8 nbl wave loads of 1 KiB
        const u32x4 *xf = (const u32x4 *)a.xf + (size_t)jb * 512;
        for (int seg = wv; seg < 8 * nbl; seg += NW)
            __builtin_amdgcn_global_load_lds((const void *)(xf + (size_t)seg * 64 + lane),
                                             (__attribute__((address_space(3))) void *)(lds + seg * 1024), 16, 0, 0);
    }
    const int n0 = (blockIdx.x * NW + wv) * 16 * T;
    // one resource per 16-row tile from the slice start of its first row (wave
    // uniform, so the descriptor stays in scalar registers); lane (q, r) reads
    // row r at r K + 128 (block) + 32 s + 8 q elements, blocks past the slice
    // at kOob
    const int n0u = (blockIdx.x * NW + __builtin_amdgcn_readfirstlane(wv)) * 16 * T;
    // (W8: codes K bytes a row, the lane's 8 bytes of a step at 32 s + 8 q;
    // scales K / 32 floats a row, the block's four at 16 bytes)
    constexpr uint32_t eb = W8 ? 1 : 2; // bytes per weight
    // A tile past N (the last tile column of an N that is not a multiple of
    // its width) gets an empty resource: its loads return zeros, and it
    // stores nothing, while its wave still takes part in the barriers.
    __amdgpu_buffer_rsrc_t Wr[T], Sr[T];
#pragma unroll
    for (int t = 0; t < T; t++) {
        const bool live = n0u + 16 * t < a.N;
        Wr[t] = buf_rsrc(live ? (const char *)a.W + ((size_t)(n0u + 16 * t) * a.K + (size_t)jb * 128) * eb
                              : (const char *)a.W,
                         live ? (uint32_t)(16 * a.K - jb * 128) * eb : 0u);
        if constexpr (W8)
            Sr[t] = buf_rsrc(live ? a.ws + (size_t)(n0u + 16 * t) * (a.K / 32) + (size_t)jb * 4 : a.ws,
                             live ? (uint32_t)(16 * (a.K / 32) - jb * 4) * 4 : 0u);
    }
    const uint32_t lofs = W8 ? (uint32_t)r * a.K + 8 * q : (uint32_t)r * a.K * 2 + 16 * q;
    const uint32_t sofs = (uint32_t)r * (a.K / 32) * 4;
    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; t++)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int jl = 0; jl < nbl; jl += P) {
        u32x4 w[P][T][4];
        u32x2 w8[P][T][4];
        float4 sc[P][T];
#pragma unroll
        for (int p = 0; p < P; p++)
#pragma unroll
            for (int t = 0; t < T; t++) {
#pragma unroll
                for (int s = 0; s < 4; s++) {
                    if constexpr (W8)
                        w8[p][t][s] = buf_load8_nt(Wr[t], jl + p < nbl ? lofs + (uint32_t)(jl + p) * 128 + 32 * s : kOob);
                    else
                        w[p][t][s] = buf_load16_nt(Wr[t], jl + p < nbl ? lofs + (uint32_t)(jl + p) * 256 + 64 * s : kOob);
                }
                if constexpr (W8) {
                    const u32x4 v = buf_load16(Sr[t], jl + p < nbl ? sofs + (uint32_t)(jl + p) * 16 : kOob);
                    sc[p][t] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                                           __uint_as_float(v.w));
                }
            }
        // all P blocks' loads are issued before the first MFMA waits on one
        // (else the scheduler moves each load next to its use)
        __builtin_amdgcn_sched_barrier(0);
        if (jl == 0) {
            if constexpr (NORM) {
                // x g as bf16 hi / lo fragments into LDS (the compiler waits
                // for the activation loads only, issued before the weights)
                float ss = 0.f;
#pragma unroll
                for (int i = 0; i < kSkUnits; i++) {
                    const int u = threadIdx.x + 64 * NW * i;
                    if (u < 256 * nbl) {
                        float e[8], f[8];
#pragma unroll
                        for (int c = 0; c < 4; c++) {
                            e[c] = __uint_as_float(xv[i][0][c]);
                            e[4 + c] = __uint_as_float(xv[i][1][c]);
                            f[c] = __uint_as_float(gv[i][0][c]);
                            f[4 + c] = __uint_as_float(gv[i][1][c]);
                        }
                        uint32_t hw[4], lw[4];
#pragma unroll
                        for (int t2 = 0; t2 < 4; t2++) {
                            const float v0 = e[2 * t2] * f[2 * t2], v1 = e[2 * t2 + 1] * f[2 * t2 + 1];
                            const uint16_t h0 = f32_to_bf16(v0), h1 = f32_to_bf16(v1);
                            hw[t2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                            lw[t2] = (uint32_t)f32_to_bf16(v0 - bf16_to_f32(h0)) |
                                     ((uint32_t)f32_to_bf16(v1 - bf16_to_f32(h1)) << 16);
                            ss += e[2 * t2] * e[2 * t2] + e[2 * t2 + 1] * e[2 * t2 + 1];
                        }
                        const int jl2 = u >> 8, s2 = (u >> 6) & 3, ln = u & 63;
                        *(u32x4 *)(lds + ((jl2 * 2 + 0) * 4 + s2) * 1024 + ln * 16) = u32x4{hw[0], hw[1], hw[2], hw[3]};
                        *(u32x4 *)(lds + ((jl2 * 2 + 1) * 4 + s2) * 1024 + ln * 16) = u32x4{lw[0], lw[1], lw[2], lw[3]};
                    }
                }
                ssr[threadIdx.x] = ss;
                __syncthreads(); // LDS only: the weight loads stay in flight
                if (blockIdx.x == 0 && threadIdx.x < 16) {
                    // row b's squares over the slice, threads b, b + 16, ... in order
                    float t3 = 0.f;
                    for (int i = 0; i < 4 * NW; i++)
                        t3 += ssr[threadIdx.x + 16 * i];
                    a.part[(size_t)a.S * a.B * a.N + ks * 16 + threadIdx.x] = t3;
                }
            } else {
                // this wave's fragment loads (issued before these weight loads,
                // loads complete in order) are done once only the weight loads
                // remain; after the barrier every wave's fragments are in LDS
                wait_vmcnt<P * T * (W8 ? 5 : 4)>(); // W8: 4 code loads + 1 scale load per (p, t)
                __builtin_amdgcn_s_barrier();
            }
        }
#pragma unroll
        for (int p = 0; p < P; p++)
            if (jl + p < nbl)
#pragma unroll
                for (int s = 0; s < 4; s++) {
                    const u32x4 xh = *(const u32x4 *)(lds + (((jl + p) * 2 + 0) * 4 + s) * 1024 + lane * 16);
                    const u32x4 xl = *(const u32x4 *)(lds + (((jl + p) * 2 + 1) * 4 + s) * 1024 + lane * 16);
                    f32x4 c0 = f32x4{0.f, 0.f, 0.f, 0.f};
                    if constexpr (W8) {
                        // c0[i] = -128 x (batch 4q + i) summed over the 32-block
                        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xh), neg128_bf16x8(), c0, 0, 0, 0);
                        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xl), neg128_bf16x8(), c0, 0, 0, 0);
                    }
#pragma unroll
                    for (int t = 0; t < T; t++) {
                        if constexpr (W8) {
                            const bf16x8 wb = i8x8_to_bf16_biased(w8[p][t][s]);
                            f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xh), wb, c0, 0, 0, 0);
                            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xl), wb, d, 0, 0, 0);
                            const float scv = sc[p][t][s];
                            acc[t][0] += scv * d[0];
                            acc[t][1] += scv * d[1];
                            acc[t][2] += scv * d[2];
                            acc[t][3] += scv * d[3];
                        } else {
                            const bf16x8 wa = __builtin_bit_cast(bf16x8, w[p][t][s]);
                            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, __builtin_bit_cast(bf16x8, xh), acc[t], 0, 0, 0);
                            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, __builtin_bit_cast(bf16x8, xl), acc[t], 0, 0, 0);
                        }
                    }
                }
    }
    if constexpr (W8) {
        // lane (q, r) holds batches 4q + i (i < 4) of row n0 + 16 t + r
#pragma unroll
        for (int t = 0; t < T; t++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                if (4 * q + i < a.B && n0 + 16 * t < a.N)
                    a.part[((size_t)ks * a.B + 4 * q + i) * a.N + n0 + 16 * t + r] = acc[t][i];
    } else if (r < a.B) {
        // lane (q, b = r) holds rows n0 + 16 t + 4q + i (i < 4) of batch column b
#pragma unroll
        for (int t = 0; t < T; t++)
            if (n0 + 16 * t < a.N)
                *(f32x4 *)(a.part + ((size_t)ks * a.B + r) * a.N + n0 + 16 * t + 4 * q) = acc[t];
    }
}

// y[b][n] = sum_s part[s][b][n] in slice order, then the projection's
// epilogue: store (+ tap, + fused merge), or SwiGLU of the interleaved
// (W1_f, W3_f) rows (+ tap, + fragment copy for the next projection).
// One thread per 4 consecutive n of one batch row.
constexpr int kSkEpiU = 32;

// One wave a workgroup: the 20..112 workgroups of the 70B shapes' reduces
// then spread their slice loads over 4x as many CUs (70B step 83.8 -> 83.1 us).
template <int EPI>
__global__ __launch_bounds__(64) void k_gemv_sk_epi(MfmaGemvArgs a)
{
    const int n4 = a.N / 4;
    const int i = blockIdx.x * 64 + threadIdx.x;
    if (i >= a.B * n4)
        return;
    const int b = i / n4, n = (i % n4) * 4;
    const size_t slice = (size_t)a.B * a.N;
    const float *p = a.part + (size_t)b * a.N + n;
    const float *ssp = a.part + (size_t)a.S * slice + b; // [S][16] row sums of squares
    // up to kSkEpiU slices per round, all their loads (and, with the RMSNorm
    // folded in, the slices' sums of squares of row b) in flight before the
    // in-order adds: one round trip for every shape with S <= kSkEpiU
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    float t = 0.f;
    for (int s0 = 0; s0 < a.S; s0 += kSkEpiU) {
        float4 u[kSkEpiU];
        float q2[kSkEpiU];
#pragma unroll
        for (int k = 0; k < kSkEpiU; k++)
            if (s0 + k < a.S) {
                u[k] = *(const float4 *)(p + (s0 + k) * slice);
                if (a.xs)
                    q2[k] = ssp[16 * (s0 + k)];
            }
#pragma unroll
        for (int k = 0; k < kSkEpiU; k++)
            if (s0 + k < a.S) {
                if (s0 + k == 0) {
                    v = u[0];
                } else {
                    v.x += u[k].x;
                    v.y += u[k].y;
                    v.z += u[k].z;
                    v.w += u[k].w;
                }
                if (a.xs)
                    t += q2[k];
            }
    }
    // RMSNorm folded in: row b times 1 / rms of input row b
    const float rs = a.xs ? 1.0f / sqrtf(t / (float)a.K + a.eps) : 1.f;
    v.x *= rs;
    v.y *= rs;
    v.z *= rs;
    v.w *= rs;
    if constexpr (EPI == EPI_SWIGLU) {
        const int f = n >> 1; // rows (n, n+1) and (n+2, n+3) are features f, f+1
        const float h0 = silu(v.x) * v.y, h1 = silu(v.z) * v.w;
        *(float2 *)(a.y + (size_t)b * a.ldy + f) = make_float2(h0, h1);
        if (a.tap)
            *(float2 *)(a.tap + (size_t)b * a.ldy + f) = make_float2(h0, h1);
        if (a.yf) {
            xf_store(a.yf, b, f, h0);
            xf_store(a.yf, b, f + 1, h1);
        }
    } else {
        const size_t o = (size_t)b * a.ldy + n;
        *(float4 *)(a.y + o) = v;
        if (a.tap)
            *(float4 *)(a.tap + o) = v;
        if (a.mo.n_wires) {
            float4 m = *(const float4 *)(a.mo.residual + o);
            for (int k0 = 0; k0 < a.mo.n_wires; k0 += kMO) {
                float4 d[kMO];
#pragma unroll
                for (int k = 0; k < kMO; k++)
                    if (k0 + k < a.mo.n_wires && k0 + k != a.mo.own)
                        d[k] = *(const float4 *)((const float *)a.mo.wires[k0 + k] + o);
#pragma unroll
                for (int k = 0; k < kMO; k++)
                    if (k0 + k < a.mo.n_wires) {
                        const float4 e = k0 + k == a.mo.own ? v : d[k];
                        m.x = m.x + e.x;
                        m.y = m.y + e.y;
                        m.z = m.z + e.z;
                        m.w = m.w + e.w;
                    }
            }
            *(float4 *)(a.mo.x_out + o) = m;
        }
    }
}

// Split-K shape for an N x K projection: tiles per wave T, 128-blocks per
// slice and slices, aiming at up to 256 workgroups; T = 0 when the shape
// does not tile (the per-tile kernel takes it).
struct SkShape {
    int T, nbs, S, R, NW;
};
static SkShape sk_shape(int N, int K)
{
    const int nb = K / 128;
    SkShape sh{0, 0, 0, 0, 0};
    // only long K: with K < 4096 the per-tile kernel's activation traffic is
    // small and the reduce launch would cost more than it saves (70B W_O and
    // W2 measured slower split)
    if (K % 128 || K < 4096)
        return sh;
    int T;
    if (N % 256 == 0 && N / 256 >= 16)
        T = 2;
    else if (N % 16 == 0) // a ragged last tile column: its tiles past N are idle
        T = 1;
    else
        return sh;
    // at most 256 workgroups: the folded-RMSNorm kernel holds one workgroup
    // per CU, so a 257th would run in a second round (70B up-projection: 280
    // -> 224 workgroups, 34.8 -> 33.5 us). Of 8 and 7 waves a workgroup, the
    // one whose grid keeps more CUs busy with live tiles (a weights-only
    // probe of the 70B W1/W3 grid: 224 workgroups of 8 waves 23.8 us, 256 of
    // 7 waves 21.5 us)
    double best = -1.0;
    for (const int NW : {8, 7}) {
        const int tiles = N / 16, R = (tiles + T * NW - 1) / (T * NW);
        const int st = 256 / R > 1 ? 256 / R : 1;
        int nbs = (nb + st - 1) / st;
        nbs = nbs < 2 ? 2 : nbs > kSkMaxNbs ? kSkMaxNbs : nbs;
        const int S = (nb + nbs - 1) / nbs;
        if (NW != 8 && R * S > 256)
            continue;
        const double busy = (double)R * S * tiles / ((double)R * T * NW);
        if (busy > best + 1e-9) {
            best = busy;
            sh = SkShape{T, nbs, S, R, NW};
        }
    }
    return sh;
}

size_t gemv_sk_part_floats(int N, int K, int B)
{
    const SkShape sh = sk_shape(N, K);
    return sh.T ? (size_t)sh.S * (B * N + 16) : 0;
}

bool gemv_sk_used(int N, int K) { return sk_shape(N, K).T != 0; }

bool gemv_mfma_ok(int B, int N, int K, int w_bf16)
{
    return w_bf16 && B > 4 && B <= 16 && N % 16 == 0 && K % 128 == 0;
}

// Host-checked preconditions: gemv_mfma_ok; ldy and the float2/float4
// stores 8/16-byte aligned (N and ldy multiples of 4).
hipError_t launch_gemv_mfma(const MfmaGemvArgs &a0, int epi, hipStream_t st)
{
    MfmaGemvArgs a = a0;
    const int nb = a.K / 128;
    const SkShape sh = sk_shape(a.N, a.K);
    if (a.xs && !(a.part && sh.T)) // the folded RMSNorm exists on the split-K path only
        return hipErrorInvalidValue;
    if (a.part && sh.T) {
        a.nbs = sh.nbs;
        a.S = sh.S;
        const dim3 grid(sh.R, sh.S), block(64 * sh.NW);
#define TPS_SK(NORM, W8)                                                             \
    do {                                                                             \
        if (sh.T == 2 && sh.NW == 7)                                                 \
            hipLaunchKernelGGL((k_gemv_sk<2, 7, NORM, W8>), grid, block, 0, st, a);  \
        else if (sh.T == 2)                                                          \
            hipLaunchKernelGGL((k_gemv_sk<2, 8, NORM, W8>), grid, block, 0, st, a);  \
        else if (sh.NW == 7)                                                         \
            hipLaunchKernelGGL((k_gemv_sk<1, 7, NORM, W8>), grid, block, 0, st, a);  \
        else                                                                         \
            hipLaunchKernelGGL((k_gemv_sk<1, 8, NORM, W8>), grid, block, 0, st, a);  \
    } while (0)
        if (a.xs) {
            if (a.ws)
                TPS_SK(true, true);
            else
                TPS_SK(true, false);
        } else {
            if (a.ws)
                TPS_SK(false, true);
            else
                TPS_SK(false, false);
        }
#undef TPS_SK
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        const dim3 eg((unsigned)((a.B * (a.N / 4) + 63) / 64));
        if (epi == EPI_SWIGLU)
            hipLaunchKernelGGL(k_gemv_sk_epi<EPI_SWIGLU>, eg, dim3(64), 0, st, a);
        else
            hipLaunchKernelGGL(k_gemv_sk_epi<EPI_STORE>, eg, dim3(64), 0, st, a);
        return hipGetLastError();
    }
    // K split so that each wave streams about 2 blocks (2 x 4 KiB of weights
    // per tile), one round of loads: a wave that must wait for one round
    // before issuing the next falls behind in the queue at the HBM, and the
    // last waves then stream alone (70B W_O 9.6 -> 8.3 us with 2 instead of 8
    // blocks per wave, W2 19.1 -> 17.6 us). Two tiles per wave when that
    // still gives every SIMD a wave, else one.
    const int wkb = (nb + 1) / 2;
    const int wk2 = wkb < 1 ? 1 : wkb > 8 ? 8 : wkb;
    const bool two = a.N % 32 == 0 && (long)(a.N / 32) * wk2 >= 1024;
    const int wmax = a.ws ? 8 : kMaxWk;
    a.wk = two ? wk2 : (wkb < 1 ? 1 : wkb > wmax ? wmax : wkb);
    const dim3 grid(a.N / (two ? 32 : 16)), block(64 * a.wk);
#define TPS_MFMA(TT, W8)                                                              \
    do {                                                                              \
        if (epi == EPI_SWIGLU)                                                        \
            hipLaunchKernelGGL((k_gemv_mfma<EPI_SWIGLU, TT, W8>), grid, block, 0, st, a); \
        else                                                                          \
            hipLaunchKernelGGL((k_gemv_mfma<EPI_STORE, TT, W8>), grid, block, 0, st, a);  \
    } while (0)
    const bool w8 = a.ws != nullptr;
    if (two) {
        if (w8)
            TPS_MFMA(2, true);
        else
            TPS_MFMA(2, false);
    } else {
        if (w8)
            TPS_MFMA(1, true);
        else
            TPS_MFMA(1, false);
    }
#undef TPS_MFMA
    return hipGetLastError();
}

} // namespace tps
