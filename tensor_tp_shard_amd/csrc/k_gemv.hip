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
#include "common.h"

namespace tps {

// One 16-byte chunk of a weight row against the matching activations xp
// (fp32: 4 weights, bf16: 8, int8: 16 codes of one half of a 32-block whose
// scale is sc: the codes' dot product, then one multiply by the scale).
template <int WT>
__device__ __forceinline__ float dot_chunk(const u32x4 &w, const float4 *xp, float sc, float acc)
{
    if constexpr (WT == WT_BF16) {
        const float4 x0 = xp[0], x1 = xp[1];
        acc += bf16_lo(w.x) * x0.x;
        acc += bf16_hi(w.x) * x0.y;
        acc += bf16_lo(w.y) * x0.z;
        acc += bf16_hi(w.y) * x0.w;
        acc += bf16_lo(w.z) * x1.x;
        acc += bf16_hi(w.z) * x1.y;
        acc += bf16_lo(w.w) * x1.z;
        acc += bf16_hi(w.w) * x1.w;
    } else if constexpr (WT == WT_I8) {
        float p = 0.f;
#pragma unroll
        for (int d = 0; d < 4; d++) {
            const uint32_t u = w[d];
            const float4 x = xp[d];
            p += (float)(int8_t)(u & 0xffu) * x.x;
            p += (float)(int8_t)((u >> 8) & 0xffu) * x.y;
            p += (float)(int8_t)((u >> 16) & 0xffu) * x.z;
            p += (float)(int8_t)(u >> 24) * x.w;
        }
        acc += sc * p;
    } else {
        const float4 x0 = xp[0];
        acc += __uint_as_float(w.x) * x0.x;
        acc += __uint_as_float(w.y) * x0.y;
        acc += __uint_as_float(w.z) * x0.z;
        acc += __uint_as_float(w.w) * x0.w;
    }
    return acc;
}

// sum over the NW waves of a block, in a fixed order (pairwise)
template <int NW>
__device__ __forceinline__ float block_sum(float v, float *red)
{
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    v = group_sum<64>(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float s4 = (red[0] + red[1]) + (red[2] + red[3]);
    if constexpr (NW == 8)
        return s4 + ((red[4] + red[5]) + (red[6] + red[7]));
    return s4;
}

// Staging of the activation rows x[b][0..K) (b < B) into LDS as fp32; with
// a.g set, as the normalised row g * x * r (r = 1/sqrt(mean x^2 + eps)),
// optionally through the int8 round trip (blocks of 32 = 8 consecutive
// float4 = 8 lanes). Row 0 and the gains are loaded by stage_x_issue BEFORE
// the weight loads are issued, so they return first (vector loads return in
// order) and the norm is computed while the weights are still in flight.
constexpr int kXV = 4; // float4 of a row per thread (K <= 4096 with 256 or more threads)

struct XRegs {
    float4 x[kXV], g[kXV];
};

template <int NT>
__device__ __forceinline__ void stage_x_issue(const GemvArgs &a, XRegs &r)
{
    const int n4 = a.K / 4;
#pragma unroll
    for (int i = 0; i < kXV; i++) {
        const int e = threadIdx.x + NT * i;
        if (e < n4) {
            r.x[i] = ((const float4 *)a.x)[e];
            if (a.g)
                r.g[i] = ((const float4 *)a.g)[e];
        }
    }
}

template <int NT>
__device__ void stage_x_finish(const GemvArgs &a, XRegs &r, float *xs, float *red4)
{
    const int n4 = a.K / 4;
    for (int b = 0; b < a.B; b++) {
        float4 *dst = (float4 *)(xs + (size_t)b * a.K);
        if (b > 0) {
            const float4 *src = (const float4 *)(a.x + (size_t)b * a.ldx);
#pragma unroll
            for (int i = 0; i < kXV; i++) {
                const int e = threadIdx.x + NT * i;
                if (e < n4)
                    r.x[i] = src[e];
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < kXV; i++) {
            const int e = threadIdx.x + NT * i;
            if (e < n4) {
                const float4 v = r.x[i];
                ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
            }
        }
        if (!a.g) {
#pragma unroll
            for (int i = 0; i < kXV; i++) {
                const int e = threadIdx.x + NT * i;
                if (e < n4)
                    dst[e] = r.x[i];
            }
            continue;
        }
        ss = block_sum<NT / 64>(ss, red4);
        const float rr = 1.0f / sqrtf(ss / (float)a.K + a.eps);
        float4 *tap = (a.xn_tap && blockIdx.x == 0) ? (float4 *)(a.xn_tap + (size_t)b * a.K) : nullptr;
        float4 *tapq = (a.xq_tap && blockIdx.x == 0) ? (float4 *)(a.xq_tap + (size_t)b * a.K) : nullptr;
#pragma unroll
        for (int i = 0; i < kXV; i++) {
            const int e = threadIdx.x + NT * i;
            if (NT * i >= n4)
                break; // uniform: no lane of this pass holds an element
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < n4) {
                const float4 x = r.x[i], g = r.g[i];
                v = make_float4(g.x * x.x * rr, g.y * x.y * rr, g.z * x.z * rr, g.w * x.w * rr);
                if (tapq)
                    tapq[e] = v;
            }
            if (a.qin) { // every lane takes part; lanes past the row hold 0
                const float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
                const float s = q8_scale(group_max<8>(m));
                v.x = q8_dequant(q8_code(v.x, s), s);
                v.y = q8_dequant(q8_code(v.y, s), s);
                v.z = q8_dequant(q8_code(v.z, s), s);
                v.w = q8_dequant(q8_code(v.w, s), s);
            }
            if (e < n4) {
                dst[e] = v;
                if (tap)
                    tap[e] = v;
            }
        }
    }
}

// NW waves per workgroup, one (RPW rows) per wave
template <int WT, int NB, int RPW, int EPI, bool MO, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemv_lds(GemvArgs a)
{
    constexpr int V = wt_per_chunk(WT); // elements per 16-byte chunk
    constexpr int KC = 8;           // chunk iterations per lane kept in flight
    extern __shared__ float xs[];   // [B][K]
    __shared__ float red4[NW];
    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index twice: uniform for the weight buffers, and as a lane
    // value for the merge's element index (proven uniform, that address
    // would turn the merge preloads into scalar loads the wave waits on
    // before it can issue its weights)
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row0 = (blockIdx.x * NW + wv) * RPW;
    const int row0v = (blockIdx.x * NW + (tid >> 6)) * RPW;
    const bool active = row0 < a.N;
    const int nchunk = a.K / V;
    // one buffer per weight row (an inactive wave's covers nothing)
    const uint32_t rowb = (uint32_t)a.K * 16 / V;
    __amdgpu_buffer_rsrc_t Wr[RPW], Sr[RPW];
#pragma unroll
    for (int r = 0; r < RPW; r++) {
        Wr[r] = buf_rsrc((const char *)a.W + (size_t)(active ? row0 + r : 0) * rowb, active ? rowb : 0u);
        // int8: the row's fp32 scales, one per 32 codes (two chunks)
        if constexpr (WT == WT_I8)
            Sr[r] = buf_rsrc(a.ws + (size_t)(active ? row0 + r : 0) * (a.K / 32), active ? (uint32_t)a.K / 8 : 0u);
    }
    // fused merge (MO): the lane that stores output (row0 + r, b) preloads the
    // residual and the other wires' elements before the weights are requested
    float mres = 0.f;
    uint2 mpre[kMO];
    // EPI_Q8: thread t < 32 NB quantises (and merges) output row
    // blockIdx.x * 32 + t % 32 of batch row t / 32
    const int qb = tid >> 5, qi = tid & 31, qrow = blockIdx.x * 32 + qi;
    const bool qact = EPI == EPI_Q8 && qb < a.B && qrow < a.N;
    if constexpr (MO && EPI == EPI_Q8) {
        if (tid < 32 * NB && qact)
            merge_preload1<true>(a.mo, (size_t)qb * a.ldy + qrow, mres, mpre);
    } else if constexpr (MO) {
        const int mr = lane / NB, mb = lane % NB;
        if (active && lane < RPW * NB && mb < a.B)
            merge_preload1<false>(a.mo, (size_t)mb * a.ldy + row0v + mr, mres, mpre);
    }

    XRegs xr;
    stage_x_issue<64 * NW>(a, xr);
    __builtin_amdgcn_sched_barrier(0); // the activation loads stay ahead of the weights
    u32x4 w[RPW][KC];
    float sc[RPW][KC];
    auto load_w = [&](int kb) {
#pragma unroll
        for (int i = 0; i < KC; i++) {
            const int c = kb + lane + 64 * i;
#pragma unroll
            for (int r = 0; r < RPW; r++) {
                w[r][i] = buf_load16_nt(Wr[r], c < nchunk ? 16u * c : kOob);
                if constexpr (WT == WT_I8)
                    sc[r][i] = __uint_as_float(buf_load4(Sr[r], c < nchunk ? 4u * (c >> 1) : kOob));
                else
                    sc[r][i] = 1.f;
            }
        }
    };
    load_w(0);
    stage_x_finish<64 * NW>(a, xr, xs, red4);
    __syncthreads();

    float acc[RPW][NB];
#pragma unroll
    for (int r = 0; r < RPW; r++)
#pragma unroll
        for (int b = 0; b < NB; b++)
            acc[r][b] = 0.f;
    for (int kb = 0; kb < nchunk; kb += 64 * KC) {
        if (kb > 0)
            load_w(kb);
#pragma unroll
        for (int i = 0; i < KC; i++) {
            const int c = kb + lane + 64 * i;
            if (active && c < nchunk) {
#pragma unroll
                for (int b = 0; b < NB; b++) {
                    if (b < a.B) {
                        const float4 *xp = (const float4 *)(xs + (size_t)b * a.K) + c * (V / 4);
#pragma unroll
                        for (int r = 0; r < RPW; r++)
                            acc[r][b] = dot_chunk<WT>(w[r][i], xp, sc[r][i], acc[r][b]);
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

    if constexpr (EPI == EPI_Q8) {
        static_assert(NW * RPW == 32, "a workgroup owns one 32-row block of the wire");
        // the block's 32 x NB partials through LDS, then one 32-lane group per
        // batch row: block max, scale, codes, and the merge of the int8 wires
        __shared__ float pq[32][NB];
        if (active && lane == 0)
#pragma unroll
            for (int r = 0; r < RPW; r++)
#pragma unroll
                for (int b = 0; b < NB; b++)
                    pq[wv * RPW + r][b] = acc[r][b];
        __syncthreads();
        if (tid < 32 * NB) { // whole 32-lane groups: the butterfly below needs every lane
            const float v = qact ? pq[qi][qb] : 0.f;
            const float sc = q8_scale(group_max<32>(fabsf(v)));
            if (qact) {
                const size_t e = (size_t)qb * a.ldy + qrow;
                const int code = q8_code(v, sc);
                a.codes[e] = (int8_t)code;
                if (qi == 0)
                    a.scales[(size_t)qb * (a.ldy / kQBlock) + qrow / kQBlock] = sc;
                if (a.tap)
                    a.tap[e] = v;
                if constexpr (MO)
                    merge_finish1<true>(a.mo, e, q8_dequant(code, sc), mres, mpre);
            }
        }
        return;
    }
    if (active) {
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
                        if constexpr (MO)
                            merge_finish1<false>(a.mo, (size_t)b * a.ldy + row0 + r, acc[r][b], mres, mpre);
                    }
                }
        }
    }
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
