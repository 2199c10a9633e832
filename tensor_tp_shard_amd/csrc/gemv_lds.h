// gemv_lds.h -- the batch <= 4 weight-streaming GEMV with activations staged
// in LDS (and the RMSNorm fused into its prologue), as a device function: the
// k_gemv_lds kernel runs it for every workgroup, and the fused QKV projection
// + attention kernel (k_qkv_attn) for its projection workgroups.
//
// Pages: aiterms.tw "Tensor Parallelism", 核心概念 items 1-2 (a column-split
// shard owns whole output rows of Wq/Wk/Wv/W1/W3; a row-split shard owns a
// column block of Wo/W2 and produces a full-size partial); distributed-llama
// issue "[Feature Suggest] Tensor Parallellism for Accelerating LLM",
// buildLlama2Arch tasks llamaRmsAttNorm / llamaRmfFfnNorm (the norm),
// llamaQuantizeRmsAtt / llamaQuantizeRmfFfn (int8 round trip of the
// normalised row), llamaQkv, llamaAttOutput, llamaFfn, llamaFfn2.
#pragma once

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

// NW waves per workgroup, one (RPW rows) per wave: the body of k_gemv_lds
// for workgroup blk, xs the workgroup's dynamic LDS
// ([B][K] floats). With hand (EPI_STORE without a merge), every output is
// also published as a hand-off word (tag << 32 | fp32 bits) by an
// agent-scope store, for the attention workgroups of the same launch that
// consume the QKV projection (k_qkv_attn).
template <int WT, int NB, int RPW, int EPI, bool MO, int NW>
__device__ __forceinline__ void gemv_lds_body(const GemvArgs &a, int blk, float *xs, uint64_t *hand,
                                              uint32_t tag)
{
    constexpr int V = wt_per_chunk(WT); // elements per 16-byte chunk
    constexpr int KC = 8;           // chunk iterations per lane kept in flight
    __shared__ float red4[NW];
    const int tid = threadIdx.x, lane = tid & 63;
    if (a.epoch && blk == 0 && tid == 0)
        a.epoch[0] = (a.epoch[0] + 1u) & 0x7fffffffu;
    // the wave index twice: uniform for the weight buffers, and as a lane
    // value for the merge's element index (proven uniform, that address
    // would turn the merge preloads into scalar loads the wave waits on
    // before it can issue its weights)
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row0 = (blk * NW + wv) * RPW;
    const int row0v = (blk * NW + (tid >> 6)) * RPW;
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
    // blk * 32 + t % 32 of batch row t / 32
    const int qb = tid >> 5, qi = tid & 31, qrow = blk * 32 + qi;
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
                        else if (hand)
                            hand_publish(hand + (size_t)b * a.ldy + row0 + r, acc[r][b], tag);
                    }
                }
        }
    }
}

} // namespace tps
