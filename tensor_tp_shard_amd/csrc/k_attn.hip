// k_attn.hip -- RoPE, KV-cache append and split-KV grouped-query decode
// attention over one shard's cache, then the fixed-order combine.
//
// Pages: distributed-llama issue "[Feature Suggest] Tensor Parallellism for
// Accelerating LLM", buildLlama2Arch task llamaMultiheadAtt ("merge kv-cache,
// add RoPE encoding, compute a part of multi-head attention locally");
// tt-metal issue "Llama-2 (meta) TT implementation" (GQA vs MHA matters for
// Llama-2); CS349E lecture 4 03_pope_partitioning.py, demo 3 observations
// (with 8 KV groups, head sharding at TP <= 8 keeps each KV head on exactly
// one shard: a shard's q heads only read its own kv heads).
//
// Readings where the pages are silent: RoPE rotates adjacent pairs
// (u_2i, u_2i+1) by pos * theta^(-2i/hd); the new token sits at index
// lens[b] and attention covers lens[b] + 1 positions; the cached K is stored
// rotated; scores are scaled by 1/sqrt(hd); the new K/V are used as stored
// (rounded to the cache type).
//
// Work split: one 256-thread workgroup per (sequence b, kv head g, chunk of
// 64 positions). The workgroup serves all G query heads of kv head g, so each
// K/V row is read from HBM once per step however many q heads share it.
//  scores : 4 threads per position, each a 16-element stride of hd, butterfly
//           over the 4 -> s[j][t] for the G heads
//  softmax: one wave per head: chunk max m, p = exp(s - m), l = sum p
//  values : hd/4 threads per row, 4 dims each, rows split into phases;
//           phases summed in fixed order through LDS
// The chunk holding position lens[b] rotates the new k, rounds k and v to the
// cache type, appends them and uses the rounded values.
// Partial record per (b, q head, chunk): m, l, -, -, o[hd] (unnormalised).
#include "common.h"

namespace tps {

constexpr int kChunk = 64;

template <bool KBF16>
__device__ __forceinline__ float4 load4(const void *base, size_t elem)
{
    if constexpr (KBF16) {
        const uint2 u = *(const uint2 *)((const uint16_t *)base + elem);
        return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
    } else {
        return *(const float4 *)((const float *)base + elem);
    }
}

template <bool KBF16>
__device__ __forceinline__ float round_kv(float v)
{
    if constexpr (KBF16)
        return bf16_to_f32(f32_to_bf16(v));
    else
        return v;
}

template <bool KBF16>
__device__ __forceinline__ void store_kv(void *base, size_t elem, float v)
{
    if constexpr (KBF16)
        ((uint16_t *)base)[elem] = f32_to_bf16(v);
    else
        ((float *)base)[elem] = v;
}

template <bool KBF16, int GM>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a)
{
    extern __shared__ float smem[];
    const int hd = a.hd, G = a.G;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int L = a.lens[b];
    if (L < 0 || L >= a.max_ctx) {
        if (c == 0 && g == 0 && tid == 0)
            atomicOr(a.err, 1u);
        return;
    }
    const int t0 = c * kChunk;
    if (t0 > L)
        return;
    const int n = min(kChunk, L + 1 - t0); // positions in this chunk
    const bool owner = L < t0 + kChunk;

    float *q_s = smem;                  // [G][hd]
    float *s_s = q_s + G * hd;          // [G][64]
    float *knew = s_s + G * kChunk;     // [hd]
    float *vnew = knew + hd;            // [hd]
    float *ml = vnew + hd;              // [G][2] (4*GM floats keep red 16-byte aligned)
    float *red = ml + 4 * GM;           // [phases][G][hd]

    const float *qkv = a.qkv + (size_t)b * a.ld_qkv;
    const float2 *rope = a.rope + (size_t)L * (hd / 2);
    const int half = hd / 2;

    // rotated queries of the G heads served by kv head g
    for (int i = tid; i < G * half; i += 256) {
        const int j = i / half, p = i % half;
        const int h = g * G + j;
        const float x0 = qkv[h * hd + 2 * p], x1 = qkv[h * hd + 2 * p + 1];
        const float2 cs = rope[p];
        const float r0 = x0 * cs.x - x1 * cs.y, r1 = x0 * cs.y + x1 * cs.x;
        q_s[j * hd + 2 * p] = r0;
        q_s[j * hd + 2 * p + 1] = r1;
        if (c == 0 && a.tap_q) {
            a.tap_q[(size_t)b * a.Hq_s * hd + h * hd + 2 * p] = r0;
            a.tap_q[(size_t)b * a.Hq_s * hd + h * hd + 2 * p + 1] = r1;
        }
    }
    const size_t head_base = ((size_t)b * a.Hkv_s + g) * a.max_ctx * hd;
    if (owner) { // rotate and append the new key / value at slot L
        const float *kq = qkv + (a.Hq_s + g) * hd;
        const float *vq = qkv + (a.Hq_s + a.Hkv_s + g) * hd;
        for (int p = tid; p < half; p += 256) {
            const float x0 = kq[2 * p], x1 = kq[2 * p + 1];
            const float2 cs = rope[p];
            const float r0 = x0 * cs.x - x1 * cs.y, r1 = x0 * cs.y + x1 * cs.x;
            const float v0 = vq[2 * p], v1 = vq[2 * p + 1];
            const size_t e = head_base + (size_t)L * hd + 2 * p;
            store_kv<KBF16>(a.kc, e, r0);
            store_kv<KBF16>(a.kc, e + 1, r1);
            store_kv<KBF16>(a.vc, e, v0);
            store_kv<KBF16>(a.vc, e + 1, v1);
            knew[2 * p] = round_kv<KBF16>(r0);
            knew[2 * p + 1] = round_kv<KBF16>(r1);
            vnew[2 * p] = round_kv<KBF16>(v0);
            vnew[2 * p + 1] = round_kv<KBF16>(v1);
            if (a.tap_k) {
                float *tk = a.tap_k + (size_t)b * a.Hkv_s * hd + g * hd;
                float *tv = a.tap_v + (size_t)b * a.Hkv_s * hd + g * hd;
                tk[2 * p] = r0;
                tk[2 * p + 1] = r1;
                tv[2 * p] = v0;
                tv[2 * p + 1] = v1;
            }
        }
    }
    __syncthreads();

    // scores: 4 threads per position; thread quarter qt covers dims 4qt + 16i
    {
        const int pl = tid >> 2, qt = tid & 3;
        const int t = t0 + pl;
        float sacc[GM];
#pragma unroll
        for (int j = 0; j < GM; j++)
            sacc[j] = 0.f;
        if (pl < n) {
            for (int d = 4 * qt; d < hd; d += 16) {
                const float4 k4 = (t == L) ? *(const float4 *)(knew + d)
                                           : load4<KBF16>(a.kc, head_base + (size_t)t * hd + d);
#pragma unroll
                for (int j = 0; j < GM; j++) {
                    if (j < G) {
                        const float4 q4 = *(const float4 *)(q_s + j * hd + d);
                        sacc[j] += q4.x * k4.x + q4.y * k4.y + q4.z * k4.z + q4.w * k4.w;
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < GM; j++) {
            const float s = group_sum<4>(sacc[j]);
            if (qt == 0 && j < G)
                s_s[j * kChunk + pl] = (pl < n) ? s * a.scale : -INFINITY;
        }
    }
    __syncthreads();

    // chunk softmax statistics, one wave per head
    {
        const int w = tid >> 6, lane = tid & 63;
        for (int j = w; j < G; j += 4) {
            const float s = s_s[j * kChunk + lane];
            const float m = group_max<64>(s);
            const float p = (lane < n) ? expf(s - m) : 0.f;
            const float l = group_sum<64>(p);
            s_s[j * kChunk + lane] = p;
            if (lane == 0) {
                ml[2 * j] = m;
                ml[2 * j + 1] = l;
            }
        }
    }
    __syncthreads();

    // o[j][d] = sum_t p[j][t] v[t][d]
    const int tpr = hd / 4;       // threads per row
    const int nph = 256 / tpr;    // row phases
    {
        const int ph = tid / tpr, d = (tid % tpr) * 4;
        if (ph < nph) {
            float4 acc[GM];
#pragma unroll
            for (int j = 0; j < GM; j++)
                acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int pl = ph; pl < n; pl += nph) {
                const int t = t0 + pl;
                const float4 v4 = (t == L) ? *(const float4 *)(vnew + d)
                                           : load4<KBF16>(a.vc, head_base + (size_t)t * hd + d);
#pragma unroll
                for (int j = 0; j < GM; j++) {
                    if (j < G) {
                        const float p = s_s[j * kChunk + pl];
                        acc[j].x += p * v4.x;
                        acc[j].y += p * v4.y;
                        acc[j].z += p * v4.z;
                        acc[j].w += p * v4.w;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < GM; j++)
                if (j < G)
                    *(float4 *)(red + ((size_t)ph * G + j) * hd + d) = acc[j];
        }
    }
    __syncthreads();
    for (int i = tid; i < G * hd; i += 256) {
        const int j = i / hd, d = i % hd;
        float o = 0.f;
        for (int ph = 0; ph < nph; ph++)
            o += red[((size_t)ph * G + j) * hd + d];
        float *rec = a.part + (((size_t)b * a.Hq_s + g * G + j) * a.n_chunks + c) * (hd + 4);
        rec[4 + d] = o;
        if (d == 0) {
            rec[0] = ml[2 * j];
            rec[1] = ml[2 * j + 1];
        }
    }
}

// att[b][h][d] = sum_c o_c[d] e^(m_c - M) / sum_c l_c e^(m_c - M), c in order.
__global__ __launch_bounds__(256) void k_combine(CombineArgs a)
{
    const int h = blockIdx.x, b = blockIdx.y, hd = a.hd;
    float *out = a.att + ((size_t)b * a.Hq_s + h) * hd;
    float *tap = a.tap ? a.tap + ((size_t)b * a.Hq_s + h) * hd : nullptr;
    const int L = a.lens[b];
    if (L < 0 || L >= a.max_ctx) {
        for (int d = threadIdx.x; d < hd; d += blockDim.x) {
            out[d] = 0.f;
            if (tap)
                tap[d] = 0.f;
        }
        return;
    }
    const int nch = L / a.chunk + 1;
    const float *rec = a.part + ((size_t)b * a.Hq_s + h) * a.n_chunks * (hd + 4);
    float M = -INFINITY;
    for (int c = 0; c < nch; c++)
        M = fmaxf(M, rec[(size_t)c * (hd + 4)]);
    float l = 0.f;
    for (int c = 0; c < nch; c++)
        l += rec[(size_t)c * (hd + 4) + 1] * expf(rec[(size_t)c * (hd + 4)] - M);
    const float inv = 1.0f / l;
    for (int d = threadIdx.x; d < hd; d += blockDim.x) {
        float o = 0.f;
        for (int c = 0; c < nch; c++)
            o += rec[(size_t)c * (hd + 4) + 4 + d] * expf(rec[(size_t)c * (hd + 4)] - M);
        out[d] = o * inv;
        if (tap)
            tap[d] = o * inv;
    }
}

static size_t attn_smem(int G, int GM, int hd)
{
    const int nph = 256 / (hd / 4);
    return sizeof(float) * ((size_t)G * hd + (size_t)G * kChunk + 2 * hd + 4 * GM +
                            (size_t)nph * G * hd);
}

template <bool KBF16>
static hipError_t launch_attn_t(const AttnArgs &a, int B, hipStream_t st)
{
    const dim3 grid(a.n_chunks, a.Hkv_s, B), block(256);
#define TPS_ATTN(GM)                                                                          \
    hipLaunchKernelGGL((k_attn<KBF16, GM>), grid, block, attn_smem(a.G, GM, a.hd), st, a)
    if (a.G <= 1)
        TPS_ATTN(1);
    else if (a.G <= 2)
        TPS_ATTN(2);
    else if (a.G <= 4)
        TPS_ATTN(4);
    else
        TPS_ATTN(8);
#undef TPS_ATTN
    return hipGetLastError();
}

// Host-checked preconditions: 1 <= G <= 8, hd % 16 == 0, hd <= 256,
// n_chunks = ceil(max_ctx / 64), chunk == 64.
hipError_t launch_attn(const AttnArgs &a, int kv_bf16, int B, hipStream_t st)
{
    return kv_bf16 ? launch_attn_t<true>(a, B, st) : launch_attn_t<false>(a, B, st);
}

hipError_t launch_combine(const CombineArgs &a, int B, hipStream_t st)
{
    hipLaunchKernelGGL(k_combine, dim3(a.Hq_s, B), dim3(a.hd < 256 ? 128 : 256), 0, st, a);
    return hipGetLastError();
}

} // namespace tps
