// k_attn.hip -- RoPE, KV-cache append and split-KV grouped-query decode
// attention over one shard's cache, with the chunk combine fused in.
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
//  load   : the chunk's K and V rows go to LDS in one round trip (16-byte
//           loads, all issued before the first is used); the chunk holding
//           position lens[b] rotates the new k, rounds k and v to the cache
//           type, appends them to the cache and to its LDS rows
//  scores : 4 threads per position, butterfly over the 4 -> s[j][t]
//  softmax: one wave per head: chunk max m, p = exp(s - m), l = sum p
//  values : hd/4 threads per row, 4 dims each, rows split into phases;
//           phases summed in fixed order through LDS
//  combine: a second kernel (one workgroup per (b, q head)) merges the
//           chunk records in chunk order: att = sum_c o_c e^(m_c - M) /
//           sum_c l_c e^(m_c - M). A separate launch is cheaper here than
//           publishing through agent-scope fences (which on this chip write
//           back and invalidate a whole XCD L2 per workgroup) or than a last-
//           arriving chunk workgroup doing it (measured slower).
#include "common.h"

namespace tps {

constexpr int kChunk = 64;
constexpr int kMaxPieces = 8; // 16-byte pieces per thread per tensor (64 rows x hd <= 128 fp32)

template <bool KBF16>
__device__ __forceinline__ float4 lds4(const char *row, int d)
{
    if constexpr (KBF16) {
        const uint2 u = *(const uint2 *)(row + 2 * d);
        return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
    } else {
        return *(const float4 *)(row + 4 * d);
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

// bytes of one padded LDS row of K or V
__host__ __device__ inline int attn_row_bytes(int hd, int kv_bf16) { return hd * (kv_bf16 ? 2 : 4) + 16; }

__host__ __device__ inline size_t attn_smem_bytes(int G, int GM, int hd, int kv_bf16, int n_chunks)
{
    const int nph = 256 / (hd / 4);
    const size_t rowb = attn_row_bytes(hd, kv_bf16);
    const size_t kr = kChunk * rowb > (size_t)nph * G * hd * 4 ? kChunk * rowb : (size_t)nph * G * hd * 4;
    (void)n_chunks;
    return sizeof(float) * ((size_t)G * hd + (size_t)G * kChunk + 4 * GM) + kChunk * rowb + kr;
}

template <bool KBF16, int GM, int HD>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a)
{
    extern __shared__ float smem[];
    constexpr int hd = HD;
    const int G = a.G;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int L = a.lens[b];
    if (L < 0 || L >= a.max_ctx) { // skipped sequence: flagged here, zeroed by the combine
        if (c == 0 && g == 0 && tid == 0)
            atomicOr(a.err, 1u);
        return;
    }
    const int t0 = c * kChunk;
    if (t0 > L)
        return;
    const int n = min(kChunk, L + 1 - t0); // positions in this chunk
    const int nch = L / kChunk + 1;        // chunks of this sequence
    const bool owner = L < t0 + kChunk;
    constexpr int esz = KBF16 ? 2 : 4;
    constexpr int rowb = hd * esz + 16;

    float *q_s = smem;                            // [G][hd]
    float *s_s = q_s + G * hd;                    // [G][64]
    float *ml = s_s + G * kChunk;                 // [G][2] (4*GM floats)
    char *V_s = (char *)(ml + 4 * GM);            // [64][rowb]
    char *K_s = V_s + kChunk * rowb;              // [64][rowb], later the value-phase sums
    float *red = (float *)K_s;

    const size_t head_base = ((size_t)b * a.Hkv_s + g) * a.max_ctx * hd;
    const float *qkv = a.qkv + (size_t)b * a.ld_qkv;
    const float2 *rope = a.rope + (size_t)L * (hd / 2);
    const int half = hd / 2;
    // 1) query pairs and their rotation factors first (they return first), then
    //    the chunk's K and V rows: all 16-byte loads issued before any is used
    constexpr int kQP = 4; // query pairs per thread: G * hd / 2 <= 8 * 64 = 512 <= 256 * kQP
    float2 qp[kQP], cs[kQP];
#pragma unroll
    for (int u = 0; u < kQP; u++) {
        const int i = tid + 256 * u;
        if (i < G * half) {
            const int j = i / half, p = i % half;
            qp[u] = *(const float2 *)(qkv + (g * G + j) * hd + 2 * p);
            cs[u] = rope[p];
        }
    }
    // the owner's new key / value pair p = tid (rotation factor cs[0] = rope[tid])
    float2 nk = make_float2(0.f, 0.f), nv = make_float2(0.f, 0.f);
    if (owner && tid < half) {
        nk = *(const float2 *)(qkv + (a.Hq_s + g) * hd + 2 * tid);
        nv = *(const float2 *)(qkv + (a.Hq_s + a.Hkv_s + g) * hd + 2 * tid);
    }
    constexpr int ppr = hd * esz / 16; // 16-byte pieces per row
    const int npc = n * ppr;
    u32x4 kv[2][kMaxPieces];
    {
        const u32x4 *kg = (const u32x4 *)((const char *)a.kc + (head_base + (size_t)t0 * hd) * esz);
        const u32x4 *vg = (const u32x4 *)((const char *)a.vc + (head_base + (size_t)t0 * hd) * esz);
#pragma unroll
        for (int i = 0; i < kMaxPieces; i++) {
            const int p = tid + 256 * i;
            if (p < npc) {
                kv[0][i] = __builtin_nontemporal_load(kg + p);
                kv[1][i] = __builtin_nontemporal_load(vg + p);
            }
        }
    }
    // 2) rotated queries of the G heads served by kv head g
#pragma unroll
    for (int u = 0; u < kQP; u++) {
        const int i = tid + 256 * u;
        if (i < G * half) {
            const int j = i / half, p = i % half;
            const float r0 = qp[u].x * cs[u].x - qp[u].y * cs[u].y;
            const float r1 = qp[u].x * cs[u].y + qp[u].y * cs[u].x;
            q_s[j * hd + 2 * p] = r0;
            q_s[j * hd + 2 * p + 1] = r1;
            if (c == 0 && a.tap_q) {
                const int h = g * G + j;
                a.tap_q[(size_t)b * a.Hq_s * hd + h * hd + 2 * p] = r0;
                a.tap_q[(size_t)b * a.Hq_s * hd + h * hd + 2 * p + 1] = r1;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kMaxPieces; i++) {
        const int p = tid + 256 * i;
        if (p < npc) {
            const int row = p / ppr, col = p % ppr;
            *(u32x4 *)(K_s + row * rowb + col * 16) = kv[0][i];
            *(u32x4 *)(V_s + row * rowb + col * 16) = kv[1][i];
        }
    }
    __syncthreads();
    // 3) the owner rotates and appends the new key / value at slot L
    if (owner) {
        char *krow = K_s + (L - t0) * rowb, *vrow = V_s + (L - t0) * rowb;
        if (tid < half) {
            const int p = tid;
            const float2 cr = cs[0];
            const float r0 = nk.x * cr.x - nk.y * cr.y, r1 = nk.x * cr.y + nk.y * cr.x;
            const float v0 = nv.x, v1 = nv.y;
            const size_t e = head_base + (size_t)L * hd + 2 * p;
            store_kv<KBF16>(a.kc, e, r0);
            store_kv<KBF16>(a.kc, e + 1, r1);
            store_kv<KBF16>(a.vc, e, v0);
            store_kv<KBF16>(a.vc, e + 1, v1);
            if constexpr (KBF16) {
                *(uint32_t *)(krow + 4 * p) = (uint32_t)f32_to_bf16(r0) | ((uint32_t)f32_to_bf16(r1) << 16);
                *(uint32_t *)(vrow + 4 * p) = (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
            } else {
                *(float2 *)(krow + 8 * p) = make_float2(r0, r1);
                *(float2 *)(vrow + 8 * p) = make_float2(v0, v1);
            }
            if (a.tap_k) {
                float *tk = a.tap_k + (size_t)b * a.Hkv_s * hd + g * hd;
                float *tv = a.tap_v + (size_t)b * a.Hkv_s * hd + g * hd;
                tk[2 * p] = r0;
                tk[2 * p + 1] = r1;
                tv[2 * p] = v0;
                tv[2 * p + 1] = v1;
            }
        }
        __syncthreads();
    }

    // 4) scores: 4 threads per position; thread quarter qt covers dims 4qt + 16i
    {
        const int pl = tid >> 2, qt = tid & 3;
        float sacc[GM];
#pragma unroll
        for (int j = 0; j < GM; j++)
            sacc[j] = 0.f;
        if (pl < n) {
            const char *krow = K_s + pl * rowb;
#pragma unroll
            for (int it = 0; it < hd / 16; it++) {
                const int d = 4 * qt + 16 * it;
                const float4 k4 = lds4<KBF16>(krow, d);
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

    // 5) chunk softmax statistics, one wave per head
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

    // 6) o[j][d] = sum_t p[j][t] v[t][d]; K_s is dead, its space holds the phase sums
    constexpr int tpr = hd / 4;    // threads per row
    constexpr int nph = 256 / tpr; // row phases
    {
        const int ph = tid / tpr, d = (tid % tpr) * 4;
        float4 acc[GM];
#pragma unroll
        for (int j = 0; j < GM; j++)
            acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ph < nph) {
#pragma unroll
            for (int it = 0; it < (kChunk + nph - 1) / nph; it++) {
                const int pl = ph + it * nph;
                if (pl >= n)
                    break;
                const float4 v4 = lds4<KBF16>(V_s + pl * rowb, d);
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
        }
        __syncthreads(); // every thread is done with K_s before it is overwritten
        if (ph < nph) {
#pragma unroll
            for (int j = 0; j < GM; j++)
                if (j < G)
                    *(float4 *)(red + ((size_t)ph * G + j) * hd + d) = acc[j];
        }
    }
    __syncthreads();
    const size_t rec_stride = (size_t)a.n_chunks * (hd + 4);
    float *rec0 = a.part + ((size_t)b * a.Hq_s + (size_t)g * G) * rec_stride;
    for (int i = tid; i < G * hd; i += 256) {
        const int j = i / hd, d = i % hd;
        float o = 0.f;
#pragma unroll
        for (int ph = 0; ph < nph; ph++)
            o += red[((size_t)ph * G + j) * hd + d];
        float *rec = rec0 + j * rec_stride + (size_t)c * (hd + 4);
        rec[4 + d] = o;
        if (d == 0) {
            rec[0] = ml[2 * j];
            rec[1] = ml[2 * j + 1];
        }
    }

}

// ---------------------------------------------------------------- GQA on MFMA
// The same work split and chunk records for a bf16 cache with G >= 4 q heads
// per kv head, where the VALU version spends its time re-reading the G
// queries from LDS for every position. Scores and values are dense
// contractions: S^T[t][j] = K[t][:] . q_j (A = the K chunk, B = the queries)
// and O[j][d] = sum_t p[j][t] V[t][d] (A = the probabilities, B = V, stored
// transposed in LDS), each on v_mfma_f32_16x16x32_bf16 with the fp32
// operand (queries, probabilities) split into bf16 hi + lo parts (two MFMAs,
// ~16 mantissa bits) and fp32 accumulation. K and V are used as stored.
// Positions past the sequence are zero in LDS (the cache may hold anything
// there) and masked out of the softmax. One wave per 16 positions for the
// scores, per 16-wide dim tiles for the values.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_pair(float lo_elem, float hi_elem)
{
    return (uint32_t)f32_to_bf16(lo_elem) | ((uint32_t)f32_to_bf16(hi_elem) << 16);
}

// LDS: queries and probabilities as bf16 hi / lo parts in 16-row MFMA
// operand form (rows past G zero), the K chunk row-major with padded rows,
// V in 8-position groups [t/8][dim][t%8] so that a B fragment (8 consecutive
// positions of one dim) is one aligned 16-byte read.
__host__ __device__ inline size_t attn_mfma_smem_bytes(int G, int hd)
{
    return (size_t)2 * 16 * (hd + 8) * 2 +    // q hi, lo (rows padded by 16 bytes)
           sizeof(float) * (size_t)G * kChunk + // scores
           (size_t)2 * 16 * (kChunk + 8) * 2 + // p hi, lo (rows padded by 16 bytes)
           sizeof(float) * 2 * 16 +            // (m, l)
           (size_t)kChunk * (hd * 2 + 16) +    // K
           (size_t)kChunk * hd * 2;            // V groups
}

template <int HD>
__global__ __launch_bounds__(256) void k_attn_mfma(AttnArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    constexpr int hd = HD;
    constexpr int rowb = hd * 2 + 16; // padded K row
    const int G = a.G;
    const int g = blockIdx.y;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, q = lane >> 4, r = lane & 15;
    // Compact chunk numbering: workgroup x takes the x-th chunk in the order
    // (sequence, chunk) over the chunks the sequences actually have, so the
    // working workgroups are the first ones dispatched and the surplus of the
    // n_chunks x B grid exits at its end. (With x = chunk and z = sequence,
    // the chunks past each sequence's end sat between working ones, and at
    // 3 workgroups per CU the last sequences' chunks waited for a second
    // round of slots.) A skipped sequence (lens outside [0, max_ctx)) has no
    // chunks; workgroup 0 of kv head 0 flags it, the combine zeroes its rows.
    // Each wave reads 64 lengths per load (lane i: sequence i0 + i) and an
    // inclusive scan of their chunk counts gives every sequence's chunk
    // range: one load round trip for up to 64 sequences, where a loop over
    // scalar loads waited for each length in turn (2-6 us at batch 16).
    int b = -1, c = 0, L = 0, before = 0;
    bool bad = false;
    for (int i0 = 0; i0 < a.B; i0 += 64) {
        const int i = i0 + lane;
        const int Li = i < a.B ? a.lens[i] : 0;
        const bool ok = Li >= 0 && Li < a.max_ctx;
        bad |= __ballot(i < a.B && !ok) != 0ull;
        const int ni = i < a.B && ok ? Li / kChunk + 1 : 0;
        int inc = ni;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(inc, o, 64);
            inc += lane >= o ? t : 0;
        }
        inc += before;
        const int x = blockIdx.x;
        const unsigned long long m = __ballot(x >= inc - ni && x < inc);
        if (b < 0 && m) {
            const int ln = __ffsll((unsigned long long)m) - 1;
            b = i0 + ln;
            L = __shfl(Li, ln, 64);
            c = x - (__shfl(inc, ln, 64) - __shfl(ni, ln, 64));
        }
        before = __shfl(inc, 63, 64);
    }
    b = __builtin_amdgcn_readfirstlane(b);
    c = __builtin_amdgcn_readfirstlane(c);
    L = __builtin_amdgcn_readfirstlane(L);
    if (bad && blockIdx.x == 0 && g == 0 && tid == 0)
        atomicOr(a.err, 1u);
    if (b < 0)
        return;
    const int t0 = c * kChunk;
    const int n = min(kChunk, L + 1 - t0);
    const bool owner = L < t0 + kChunk;

    // operand rows padded by 16 bytes: the 16 lanes that read one 16-byte
    // slice of 16 consecutive rows then hit 16 different bank groups (with
    // 256- and 128-byte rows they hit one or two)
    constexpr int qld = hd + 8, pld = kChunk + 8;
    uint16_t *qh_s = (uint16_t *)lds_raw;          // [16][qld]
    uint16_t *ql_s = qh_s + 16 * qld;              // [16][qld]
    float *s_s = (float *)(ql_s + 16 * qld);       // [G][64]
    uint16_t *ph_s = (uint16_t *)(s_s + G * kChunk); // [16][pld]
    uint16_t *pl_s = ph_s + 16 * pld;              // [16][pld]
    float *ml = (float *)(pl_s + 16 * pld);        // [16][2]
    char *K_s = (char *)(ml + 2 * 16);             // [64][rowb]
    uint16_t *V_g = (uint16_t *)(K_s + kChunk * rowb); // [8][hd][8]

    const size_t head_base = ((size_t)b * a.Hkv_s + g) * a.max_ctx * hd;
    const float *qkv = a.qkv + (size_t)b * a.ld_qkv;
    const float2 *rope = a.rope + (size_t)L * (hd / 2);
    const int half = hd / 2;
    constexpr int kQP = 16 * (HD / 2) / 256; // q pairs per thread over all 16 operand rows
    float2 qp[kQP], cs[kQP];
#pragma unroll
    for (int u = 0; u < kQP; u++) {
        const int i = tid + 256 * u;
        const int j = i / half, p = i % half;
        cs[u] = rope[p];
        if (j < G)
            qp[u] = *(const float2 *)(qkv + (g * G + j) * hd + 2 * p);
    }
    float2 nk = make_float2(0.f, 0.f), nv = make_float2(0.f, 0.f);
    if (owner && tid < half) {
        nk = *(const float2 *)(qkv + (a.Hq_s + g) * hd + 2 * tid);
        nv = *(const float2 *)(qkv + (a.Hq_s + a.Hkv_s + g) * hd + 2 * tid);
    }
    constexpr int ppr = hd / 8;                 // 16-byte pieces per row
    constexpr int kPieces = kChunk * ppr / 256; // per thread (64 rows)
    u32x4 kv[2][kPieces];
    {
        const u32x4 *kg = (const u32x4 *)((const char *)a.kc + (head_base + (size_t)t0 * hd) * 2);
        const u32x4 *vg = (const u32x4 *)((const char *)a.vc + (head_base + (size_t)t0 * hd) * 2);
#pragma unroll
        for (int i = 0; i < kPieces; i++) {
            const int p = tid + 256 * i;
            if (p < n * ppr) {
                kv[0][i] = __builtin_nontemporal_load(kg + p);
                kv[1][i] = __builtin_nontemporal_load(vg + p);
            } else {
                kv[0][i] = kv[1][i] = u32x4{0u, 0u, 0u, 0u}; // positions past the sequence
            }
        }
    }
    // rotated queries -> hi / lo operand rows (rows >= G zero); p rows >= G zero
#pragma unroll
    for (int u = 0; u < kQP; u++) {
        const int i = tid + 256 * u;
        const int j = i / half, p = i % half;
        float r0 = 0.f, r1 = 0.f;
        if (j < G) {
            r0 = qp[u].x * cs[u].x - qp[u].y * cs[u].y;
            r1 = qp[u].x * cs[u].y + qp[u].y * cs[u].x;
            if (c == 0 && a.tap_q) {
                const int h = g * G + j;
                a.tap_q[(size_t)b * a.Hq_s * hd + h * hd + 2 * p] = r0;
                a.tap_q[(size_t)b * a.Hq_s * hd + h * hd + 2 * p + 1] = r1;
            }
        }
        const uint16_t h0 = f32_to_bf16(r0), h1 = f32_to_bf16(r1);
        *(uint32_t *)(qh_s + j * qld + 2 * p) = (uint32_t)h0 | ((uint32_t)h1 << 16);
        *(uint32_t *)(ql_s + j * qld + 2 * p) = bf16_pair(r0 - bf16_to_f32(h0), r1 - bf16_to_f32(h1));
    }
    for (int i = tid; i < (16 - G) * kChunk / 2; i += 256) {
        const int e = (G + 2 * i / kChunk) * pld + (2 * i) % kChunk;
        *(uint32_t *)(ph_s + e) = 0u;
        *(uint32_t *)(pl_s + e) = 0u;
    }
    // K rows as loaded; V into 8-position groups, the element order rotated by
    // the piece's column so the 16 lanes of a row write 8 different banks
#pragma unroll
    for (int i = 0; i < kPieces; i++) {
        const int p = tid + 256 * i;
        const int row = p / ppr, col = p % ppr;
        *(u32x4 *)(K_s + row * rowb + col * 16) = kv[0][i];
        const u32x4 v = kv[1][i];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        uint16_t *vb = V_g + (size_t)(row >> 3) * hd * 8 + (row & 7);
#pragma unroll
        for (int e0 = 0; e0 < 8; e0++) {
            const int e = (e0 + col) & 7;
            vb[(8 * col + e) * 8] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
        }
    }
    __syncthreads();
    if (owner) { // rotate and append the new key / value at slot L (cache and LDS)
        if (tid < half) {
            const int p = tid, tl = L - t0;
            const float2 cr = cs[0];
            const float r0 = nk.x * cr.x - nk.y * cr.y, r1 = nk.x * cr.y + nk.y * cr.x;
            const size_t e = head_base + (size_t)L * hd + 2 * p;
            const uint16_t k0 = f32_to_bf16(r0), k1 = f32_to_bf16(r1);
            const uint16_t v0 = f32_to_bf16(nv.x), v1 = f32_to_bf16(nv.y);
            ((uint16_t *)a.kc)[e] = k0;
            ((uint16_t *)a.kc)[e + 1] = k1;
            ((uint16_t *)a.vc)[e] = v0;
            ((uint16_t *)a.vc)[e + 1] = v1;
            *(uint32_t *)(K_s + tl * rowb + 4 * p) = (uint32_t)k0 | ((uint32_t)k1 << 16);
            uint16_t *vb = V_g + (size_t)(tl >> 3) * hd * 8 + (tl & 7);
            vb[(2 * p) * 8] = v0;
            vb[(2 * p + 1) * 8] = v1;
            if (a.tap_k) {
                float *tk = a.tap_k + (size_t)b * a.Hkv_s * hd + g * hd;
                float *tv = a.tap_v + (size_t)b * a.Hkv_s * hd + g * hd;
                tk[2 * p] = r0;
                tk[2 * p + 1] = r1;
                tv[2 * p] = nv.x;
                tv[2 * p + 1] = nv.y;
            }
        }
        __syncthreads();
    }

    // scores: wave wv takes positions 16 wv .. 16 wv + 15; column r = head r
    {
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < hd / 32; s++) {
            const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, *(const u32x4 *)(K_s + (16 * wv + r) * rowb + (4 * s + q) * 16));
            const bf16x8_t qh = __builtin_bit_cast(bf16x8_t, *(const u32x4 *)(qh_s + r * qld + 32 * s + 8 * q));
            const bf16x8_t ql = __builtin_bit_cast(bf16x8_t, *(const u32x4 *)(ql_s + r * qld + 32 * s + 8 * q));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ql, acc, 0, 0, 0);
        }
        if (r < G) // acc[i] = score of position 16 wv + 4q + i for head r
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int pl = 16 * wv + 4 * q + i;
                s_s[r * kChunk + pl] = pl < n ? acc[i] * a.scale : -INFINITY;
            }
    }
    __syncthreads();
    // chunk softmax statistics, one wave per head; p as hi / lo operand rows
    for (int j = wv; j < G; j += 4) {
        const float sv = s_s[j * kChunk + lane];
        const float m = group_max<64>(sv);
        const float p = (lane < n) ? expf(sv - m) : 0.f;
        const float l = group_sum<64>(p);
        const uint16_t h = f32_to_bf16(p);
        ph_s[j * pld + lane] = h;
        pl_s[j * pld + lane] = f32_to_bf16(p - bf16_to_f32(h));
        if (lane == 0) {
            ml[2 * j] = m;
            ml[2 * j + 1] = l;
        }
    }
    __syncthreads();
    // values: wave wv takes dim tiles dt = wv, wv + 4, ...; row (4q + i) = head
    const size_t rec_stride = (size_t)a.n_chunks * (hd + 4);
    float *rec0 = a.part + ((size_t)b * a.Hq_s + (size_t)g * G) * rec_stride + (size_t)c * (hd + 4);
    for (int dt = wv; dt < hd / 16; dt += 4) {
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kChunk / 32; ks++) {
            const bf16x8_t ph = __builtin_bit_cast(bf16x8_t, *(const u32x4 *)(ph_s + r * pld + 32 * ks + 8 * q));
            const bf16x8_t pl = __builtin_bit_cast(bf16x8_t, *(const u32x4 *)(pl_s + r * pld + 32 * ks + 8 * q));
            const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, *(const u32x4 *)(V_g + ((size_t)(4 * ks + q) * hd + 16 * dt + r) * 8));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int j = 4 * q + i;
            if (j < G)
                rec0[j * rec_stride + 4 + 16 * dt + r] = acc[i];
        }
    }
    if (tid < G) {
        rec0[tid * rec_stride] = ml[2 * tid];
        rec0[tid * rec_stride + 1] = ml[2 * tid + 1];
    }
}

// Combine of the chunk partials of one (sequence b, query head h): its output
// att = sum_c o_c e^(m_c - M) / sum_c l_c e^(m_c - M), chunks summed in chunk
// order. The (m, l) of the first 64 chunks (wave 0) and the first kCU chunks
// of every output quad are loaded in one batch before any arithmetic; wave 0
// then forms M, the weights e^(m_c - M) and l across its lanes.
constexpr int kCombThreads = 512;

__global__ __launch_bounds__(kCombThreads) void k_combine(AttnArgs a)
{
    extern __shared__ float smem[];
    const int hd = a.hd, h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int L = a.lens[b];
    const size_t ob = (size_t)b * a.Hq_s * hd + (size_t)h * hd;
    if (L < 0 || L >= a.max_ctx) { // skipped sequence: its attention output is 0
        for (int i = tid; i < hd; i += kCombThreads) {
            a.att[ob + i] = 0.f;
            if (a.tap_att)
                a.tap_att[ob + i] = 0.f;
            if (a.att_xf)
                xf_store(a.att_xf, b, h * hd + i, 0.f);
        }
        return;
    }
    const int nch = L / kChunk + 1;
    const float *rec = a.part + ((size_t)b * a.Hq_s + h) * (size_t)a.n_chunks * (hd + 4);
    float *wts = smem;                                // [n_chunks] e^(m_c - M)
    float *inv_l = wts + a.n_chunks;                  // [1]
    float *osum = smem + ((a.n_chunks + 4 + 3) & ~3); // [phases][hd]
    const int w = tid >> 6, lane = tid & 63;
    float2 ml0 = make_float2(-INFINITY, 0.f);
    if (w == 0 && lane < nch)
        ml0 = *(const float2 *)(rec + (size_t)lane * (hd + 4));
    const int quads = hd / 4;
    const int cph = kCombThreads / quads;             // chunk phases (quads <= 32)
    constexpr int kCU = 16;                           // chunks per phase loaded together
    const int cp = tid / quads, d = (tid % quads) * 4;
    const bool qact = cp < cph; // hd = 48: 512 is not a multiple of 12 quads
    const float *rd = rec + 4 + d;
    float4 v[kCU];
#pragma unroll
    for (int u = 0; u < kCU; u++) {
        const int cc = cp + u * cph;
        if (qact && cc < nch)
            v[u] = *(const float4 *)(rd + (size_t)cc * (hd + 4));
    }
    if (w == 0) {
        float m = ml0.x;
        for (int cc = lane + 64; cc < nch; cc += 64) // sequences longer than 64 chunks
            m = fmaxf(m, rec[(size_t)cc * (hd + 4)]);
        const float M = group_max<64>(m);
        float l = 0.f;
        if (lane < nch) {
            const float e = expf(ml0.x - M);
            wts[lane] = e;
            l = e * ml0.y;
        }
        for (int cc = lane + 64; cc < nch; cc += 64) {
            const float2 q = *(const float2 *)(rec + (size_t)cc * (hd + 4));
            const float e = expf(q.x - M);
            wts[cc] = e;
            l += e * q.y;
        }
        l = group_sum<64>(l);
        if (lane == 0)
            inv_l[0] = 1.0f / l;
    }
    __syncthreads();
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c0 = cp; qact && c0 < nch; c0 += cph * kCU) {
        if (c0 != cp) { // chunks past the first batch (long sequences)
#pragma unroll
            for (int u = 0; u < kCU; u++) {
                const int cc = c0 + u * cph;
                if (cc < nch)
                    v[u] = *(const float4 *)(rd + (size_t)cc * (hd + 4));
            }
        }
#pragma unroll
        for (int u = 0; u < kCU; u++) {
            const int cc = c0 + u * cph;
            if (cc < nch) {
                const float wv = wts[cc];
                o.x += wv * v[u].x;
                o.y += wv * v[u].y;
                o.z += wv * v[u].z;
                o.w += wv * v[u].w;
            }
        }
    }
    if (qact)
        *(float4 *)(osum + (size_t)cp * hd + d) = o;
    __syncthreads();
    for (int i = tid; i < hd; i += kCombThreads) {
        float t = 0.f;
        for (int p = 0; p < cph; p++)
            t += osum[(size_t)p * hd + i];
        const float r = t * inv_l[0];
        a.att[ob + i] = r;
        if (a.tap_att)
            a.tap_att[ob + i] = r;
        if (a.att_xf)
            xf_store(a.att_xf, b, h * hd + i, r);
    }
}

static size_t combine_smem_bytes(int G, int hd, int n_chunks)
{
    (void)G;
    const int cph = kCombThreads / (hd / 4);
    return (((size_t)n_chunks + 4 + 3) / 4 * 4 + (size_t)cph * hd) * sizeof(float);
}

template <bool KBF16, int HD>
static hipError_t launch_attn_hd(const AttnArgs &a, int B, hipStream_t st)
{
    const dim3 grid(a.n_chunks, a.Hkv_s, B), block(256);
#define TPS_ATTN(GM)                                                                          \
    hipLaunchKernelGGL((k_attn<KBF16, GM, HD>), grid, block,                                   \
                       attn_smem_bytes(a.G, GM, HD, KBF16, a.n_chunks), st, a)
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

static bool attn_use_mfma(int G, int hd, int kv_bf16) { return kv_bf16 && G >= 4 && (hd == 64 || hd == 128); }

template <bool KBF16>
static hipError_t launch_attn_t(const AttnArgs &a, int B, hipStream_t st)
{
    if (attn_use_mfma(a.G, a.hd, KBF16)) {
        const dim3 grid(a.n_chunks * B, a.Hkv_s), block(256);
        const size_t sm = attn_mfma_smem_bytes(a.G, a.hd);
        if (a.hd == 128)
            hipLaunchKernelGGL(k_attn_mfma<128>, grid, block, sm, st, a);
        else
            hipLaunchKernelGGL(k_attn_mfma<64>, grid, block, sm, st, a);
        return hipGetLastError();
    }
    switch (a.hd) {
    case 16: return launch_attn_hd<KBF16, 16>(a, B, st);
    case 32: return launch_attn_hd<KBF16, 32>(a, B, st);
    case 48: return launch_attn_hd<KBF16, 48>(a, B, st);
    case 64: return launch_attn_hd<KBF16, 64>(a, B, st);
    case 128: return launch_attn_hd<KBF16, 128>(a, B, st);
    default: return hipErrorInvalidValue;
    }
}

bool attn_hd_supported(int hd) { return hd == 16 || hd == 32 || hd == 48 || hd == 64 || hd == 128; }

// Host-checked preconditions: 1 <= G <= 8, attn_hd_supported(hd),
// n_chunks = ceil(max_ctx / 64), attn_lds_bytes(...) <= 64 KiB.
hipError_t launch_attn(const AttnArgs &args, int kv_bf16, int B, hipStream_t st)
{
    AttnArgs a = args;
    a.B = B;
    const hipError_t e = kv_bf16 ? launch_attn_t<true>(a, B, st) : launch_attn_t<false>(a, B, st);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_combine, dim3(a.Hq_s, B), dim3(kCombThreads),
                       combine_smem_bytes(a.G, a.hd, a.n_chunks), st, a);
    return hipGetLastError();
}

size_t attn_lds_bytes(int G, int hd, int kv_bf16, int n_chunks)
{
    if (attn_use_mfma(G, hd, kv_bf16)) {
        const size_t a = attn_mfma_smem_bytes(G, hd), c = combine_smem_bytes(G, hd, n_chunks);
        return a > c ? a : c;
    }
    const int GM = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
    const size_t a = attn_smem_bytes(G, GM, hd, kv_bf16, n_chunks), c = combine_smem_bytes(G, hd, n_chunks);
    return a > c ? a : c;
}

} // namespace tps
