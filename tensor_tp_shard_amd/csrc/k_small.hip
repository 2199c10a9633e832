// k_small.hip -- the short, latency-bound kernels of the shard step:
// RMSNorm (+ int8 round trip of the normalised row), block-32 int8
// quantisation of a partial, the merge of shard partials, the RoPE table and
// a small fill kernel.
//
// Pages: distributed-llama issue "[Feature Suggest] Tensor Parallellism for
// Accelerating LLM", buildLlama2Arch task list: llamaRmsAttNorm /
// llamaRmfFfnNorm (RMSNorm), llamaQuantizeRmsAtt / llamaQuantizeRmfFfn (the
// normalised input is quantised before it is broadcast), llamaQuantizeAtt /
// llamaQuantizeFfn2 + llamaDequantize* (partials travel as int8),
// llamaMergeAtt / llamaMergeFfn2 (the partials are merged); aiterms.tw
// "Tensor Parallelism", 運作原理 step 3 (row-split partials need an
// all-reduce: here a fixed-order on-device sum).
#include "common.h"

namespace tps {

// One block of kNormThreads (1024) threads per row; a thread owns runs of 8
// consecutive elements (two float4), up to kNormRuns runs (D <= 32768 in one
// pass: all of the row's x and gain loads are issued before any is used and
// the row stays in registers). Longer rows take further passes, re-reading x.
// Sum of squares in fp32 (wave butterflies, then the 16 wave sums in order),
// y = g * x * r with r = 1 / sqrt(ms + eps). With quant set, each block of 32
// elements (4 consecutive threads) is quantised and dequantised in place (the
// receiver of the broadcast sees these values). Optionally the row is also
// written in the MFMA fragment layout (8 consecutive k are 16 contiguous bytes
// there).
constexpr int kNormRuns = 4;
constexpr int kNormThreads = 1024;
constexpr int kNormWaves = kNormThreads / 64;

__device__ __forceinline__ void norm_store_run(const NormArgs &a, int b, int run, float (&e)[8], float4 *y,
                                               float4 *tap)
{
    const float4 lo4 = make_float4(e[0], e[1], e[2], e[3]);
    const float4 hi4 = make_float4(e[4], e[5], e[6], e[7]);
    y[2 * run] = lo4;
    y[2 * run + 1] = hi4;
    if (tap) {
        tap[2 * run] = lo4;
        tap[2 * run + 1] = hi4;
    }
    if (a.xf) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const uint16_t h0 = f32_to_bf16(e[2 * t]), h1 = f32_to_bf16(e[2 * t + 1]);
            const uint16_t l0 = f32_to_bf16(e[2 * t] - bf16_to_f32(h0));
            const uint16_t l1 = f32_to_bf16(e[2 * t + 1] - bf16_to_f32(h1));
            hw[t] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lw[t] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        *(u32x4 *)(a.xf + xf_index(b, 8 * run, 0)) = u32x4{hw[0], hw[1], hw[2], hw[3]};
        *(u32x4 *)(a.xf + xf_index(b, 8 * run, 1)) = u32x4{lw[0], lw[1], lw[2], lw[3]};
    }
}

__global__ __launch_bounds__(kNormThreads) void k_rmsnorm(NormArgs a)
{
    const int b = blockIdx.x, tid = threadIdx.x;
    const int nruns = a.D / 8;
    const bool one_pass = nruns <= kNormThreads * kNormRuns;
    const float4 *x = (const float4 *)(a.x + (size_t)b * a.D);
    const float4 *g = (const float4 *)a.g;
    __shared__ float red[kNormWaves];
    float4 v[kNormRuns][2], gv[kNormRuns][2];
    float ss = 0.f;
    for (int r0 = 0; r0 < nruns; r0 += kNormThreads * kNormRuns) {
#pragma unroll
        for (int i = 0; i < kNormRuns; i++) {
            const int run = r0 + tid + kNormThreads * i;
            if (run < nruns) {
                v[i][0] = x[2 * run];
                v[i][1] = x[2 * run + 1];
                if (one_pass) {
                    gv[i][0] = g[2 * run];
                    gv[i][1] = g[2 * run + 1];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kNormRuns; i++) {
            const int run = r0 + tid + kNormThreads * i;
            if (run < nruns)
#pragma unroll
                for (int h = 0; h < 2; h++)
                    ss += v[i][h].x * v[i][h].x + v[i][h].y * v[i][h].y + v[i][h].z * v[i][h].z +
                          v[i][h].w * v[i][h].w;
        }
    }
    ss = group_sum<64>(ss);
    if ((tid & 63) == 0)
        red[tid >> 6] = ss;
    __syncthreads();
    ss = 0.f;
#pragma unroll
    for (int w = 0; w < kNormWaves; w++)
        ss += red[w];
    const float r = 1.0f / sqrtf(ss / (float)a.D + a.eps);
    float4 *y = (float4 *)(a.xn + (size_t)b * a.D);
    float4 *tap = a.tap ? (float4 *)(a.tap + (size_t)b * a.D) : nullptr;
    for (int r0 = 0; r0 < nruns; r0 += kNormThreads * kNormRuns) {
        if (!one_pass) {
#pragma unroll
            for (int i = 0; i < kNormRuns; i++) {
                const int run = r0 + tid + kNormThreads * i;
                if (run < nruns) {
                    v[i][0] = x[2 * run];
                    v[i][1] = x[2 * run + 1];
                    gv[i][0] = g[2 * run];
                    gv[i][1] = g[2 * run + 1];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kNormRuns; i++) {
            const int run = r0 + tid + kNormThreads * i;
            if (r0 + kNormThreads * i >= nruns)
                break; // uniform: no thread of this pass holds a run
            float e[8];
            if (run < nruns) {
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    e[4 * h + 0] = gv[i][h].x * v[i][h].x * r;
                    e[4 * h + 1] = gv[i][h].y * v[i][h].y * r;
                    e[4 * h + 2] = gv[i][h].z * v[i][h].z * r;
                    e[4 * h + 3] = gv[i][h].w * v[i][h].w * r;
                }
            } else {
#pragma unroll
                for (int t = 0; t < 8; t++)
                    e[t] = 0.f;
            }
            if (a.tap_pre && run < nruns) { // the row the quantiser sees
                float4 *tp = (float4 *)(a.tap_pre + (size_t)b * a.D);
                tp[2 * run] = make_float4(e[0], e[1], e[2], e[3]);
                tp[2 * run + 1] = make_float4(e[4], e[5], e[6], e[7]);
            }
            if (a.quant) { // every lane takes part; 4 consecutive threads hold a block of 32
                float m = 0.f;
#pragma unroll
                for (int t = 0; t < 8; t++)
                    m = fmaxf(m, fabsf(e[t]));
                const float sc = q8_scale(group_max<4>(m));
#pragma unroll
                for (int t = 0; t < 8; t++)
                    e[t] = q8_dequant(q8_code(e[t], sc), sc);
            }
            if (run < nruns)
                norm_store_run(a, b, run, e, y, tap);
        }
    }
}

// One half-wave per block of 32 consecutive elements of p (rows are
// D-contiguous and D % 32 == 0, so block j of the flat array is block
// j % (D/32) of row j / (D/32)). With a fused merge, each lane also writes
// x_out = residual + sum of the wires in order, its own wire's value being
// the dequantised code it just wrote (the other wires' elements are requested
// together with p). The wires of a quantised exchange are all int8.
__global__ __launch_bounds__(64) void k_wire(WireArgs a)
{
    const int blk = blockIdx.x * 2 + (threadIdx.x >> 5);
    const int nblk = a.B * (a.D / kQBlock);
    const int lane = threadIdx.x & 31;
    const bool ok = blk < nblk;
    const size_t i = (size_t)blk * kQBlock + lane;
    float mres = 0.f;
    uint2 mpre[kMO];
    if (ok && a.mo.n_wires)
        merge_preload1<true>(a.mo, i, mres, mpre);
    const float v = ok ? a.p[i] : 0.f;
    const float s = q8_scale(group_max<32>(fabsf(v)));
    if (ok) {
        const int c = q8_code(v, s);
        a.codes[i] = (int8_t)c;
        if (lane == 0)
            a.scales[blk] = s;
        if (a.mo.n_wires)
            merge_finish1<true>(a.mo, i, q8_dequant(c, s), mres, mpre);
    }
}

// Weight quantisation at load time: rows of a bf16 or fp32 matrix (pitch
// src_pitch elements) to int8 codes and one fp32 scale per 32 consecutive
// elements of a row, with the block-32 codec of the exchanged activations.
// One 32-lane group per block (the group's max |w| by butterfly), as k_wire.
__global__ __launch_bounds__(256) void k_quant_rows(QuantRowsArgs a)
{
    const int nb = a.cols / kQBlock;
    const long blk = (long)blockIdx.x * 8 + (threadIdx.x >> 5);
    const int lane = threadIdx.x & 31;
    const bool ok = blk < (long)a.rows * nb;
    const long row = ok ? blk / nb : 0;
    const int c = ok ? (int)(blk % nb) * kQBlock + lane : 0;
    float v = 0.f;
    if (ok) {
        const size_t e = (size_t)row * a.src_pitch + c;
        v = a.src_bf16 ? bf16_to_f32(((const uint16_t *)a.src)[e]) : ((const float *)a.src)[e];
    }
    const float s = q8_scale(group_max<32>(fabsf(v)));
    if (ok) {
        a.codes[(size_t)row * a.code_pitch + c] = (int8_t)q8_code(v, s);
        if (lane == 0)
            a.scales[(size_t)row * a.scale_pitch + c / kQBlock] = s;
    }
}

hipError_t launch_quant_rows(const QuantRowsArgs &a, hipStream_t st)
{
    const long n = (long)a.rows * (a.cols / kQBlock);
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_quant_rows, dim3((unsigned)((n + 7) / 8)), dim3(256), 0, st, a);
    return hipGetLastError();
}

// out = residual + d_0 + d_1 + ... (array order), 4 elements per thread;
// the wires are read 8 at a time so their loads are in flight together.
__global__ __launch_bounds__(256) void k_merge(MergeArgs a)
{
    constexpr int U = 8;
    const MergeIn &m = a.m;
    const size_t n = (size_t)a.B * a.D;
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n)
        return;
    float4 acc = *(const float4 *)(m.residual + i);
    for (int s0 = 0; s0 < m.n_wires; s0 += U) {
        u32x4 r[U];
#pragma unroll
        for (int u = 0; u < U; u++)
            if (s0 + u < m.n_wires)
                r[u] = wire_load(m, s0 + u, i);
#pragma unroll
        for (int u = 0; u < U; u++)
            if (s0 + u < m.n_wires)
                wire_add(acc, m, r[u]);
    }
    *(float4 *)(m.x_out + i) = acc;
}

// Logits merge: 4 elements of shard blockIdx.y's slice per thread, read from
// its wire (int8 codes + block scale, or fp32) and stored at their place in
// the full row. The shard index is uniform over the workgroup, so the wire's
// address comes from the kernel arguments with a scalar load.
__global__ __launch_bounds__(256) void k_merge_logits(LogitsMergeArgs a)
{
    const int s = blockIdx.y;
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= (size_t)a.B * a.Vs)
        return;
    const size_t b = i / a.Vs, j = i % a.Vs;
    const u32x4 r = wire_load(a.m, s, i);
    float4 v;
    if (a.m.quant) {
        const float sc = __uint_as_float(r.y);
        v.x = q8_dequant((int)(int8_t)(r.x & 0xffu), sc);
        v.y = q8_dequant((int)(int8_t)((r.x >> 8) & 0xffu), sc);
        v.z = q8_dequant((int)(int8_t)((r.x >> 16) & 0xffu), sc);
        v.w = q8_dequant((int)(int8_t)(r.x >> 24), sc);
    } else {
        v = make_float4(__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z),
                        __uint_as_float(r.w));
    }
    *(float4 *)(a.out + b * a.V + (size_t)s * a.Vs + j) = v;
}

// All-to-all: 4 consecutive columns of one row of source blockIdx.y per
// thread (the source index is uniform over the workgroup: a scalar load of
// its address from the kernel arguments).
__global__ __launch_bounds__(256) void k_a2a(A2aArgs a)
{
    const int i = blockIdx.y, c4 = a.C / 4;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= a.nb * c4)
        return;
    const int b = t / c4, c = (t % c4) * 4;
    size_t so, dof;
    if (a.dir == 0) {
        so = (size_t)(a.r * a.nb + b) * a.ld_src + c;
        dof = (size_t)b * a.ld_dst + (size_t)i * a.C + c;
    } else {
        so = (size_t)b * a.ld_src + (size_t)a.r * a.C + c;
        dof = (size_t)(i * a.nb + b) * a.ld_dst + c;
    }
    *(float4 *)(a.dst + dof) = *(const float4 *)(a.src[i] + so);
}

// cos / sin of p * theta^(-2i/hd) in fp64, stored fp32: [max_ctx][hd/2].
__global__ __launch_bounds__(256) void k_rope_table(RopeArgs a)
{
    const int half = a.hd / 2;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.max_ctx * half)
        return;
    const int p = idx / half, i = idx % half;
    const double ang = (double)p * pow(a.theta, -2.0 * (double)i / (double)a.hd);
    a.table[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

__global__ void k_clear_u32(unsigned *p, int n)
{
    const int i = blockIdx.x * 64 + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

hipError_t launch_rmsnorm(const NormArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL(k_rmsnorm, dim3(a.B), dim3(kNormThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_wire(const WireArgs &a, hipStream_t st)
{
    // two 32-element blocks (one wave) a workgroup: the 128 blocks of a 7B
    // row spread over 64 CUs rather than 16
    const int nblk = a.B * (a.D / kQBlock);
    hipLaunchKernelGGL(k_wire, dim3((nblk + 1) / 2), dim3(64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs &a, hipStream_t st)
{
    const size_t n4 = (size_t)a.B * a.D / 4;
    if (n4 == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_merge, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

// Host-checked: Vs % 4 == 0, V = T * Vs, out and the wires 16-byte aligned.
hipError_t launch_merge_logits(const LogitsMergeArgs &a, int T, hipStream_t st)
{
    const size_t n4 = (size_t)a.B * a.Vs / 4;
    if (n4 == 0 || T < 1)
        return hipSuccess;
    hipLaunchKernelGGL(k_merge_logits, dim3((unsigned)((n4 + 255) / 256), (unsigned)T), dim3(256), 0,
                       st, a);
    return hipGetLastError();
}

// Host-checked: C, ld_src, ld_dst multiples of 4, buffers 16-byte aligned,
// every source holding the rows and columns the direction reads.
hipError_t launch_a2a(const A2aArgs &a, hipStream_t st)
{
    const long n = (long)a.nb * (a.C / 4);
    if (n == 0 || a.T < 1)
        return hipSuccess;
    hipLaunchKernelGGL(k_a2a, dim3((unsigned)((n + 255) / 256), (unsigned)a.T), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_rope_table(const RopeArgs &a, hipStream_t st)
{
    const int n = a.max_ctx * (a.hd / 2);
    hipLaunchKernelGGL(k_rope_table, dim3((n + 255) / 256), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_clear_u32(unsigned *p, int n, hipStream_t st)
{
    hipLaunchKernelGGL(k_clear_u32, dim3((n + 63) / 64), dim3(64), 0, st, p, n);
    return hipGetLastError();
}

} // namespace tps
