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

// One 256-thread block per row. Sum of squares in fp32 (wave butterflies,
// then the 4 wave sums in order), y = g * x * r with r = 1 / sqrt(ms + eps).
// With quant set, each run of 32 elements (one half-wave) is quantised and
// dequantised in place (the receiver of the broadcast sees these values).
__global__ __launch_bounds__(256) void k_rmsnorm(NormArgs a)
{
    const int b = blockIdx.x;
    const float *x = a.x + (size_t)b * a.D;
    __shared__ float red[4];
    float ss = 0.f;
    for (int i = threadIdx.x; i < a.D; i += 256) {
        const float v = x[i];
        ss += v * v;
    }
    ss = group_sum<64>(ss);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = (red[0] + red[1]) + (red[2] + red[3]);
    const float r = 1.0f / sqrtf(ss / (float)a.D + a.eps);
    float *y = a.xn + (size_t)b * a.D;
    float *tap = a.tap ? a.tap + (size_t)b * a.D : nullptr;
    for (int i0 = 0; i0 < a.D; i0 += 256) {
        const int i = i0 + threadIdx.x;
        float v = 0.f;
        if (i < a.D)
            v = a.g[i] * x[i] * r;
        if (a.quant) { // every lane takes part; lanes past D hold 0
            const float s = q8_scale(group_max<32>(fabsf(v)));
            v = q8_dequant(q8_code(v, s), s);
        }
        if (i < a.D) {
            y[i] = v;
            if (tap)
                tap[i] = v;
        }
    }
}

// One half-wave per block of 32 consecutive elements of p (rows are
// D-contiguous and D % 32 == 0, so block j of the flat array is block
// j % (D/32) of row j / (D/32)).
__global__ __launch_bounds__(256) void k_wire(WireArgs a)
{
    const int blk = blockIdx.x * 8 + (threadIdx.x >> 5);
    const int nblk = a.B * (a.D / kQBlock);
    const int lane = threadIdx.x & 31;
    const bool ok = blk < nblk;
    const float v = ok ? a.p[(size_t)blk * kQBlock + lane] : 0.f;
    const float s = q8_scale(group_max<32>(fabsf(v)));
    if (ok) {
        a.codes[(size_t)blk * kQBlock + lane] = (int8_t)q8_code(v, s);
        if (lane == 0)
            a.scales[blk] = s;
    }
}

// out = residual + d_0 + d_1 + ... (array order), 4 elements per thread;
// the wires are read 8 at a time so their loads are in flight together.
__global__ __launch_bounds__(256) void k_merge(MergeArgs a)
{
    constexpr int U = 8;
    const size_t n = (size_t)a.B * a.D;
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n)
        return;
    float4 acc = *(const float4 *)(a.residual + i);
    for (int s0 = 0; s0 < a.n_wires; s0 += U) {
        if (a.quant) {
            char4 c[U];
            float sc[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                if (s0 + u < a.n_wires) {
                    const char *w = (const char *)a.wires[s0 + u];
                    c[u] = *(const char4 *)(w + i);
                    sc[u] = ((const float *)(w + a.scales_off))[i / kQBlock];
                }
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                if (s0 + u < a.n_wires) {
                    acc.x = acc.x + q8_dequant(c[u].x, sc[u]);
                    acc.y = acc.y + q8_dequant(c[u].y, sc[u]);
                    acc.z = acc.z + q8_dequant(c[u].z, sc[u]);
                    acc.w = acc.w + q8_dequant(c[u].w, sc[u]);
                }
            }
        } else {
            float4 f[U];
#pragma unroll
            for (int u = 0; u < U; u++)
                if (s0 + u < a.n_wires)
                    f[u] = *(const float4 *)((const char *)a.wires[s0 + u] + i * 4);
#pragma unroll
            for (int u = 0; u < U; u++) {
                if (s0 + u < a.n_wires) {
                    acc.x = acc.x + f[u].x;
                    acc.y = acc.y + f[u].y;
                    acc.z = acc.z + f[u].z;
                    acc.w = acc.w + f[u].w;
                }
            }
        }
    }
    *(float4 *)(a.out + i) = acc;
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
    hipLaunchKernelGGL(k_rmsnorm, dim3(a.B), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_wire(const WireArgs &a, hipStream_t st)
{
    const int nblk = a.B * (a.D / kQBlock);
    hipLaunchKernelGGL(k_wire, dim3((nblk + 7) / 8), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs &a, hipStream_t st)
{
    const size_t n4 = (size_t)a.B * a.D / 4;
    hipLaunchKernelGGL(k_merge, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a);
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
