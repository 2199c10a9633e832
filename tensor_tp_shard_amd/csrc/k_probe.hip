// k_probe.hip -- the two measured-peak probes behind the benchmark's "% of
// measured peak" denominators: a plain read stream (what HBM delivers to
// 16-byte nontemporal vector loads with many in flight) and an MFMA loop
// (what the bf16 matrix cores deliver at the clock the chip runs, with no
// memory traffic). Neither is part of the shard step.
#include "common.h"

namespace tps {

typedef __bf16 bf16x8p_t __attribute__((ext_vector_type(8)));

// Each workgroup reads a contiguous span in rounds of kProbeIn 16-byte
// loads per thread, all issued before any is used; lanes past the span read
// through an empty part of the buffer resource (zeros, no access). The XOR of
// everything read goes to out[block] so the loads cannot be removed.
constexpr int kProbeIn = 8;

__global__ __launch_bounds__(256) void k_probe_read(const char *buf, uint64_t bytes, uint64_t span,
                                                    uint32_t *out)
{
    const uint64_t b0 = (uint64_t)blockIdx.x * span;
    const uint64_t b1 = b0 + span < bytes ? b0 + span : bytes;
    uint32_t acc = 0;
    for (uint64_t base = b0; base < b1; base += (uint64_t)256 * 16 * kProbeIn) {
        const uint64_t left = b1 - base;
        const __amdgpu_buffer_rsrc_t r =
            buf_rsrc(buf + base, left < 0x7fffffffull ? (uint32_t)left : 0x7fffffffu);
        u32x4 v[kProbeIn];
#pragma unroll
        for (int i = 0; i < kProbeIn; i++)
            v[i] = buf_load16_nt(r, (uint32_t)(16 * (threadIdx.x + 256 * i)));
#pragma unroll
        for (int i = 0; i < kProbeIn; i++)
            acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
    acc = (uint32_t)__shfl_xor((int)acc, 1, 64) ^ acc;
    if (threadIdx.x == 0)
        out[blockIdx.x] = acc;
}

// Four independent accumulator chains per wave of v_mfma_f32_32x32x16_bf16
// (32 x 32 x 16 x 2 = 32768 flops each) for `iters` rounds; operands come
// from registers (values derived from the thread index), results to out.
// (The 16 x 16 x 32 form needs more independent chains per wave than a
// register-only loop gives it to reach the same rate; measured 1.2 against
// 2.2 PFLOP/s here, while in a GEMM both forms run 1024 flops per busy cycle.)
typedef float f32x16p_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float *out)
{
    const float s = (float)(threadIdx.x & 15) * 0.0625f;
    bf16x8p_t a, b;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        a[i] = (__bf16)(s + (float)i * 0.125f);
        b[i] = (__bf16)(s - (float)i * 0.125f);
    }
    f32x16p_t c[4];
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
        for (int e = 0; e < 16; e++)
            c[j][e] = 0.f;
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int j = 0; j < 4; j++)
            c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
    }
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++)
        t += c[j][0] + c[j][15];
    out[blockIdx.x * 256 + threadIdx.x] = t;
}

hipError_t launch_probe_read(const void *buf, uint64_t bytes, uint32_t *out, int blocks, hipStream_t st)
{
    const uint64_t span = (bytes + (uint64_t)blocks - 1) / (uint64_t)blocks;
    const uint64_t round = (uint64_t)256 * 16 * kProbeIn;
    hipLaunchKernelGGL(k_probe_read, dim3(blocks), dim3(256), 0, st, (const char *)buf, bytes,
                       (span + round - 1) / round * round, out);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(int blocks, int iters, float *out, hipStream_t st)
{
    hipLaunchKernelGGL(k_probe_mfma, dim3(blocks), dim3(256), 0, st, iters, out);
    return hipGetLastError();
}

} // namespace tps
