// common.h -- device helpers and launch-argument records shared by the
// library's HIP sources (gfx950, wave64). Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {

constexpr int kWave = 64;

// 16-byte vector of a native vector type (usable with the nontemporal builtins)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kMaxWires = 64;
constexpr int kQBlock = 32;

// ---------------------------------------------------------------- bf16

// bf16 is the upper half of an fp32: widening is a shift, exact.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest, ties to even (gfx950's conversion
// instruction, v_cvt_pk_bf16_f32; NaN gives a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// ---------------------------------------------------------------- buffer loads
// A raw buffer resource over [p, p + bytes): a load at an offset at or past
// `bytes` returns zeros without touching memory. The decode projections issue
// their weight loads through these unconditionally (out-of-range lanes get
// kOob), which lets the compiler count outstanding loads exactly: a wait for
// an earlier small load (an activation row) then does not also wait for the
// weights behind it.
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes)
{
    // 0x00020000: the third descriptor word of a raw 32-bit-format buffer on CDNA
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 buf_load8_nt(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2); // nontemporal
}
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2); // nontemporal
}

// s_waitcnt vmcnt(0), the other counters unconstrained (gfx9 encoding): no
// vector memory operation of this wave in flight afterwards
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }

// ---------------------------------------------------------------- RoPE
// The rotation of one pair (x, y) by (c, s) = (cos, sin):
// (x c - y s, x s + y c), each as one fused multiply-add over the other,
// rounded, product. Written out so that every kernel rounds it the same way:
// left to the compiler's contraction, which of the two products was fused
// differed between kernels, by one ulp of the result.
__device__ __forceinline__ float2 rope_pair(float x, float y, float c, float s)
{
    return make_float2(fmaf(x, c, -(y * s)), fmaf(x, s, y * c));
}

// ---------------------------------------------------------------- hand-off words
// A value passed from one workgroup to another inside one launch: the fp32
// bits in the low half and the launch's tag in the high half of one 8-byte
// word, written and read by single agent-scope atomic accesses. These keep
// the word coherent across the XCDs' separate L2 caches, and a reader that
// sees the tag sees the value stored with it, so no fence is needed. The
// tag is the stage's epoch + 1, never 0 (the zeroed region matches no tag).
__device__ __forceinline__ void hand_publish(uint64_t *w, float v, uint32_t tag)
{
    __hip_atomic_store(w, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
// Two aligned hand-off words in one 16-byte load with the device-scope cache
// policy (sc1, the bits the compiler gives an agent-scope atomic load): each
// 8-byte word arrives whole, as it was stored, so its tag vouches for its
// value; all of a lane's loads are issued before the first is waited on (a
// chain of atomic loads would wait for each in turn).
constexpr int kCpolSc1 = 16;
__device__ __forceinline__ u32x4 hand_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1);
}
// error-word bits (the C header's TP_DERR_*)
constexpr uint32_t kDerrLen = 1u, kDerrHandoff = 2u;
// longest wait for hand-off words: 2^24 ticks of the 100 MHz real-time
// counter (0.17 s), then kDerrHandoff is set and the waiter goes on
constexpr uint64_t kHandWaitTicks = 1ull << 24;

// ---------------------------------------------------------------- wave reductions

// Rotation right by N lanes inside each 16-lane row (DPP row_ror:N, a VALU
// operand modifier: no LDS round trip).
template <int N>
__device__ __forceinline__ float row_ror(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_value(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// DPP lane permutations inside 16-lane rows (VALU operand modifiers, no LDS
// round trip): swap neighbours (lane i ^ 1), swap pairs (i ^ 2), mirror each
// 8-lane half (i -> 7 - i) and mirror the row (i -> 15 - i).
template <int CTRL>
__device__ __forceinline__ float dpp_perm(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppRowMirror = 0x140;

// Reductions over groups of W consecutive lanes (W a power of two <= 64),
// result in every lane of the group; all lanes of the wave active. W = 64:
// rotations by 8, 4, 2, 1 leave each 16-lane row's total in its lanes, then
// the four row totals (lanes 0, 16, 32, 48) are combined as wave-uniform
// values, (r0 + r1) + (r2 + r3). Smaller W: a butterfly, each step adding
// the partner lane's value: lanes i ^ 1 and i ^ 2 by DPP, then, with every
// 4- (8-) lane group already uniform, the mirrored lane stands for lane i ^ 4
// (i ^ 8), also by DPP; the step across 16-lane rows (W = 32) through
// ds_bpermute. Each lane adds the same two values as in a plain xor
// butterfly, so the results are those of one.
template <int W>
__device__ __forceinline__ float group_sum(float v)
{
    if constexpr (W == 64) {
        v += row_ror<8>(v);
        v += row_ror<4>(v);
        v += row_ror<2>(v);
        v += row_ror<1>(v);
        return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
    } else {
        static_assert(W == 2 || W == 4 || W == 8 || W == 16 || W == 32, "group width");
        v += dpp_perm<kDppXor1>(v);
        if constexpr (W >= 4)
            v += dpp_perm<kDppXor2>(v);
        if constexpr (W >= 8)
            v += dpp_perm<kDppHalfMirror>(v);
        if constexpr (W >= 16)
            v += dpp_perm<kDppRowMirror>(v);
        if constexpr (W >= 32)
            v += __shfl_xor(v, 16, kWave);
        return v;
    }
}

template <int W>
__device__ __forceinline__ float group_max(float v)
{
    if constexpr (W == 64) {
        v = fmaxf(v, row_ror<8>(v));
        v = fmaxf(v, row_ror<4>(v));
        v = fmaxf(v, row_ror<2>(v));
        v = fmaxf(v, row_ror<1>(v));
        return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
    } else {
        static_assert(W == 2 || W == 4 || W == 8 || W == 16 || W == 32, "group width");
        v = fmaxf(v, dpp_perm<kDppXor1>(v));
        if constexpr (W >= 4)
            v = fmaxf(v, dpp_perm<kDppXor2>(v));
        if constexpr (W >= 8)
            v = fmaxf(v, dpp_perm<kDppHalfMirror>(v));
        if constexpr (W >= 16)
            v = fmaxf(v, dpp_perm<kDppRowMirror>(v));
        if constexpr (W >= 32)
            v = fmaxf(v, __shfl_xor(v, 16, kWave));
        return v;
    }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- block-32 int8 codec
// scale = max|x| / 127 (IEEE fp32 division); code = round-half-away(x / scale)
// clamped to +-127; zero scale -> zero code. `amax` is the block's max |x|.
__device__ __forceinline__ float q8_scale(float amax) { return amax / 127.0f; }
__device__ __forceinline__ int q8_code(float x, float scale)
{
    if (scale == 0.0f)
        return 0;
    float r = roundf(x / scale);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}
// dequantisation: one rounded fp32 multiply, never contracted into the add
// that consumes it (the contract flag is off for this product, so the
// compiler's default fp-contract cannot fuse it into an FMA)
__device__ __forceinline__ float q8_dequant(int code, float scale)
{
#pragma clang fp contract(off)
    return (float)code * scale;
}

// ---------------------------------------------------------------- merge of shard partials
// x = residual + d_0 + d_1 + ... in wire order, one fp32 add per element and
// wire, d_s the (dequantised) partial carried by wire s. The merge kernel and
// the merge fused into the kernel that produces a shard's own partial both
// use these helpers, so their results are bitwise equal.
struct MergeIn {
    const void *wires[kMaxWires];
    const float *residual; // [B][D]
    float *x_out;          // [B][D] merged rows
    int n_wires;           // 0: no merge
    int quant;             // wires hold int8 codes [B][D] + fp32 block scales
    int own;               // wire whose values the producing kernel holds (-1: none)
    uint64_t scales_off;   // byte offset of the scales inside a wire
};

// raw load of the 4 elements at flat index i (= b * D + k, i % 4 == 0) of wire s
__device__ __forceinline__ u32x4 wire_load(const MergeIn &m, int s, size_t i)
{
    const char *w = (const char *)m.wires[s];
    if (m.quant)
        return u32x4{*(const uint32_t *)(w + i),
                     __float_as_uint(((const float *)(w + m.scales_off))[i / kQBlock]), 0u, 0u};
    return *(const u32x4 *)(w + 4 * i);
}

__device__ __forceinline__ void wire_add(float4 &acc, const MergeIn &m, const u32x4 &r)
{
    if (m.quant) {
        const float sc = __uint_as_float(r.y);
        acc.x = acc.x + q8_dequant((int)(int8_t)(r.x & 0xffu), sc);
        acc.y = acc.y + q8_dequant((int)(int8_t)((r.x >> 8) & 0xffu), sc);
        acc.z = acc.z + q8_dequant((int)(int8_t)((r.x >> 16) & 0xffu), sc);
        acc.w = acc.w + q8_dequant((int)(int8_t)(r.x >> 24), sc);
    } else {
        acc.x = acc.x + __uint_as_float(r.x);
        acc.y = acc.y + __uint_as_float(r.y);
        acc.z = acc.z + __uint_as_float(r.z);
        acc.w = acc.w + __uint_as_float(r.w);
    }
}

// One element of wire s at flat index i: (code, scale) of an int8 wire (Q)
// or the fp32 bits.
template <bool Q>
__device__ __forceinline__ uint2 wire_load1(const MergeIn &m, int s, size_t i)
{
    const char *w = (const char *)m.wires[s];
    if constexpr (Q)
        return make_uint2((uint32_t)(uint8_t)w[i], __float_as_uint(((const float *)(w + m.scales_off))[i / kQBlock]));
    else
        return make_uint2(((const uint32_t *)w)[i], 0u);
}

template <bool Q>
__device__ __forceinline__ float wire_value1(uint2 r)
{
    if constexpr (Q)
        return q8_dequant((int)(int8_t)(r.x & 0xffu), __uint_as_float(r.y));
    else
        return __uint_as_float(r.x);
}

// Fused merge of one element at flat index i by the lane that holds the own
// partial's value v: the residual and wires 0..kMO-1 are requested by
// merge_preload1 (early, so they are in flight with the kernel's other
// loads), later wires by merge_finish1.
constexpr int kMO = 8;

template <bool Q>
__device__ __forceinline__ void merge_preload1(const MergeIn &m, size_t i, float &res, uint2 (&pre)[kMO])
{
    res = m.residual[i];
#pragma unroll
    for (int k = 0; k < kMO; k++)
        if (k < m.n_wires && k != m.own)
            pre[k] = wire_load1<Q>(m, k, i);
}

template <bool Q>
__device__ __forceinline__ void merge_finish1(const MergeIn &m, size_t i, float v, float res,
                                              const uint2 (&pre)[kMO])
{
    float acc = res;
#pragma unroll
    for (int k = 0; k < kMO; k++)
        if (k < m.n_wires)
            acc = acc + (k == m.own ? v : wire_value1<Q>(pre[k]));
    for (int k = kMO; k < m.n_wires; k++)
        acc = acc + (k == m.own ? v : wire_value1<Q>(wire_load1<Q>(m, k, i)));
    m.x_out[i] = acc;
}

// ---------------------------------------------------------------- launch records

struct NormArgs {
    const float *x;      // [B][D]
    const float *g;      // [D]
    float *xn;           // [B][D]
    float *tap;          // optional [B][D]
    uint16_t *xf;        // optional: xn in the MFMA fragment layout (hi/lo bf16)
    int B, D;
    float eps;
    int quant;           // int8 round trip of the normalised row
    float *tap_pre;      // optional [B][D]: the normalised row before that round trip
};

// ---------------------------------------------------------------- MFMA fragment layout
// Activations of a batch of <= 16 rows, K a multiple of 128, as the B operand
// of v_mfma_f32_16x16x32_bf16: the fp32 value v is split into hi = bf16(v)
// and lo = bf16(v - hi) (hi + lo carries ~16 mantissa bits). Element (b, k)
// of part hl sits at [k/128][hl][s][q][b][e] with k % 128 = 32s + 8q + e, so
// lane (q, b) of a wave reads its 8 values for step s as 16 contiguous bytes
// and a wave reads 1 KiB contiguous per step. The same k-slot order on the
// weight side makes the 4 lanes that share a weight row read 64 contiguous
// bytes of it per step (32s + 8q), half a 128-byte line, instead of 16
// bytes from each of 4 places (measured: the 70B up-projection 48 -> 41 us).
__host__ __device__ inline size_t xf_index(int b, int k, int hl)
{
    const int j = k >> 7, r = k & 127, q = (r >> 3) & 3, s = r >> 5, e = k & 7;
    return ((((((size_t)j * 2 + hl) * 4 + s) * 4 + q) * 16 + b) << 3) + e;
}
__host__ __device__ inline size_t xf_elems(int K) { return (size_t)K * 32; } // 16 rows x K x {hi, lo}

__device__ __forceinline__ void xf_store(uint16_t *xf, int b, int k, float v)
{
    const uint16_t hi = f32_to_bf16(v);
    const uint16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
    xf[xf_index(b, k, 0)] = hi;
    xf[xf_index(b, k, 1)] = lo;
}

struct MfmaGemvArgs {
    const uint16_t *W;   // bf16 [N][K] (or int8 codes [N][K] with ws), N % 16 == 0, K % 128 == 0
    const uint16_t *xf;  // activations in the fragment layout
    float *y;            // EPI_STORE: y[b][n] (ld ldy); EPI_SWIGLU: y[b][n/2]
    float *tap;          // optional copy of y
    uint16_t *yf;        // EPI_SWIGLU: optional y in the fragment layout (K' = N/2)
    int N, K, B, ldy, wk; // wk = waves per 16-row tile (K split)
    MergeIn mo;          // EPI_STORE, fp32 wires: fused merge (y is wire mo.own)
    float *part;         // split-K partials [S][B][N] then [S][16] row sums of squares
                         // (gemv_sk_part_floats floats), or null
    int nbs, S;          // split-K: 128-blocks per K slice, number of slices (set by the launcher)
    // split-K with the RMSNorm folded in (xs != null, instead of xf): the
    // operand is xs[b][k] * g[k] (xs the raw fp32 stage input, row stride K)
    // and the epilogue scales row b by 1 / sqrt(mean_k xs[b][k]^2 + eps)
    const float *xs;
    const float *g;
    float eps;
    const float *ws;     // int8 weights: W holds the codes, ws the scales [N][K/32]
};

// EPI_Q8 (batch <= 4, LDS-staged GEMV only): the row-split projection's
// partial goes straight into the block-32 int8 wire (codes + scales), each
// workgroup owning whole 32-row blocks; with a merge request the int8 wires
// are merged in the same epilogue.
enum GemvEpi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_Q8 = 2 };

// Weight types of the projections: fp32, bf16, or int8 codes with one fp32
// scale per 32 consecutive k of a row (the block-32 codec applied to the
// weights at load time).
enum WeightType { WT_F32 = 0, WT_BF16 = 1, WT_I8 = 2 };
__host__ __device__ constexpr int wt_per_chunk(int wt) { return wt == WT_I8 ? 16 : wt == WT_BF16 ? 8 : 4; }

struct GemvArgs {
    const void *W;       // [N][K] row-major, 16-byte aligned rows
    const float *ws;     // WT_I8: scales [N][K/32]
    const float *x;      // [B][ldx]
    float *y;            // [B][ldy]; SwiGLU: y[b][n/2]
    float *tap;          // optional copy of y, same layout
    int N, K, B, ldx, ldy;
    // fused RMSNorm prologue (g != null): x is the raw stage input and the
    // product uses xn = g * x / sqrt(mean(x^2) + eps) [int8 round trip if qin]
    const float *g;
    float eps;
    int qin;
    float *xn_tap;       // [B][K]: the normalised rows, written by block 0
    float *xq_tap;       // [B][K]: the same before the int8 round trip, block 0
    // EPI_STORE, fp32 wires: merge of the stage's partials (this kernel's
    // output y is wire mo.own), written to mo.x_out [B][ldy]; EPI_Q8: the
    // same with int8 wires
    MergeIn mo;
    int8_t *codes;       // EPI_Q8: [B][ldy] int8 codes of the wire
    float *scales;       // EPI_Q8: [B][ldy/32] block scales
    // after a one-launch QKV + attention (the stage's W_O): the epoch whose
    // + 1 tagged that launch's hand-off words, advanced by thread 0 of
    // workgroup 0 (this kernel starts after every workgroup of that launch
    // has read it); null otherwise
    uint32_t *epoch;
};

struct AttnArgs {
    const float *qkv;    // [B][ld_qkv]: q heads, then k heads, then v heads (raw, unrotated)
    const int *lens;     // [B]
    void *kc, *vc;       // [max_batch][Hkv_s][max_ctx][hd]
    const float2 *rope;  // [max_ctx][hd/2] (cos, sin)
    float *part;         // [B][Hq_s][n_chunks][hd + 4]: (m, l, -, -, o[hd])
    unsigned *err;
    float *att;          // [B][Hq_s*hd] combined attention output
    float *tap_q, *tap_k, *tap_v, *tap_att;
    uint16_t *att_xf;    // optional: att in the MFMA fragment layout
    int ld_qkv, max_ctx, Hq_s, Hkv_s, G, hd, n_chunks;
    float scale;
    int B;               // sequences (set by launch_attn)
    // one-launch QKV + attention, for the error-path test only (0, 0 otherwise):
    // the longest wait for hand-off words in ticks (0: kHandWaitTicks) and a
    // mask applied to the tag the waiting workgroups look for (nonzero: a tag
    // no word carries, so every wait runs out)
    uint32_t hand_wait_ticks, hand_tag_xor;
};

__device__ __forceinline__ uint64_t hand_wait_ticks(const AttnArgs &a)
{
    return a.hand_wait_ticks ? (uint64_t)a.hand_wait_ticks : kHandWaitTicks;
}

struct WireArgs {
    const float *p;      // [B][D]
    int8_t *codes;       // [B][D]
    float *scales;       // [B][D/32]
    int B, D;
    MergeIn mo;          // fused merge (codes/scales are wire mo.own), n_wires 0: none
};

struct MergeArgs {
    MergeIn m;           // out = m.x_out
    int B, D;
};

// All-to-all around batch-sharded attention, shard r of T: nb rows x C
// columns from each source i (grid.y) to its place in dst. dir 0 (heads to
// batch): source row r*nb + b, columns [0, C) -> dst row b, columns
// [i*C, (i+1)*C); dir 1 (batch to heads): source row b, columns
// [r*C, (r+1)*C) -> dst row i*nb + b, columns [0, C).
struct A2aArgs {
    const float *src[kMaxWires];
    float *dst;
    int64_t ld_src, ld_dst; // row strides in elements
    int nb, C, r, T, dir;
};

// Logits merge: wire s's rows [B][Vs] (dequantised) into columns
// [s*Vs, (s+1)*Vs) of out [B][V]; m.wires / quant / scales_off as in a merge.
struct LogitsMergeArgs {
    MergeIn m;
    float *out;          // [B][V]
    int B, Vs, V;
};

// int8 weight packing: rows x cols (cols % 32 == 0) of src -> codes / scales
struct QuantRowsArgs {
    const void *src;
    int src_bf16;
    size_t src_pitch;   // elements
    int rows, cols;
    int8_t *codes;
    size_t code_pitch;  // bytes
    float *scales;
    size_t scale_pitch; // floats
};

struct RopeArgs {
    float2 *table;       // [max_ctx][hd/2]
    int max_ctx, hd;
    double theta;
};

struct Ffn2dArgs {
    const uint16_t *x;   // [B][E] bf16
    const uint16_t *w13; // [F/8][2][8][E] bf16: 8 gate rows, then the 8 matching up rows
    const uint16_t *w2;  // [E][F] bf16
    uint16_t *h;         // [B][F] bf16 workspace
    float *part;         // [splits][B][E] fp32 workspace (split-K partials)
    float *y;            // [B][E]
    int B, E, F;
};

// ---------------------------------------------------------------- launchers

hipError_t launch_rmsnorm(const NormArgs &a, hipStream_t st);
hipError_t launch_gemv(const GemvArgs &a, int wt, int epi, hipStream_t st);
hipError_t launch_gemv_mfma(const MfmaGemvArgs &a, int epi, hipStream_t st);
size_t gemv_sk_part_floats(int N, int K, int B);
bool gemv_sk_used(int N, int K); // the batch-16 N x K projection takes the split-K kernels
bool gemv_mfma_ok(int B, int N, int K, int w_bf16);
hipError_t launch_attn(const AttnArgs &a, int kv_bf16, int B, hipStream_t st);
bool qkv_attn_fusable(int wt, int B, int K, int N, int G, int hd, int kv_bf16);
hipError_t launch_qkv_attn(const GemvArgs &g, const AttnArgs &a, uint64_t *hand, uint64_t *recw,
                           const uint32_t *epoch, int wt, int B, hipStream_t st);
size_t attn_lds_bytes(int G, int hd, int kv_bf16, int n_chunks);
bool attn_hd_supported(int hd);
size_t gemv_lds_bytes(int B, int K);
bool gemv_fused_ok(int B, int K);
hipError_t launch_wire(const WireArgs &a, hipStream_t st);
hipError_t launch_merge(const MergeArgs &a, hipStream_t st);
hipError_t launch_merge_logits(const LogitsMergeArgs &a, int T, hipStream_t st);
hipError_t launch_a2a(const A2aArgs &a, hipStream_t st);
hipError_t launch_rope_table(const RopeArgs &a, hipStream_t st);
hipError_t launch_quant_rows(const QuantRowsArgs &a, hipStream_t st);
hipError_t launch_clear_u32(unsigned *p, int n, hipStream_t st);
hipError_t launch_ffn2d(const Ffn2dArgs &a, hipStream_t st, int which);
int ffn2d_splits(int B, int E, int F);

// measured-peak probes (k_probe.hip)
hipError_t launch_probe_read(const void *buf, uint64_t bytes, uint32_t *out, int blocks, hipStream_t st);
hipError_t launch_probe_mfma(int blocks, int iters, float *out, hipStream_t st);

// The static device buffer behind decode_step_noalloc (scratch.hip): its size,
// and its address on the current device (looked up once per device, then cached).
constexpr size_t kScratchBytes = (size_t)16 << 20;
hipError_t scratch_address(void **ptr);

} // namespace tps
