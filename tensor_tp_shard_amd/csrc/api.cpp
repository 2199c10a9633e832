// api.cpp -- the C ABI of the shard library (include/tpshard.h): argument
// validation, the shard's slice plan, weight packing, workspace layout and
// the launch sequence of each stage on the caller's stream.
//
// The slice plan follows aiterms.tw "Tensor Parallelism", 核心概念 items 1-2:
// column-split weights (Wq, Wk, Wv, W1, W3) keep whole output rows of the
// shard's heads / FFN features; row-split weights (Wo, W2) keep the column
// block that multiplies the shard's slice of the activation, giving a
// full-size partial. The stage order follows distributed-llama issue
// "[Feature Suggest] Tensor Parallellism for Accelerating LLM",
// buildLlama2Arch (per layer: norm, quantise, QKV, attention, W_O, quantise,
// dequantise + merge; then norm, quantise, SwiGLU FFN, W2, quantise,
// dequantise + merge).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/tpshard.h"
#include "common.h"

using namespace tps;

namespace {

thread_local std::string g_err;

int32_t fail(int32_t st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

int32_t hip_fail(hipError_t e, const char *what)
{
    return fail(TP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

enum KernelId {
    KID_RMSNORM = 0,
    KID_GEMV_QKV,
    KID_ATTN,
    KID_GEMV_WO,
    KID_WIRE,
    KID_GEMV_W13,
    KID_GEMV_W2,
    KID_MERGE,
    KID_FFN2D_UP,
    KID_FFN2D_DOWN,
    KID_ROPE_TABLE,
    KID_GEMV_LOGITS,
    KID_MERGE_LOGITS,
    KID_A2A,
    KID_QKV_ATTN,
    KID_COUNT
};

const char *const kKernelNames[KID_COUNT] = {
    "rmsnorm",    "gemv_qkv", "attention", "gemv_wo",  "q8_wire",    "gemv_w13_swiglu",
    "gemv_w2",    "merge",    "ffn2d_up",  "ffn2d_down", "rope_table", "gemv_logits",
    "merge_logits", "all_to_all", "qkv_attention"};

} // namespace

struct tp_shard {
    tp_config cfg;
    // derived shape
    // (TP_LOGITS: F = vocabulary, Fs = the shard's V/T logits)
    int T, r, D, hd, Hq, Hkv, G, Hq_s, Hkv_s, F, Fs, n_qkv, esz, kv_esz;
    bool w8; // TP_Q_WEIGHTS: packed projections are int8 codes + fp32 scales per 32 k
    int nb = 0; // TP_ATTN_BATCH: sequences per shard (Hq_s, Hkv_s then hold every head)
    // packed layout (byte offsets)
    // (TP_LOGITS: the classifier rows at o_w13 / o_sw13, the final gain at o_gatt)
    uint64_t o_wqkv, o_wo, o_w13, o_w2, o_gatt, o_gffn, o_rope, packed_bytes;
    uint64_t o_sqkv, o_swo, o_sw13, o_sw2; // w8: scale arrays [N][K/32]
    // workspace layout (byte offsets)
    uint64_t w_err, w_xfx, w_xfatt, w_xfa, w_skp, w_xn, w_qkv, w_part, w_att, w_a, w_p, ws_bytes;
    // one-launch QKV + attention (batch <= 4): the stage's epoch (one word,
    // 256 bytes reserved), then hand-off words [min(max_batch, 4)][n_qkv],
    // then the chunk records as words [min(max_batch, 4)][Hq_s][n_chunks][hd
    // + 4] (at w_hand + hand_rec); 0: none
    uint64_t w_hand = 0, hand_bytes = 0, hand_rec = 0;
    bool hand_dirty = false; // a stage failed after its fused launch: clear before the next
    uint32_t hand_wait_ticks = 0, hand_tag_xor = 0; // tp_handoff_test (0, 0: normal)
    int n_chunks;
    bool mfma_ok = false; // the batch 5..16 MFMA path applies to this shape
    uint64_t kv_bytes, wire_bytes, part_rows = 0;
    // bound buffers
    char *packed = nullptr, *ws = nullptr;
    void *kc = nullptr, *vc = nullptr;
    bool loaded = false;
    // kernel timing probe
    int timing_kernel = -1;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> ev_pool;
    size_t ev_used = 0;
};

namespace {

// The final stage: the shard's V/T classifier rows (column split over the
// vocabulary) and the final gain; workspace for the normalised rows, their
// MFMA fragments, split-K partials and the fp32 logits before quantisation.
int32_t plan_logits(const tp_config &c, tp_shard &s)
{
    const int T = c.tp_size;
    if (T < 1 || c.tp_rank < 0 || c.tp_rank >= T)
        return fail(TP_EINVAL, "tp_rank %d outside [0, tp_size=%d)", c.tp_rank, T);
    if (c.ffn_hidden % T)
        return fail(TP_EINVAL, "tp_size must divide the vocabulary (ffn_hidden)");
    if (c.max_batch > 16)
        return fail(TP_EINVAL, "decode batch is at most 16");
    if (c.quant & TP_Q_INPUTS)
        return fail(TP_EINVAL, "TP_LOGITS has no int8 round trip of the normalised input");
    if (!(c.norm_eps >= 0.f))
        return fail(TP_EINVAL, "norm_eps must be >= 0");
    s.T = T;
    s.r = c.tp_rank;
    s.Fs = s.F / T;
    s.esz = c.w_dtype == TP_BF16 ? 2 : 4;
    s.w8 = (c.quant & TP_Q_WEIGHTS) != 0;
    const bool qpart = c.quant & TP_Q_PARTIALS;
    const int vec = 16 / s.esz;
    if (s.D % 8 || s.Fs % 8 || s.Fs % vec)
        return fail(TP_EINVAL, "dim and vocab/tp_size must be multiples of 8");
    if ((s.w8 && s.D % kQBlock) || (qpart && s.Fs % kQBlock))
        return fail(TP_EINVAL, "int8 weights need dim, an int8 wire vocab/tp_size, multiples of 32");
    const uint64_t D = s.D, B = c.max_batch, Vs = s.Fs, e = s.w8 ? 1 : s.esz;
    uint64_t o = 0;
    s.o_wqkv = s.o_wo = s.o_w2 = s.o_gffn = s.o_rope = 0;
    s.o_sqkv = s.o_swo = s.o_sw13 = s.o_sw2 = 0;
    s.o_w13 = o; o = align_up(o + Vs * D * e, 256);
    if (s.w8) {
        s.o_sw13 = o; o = align_up(o + Vs * (D / kQBlock) * 4, 256);
    }
    s.o_gatt = o; o = align_up(o + D * 4, 256);
    s.packed_bytes = o;
    s.mfma_ok = (c.w_dtype == TP_BF16 || s.w8) && c.max_batch > 4 && gemv_mfma_ok(16, s.Fs, s.D, 1);
    o = 0;
    s.w_err = o;  o = 256;
    s.w_xfx = s.w_xfatt = s.w_xfa = s.w_skp = 0;
    if (s.mfma_ok) {
        s.w_xfx = o; o = align_up(o + xf_elems(s.D) * 2, 256);
        const size_t skp = gemv_sk_part_floats(s.Fs, s.D, c.max_batch);
        s.w_skp = skp ? o : 0;
        o = align_up(o + skp * 4, 256);
    }
    s.w_xn = o; o = align_up(o + B * D * 4, 256);
    s.w_p = o;  o = align_up(o + B * Vs * 4, 256);
    s.w_qkv = s.w_part = s.w_att = s.w_a = 0;
    s.ws_bytes = o;
    s.kv_bytes = 0;
    s.wire_bytes = qpart ? align_up(B * Vs, 16) + B * (Vs / kQBlock) * 4 : B * Vs * 4;
    return TP_OK;
}

// Batch-sharded attention: the shard's nb = B/T sequences with every head;
// packed holds only the RoPE table; workspace the chunk records.
int32_t plan_attn_batch(const tp_config &c, tp_shard &s)
{
    const int T = c.tp_size;
    if (c.kv_dtype != TP_F32 && c.kv_dtype != TP_BF16)
        return fail(TP_EINVAL, "unknown kv_dtype %d", c.kv_dtype);
    if (T < 1 || c.tp_rank < 0 || c.tp_rank >= T)
        return fail(TP_EINVAL, "tp_rank %d outside [0, tp_size=%d)", c.tp_rank, T);
    if (c.max_batch % T || c.max_batch > 16 * T)
        return fail(TP_EINVAL, "TP_ATTN_BATCH: tp_size must divide max_batch, at most 16 sequences a shard");
    if (c.quant)
        return fail(TP_EINVAL, "TP_ATTN_BATCH has no int8 exchange");
    if (c.n_heads < 1 || c.n_kv_heads < 1 || c.max_ctx < 1)
        return fail(TP_EINVAL, "heads and max_ctx must be positive");
    if (c.n_heads % c.n_kv_heads || c.n_heads % T)
        return fail(TP_EINVAL, "n_kv_heads and tp_size must divide n_heads");
    if (!attn_hd_supported(c.head_dim))
        return fail(TP_EINVAL, "head_dim must be 16, 32, 48, 64 or 128");
    if (c.n_heads / c.n_kv_heads > 8)
        return fail(TP_EINVAL, "at most 8 q heads per kv head");
    if (!(c.rope_theta > 0.f))
        return fail(TP_EINVAL, "rope_theta must be > 0");
    s.T = T;
    s.r = c.tp_rank;
    s.nb = c.max_batch / T;
    s.hd = c.head_dim;
    s.Hq = s.Hq_s = c.n_heads;
    s.Hkv = s.Hkv_s = c.n_kv_heads;
    s.G = s.Hq / s.Hkv;
    s.n_qkv = (s.Hq + 2 * s.Hkv) * s.hd;
    s.kv_esz = c.kv_dtype == TP_BF16 ? 2 : 4;
    s.esz = 4;
    s.w8 = false;
    s.n_chunks = (c.max_ctx + 63) / 64;
    if (attn_lds_bytes(s.G, s.hd, c.kv_dtype == TP_BF16, s.n_chunks) > 64 * 1024)
        return fail(TP_EINVAL, "attention workgroup would need more than 64 KiB of LDS");
    const uint64_t nb = s.nb;
    s.o_wqkv = s.o_wo = s.o_w13 = s.o_w2 = s.o_gatt = s.o_gffn = 0;
    s.o_sqkv = s.o_swo = s.o_sw13 = s.o_sw2 = 0;
    s.o_rope = 0;
    s.packed_bytes = align_up((uint64_t)c.max_ctx * (s.hd / 2) * 8, 256);
    s.mfma_ok = false;
    s.w_xfx = s.w_xfatt = s.w_xfa = s.w_skp = s.w_xn = s.w_qkv = s.w_att = s.w_a = s.w_p = 0;
    s.w_err = 0;
    s.w_part = 256;
    s.ws_bytes = align_up(s.w_part + nb * s.Hq * (uint64_t)s.n_chunks * (s.hd + 4) * 4, 256);
    s.kv_bytes = nb * s.Hkv * (uint64_t)c.max_ctx * s.hd * s.kv_esz;
    s.wire_bytes = nb * s.Hq * s.hd * 4;
    return TP_OK;
}

int32_t plan(const tp_config &c, tp_shard &s)
{
    if (c.kind != TP_LLAMA_BLOCK && c.kind != TP_FFN_2D && c.kind != TP_LOGITS && c.kind != TP_ATTN_BATCH)
        return fail(TP_EINVAL, "unknown kind %d", c.kind);
    const bool weights = c.kind != TP_ATTN_BATCH; // batch-sharded attention has none
    if (weights && c.w_dtype != TP_F32 && c.w_dtype != TP_BF16)
        return fail(TP_EINVAL, "unknown w_dtype %d", c.w_dtype);
    if (c.quant & ~(TP_Q_PARTIALS | TP_Q_INPUTS | TP_Q_WEIGHTS))
        return fail(TP_EINVAL, "unknown quant bits 0x%x", c.quant);
    if (c.quant && c.quant_block != kQBlock)
        return fail(TP_EINVAL, "quant_block must be 32 (got %d)", c.quant_block);
    if (c.max_batch < 1 || c.max_batch > (1 << 20) || (weights && (c.dim < 1 || c.ffn_hidden < 1)))
        return fail(TP_EINVAL, "dim, ffn_hidden and max_batch must be positive");
    s.cfg = c;
    s.D = c.dim;
    s.F = c.ffn_hidden;
    if (c.kind == TP_FFN_2D) {
        if (c.w_dtype != TP_BF16)
            return fail(TP_EINVAL, "TP_FFN_2D needs bf16 weights");
        if (c.tp_size != 1 || c.tp_rank != 0)
            return fail(TP_EINVAL, "TP_FFN_2D takes an already-cut block: tp_size 1, tp_rank 0");
        if (c.quant)
            return fail(TP_EINVAL, "TP_FFN_2D has no int8 exchange");
        if (c.dim % 288 || c.dim % 64 || (2 * c.ffn_hidden) % 288 || c.ffn_hidden % 64)
            return fail(TP_EINVAL, "TP_FFN_2D needs E a multiple of 576, 2F of 288 and F of 64");
        s.T = 1;
        s.r = 0;
        s.esz = 2;
        s.o_w13 = 0;
        s.o_w2 = align_up(2ull * s.F * s.D * 2, 256);
        s.packed_bytes = align_up(s.o_w2 + (uint64_t)s.D * s.F * 2, 256);
        s.w_err = 0;
        s.w_a = 256; // H = silu(X Wg^T) * (X Win^T), bf16 [max_batch][F]
        s.w_p = align_up(s.w_a + (uint64_t)c.max_batch * s.F * 2, 256);
        uint64_t part_rows = 0; // split-K partial rows: the most any batch <= max_batch needs
        for (int b = 1; b <= c.max_batch; b++) {
            const int S = ffn2d_splits(b, s.D, s.F);
            if (S > 1 && (uint64_t)S * b > part_rows)
                part_rows = (uint64_t)S * b;
        }
        s.part_rows = part_rows;
        s.ws_bytes = align_up(s.w_p + part_rows * s.D * 4, 256);
        s.kv_bytes = 0;
        s.wire_bytes = (uint64_t)c.max_batch * s.D * 4;
        return TP_OK;
    }
    if (c.kind == TP_LOGITS)
        return plan_logits(c, s);
    if (c.kind == TP_ATTN_BATCH)
        return plan_attn_batch(c, s);
    if (c.kv_dtype != TP_F32 && c.kv_dtype != TP_BF16)
        return fail(TP_EINVAL, "unknown kv_dtype %d", c.kv_dtype);
    const int T = c.tp_size;
    if (T < 1 || c.tp_rank < 0 || c.tp_rank >= T)
        return fail(TP_EINVAL, "tp_rank %d outside [0, tp_size=%d)", c.tp_rank, T);
    if (c.n_heads < 1 || c.n_kv_heads < 1 || c.head_dim < 1 || c.max_ctx < 1)
        return fail(TP_EINVAL, "heads, head_dim and max_ctx must be positive");
    if (c.n_heads % c.n_kv_heads)
        return fail(TP_EINVAL, "n_heads %% n_kv_heads != 0");
    if (c.n_heads % T || c.n_kv_heads % T || c.ffn_hidden % T)
        return fail(TP_EINVAL, "tp_size must divide n_heads, n_kv_heads and ffn_hidden");
    if (!attn_hd_supported(c.head_dim))
        return fail(TP_EINVAL, "head_dim must be 16, 32, 48, 64 or 128");
    if (c.n_heads / c.n_kv_heads > 8)
        return fail(TP_EINVAL, "at most 8 q heads per kv head");
    if (c.max_batch > 16)
        return fail(TP_EINVAL, "decode batch is at most 16");
    if (c.quant && c.dim % kQBlock)
        return fail(TP_EINVAL, "dim must be a multiple of 32 when quantising");
    if (!(c.norm_eps >= 0.f) || !(c.rope_theta > 0.f))
        return fail(TP_EINVAL, "norm_eps must be >= 0 and rope_theta > 0");
    s.T = T;
    s.r = c.tp_rank;
    s.hd = c.head_dim;
    s.Hq = c.n_heads;
    s.Hkv = c.n_kv_heads;
    s.G = s.Hq / s.Hkv;
    s.Hq_s = s.Hq / T;
    s.Hkv_s = s.Hkv / T;
    s.Fs = s.F / T;
    s.n_qkv = (s.Hq_s + 2 * s.Hkv_s) * s.hd;
    s.esz = c.w_dtype == TP_BF16 ? 2 : 4;
    s.kv_esz = c.kv_dtype == TP_BF16 ? 2 : 4;
    s.w8 = (c.quant & TP_Q_WEIGHTS) != 0;
    if (s.w8 && (s.D % kQBlock || (s.Hq_s * s.hd) % kQBlock || s.Fs % kQBlock))
        return fail(TP_EINVAL, "int8 weights need dim, Hq/T*head_dim and ffn_hidden/T multiples of 32");
    const int vec = 16 / s.esz;
    if (s.D % 8 || (s.Hq_s * s.hd) % vec || s.Fs % vec)
        return fail(TP_EINVAL, "dim must be a multiple of 8, Hq/T*head_dim and ffn_hidden/T of %d",
                    vec);
    s.n_chunks = (c.max_ctx + 63) / 64;
    if (attn_lds_bytes(s.G, s.hd, c.kv_dtype == TP_BF16, s.n_chunks) > 64 * 1024)
        return fail(TP_EINVAL, "attention workgroup would need more than 64 KiB of LDS");
    const uint64_t D = s.D, B = c.max_batch, e = s.w8 ? 1 : s.esz; // packed bytes per weight
    uint64_t o = 0;
    s.o_wqkv = o; o = align_up(o + (uint64_t)s.n_qkv * D * e, 256);
    s.o_wo = o;   o = align_up(o + D * s.Hq_s * s.hd * e, 256);
    s.o_w13 = o;  o = align_up(o + 2ull * s.Fs * D * e, 256);
    s.o_w2 = o;   o = align_up(o + D * s.Fs * e, 256);
    s.o_sqkv = s.o_swo = s.o_sw13 = s.o_sw2 = 0;
    if (s.w8) { // one fp32 scale per 32 weights of a row
        s.o_sqkv = o; o = align_up(o + (uint64_t)s.n_qkv * (D / kQBlock) * 4, 256);
        s.o_swo = o;  o = align_up(o + D * (s.Hq_s * s.hd / kQBlock) * 4, 256);
        s.o_sw13 = o; o = align_up(o + 2ull * s.Fs * (D / kQBlock) * 4, 256);
        s.o_sw2 = o;  o = align_up(o + D * (s.Fs / kQBlock) * 4, 256);
    }
    s.o_gatt = o; o = align_up(o + D * 4, 256);
    s.o_gffn = o; o = align_up(o + D * 4, 256);
    s.o_rope = o; o = align_up(o + (uint64_t)c.max_ctx * (s.hd / 2) * 8, 256);
    s.packed_bytes = o;
    s.mfma_ok = (c.w_dtype == TP_BF16 || s.w8) && c.max_batch > 4 && gemv_mfma_ok(16, s.n_qkv, s.D, 1) &&
                gemv_mfma_ok(16, s.D, s.Hq_s * s.hd, 1) && gemv_mfma_ok(16, 2 * s.Fs, s.D, 1) &&
                gemv_mfma_ok(16, s.D, s.Fs, 1);
    o = 0;
    s.w_err = o;  o = 256;
    s.w_xfx = s.w_xfatt = s.w_xfa = s.w_skp = 0;
    if (s.mfma_ok) { // activations in the MFMA fragment layout
        s.w_xfx = o;   o = align_up(o + xf_elems(s.D) * 2, 256);
        s.w_xfatt = o; o = align_up(o + xf_elems(s.Hq_s * s.hd) * 2, 256);
        s.w_xfa = o;   o = align_up(o + xf_elems(s.Fs) * 2, 256);
        // split-K partials of the largest batch-16 projection
        size_t skp = gemv_sk_part_floats(s.n_qkv, s.D, c.max_batch);
        const size_t sk[] = {gemv_sk_part_floats(s.D, s.Hq_s * s.hd, c.max_batch),
                             gemv_sk_part_floats(2 * s.Fs, s.D, c.max_batch),
                             gemv_sk_part_floats(s.D, s.Fs, c.max_batch)};
        for (size_t v : sk)
            skp = v > skp ? v : skp;
        s.w_skp = skp ? o : 0;
        o = align_up(o + skp * 4, 256);
    }
    s.w_xn = o;   o = align_up(o + B * D * 4, 256);
    s.w_qkv = o;  o = align_up(o + B * s.n_qkv * 4, 256);
    s.w_part = o; o = align_up(o + B * s.Hq_s * (uint64_t)s.n_chunks * (s.hd + 4) * 4, 256);
    s.w_att = o;  o = align_up(o + B * s.Hq_s * s.hd * 4, 256);
    s.w_a = o;    o = align_up(o + B * s.Fs * 4, 256);
    s.w_p = o;    o = align_up(o + B * D * 4, 256);
    {
        const int wt = s.w8 ? WT_I8 : c.w_dtype == TP_BF16 ? WT_BF16 : WT_F32;
        const int hb = c.max_batch < 4 ? c.max_batch : 4;
        if (qkv_attn_fusable(wt, 1, s.D, s.n_qkv, s.G, s.hd, c.kv_dtype == TP_BF16)) {
            s.w_hand = o;
            s.hand_rec = align_up(256 + (uint64_t)hb * s.n_qkv * 8, 256);
            s.hand_bytes = s.hand_rec + (uint64_t)hb * s.Hq_s * s.n_chunks * (s.hd + 4) * 8;
            o = align_up(o + s.hand_bytes, 256);
        }
    }
    s.ws_bytes = o;
    s.kv_bytes = B * s.Hkv_s * (uint64_t)c.max_ctx * s.hd * s.kv_esz;
    const uint64_t wq = align_up(B * D, 16) + B * (D / kQBlock) * 4;
    s.wire_bytes = (c.quant & TP_Q_PARTIALS) ? wq : B * D * 4;
    return TP_OK;
}

int32_t check_device()
{
    int dev = -1, n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1)
        return fail(TP_ENODEV, "no HIP device");
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(TP_ENODEV, "no current HIP device");
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess)
        return fail(TP_ENODEV, "hipGetDeviceProperties failed");
    if (strncmp(p.gcnArchName, "gfx950", 6) != 0)
        return fail(TP_ENODEV, "device %d is %s, the library is built for gfx950", dev,
                    p.gcnArchName);
    return TP_OK;
}

// Runs `launch` with the timing probe's events around it when armed.
template <typename F>
int32_t timed(tp_shard *s, int kid, hipStream_t st, const char *what, F &&launch)
{
    const bool arm = s->timing_kernel == kid;
    if (arm) {
        if (s->ev_used == s->ev_pool.size()) {
            hipEvent_t a, b;
            // no system-scope fence at the record: the pair then brackets the
            // kernel within ~0.5 us of its execution time (a default event adds
            // a few microseconds of its own)
            if (hipEventCreateWithFlags(&a, hipEventDisableSystemFence) != hipSuccess ||
                hipEventCreateWithFlags(&b, hipEventDisableSystemFence) != hipSuccess)
                return fail(TP_EHIP, "hipEventCreate failed");
            s->ev_pool.emplace_back(a, b);
        }
        hipEventRecord(s->ev_pool[s->ev_used].first, st);
    }
    const hipError_t e = launch();
    if (e != hipSuccess)
        return hip_fail(e, what);
    if (arm) {
        hipEventRecord(s->ev_pool[s->ev_used].second, st);
        s->ev_used++;
    }
    return TP_OK;
}

hipError_t copy2d(void *dst, size_t dpitch, const void *src, size_t spitch, size_t width,
                  size_t rows, hipStream_t st)
{
    return hipMemcpy2DAsync(dst, dpitch, src, spitch, width, rows, hipMemcpyDeviceToDevice, st);
}

} // namespace

extern "C" {

int32_t init_shard(const tp_config *cfg, tp_shard **out, tp_sizes *sizes)
{
    if (!cfg || !out || !sizes)
        return fail(TP_EINVAL, "init_shard: null argument");
    *out = nullptr;
    tp_shard *s = new (std::nothrow) tp_shard();
    if (!s)
        return fail(TP_EINVAL, "init_shard: out of host memory");
    const int32_t st = plan(*cfg, *s);
    if (st != TP_OK) {
        delete s;
        return st;
    }
    sizes->packed_weights = s->packed_bytes;
    sizes->kv_cache_each = s->kv_bytes;
    sizes->workspace = s->ws_bytes;
    sizes->wire = s->wire_bytes;
    *out = s;
    return TP_OK;
}

void destroy_shard(tp_shard *s)
{
    if (!s)
        return;
    for (auto &p : s->ev_pool) {
        hipEventDestroy(p.first);
        hipEventDestroy(p.second);
    }
    delete s;
}

uint64_t tp_wire_scales_offset(const tp_config *cfg, int32_t batch)
{
    if (!cfg || batch < 0)
        return 0;
    const uint64_t row = cfg->kind == TP_LOGITS ? (cfg->tp_size > 0 ? cfg->ffn_hidden / cfg->tp_size : 0)
                                                : (uint64_t)cfg->dim;
    return align_up((uint64_t)batch * row, 16);
}

// TP_LOGITS: the classifier rows [r*V/T, (r+1)*V/T) are one contiguous block
// of W_cls (copied, or cut into int8 blocks of 32 along k) and the final gain.
static int32_t load_logits(tp_shard *s, const tp_layer_weights *w, void *packed, void *workspace,
                           hipStream_t st)
{
    if (!w->w1 || !w->g_att)
        return fail(TP_EINVAL, "load_weights: null classifier or final gain");
    const void *ptrs[] = {packed, workspace, w->w1, w->g_att};
    for (const void *p : ptrs)
        if (!aligned16(p))
            return fail(TP_EALIGN, "load_weights: device buffer not 16-byte aligned");
    const int32_t dv = check_device();
    if (dv != TP_OK)
        return dv;
    char *P = (char *)packed;
    const size_t D = s->D, Vs = s->Fs, e = s->esz;
    const char *src = (const char *)w->w1 + (size_t)s->r * Vs * D * e;
    hipError_t err;
    if (s->w8) {
        const QuantRowsArgs qa{src, s->cfg.w_dtype == TP_BF16, D, (int)Vs, (int)D, (int8_t *)(P + s->o_w13),
                               D, (float *)(P + s->o_sw13), D / kQBlock};
        err = launch_quant_rows(qa, st);
    } else {
        err = hipMemcpyAsync(P + s->o_w13, src, Vs * D * e, hipMemcpyDeviceToDevice, st);
    }
    if (!err)
        err = hipMemcpyAsync(P + s->o_gatt, w->g_att, D * 4, hipMemcpyDeviceToDevice, st);
    if (!err)
        err = launch_clear_u32((unsigned *)((char *)workspace + s->w_err), 1, st);
    if (err)
        return hip_fail(err, "load_weights: classifier packing");
    s->packed = P;
    s->ws = (char *)workspace;
    s->kc = s->vc = nullptr;
    s->loaded = true;
    return TP_OK;
}

// TP_ATTN_BATCH: no weights; the RoPE table, the error word and the caches.
static int32_t load_attn_batch(tp_shard *s, void *packed, void *k_cache, void *v_cache,
                               void *workspace, hipStream_t st)
{
    if (!k_cache || !v_cache)
        return fail(TP_EINVAL, "load_weights: null cache pointer");
    const void *ptrs[] = {packed, workspace, k_cache, v_cache};
    for (const void *p : ptrs)
        if (!aligned16(p))
            return fail(TP_EALIGN, "load_weights: device buffer not 16-byte aligned");
    const int32_t dv = check_device();
    if (dv != TP_OK)
        return dv;
    char *P = (char *)packed;
    RopeArgs ra{(float2 *)(P + s->o_rope), s->cfg.max_ctx, s->hd, (double)s->cfg.rope_theta};
    int32_t rc = timed(s, KID_ROPE_TABLE, st, "rope table", [&] { return launch_rope_table(ra, st); });
    if (rc)
        return rc;
    const hipError_t ce = launch_clear_u32((unsigned *)((char *)workspace + s->w_err), 1, st);
    if (ce)
        return hip_fail(ce, "load_weights: clear error word");
    s->packed = P;
    s->ws = (char *)workspace;
    s->kc = k_cache;
    s->vc = v_cache;
    s->loaded = true;
    return TP_OK;
}

int32_t load_weights(tp_shard *s, const tp_layer_weights *w, void *packed, void *k_cache,
                     void *v_cache, void *workspace, void *hip_stream)
{
    const bool llama = s && s->cfg.kind == TP_LLAMA_BLOCK;
    // a Llama block may be loaded without a workspace: its stages then run only
    // through decode_step_noalloc, on the library's static scratch
    if (!s || !w || !packed || (!workspace && !llama))
        return fail(TP_EINVAL, "load_weights: null argument");
    if (s->cfg.kind == TP_LOGITS)
        return load_logits(s, w, packed, workspace, (hipStream_t)hip_stream);
    if (s->cfg.kind == TP_ATTN_BATCH)
        return load_attn_batch(s, packed, k_cache, v_cache, workspace, (hipStream_t)hip_stream);
    if (!w->w1 || !w->w3 || !w->w2 ||
        (llama && (!w->wq || !w->wk || !w->wv || !w->wo || !w->g_att || !w->g_ffn || !k_cache ||
                   !v_cache)))
        return fail(TP_EINVAL, "load_weights: null weight or cache pointer");
    const void *ptrs[] = {packed, workspace, w->w1, w->w3, w->w2};
    for (const void *p : ptrs)
        if (!aligned16(p))
            return fail(TP_EALIGN, "load_weights: device buffer not 16-byte aligned");
    if (llama) {
        const void *lp[] = {w->wq, w->wk, w->wv, w->wo, w->g_att, w->g_ffn, k_cache, v_cache};
        for (const void *p : lp)
            if (!aligned16(p))
                return fail(TP_EALIGN, "load_weights: device buffer not 16-byte aligned");
    }
    const int32_t dv = check_device();
    if (dv != TP_OK)
        return dv;
    hipStream_t st = (hipStream_t)hip_stream;
    char *P = (char *)packed;
    const size_t e = s->esz, D = s->D;
    hipError_t err = hipSuccess;
    if (llama && s->w8) {
        // int8 weights: the same slices and interleave as below, each row cut
        // into blocks of 32 along k and quantised (codes and scales packed
        // separately, [N][K] and [N][K/32]); the shard's column slices start at
        // multiples of 32, so the blocks are those of the unsharded rows
        const size_t hd = s->hd, nb = D / kQBlock, wo_cols = (size_t)s->Hq_s * hd;
        const int bf = s->cfg.w_dtype == TP_BF16;
        auto quant = [&](const void *src, size_t src_pitch, size_t rows, size_t cols, uint64_t code_off,
                         size_t code_pitch, uint64_t scale_off, size_t scale_pitch) {
            const QuantRowsArgs qa{src, bf, src_pitch, (int)rows, (int)cols, (int8_t *)(P + code_off),
                                   code_pitch, (float *)(P + scale_off), scale_pitch};
            return launch_quant_rows(qa, st);
        };
        const size_t nq = (size_t)s->Hq_s * hd, nk = (size_t)s->Hkv_s * hd;
        err = quant((const char *)w->wq + s->r * nq * D * e, D, nq, D, s->o_wqkv, D, s->o_sqkv, nb);
        if (!err)
            err = quant((const char *)w->wk + s->r * nk * D * e, D, nk, D, s->o_wqkv + nq * D, D,
                        s->o_sqkv + nq * nb * 4, nb);
        if (!err)
            err = quant((const char *)w->wv + s->r * nk * D * e, D, nk, D, s->o_wqkv + (nq + nk) * D, D,
                        s->o_sqkv + (nq + nk) * nb * 4, nb);
        if (!err) // W_O: columns [r*Hq_s*hd, (r+1)*Hq_s*hd) of every row
            err = quant((const char *)w->wo + s->r * wo_cols * e, (size_t)s->Hq * hd, D, wo_cols, s->o_wo,
                        wo_cols, s->o_swo, wo_cols / kQBlock);
        if (!err) // W1_f and W3_f rows interleaved
            err = quant((const char *)w->w1 + (size_t)s->r * s->Fs * D * e, D, s->Fs, D, s->o_w13, 2 * D,
                        s->o_sw13, 2 * nb);
        if (!err)
            err = quant((const char *)w->w3 + (size_t)s->r * s->Fs * D * e, D, s->Fs, D, s->o_w13 + D,
                        2 * D, s->o_sw13 + nb * 4, 2 * nb);
        if (!err) // W2: columns [r*Fs, (r+1)*Fs)
            err = quant((const char *)w->w2 + (size_t)s->r * s->Fs * e, (size_t)s->F, D, s->Fs, s->o_w2,
                        s->Fs, s->o_sw2, s->Fs / kQBlock);
        if (!err)
            err = hipMemcpyAsync(P + s->o_gatt, w->g_att, D * 4, hipMemcpyDeviceToDevice, st);
        if (!err)
            err = hipMemcpyAsync(P + s->o_gffn, w->g_ffn, D * 4, hipMemcpyDeviceToDevice, st);
        if (err)
            return hip_fail(err, "load_weights: int8 packing");
        RopeArgs ra{(float2 *)(P + s->o_rope), s->cfg.max_ctx, s->hd, (double)s->cfg.rope_theta};
        const int32_t rc =
            timed(s, KID_ROPE_TABLE, st, "rope table", [&] { return launch_rope_table(ra, st); });
        if (rc)
            return rc;
    } else if (llama) {
        const size_t hd = s->hd;
        // column split: rows of the shard's q heads, kv heads (contiguous blocks)
        err = hipMemcpyAsync(P + s->o_wqkv, (const char *)w->wq + (size_t)s->r * s->Hq_s * hd * D * e,
                             (size_t)s->Hq_s * hd * D * e, hipMemcpyDeviceToDevice, st);
        if (!err)
            err = hipMemcpyAsync(P + s->o_wqkv + (size_t)s->Hq_s * hd * D * e,
                                 (const char *)w->wk + (size_t)s->r * s->Hkv_s * hd * D * e,
                                 (size_t)s->Hkv_s * hd * D * e, hipMemcpyDeviceToDevice, st);
        if (!err)
            err = hipMemcpyAsync(P + s->o_wqkv + (size_t)(s->Hq_s + s->Hkv_s) * hd * D * e,
                                 (const char *)w->wv + (size_t)s->r * s->Hkv_s * hd * D * e,
                                 (size_t)s->Hkv_s * hd * D * e, hipMemcpyDeviceToDevice, st);
        // row split of W_O: columns [r*Hq_s*hd, (r+1)*Hq_s*hd) of every row
        const size_t wo_cols = (size_t)s->Hq_s * hd;
        if (!err)
            err = copy2d(P + s->o_wo, wo_cols * e, (const char *)w->wo + s->r * wo_cols * e,
                         (size_t)s->Hq * hd * e, wo_cols * e, D, st);
        // up-projection: rows W1_f and W3_f interleaved (f in the shard's slice)
        if (!err)
            err = copy2d(P + s->o_w13, 2 * D * e, (const char *)w->w1 + (size_t)s->r * s->Fs * D * e,
                         D * e, D * e, s->Fs, st);
        if (!err)
            err = copy2d(P + s->o_w13 + D * e, 2 * D * e,
                         (const char *)w->w3 + (size_t)s->r * s->Fs * D * e, D * e, D * e, s->Fs,
                         st);
        // row split of W2: columns [r*Fs, (r+1)*Fs)
        if (!err)
            err = copy2d(P + s->o_w2, (size_t)s->Fs * e, (const char *)w->w2 + (size_t)s->r * s->Fs * e,
                         (size_t)s->F * e, (size_t)s->Fs * e, D, st);
        if (!err)
            err = hipMemcpyAsync(P + s->o_gatt, w->g_att, D * 4, hipMemcpyDeviceToDevice, st);
        if (!err)
            err = hipMemcpyAsync(P + s->o_gffn, w->g_ffn, D * 4, hipMemcpyDeviceToDevice, st);
        if (err)
            return hip_fail(err, "load_weights: packing copy");
        RopeArgs ra{(float2 *)(P + s->o_rope), s->cfg.max_ctx, s->hd, (double)s->cfg.rope_theta};
        const int32_t rc =
            timed(s, KID_ROPE_TABLE, st, "rope table", [&] { return launch_rope_table(ra, st); });
        if (rc)
            return rc;
    } else {
        // 2D FFN block: gate rows and up rows interleaved in groups of 8
        // ([F/8][2][8][E]), so every 16-row MFMA tile holds 8 features' gate
        // and up rows
        const size_t E = s->D, F = s->F;
        err = copy2d(P + s->o_w13, 16 * E * e, w->w1, 8 * E * e, 8 * E * e, F / 8, st);
        if (!err)
            err = copy2d(P + s->o_w13 + 8 * E * e, 16 * E * e, w->w3, 8 * E * e, 8 * E * e, F / 8,
                         st);
        if (!err)
            err = hipMemcpyAsync(P + s->o_w2, w->w2, E * F * e, hipMemcpyDeviceToDevice, st);
        if (err)
            return hip_fail(err, "load_weights: packing copy");
    }
    s->packed = P;
    s->ws = (char *)workspace;
    s->kc = k_cache;
    s->vc = v_cache;
    if (llama) { // set-up of decode_step_noalloc: this device's scratch address, once per device
        void *sp = nullptr;
        const hipError_t se = scratch_address(&sp);
        if (se)
            return hip_fail(se, "load_weights: scratch address");
    }
    if (s->ws) {
        hipError_t ce = launch_clear_u32((unsigned *)(s->ws + s->w_err), 1, st);
        if (!ce && s->w_hand) // epoch 0 and no word carrying a tag
            ce = launch_clear_u32((unsigned *)(s->ws + s->w_hand), (int)(s->hand_bytes / 4), st);
        if (ce)
            return hip_fail(ce, "load_weights: clear error word");
    }
    s->loaded = true;
    return TP_OK;
}

// The final stage of shard r (distributed-llama issue, buildLlama2Arch:
// llamaRmsFinal + llamaRmsFinalNorm, llamaLogits, llamaQuantizeLogits): the
// final RMSNorm of x and the shard's V/T classifier rows times it, with the
// projection kernels and norm placement of the block's up-projections (norm
// fused into the GEMV prologue below batch 5, folded into a split-K MFMA GEMV
// where that applies, else a kernel of its own), then the int8 wire.
static int32_t logits_step(tp_shard *s, const float *x, int B, void *wire_out, const tp_taps &tp,
                           hipStream_t st)
{
    const int wt = s->w8 ? WT_I8 : s->cfg.w_dtype == TP_BF16 ? WT_BF16 : WT_F32;
    const bool qpart = s->cfg.quant & TP_Q_PARTIALS;
    const float *gain = (const float *)(s->packed + s->o_gatt);
    float *p = qpart ? (float *)(s->ws + s->w_p) : (float *)wire_out;
    const bool mfma = s->mfma_ok && B > 4;
    const bool sk_norm = mfma && s->w_skp && gemv_sk_used(s->Fs, s->D);
    const bool fuse_norm = !mfma && gemv_fused_ok(B, s->D);
    uint16_t *xfx = mfma ? (uint16_t *)(s->ws + s->w_xfx) : nullptr;
    GemvArgs g{};
    g.W = s->packed + s->o_w13;
    g.ws = s->w8 ? (const float *)(s->packed + s->o_sw13) : nullptr;
    g.x = x;
    g.ldx = s->D;
    g.K = s->D;
    g.B = B;
    g.y = p;
    g.tap = tp.p_pre;
    g.N = s->Fs;
    g.ldy = s->Fs;
    int32_t rc;
    if (fuse_norm) {
        g.g = gain;
        g.eps = s->cfg.norm_eps;
        g.xn_tap = tp.xn;
        g.xq_tap = tp.xq;
    } else if (!sk_norm || tp.xn || tp.xq) {
        float *xn = (float *)(s->ws + s->w_xn);
        NormArgs na{x, gain, xn, tp.xn, xfx, B, s->D, s->cfg.norm_eps, 0, tp.xq};
        rc = timed(s, KID_RMSNORM, st, "rmsnorm", [&] { return launch_rmsnorm(na, st); });
        if (rc)
            return rc;
        g.x = xn;
    }
    rc = timed(s, KID_GEMV_LOGITS, st, "gemv logits", [&] {
        if (!mfma)
            return launch_gemv(g, wt, EPI_STORE, st);
        MfmaGemvArgs m{(const uint16_t *)g.W, xfx, g.y, g.tap, nullptr, g.N, g.K, g.B, g.ldy, 1, g.mo,
                       s->w_skp ? (float *)(s->ws + s->w_skp) : nullptr, 0, 0,
                       sk_norm ? x : nullptr, sk_norm ? gain : nullptr, s->cfg.norm_eps, g.ws};
        return launch_gemv_mfma(m, EPI_STORE, st);
    });
    if (rc || !qpart)
        return rc;
    WireArgs wa{p, (int8_t *)wire_out,
                (float *)((char *)wire_out + tp_wire_scales_offset(&s->cfg, B)), B, s->Fs, {}};
    return timed(s, KID_WIRE, st, "q8 wire", [&] { return launch_wire(wa, st); });
}

// Batch-sharded attention of the shard's sequences (CS349E lecture 4, demo 3
// observations): the attention kernels of the head-sharded stage run over
// every head of nb sequences; x holds their raw q / k / v rows.
static int32_t attn_batch_step(tp_shard *s, const float *x, const int32_t *lens, int B, float *out,
                               const tp_taps &tp, hipStream_t st)
{
    if (!lens)
        return fail(TP_EINVAL, "decode_step: attention stage needs lens");
    AttnArgs aa{};
    aa.qkv = x;
    aa.lens = lens;
    aa.kc = s->kc;
    aa.vc = s->vc;
    aa.rope = (const float2 *)(s->packed + s->o_rope);
    aa.part = (float *)(s->ws + s->w_part);
    aa.err = (unsigned *)(s->ws + s->w_err);
    aa.att = out;
    aa.tap_q = tp.q;
    aa.tap_k = tp.k;
    aa.tap_v = tp.v;
    aa.tap_att = tp.att;
    aa.att_xf = nullptr;
    aa.ld_qkv = s->n_qkv;
    aa.max_ctx = s->cfg.max_ctx;
    aa.Hq_s = s->Hq;
    aa.Hkv_s = s->Hkv;
    aa.G = s->G;
    aa.hd = s->hd;
    aa.n_chunks = s->n_chunks;
    aa.scale = (float)(1.0 / std::sqrt((double)s->hd));
    return timed(s, KID_ATTN, st, "attention",
                 [&] { return launch_attn(aa, s->cfg.kv_dtype == TP_BF16, B, st); });
}

// One stage of the shard step on input x. With mo (llama blocks only) the
// stage's partials are also merged, mo->x_out = x + sum of mo's wires, by the
// kernel that writes this shard's own partial (wire mo->own = wire_out).
static int32_t step_impl(tp_shard *s, int32_t stage, const void *x, const MergeIn *mo,
                         const int32_t *lens, int32_t batch, void *wire_out, const tp_taps *taps,
                         void *hip_stream, char *ws = nullptr, unsigned *err_word = nullptr)
{
    if (!s)
        return fail(TP_EINVAL, "decode_step: null handle");
    if (!s->loaded)
        return fail(TP_ESTATE, "decode_step before load_weights");
    // the workspace: the handle's, or (decode_step_noalloc) the static scratch
    if (!ws)
        ws = s->ws;
    if (!ws)
        return fail(TP_ESTATE, "no workspace was bound at load_weights: use decode_step_noalloc");
    if (!err_word)
        err_word = (unsigned *)(ws + s->w_err);
    if (stage != TP_STAGE_ATTN && stage != TP_STAGE_FFN && stage != TP_STAGE_LOGITS)
        return fail(TP_EINVAL, "unknown stage %d", stage);
    if ((stage == TP_STAGE_LOGITS) != (s->cfg.kind == TP_LOGITS))
        return fail(TP_EINVAL, "TP_STAGE_LOGITS goes with (and only with) a TP_LOGITS handle");
    if (s->cfg.kind == TP_ATTN_BATCH && stage != TP_STAGE_ATTN)
        return fail(TP_EINVAL, "TP_ATTN_BATCH has only the attention stage");
    const int max_rows = s->cfg.kind == TP_ATTN_BATCH ? s->nb : s->cfg.max_batch;
    if (batch < 1 || batch > max_rows)
        return fail(TP_EINVAL, "batch %d outside [1, %d]", batch, max_rows);
    if (mo && s->cfg.kind != TP_LLAMA_BLOCK)
        return fail(TP_EINVAL, "decode_merge_step applies to TP_LLAMA_BLOCK shards");
    if (!x || !wire_out)
        return fail(TP_EINVAL, "decode_step: null x or wire_out");
    if (!aligned16(x) || !aligned16(wire_out))
        return fail(TP_EALIGN, "decode_step: x / wire_out not 16-byte aligned");
    const tp_taps nt{};
    const tp_taps &tp = taps ? *taps : nt;
    const float *tp_ptrs[] = {tp.xn, tp.q, tp.k, tp.v, tp.att, tp.a, tp.p_pre, tp.xq};
    for (const float *p : tp_ptrs)
        if (p && !aligned16(p))
            return fail(TP_EALIGN, "decode_step: tap not 16-byte aligned");
    if ((tp.k == nullptr) != (tp.v == nullptr))
        return fail(TP_EINVAL, "decode_step: taps k and v go together");
    hipStream_t st = (hipStream_t)hip_stream;
    const int B = batch;

    if (s->cfg.kind == TP_FFN_2D) {
        if (stage != TP_STAGE_FFN)
            return fail(TP_EINVAL, "TP_FFN_2D has only the FFN stage");
        const int S = ffn2d_splits(B, s->D, s->F);
        if (S > 1 && (uint64_t)S * B > s->part_rows) // cannot happen with plan()'s sizing
            return fail(TP_EINVAL, "split-K partials of batch %d exceed the workspace", B);
        Ffn2dArgs fa{(const uint16_t *)x,
                     (const uint16_t *)(s->packed + s->o_w13),
                     (const uint16_t *)(s->packed + s->o_w2),
                     (uint16_t *)(ws + s->w_a),
                     (float *)(ws + s->w_p),
                     (float *)wire_out,
                     B,
                     s->D,
                     s->F};
        int32_t rc = timed(s, KID_FFN2D_UP, st, "ffn2d up", [&] { return launch_ffn2d(fa, st, 0); });
        if (rc)
            return rc;
        return timed(s, KID_FFN2D_DOWN, st, "ffn2d down", [&] { return launch_ffn2d(fa, st, 1); });
    }

    if (s->cfg.kind == TP_LOGITS)
        return logits_step(s, (const float *)x, batch, wire_out, tp, st);
    if (s->cfg.kind == TP_ATTN_BATCH)
        return attn_batch_step(s, (const float *)x, lens, batch, (float *)wire_out, tp, st);

    const bool wbf = s->cfg.w_dtype == TP_BF16;
    const int wt = s->w8 ? WT_I8 : wbf ? WT_BF16 : WT_F32;
    const char *Pk = s->packed;
    auto wscales = [&](uint64_t off) { return s->w8 ? (const float *)(Pk + off) : nullptr; };
    const bool qin = s->cfg.quant & TP_Q_INPUTS, qpart = s->cfg.quant & TP_Q_PARTIALS;
    const float *gain = (const float *)(s->packed + (stage == TP_STAGE_ATTN ? s->o_gatt : s->o_gffn));
    // the partial goes straight into the wire unless it is quantised
    float *p = qpart ? (float *)(ws + s->w_p) : (float *)wire_out;
    int8_t *codes = qpart ? (int8_t *)wire_out : nullptr;
    float *scales = qpart ? (float *)((char *)wire_out + tp_wire_scales_offset(&s->cfg, B)) : nullptr;
    int32_t rc;

    // batch 5..16: MFMA projections. A split-K up-projection folds the
    // RMSNorm in (fragments of x g built per K slice, each row scaled by its
    // 1 / rms in the epilogue); otherwise a RMSNorm kernel writes xn and its
    // fragments. The int8 round trip of quantised inputs needs the kernel.
    const bool mfma = s->mfma_ok && B > 4;
    const int up_n = stage == TP_STAGE_ATTN ? s->n_qkv : 2 * s->Fs;
    const bool sk_norm = mfma && !qin && s->w_skp && gemv_sk_used(up_n, s->D);
    // RMSNorm below batch 5: fused into the projection's prologue when the
    // batch's rows fit in LDS, else a kernel of its own writing xn
    const bool fuse_norm = !mfma && gemv_fused_ok(B, s->D);
    const float *in = (const float *)x;
    uint16_t *xfx = mfma ? (uint16_t *)(ws + s->w_xfx) : nullptr;
    uint16_t *xfatt = mfma ? (uint16_t *)(ws + s->w_xfatt) : nullptr;
    uint16_t *xfa = mfma ? (uint16_t *)(ws + s->w_xfa) : nullptr;
    GemvArgs up{};
    up.x = in;
    up.ldx = s->D;
    up.K = s->D;
    up.B = B;
    if (fuse_norm) {
        up.g = gain;
        up.eps = s->cfg.norm_eps;
        up.qin = qin ? 1 : 0;
        up.xn_tap = tp.xn;
        up.xq_tap = tp.xq;
    } else if (!sk_norm || tp.xn || tp.xq) { // with sk_norm only for the xn / xq taps
        float *xn = (float *)(ws + s->w_xn);
        NormArgs na{in, gain, xn, tp.xn, xfx, B, s->D, s->cfg.norm_eps, qin ? 1 : 0, tp.xq};
        rc = timed(s, KID_RMSNORM, st, "rmsnorm", [&] { return launch_rmsnorm(na, st); });
        if (rc)
            return rc;
        up.x = xn;
    }
    // row-split projection; its fp32 partial is quantised into the wire after it
    GemvArgs down{};
    down.y = p;
    down.tap = tp.p_pre;
    down.N = s->D;
    down.ldy = s->D;
    down.B = B;
    const int Kd = stage == TP_STAGE_ATTN ? s->Hq_s * s->hd : s->Fs;
    // int8 wire below batch 5: the down-projection's epilogue quantises its
    // partial into the wire (and merges the int8 wires), no k_wire launch
    const bool wire_epi = qpart && !mfma && gemv_fused_ok(B, Kd);
    if (mo && (!qpart || wire_epi)) // the down-projection's epilogue merges
        down.mo = *mo;
    if (wire_epi) {
        down.codes = codes;
        down.scales = scales;
    }
    const int down_epi = wire_epi ? EPI_Q8 : EPI_STORE;
    auto run_gemv = [&](const GemvArgs &g, const uint16_t *xf, uint16_t *yf, int epi, bool norm) {
        if (!mfma)
            return launch_gemv(g, wt, epi, st);
        MfmaGemvArgs m{(const uint16_t *)g.W, xf, g.y, g.tap, yf, g.N, g.K, g.B, g.ldy, 1, g.mo,
                       s->w_skp ? (float *)(ws + s->w_skp) : nullptr, 0, 0,
                       norm ? in : nullptr, norm ? gain : nullptr, s->cfg.norm_eps, g.ws};
        return launch_gemv_mfma(m, epi, st);
    };

    if (stage == TP_STAGE_ATTN) {
        if (!lens)
            return fail(TP_EINVAL, "decode_step: attention stage needs lens");
        float *qkv = (float *)(ws + s->w_qkv);
        up.W = s->packed + s->o_wqkv;
        up.ws = wscales(s->o_sqkv);
        up.y = qkv;
        up.N = s->n_qkv;
        up.ldy = s->n_qkv;
        // batch <= 4 on the handle's own workspace (the hand-off words and
        // the epoch live there): the projection and the chunk attention in
        // one launch
        const bool fused_qa = s->w_hand && ws == s->ws && fuse_norm &&
                              qkv_attn_fusable(wt, B, s->D, s->n_qkv, s->G, s->hd, s->cfg.kv_dtype == TP_BF16);
        if (!fused_qa) {
            rc = timed(s, KID_GEMV_QKV, st, "gemv qkv",
                       [&] { return run_gemv(up, xfx, nullptr, EPI_STORE, sk_norm); });
            if (rc)
                return rc;
        }
        float *att = (float *)(ws + s->w_att);
        AttnArgs aa{};
        aa.qkv = qkv;
        aa.lens = lens;
        aa.kc = s->kc;
        aa.vc = s->vc;
        aa.rope = (const float2 *)(s->packed + s->o_rope);
        aa.part = (float *)(ws + s->w_part);
        aa.err = err_word;
        aa.att = att;
        aa.tap_q = tp.q;
        aa.tap_k = tp.k;
        aa.tap_v = tp.v;
        aa.tap_att = tp.att;
        aa.att_xf = xfatt;
        aa.ld_qkv = s->n_qkv;
        aa.max_ctx = s->cfg.max_ctx;
        aa.Hq_s = s->Hq_s;
        aa.Hkv_s = s->Hkv_s;
        aa.G = s->G;
        aa.hd = s->hd;
        aa.n_chunks = s->n_chunks;
        aa.scale = (float)(1.0 / std::sqrt((double)s->hd));
        aa.hand_wait_ticks = s->hand_wait_ticks;
        aa.hand_tag_xor = s->hand_tag_xor;
        if (fused_qa) {
            char *hb = ws + s->w_hand;
            if (s->hand_dirty) { // epoch 0 and no word carrying a tag again
                const hipError_t ce = launch_clear_u32((unsigned *)hb, (int)(s->hand_bytes / 4), st);
                if (ce)
                    return hip_fail(ce, "decode_step: clear hand-off words");
                s->hand_dirty = false;
            }
            rc = timed(s, KID_QKV_ATTN, st, "qkv + attention", [&] {
                return launch_qkv_attn(up, aa, (uint64_t *)(hb + 256), (uint64_t *)(hb + s->hand_rec),
                                       (const uint32_t *)hb, wt, B, st);
            });
            down.epoch = (uint32_t *)hb; // W_O advances the epoch for the next launch
            s->hand_dirty = rc != TP_OK;
        } else {
            rc = timed(s, KID_ATTN, st, "attention",
                       [&] { return launch_attn(aa, s->cfg.kv_dtype == TP_BF16, B, st); });
        }
        if (rc)
            return rc;
        down.W = s->packed + s->o_wo;
        down.ws = wscales(s->o_swo);
        down.x = att;
        down.K = Kd;
        down.ldx = Kd;
        rc = timed(s, KID_GEMV_WO, st, "gemv wo", [&] { return run_gemv(down, xfatt, nullptr, down_epi, false); });
        if (rc) {
            if (down.epoch)
                s->hand_dirty = true;
            return rc;
        }
    } else {
        float *a = (float *)(ws + s->w_a);
        up.W = s->packed + s->o_w13;
        up.ws = wscales(s->o_sw13);
        up.y = a;
        up.tap = tp.a;
        up.N = 2 * s->Fs;
        up.ldy = s->Fs;
        rc = timed(s, KID_GEMV_W13, st, "gemv w13", [&] { return run_gemv(up, xfx, xfa, EPI_SWIGLU, sk_norm); });
        if (rc)
            return rc;
        down.W = s->packed + s->o_w2;
        down.ws = wscales(s->o_sw2);
        down.x = a;
        down.K = Kd;
        down.ldx = Kd;
        rc = timed(s, KID_GEMV_W2, st, "gemv w2", [&] { return run_gemv(down, xfa, nullptr, down_epi, false); });
        if (rc)
            return rc;
    }

    if (qpart && !wire_epi) {
        WireArgs wa{p, codes, scales, B, s->D, {}};
        if (mo) // int8 wires: the quantiser merges
            wa.mo = *mo;
        return timed(s, KID_WIRE, st, "q8 wire", [&] { return launch_wire(wa, st); });
    }
    return TP_OK;
}

int32_t decode_step(tp_shard *s, int32_t stage, const void *x, const int32_t *lens,
                    int32_t batch, void *wire_out, const tp_taps *taps, void *hip_stream)
{
    return step_impl(s, stage, x, nullptr, lens, batch, wire_out, taps, hip_stream);
}

// decode_step on the static scratch (scratch.hip) instead of the handle's
// workspace: the same kernels and arguments, the workspace regions at the
// same offsets inside the scratch. Allocates nothing: the scratch address was
// looked up when the handle was loaded; the kernel-timing probe is bypassed
// (it would create events). No region of the workspace carries anything from
// one call to the next (every kernel writes what a later one reads), and
// device errors go to the caller's err_out (or to an unread word of the
// scratch), so nothing in the scratch needs clearing.
int32_t decode_step_noalloc(tp_shard *s, int32_t stage, const void *x, const int32_t *lens,
                            int32_t batch, void *wire_out, const tp_taps *taps, uint32_t *err_out,
                            void *hip_stream)
{
    if (!s)
        return fail(TP_EINVAL, "decode_step_noalloc: null handle");
    if (s->cfg.kind != TP_LLAMA_BLOCK)
        return fail(TP_EINVAL, "decode_step_noalloc applies to TP_LLAMA_BLOCK shards");
    if (!s->loaded)
        return fail(TP_ESTATE, "decode_step_noalloc before load_weights");
    // (the hand-off region, last in the workspace, is not used here)
    const uint64_t need = s->w_hand ? s->w_hand : s->ws_bytes;
    if (need > kScratchBytes)
        return fail(TP_EINVAL,
                    "decode_step_noalloc: this shard needs %llu bytes of workspace, the static "
                    "scratch holds %llu (use decode_step with a workspace)",
                    (unsigned long long)need, (unsigned long long)kScratchBytes);
    if (err_out && ((uintptr_t)err_out & 3u))
        return fail(TP_EALIGN, "decode_step_noalloc: err_out not 4-byte aligned");
    void *sp = nullptr;
    const hipError_t se = scratch_address(&sp);
    if (se)
        return hip_fail(se, "decode_step_noalloc: scratch address");
    const int armed = s->timing_kernel;
    s->timing_kernel = -1;
    const int32_t rc = step_impl(s, stage, x, nullptr, lens, batch, wire_out, taps, hip_stream,
                                 (char *)sp, (unsigned *)err_out);
    s->timing_kernel = armed;
    return rc;
}

// Validates a merge request and fills mi (x_out = residual + sum of the wires).
static int32_t merge_request(const tp_shard *s, int32_t stage, const void *const *wires,
                             int32_t n_wires, const float *residual, float *x_out, int32_t batch,
                             const char *fn, MergeIn &mi)
{
    if (!s)
        return fail(TP_EINVAL, "%s: null handle", fn);
    if (s->cfg.kind != TP_LLAMA_BLOCK)
        return fail(TP_EINVAL, "%s applies to TP_LLAMA_BLOCK shards", fn);
    if (stage != TP_STAGE_ATTN && stage != TP_STAGE_FFN)
        return fail(TP_EINVAL, "unknown stage %d", stage);
    if (!wires || n_wires < 1 || n_wires > kMaxWires)
        return fail(TP_EINVAL, "%s: n_wires %d outside [1, %d]", fn, n_wires, kMaxWires);
    if (batch < 1 || batch > s->cfg.max_batch)
        return fail(TP_EINVAL, "batch %d outside [1, max_batch=%d]", batch, s->cfg.max_batch);
    if (!residual || !x_out)
        return fail(TP_EINVAL, "%s: null residual / out", fn);
    if (!aligned16(residual) || !aligned16(x_out))
        return fail(TP_EALIGN, "%s: residual / out not 16-byte aligned", fn);
    mi = MergeIn{};
    for (int i = 0; i < n_wires; i++) {
        if (!wires[i])
            return fail(TP_EINVAL, "%s: wire %d is null", fn, i);
        if (!aligned16(wires[i]))
            return fail(TP_EALIGN, "%s: wire %d not 16-byte aligned", fn, i);
        mi.wires[i] = wires[i];
    }
    mi.residual = residual;
    mi.x_out = x_out;
    mi.n_wires = n_wires;
    mi.quant = (s->cfg.quant & TP_Q_PARTIALS) ? 1 : 0;
    mi.own = -1;
    mi.scales_off = tp_wire_scales_offset(&s->cfg, batch);
    return TP_OK;
}

int32_t decode_merge_step(tp_shard *s, int32_t stage, const void *x, const int32_t *lens,
                          int32_t batch, void *wire_out, const void *const *wires,
                          int32_t n_wires, float *x_out, const tp_taps *taps, void *hip_stream)
{
    MergeIn mo;
    const int32_t rc = merge_request(s, stage, wires, n_wires, (const float *)x, x_out, batch,
                                     "decode_merge_step", mo);
    if (rc)
        return rc;
    mo.own = -1;
    for (int i = 0; i < n_wires; i++) {
        if (wires[i] == wire_out) {
            if (mo.own >= 0)
                return fail(TP_EINVAL, "decode_merge_step: wire_out appears twice in wires");
            mo.own = i;
        }
        // the kernel that writes x_out still reads the other wires
        if ((const void *)x_out == wires[i])
            return fail(TP_EINVAL, "decode_merge_step: x_out aliases wire %d", i);
    }
    if (mo.own < 0)
        return fail(TP_EINVAL, "decode_merge_step: wire_out is not one of the wires");
    return step_impl(s, stage, x, &mo, lens, batch, wire_out, taps, hip_stream);
}

int32_t merge_partials(const tp_shard *s, int32_t stage, const void *const *wires,
                       int32_t n_wires, const float *residual, float *out, int32_t batch,
                       void *hip_stream)
{
    MergeArgs m{};
    const int32_t rc = merge_request(s, stage, wires, n_wires, residual, out, batch,
                                     "merge_partials", m.m);
    if (rc)
        return rc;
    m.B = batch;
    m.D = s->D;
    hipStream_t st = (hipStream_t)hip_stream;
    return timed(const_cast<tp_shard *>(s), KID_MERGE, st, "merge",
                 [&] { return launch_merge(m, st); });
}

int32_t merge_logits(const tp_shard *s, const void *const *wires, int32_t n_wires, float *out,
                     int32_t batch, void *hip_stream)
{
    if (!s)
        return fail(TP_EINVAL, "merge_logits: null handle");
    if (s->cfg.kind != TP_LOGITS)
        return fail(TP_EINVAL, "merge_logits applies to TP_LOGITS shards");
    if (!wires || n_wires != s->T)
        return fail(TP_EINVAL, "merge_logits: n_wires %d, the handle has %d shards", n_wires, s->T);
    if (batch < 1 || batch > s->cfg.max_batch)
        return fail(TP_EINVAL, "batch %d outside [1, max_batch=%d]", batch, s->cfg.max_batch);
    if (!out)
        return fail(TP_EINVAL, "merge_logits: null out");
    if (!aligned16(out))
        return fail(TP_EALIGN, "merge_logits: out not 16-byte aligned");
    LogitsMergeArgs a{};
    for (int i = 0; i < n_wires; i++) {
        if (!wires[i])
            return fail(TP_EINVAL, "merge_logits: wire %d is null", i);
        if (!aligned16(wires[i]))
            return fail(TP_EALIGN, "merge_logits: wire %d not 16-byte aligned", i);
        if (wires[i] == (const void *)out)
            return fail(TP_EINVAL, "merge_logits: out aliases wire %d", i);
        a.m.wires[i] = wires[i];
    }
    a.m.n_wires = n_wires;
    a.m.quant = (s->cfg.quant & TP_Q_PARTIALS) ? 1 : 0;
    a.m.own = -1;
    a.m.scales_off = tp_wire_scales_offset(&s->cfg, batch);
    a.out = out;
    a.B = batch;
    a.Vs = s->Fs;
    a.V = s->F;
    hipStream_t st = (hipStream_t)hip_stream;
    return timed(const_cast<tp_shard *>(s), KID_MERGE_LOGITS, st, "merge logits",
                 [&] { return launch_merge_logits(a, n_wires, st); });
}

int32_t tp_all_to_all(const tp_shard *s, int32_t dir, const void *const *srcs, int32_t n_srcs,
                      int64_t ld_src, float *dst, int64_t ld_dst, void *hip_stream)
{
    if (!s)
        return fail(TP_EINVAL, "tp_all_to_all: null handle");
    if (s->cfg.kind != TP_ATTN_BATCH)
        return fail(TP_EINVAL, "tp_all_to_all applies to TP_ATTN_BATCH shards");
    if (dir != TP_A2A_HEADS_TO_BATCH && dir != TP_A2A_BATCH_TO_HEADS)
        return fail(TP_EINVAL, "tp_all_to_all: unknown direction %d", dir);
    if (!srcs || n_srcs != s->T)
        return fail(TP_EINVAL, "tp_all_to_all: n_srcs %d, the handle has %d shards", n_srcs, s->T);
    if (!dst)
        return fail(TP_EINVAL, "tp_all_to_all: null dst");
    const int64_t C = (int64_t)(s->Hq / s->T) * s->hd;
    const int64_t need_src = dir == TP_A2A_HEADS_TO_BATCH ? C : s->T * C;
    const int64_t need_dst = dir == TP_A2A_HEADS_TO_BATCH ? s->T * C : C;
    if (ld_src < need_src || ld_dst < need_dst || ld_src % 4 || ld_dst % 4)
        return fail(TP_EINVAL, "tp_all_to_all: row strides %lld / %lld (need >= %lld / %lld, multiples of 4)",
                    (long long)ld_src, (long long)ld_dst, (long long)need_src, (long long)need_dst);
    if (!aligned16(dst))
        return fail(TP_EALIGN, "tp_all_to_all: dst not 16-byte aligned");
    A2aArgs a{};
    for (int i = 0; i < n_srcs; i++) {
        if (!srcs[i])
            return fail(TP_EINVAL, "tp_all_to_all: source %d is null", i);
        if (!aligned16(srcs[i]))
            return fail(TP_EALIGN, "tp_all_to_all: source %d not 16-byte aligned", i);
        if (srcs[i] == (const void *)dst)
            return fail(TP_EINVAL, "tp_all_to_all: dst aliases source %d", i);
        a.src[i] = (const float *)srcs[i];
    }
    a.dst = dst;
    a.ld_src = ld_src;
    a.ld_dst = ld_dst;
    a.nb = s->nb;
    a.C = (int)C;
    a.r = s->r;
    a.T = s->T;
    a.dir = dir;
    hipStream_t st = (hipStream_t)hip_stream;
    return timed(const_cast<tp_shard *>(s), KID_A2A, st, "all-to-all", [&] { return launch_a2a(a, st); });
}

int32_t tp_packed_int8_view(const tp_shard *s, int32_t proj, uint64_t *codes_off,
                            uint64_t *scales_off, int32_t *rows, int32_t *cols)
{
    if (!s || !codes_off || !scales_off || !rows || !cols)
        return fail(TP_EINVAL, "tp_packed_int8_view: null argument");
    if (!s->w8)
        return fail(TP_EINVAL, "tp_packed_int8_view: the shard has no int8 weights");
    if (s->cfg.kind == TP_LOGITS) {
        if (proj != 0)
            return fail(TP_EINVAL, "tp_packed_int8_view: a TP_LOGITS shard has only projection 0");
        *codes_off = s->o_w13;
        *scales_off = s->o_sw13;
        *rows = s->Fs;
        *cols = s->D;
        return TP_OK;
    }
    switch (proj) {
    case 0: *codes_off = s->o_wqkv; *scales_off = s->o_sqkv; *rows = s->n_qkv; *cols = s->D; break;
    case 1: *codes_off = s->o_wo; *scales_off = s->o_swo; *rows = s->D; *cols = s->Hq_s * s->hd; break;
    case 2: *codes_off = s->o_w13; *scales_off = s->o_sw13; *rows = 2 * s->Fs; *cols = s->D; break;
    case 3: *codes_off = s->o_w2; *scales_off = s->o_sw2; *rows = s->D; *cols = s->Fs; break;
    default: return fail(TP_EINVAL, "tp_packed_int8_view: unknown projection %d", proj);
    }
    return TP_OK;
}

int32_t tp_read_error_word(tp_shard *s, uint32_t *word, int32_t clear, void *hip_stream)
{
    if (!s || !word)
        return fail(TP_EINVAL, "tp_read_error_word: null argument");
    if (!s->loaded)
        return fail(TP_ESTATE, "tp_read_error_word before load_weights");
    if (!s->ws)
        return fail(TP_ESTATE, "tp_read_error_word: no workspace was bound at load_weights");
    hipStream_t st = (hipStream_t)hip_stream;
    hipError_t e = hipMemcpyAsync(word, s->ws + s->w_err, 4, hipMemcpyDeviceToHost, st);
    if (!e && clear)
        e = launch_clear_u32((unsigned *)(s->ws + s->w_err), 1, st);
    if (!e)
        e = hipStreamSynchronize(st);
    return e ? hip_fail(e, "tp_read_error_word") : TP_OK;
}

int32_t tp_kernel_timing_arm(tp_shard *s, int32_t kernel_id)
{
    if (!s)
        return fail(TP_EINVAL, "tp_kernel_timing_arm: null handle");
    if (kernel_id < -1 || kernel_id >= KID_COUNT)
        return fail(TP_EINVAL, "unknown kernel id %d", kernel_id);
    s->timing_kernel = kernel_id;
    s->ev_used = 0;
    return TP_OK;
}

int32_t tp_kernel_timing_read(tp_shard *s, double *total_ms, int32_t *launches)
{
    if (!s || !total_ms || !launches)
        return fail(TP_EINVAL, "tp_kernel_timing_read: null argument");
    double tot = 0.0;
    for (size_t i = 0; i < s->ev_used; i++) {
        if (hipEventSynchronize(s->ev_pool[i].second) != hipSuccess)
            return fail(TP_EHIP, "hipEventSynchronize failed");
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, s->ev_pool[i].first, s->ev_pool[i].second) != hipSuccess)
            return fail(TP_EHIP, "hipEventElapsedTime failed");
        tot += ms;
    }
    *total_ms = tot;
    *launches = (int32_t)s->ev_used;
    return TP_OK;
}

int32_t tp_handoff_test(tp_shard *s, uint32_t wait_ticks, uint32_t tag_xor)
{
    if (!s)
        return fail(TP_EINVAL, "tp_handoff_test: null handle");
    s->hand_wait_ticks = wait_ticks;
    s->hand_tag_xor = tag_xor;
    return TP_OK;
}

const char *tp_kernel_name(int32_t kernel_id)
{
    return (kernel_id >= 0 && kernel_id < KID_COUNT) ? kKernelNames[kernel_id] : nullptr;
}

int32_t tp_probe_read(const void *buf, uint64_t bytes, uint32_t *out, int32_t blocks, void *hip_stream)
{
    if (!buf || !out || bytes == 0 || blocks < 1 || blocks > (1 << 20))
        return fail(TP_EINVAL, "tp_probe_read: null buffer, no bytes or blocks outside [1, 2^20]");
    if (!aligned16(buf) || !aligned16(out))
        return fail(TP_EALIGN, "tp_probe_read: buffers not 16-byte aligned");
    const int32_t rc = check_device();
    if (rc)
        return rc;
    const hipError_t e = launch_probe_read(buf, bytes, out, blocks, (hipStream_t)hip_stream);
    return e ? hip_fail(e, "tp_probe_read") : TP_OK;
}

int32_t tp_probe_mfma(int32_t blocks, int32_t iters, float *out, void *hip_stream)
{
    if (!out || blocks < 1 || blocks > (1 << 20) || iters < 1)
        return fail(TP_EINVAL, "tp_probe_mfma: null out, blocks outside [1, 2^20] or iters < 1");
    if (!aligned16(out))
        return fail(TP_EALIGN, "tp_probe_mfma: out not 16-byte aligned");
    const int32_t rc = check_device();
    if (rc)
        return rc;
    const hipError_t e = launch_probe_mfma(blocks, iters, out, (hipStream_t)hip_stream);
    return e ? hip_fail(e, "tp_probe_mfma") : TP_OK;
}

const char *tp_status_str(int32_t st)
{
    switch (st) {
    case TP_OK: return "TP_OK";
    case TP_EINVAL: return "TP_EINVAL";
    case TP_EALIGN: return "TP_EALIGN";
    case TP_ESTATE: return "TP_ESTATE";
    case TP_ENODEV: return "TP_ENODEV";
    case TP_EHIP: return "TP_EHIP";
    case TP_ENOTIMPL: return "TP_ENOTIMPL";
    default: return "TP_UNKNOWN";
    }
}

const char *tp_last_error(void) { return g_err.c_str(); }

} // extern "C"
