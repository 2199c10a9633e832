"""The block-32 int8 codec on the GPU, bit for bit, on the hand-worked edge
blocks of tests/golden/q8_blocks.txt (half-away ties, clamping, a negative
maximum, an all-zero block, a single nonzero, a subnormal scale).

Source of the codec: distributed-llama issue "[Feature Suggest] Tensor
Parallellism for Accelerating LLM", buildLlama2Arch (a quantise task before
each sync, a dequantise task before each merge); the arithmetic is the
reading the oracle states (scale = max|x|/127, code = x/scale rounded half
away from zero, clamped to +-127; a zero block has scale 0).

Each path of the library that codes or decodes int8 gets the golden values
exactly as its fp32 input, by construction:
  - the normalised-input round trip (TP_Q_INPUTS): a stage input of +-1 in
    every element with eps = 0 normalises to g * (+-1) exactly, so the gain
    vector carries the golden blocks; the fused projection prologue (batch
    <= 4), the RMSNorm kernel (batch 5 with fp32 weights) and the RMSNorm
    kernel that also writes the MFMA fragments (batch 16, bf16 weights);
  - the wire quantiser (TP_Q_PARTIALS) on a final-stage shard with fp32
    classifier weights: an input of 8 * e_0 with eps = 0 and final gain 1/8
    in element 0 normalises to exactly e_0, so each logit is column 0 of the
    classifier, which carries the golden blocks (batch 1: fused prologue,
    batch 5: RMSNorm kernel + global-activation GEMV);
  - the dequantising merges (merge_partials, the int8-wire merge fused into
    the quantiser, merge_logits) on wires assembled on the host from the
    golden codes and scales.
Expected codes and scales are the file's hand-worked values; expected
dequantised values are float32(code) * scale and expected merges the
float32 sum residual + d_0 + d_1 + ... in wire order, computed here in numpy.
"""
import sys

import numpy as np
import pytest

import tensor_tp_shard_amd as tp
from conftest import golden_q8_blocks
from gpu_harness import dev_tensor, to_np

pytestmark = pytest.mark.gpu

F32 = np.float32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    tp.lib()


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def golden_rows(order, signs):
    """Rows of golden blocks: row i holds the blocks `order` (an index into
    the file's blocks, negative = that block negated), times signs[i].
    -> (values fp32 [R][32n], codes int [R][32n], scales fp32 [R][n])."""
    blocks = golden_q8_blocks()
    vals, codes, scales = [], [], []
    for sg in signs:
        v, c, s = [], [], []
        for k in order:
            b = blocks[abs(k) - 1]
            m = -sg if k < 0 else sg
            v += [m * x for x in b["x"]]
            c += [m * q for q in b["codes"]]
            s.append(b["scale"])
        vals.append(v)
        codes.append(c)
        scales.append(s)
    return np.array(vals, F32), np.array(codes, np.int64), np.array(scales, F32)


def dequant(codes, scales):
    """float32(code) * scale, one float32 multiply per element."""
    R, n = scales.shape
    c = codes.reshape(R, n, 32).astype(F32)
    return (c * scales[:, :, None]).reshape(R, n * 32)


# blocks 1..6 of the file, then blocks 1 and 3 negated (a maximum at a
# positive value, negative ties): 8 blocks = 256 elements
ORDER_ATT = [1, 2, 3, 4, 5, 6, -1, -3]
ORDER_FFN = [6, 5, -2, 4, 3, 2, 1, -6]


def _rows_equal_bits(got, ref):
    return np.array_equal(np.ascontiguousarray(got, F32).view(np.uint32),
                          np.ascontiguousarray(ref, F32).view(np.uint32))


@pytest.mark.parametrize("case", ["fused_b2", "rmsnorm_b5", "rmsnorm_fragments_b16"])
def test_golden_blocks_input_round_trip(case):
    import torch
    B, wdt = {"fused_b2": (2, tp.TP_F32), "rmsnorm_b5": (5, tp.TP_F32),
              "rmsnorm_fragments_b16": (16, tp.TP_BF16)}[case]
    D, H, hd, F = 256, 8, 32, 512
    say(f"golden input round trip {case}")
    cfg = tp.make_config(dim=D, n_heads=H, n_kv_heads=H, head_dim=hd, ffn_hidden=F, tp_size=1,
                         tp_rank=0, max_batch=16, max_ctx=4, w_dtype=wdt, kv_dtype=tp.TP_F32,
                         quant=tp.TP_Q_INPUTS, norm_eps=0.0)
    rng = np.random.default_rng(901)

    def w(*s):
        a = (0.02 * rng.standard_normal(s)).astype(F32)
        t = torch.from_numpy(a).cuda()
        return t.to(torch.bfloat16) if wdt == tp.TP_BF16 else t

    g_att, c_att, s_att = golden_rows(ORDER_ATT, [1])
    g_ffn, c_ffn, s_ffn = golden_rows(ORDER_FFN, [1])
    W = {"wq": w(D, D), "wk": w(D, D), "wv": w(D, D), "wo": w(D, D), "w1": w(F, D), "w3": w(F, D),
         "w2": w(D, F), "g_att": dev_tensor(g_att[0]), "g_ffn": dev_tensor(g_ffn[0])}
    sh = tp.Shard(cfg)
    sh.k_cache.zero_()
    sh.v_cache.zero_()
    sh.load(W)
    signs = [1 if b % 2 == 0 else -1 for b in range(B)]
    x_np = np.repeat(np.array(signs, F32)[:, None], D, axis=1)
    x = dev_tensor(x_np)
    lens = dev_tensor(np.zeros(B, np.int32))
    for stage, gain, codes, scales in ((tp.TP_STAGE_ATTN, g_att, c_att, s_att),
                                       (tp.TP_STAGE_FFN, g_ffn, c_ffn, s_ffn)):
        taps = {"xn": torch.full((B, D), float("nan"), device="cuda"),
                "xq": torch.full((B, D), float("nan"), device="cuda")}
        sh.step(stage, x, lens if stage == tp.TP_STAGE_ATTN else None, B, sh.new_wire(), taps)
        torch.cuda.synchronize()
        xq, xn = to_np(taps["xq"]), to_np(taps["xn"])
        sg = np.array(signs, np.int64)[:, None]
        # the normalised row is g * x * (1 / sqrt(mean x^2 + 0)) = g * (+-1) exactly
        assert _rows_equal_bits(xq, (gain * x_np) * F32(1.0)), f"{case} stage {stage}: xq"
        # its round trip is the golden codes times the golden scales, bit for bit
        ref = dequant(codes * sg, np.repeat(scales, B, axis=0))
        assert _rows_equal_bits(xn, ref), (
            f"{case} stage {stage}: {np.sum(xn.view(np.uint32) != ref.view(np.uint32))} values differ")


@pytest.mark.parametrize("B", [1, 5])
def test_golden_blocks_wire_and_logits_merge(B):
    """Two vocabulary shards of 192 logits: shard 0's column 0 holds the six
    golden blocks, shard 1's the blocks in another order, some negated."""
    import torch
    T, D = 2, 64
    order = ([1, 2, 3, 4, 5, 6], [-6, 4, -3, 2, 5, -1])
    say(f"golden wire quantiser + logits merge, batch {B}")
    rng = np.random.default_rng(902)
    w_cls = (0.02 * rng.standard_normal((T * 192, D))).astype(F32)
    gv = [golden_rows(o, [1]) for o in order]
    w_cls[:, 0] = np.concatenate([v[0][0] for v in gv])
    g_fin = (1 + 0.02 * rng.standard_normal(D)).astype(F32)
    g_fin[0] = 0.125
    signs = [1 if b % 3 != 1 else -1 for b in range(B)]
    x_np = np.zeros((B, D), F32)
    x_np[:, 0] = 8.0 * np.array(signs, F32)
    WL = {"w1": dev_tensor(w_cls), "g_att": dev_tensor(g_fin)}
    shards = []
    for r in range(T):
        cfg = tp.make_config(kind=tp.TP_LOGITS, dim=D, ffn_hidden=T * 192, tp_size=T, tp_rank=r,
                             max_batch=16, w_dtype=tp.TP_F32, quant=tp.TP_Q_PARTIALS, norm_eps=0.0)
        sh = tp.Shard(cfg, caches=False)
        sh.load(WL)
        shards.append(sh)
    x = dev_tensor(x_np)
    wires, pres = [], []
    for sh in shards:
        wires.append(sh.new_wire())
        pres.append(torch.full((B, 192), float("nan"), device="cuda"))
        sh.step(tp.TP_STAGE_LOGITS, x, None, B, wires[-1], {"p_pre": pres[-1]})
    out = torch.full((B, T * 192), float("nan"), device="cuda")
    shards[0].merge_logits(wires, out, B)
    torch.cuda.synchronize()
    off = tp.wire_scales_offset(shards[0].cfg, B)
    sg = np.array(signs, np.int64)[:, None]
    ref_out = []
    for r in range(T):
        vals, codes, scales = gv[r]
        # each logit is column 0 of the classifier times +-1 (zeros may carry either sign)
        assert np.array_equal(to_np(pres[r]), vals * sg.astype(F32)), f"shard {r} logits"
        raw = to_np(wires[r])
        got_c = raw[:B * 192].view(np.int8).reshape(B, 192)
        got_s = raw[off:off + B * 6 * 4].view(F32).reshape(B, 6)
        assert np.array_equal(got_c.astype(np.int64), codes * sg), f"shard {r} codes"
        assert _rows_equal_bits(got_s, np.repeat(scales, B, axis=0)), f"shard {r} scales"
        ref_out.append(dequant(codes * sg, np.repeat(scales, B, axis=0)))
    assert _rows_equal_bits(to_np(out), np.concatenate(ref_out, axis=1)), "merged logits"


def test_golden_wires_through_the_merges():
    """int8 wires assembled on the host from the golden blocks, merged onto a
    residual by merge_partials (the merge kernel) and, as the other ranks'
    wires, by decode_merge_step (the merge fused into the quantiser of this
    shard's own partial): every output element is the float32 sum of the
    residual and each wire's float32(code) * scale, in wire order."""
    import torch
    D, B, T = 256, 3, 2
    say("golden wires through merge_partials and the fused int8 merge")
    cfg = tp.make_config(dim=D, n_heads=8, n_kv_heads=8, head_dim=32, ffn_hidden=512, tp_size=T,
                         tp_rank=0, max_batch=4, max_ctx=4, w_dtype=tp.TP_F32,
                         kv_dtype=tp.TP_F32, quant=tp.TP_Q_PARTIALS)
    rng = np.random.default_rng(903)
    f = lambda *s: torch.from_numpy((0.02 * rng.standard_normal(s)).astype(F32)).cuda()  # noqa: E731
    W = {"wq": f(D, D), "wk": f(D, D), "wv": f(D, D), "wo": f(D, D), "w1": f(512, D),
         "w3": f(512, D), "w2": f(D, 512),
         "g_att": dev_tensor((1 + 0.02 * rng.standard_normal(D)).astype(F32)),
         "g_ffn": dev_tensor((1 + 0.02 * rng.standard_normal(D)).astype(F32))}
    sh = tp.Shard(cfg)
    sh.load(W)
    off = tp.wire_scales_offset(cfg, B)
    signs = [1, -1, 1]

    def host_wire(order):
        _, codes, scales = golden_rows(order, signs)
        raw = np.zeros(int(sh.sizes.wire), np.uint8)
        raw[:B * D] = codes.astype(np.int8).reshape(-1).view(np.uint8)
        raw[off:off + B * (D // 32) * 4] = scales.reshape(-1).view(np.uint8)
        return raw, dequant(codes, scales)

    (r0, d0), (r1, d1) = host_wire(ORDER_ATT), host_wire(ORDER_FFN)
    wires = [torch.from_numpy(r0).cuda(), torch.from_numpy(r1).cuda()]
    res = rng.standard_normal((B, D)).astype(F32)
    res[0] = 0.0  # row 0: the merge is the dequantised codes themselves
    out = torch.full((B, D), float("nan"), device="cuda")
    sh.merge(tp.TP_STAGE_ATTN, wires, dev_tensor(res), out, B)
    torch.cuda.synchronize()
    assert _rows_equal_bits(to_np(out), (res + d0) + d1), "merge_partials"
    # fused: this shard's own partial (wire `own`) is quantised and merged by
    # the same kernel, the golden wire read from memory
    for own in (0, 1):
        x = dev_tensor(res)
        mine = sh.new_wire()
        ws = [mine, wires[1]] if own == 0 else [wires[0], mine]
        xo = torch.full((B, D), float("nan"), device="cuda")
        sh.step_merge(tp.TP_STAGE_FFN, x, None, B, mine, ws, xo)
        torch.cuda.synchronize()
        raw = to_np(mine)
        dm = dequant(raw[:B * D].view(np.int8).astype(np.int64),
                     raw[off:off + B * (D // 32) * 4].view(F32).reshape(B, D // 32))
        parts = [dm, d1] if own == 0 else [d0, dm]
        assert _rows_equal_bits(to_np(xo), (res + parts[0]) + parts[1]), f"fused merge, own {own}"
