"""decode_merge_step (the merge of a stage's partials done by the kernel that
produces this shard's own partial) against decode_step followed by
merge_partials. Both use the same per-element fp32 sum in wire order, so the
merged rows and the stage's own wire must be bitwise equal. Cases cover every
producer that can carry the merge: the down-projection with LDS-staged
activations (batch <= 4), the one reading activations from global memory
(fp32 batch 8), the MFMA ones (bf16 batch 16: one and two 16-row tiles per
wave, and split K with the merge in the reduce), and the int8 quantiser; the
own wire at the first, the last and a middle position, x_out aliasing x, and
more wires than the producer requests ahead of time (8)."""
import sys

import numpy as np
import pytest

import synth
import tensor_tp_shard_amd as tp
from gpu_harness import Layer, dev_tensor, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    tp.lib()


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _wire_bytes(w, wire, B):
    """The bytes of a wire that carry data for `batch` rows."""
    a = to_np(wire)
    if w.quant & synth.Q_PARTIALS:
        off = tp.wire_scales_offset(tp.make_config(dim=w.dim), B)
        return np.concatenate([a[:B * w.dim], a[off:off + B * (w.dim // 32) * 4]])
    return a[:B * w.dim * 4]


def _bits(t):
    return to_np(t).view(np.uint32)


CASES = {
    # LDS-staged down-projection, fp32 wires
    "tiny_fp32_b1": synth.TINY,
    # int8 wires: the quantiser merges
    "micro_q8_b3": synth.small_llama(name="micro_q8", dim=256, n_heads=8, n_kv_heads=4,
                                     head_dim=32, ffn_hidden=512, tp=4, batch=3, past=(1, 100),
                                     w_dtype=synth.BF16, kv_dtype=synth.BF16,
                                     quant=synth.Q_PARTIALS | synth.Q_INPUTS, seed=301),
    # MFMA down-projection (bf16, batch 16)
    "micro_bf16_b16": synth.small_llama(name="micro_b16m", dim=256, n_heads=8, n_kv_heads=4,
                                        head_dim=32, ffn_hidden=512, tp=2, batch=16,
                                        past=(1, 90), w_dtype=synth.BF16, kv_dtype=synth.BF16,
                                        seed=302),
    # down-projection reading activations from global memory (fp32, batch 8)
    "micro_fp32_b8": synth.small_llama(name="micro_b8", dim=128, n_heads=4, n_kv_heads=4,
                                       head_dim=32, ffn_hidden=256, tp=2, batch=8, past=(3, 70),
                                       seed=303),
    # MFMA down-projection with two 16-row tiles per wave (dim 8192, F/T 3584)
    "wide_bf16_b16": synth.small_llama(name="wide_b16", dim=8192, n_heads=8, n_kv_heads=8,
                                       head_dim=128, ffn_hidden=7168, tp=2, batch=16,
                                       past=(1, 40), w_dtype=synth.BF16, kv_dtype=synth.BF16,
                                       seed=305),
    # split-K MFMA down-projection (F/T 4096: long K) with the merge in its reduce
    "splitk_bf16_b16": synth.small_llama(name="splitk_b16", dim=1024, n_heads=8, n_kv_heads=8,
                                         head_dim=128, ffn_hidden=8192, tp=2, batch=16,
                                         past=(1, 40), w_dtype=synth.BF16, kv_dtype=synth.BF16,
                                         seed=306),
    # QKV, attention, combine and W_O in one launch (bf16 cache of head dim
    # 128, batch <= 4): W_O's merging store there
    "fused_qkv_attn_b3": synth.small_llama(name="fused_qa", dim=512, n_heads=8, n_kv_heads=8,
                                           head_dim=128, ffn_hidden=512, tp=4, batch=3,
                                           past=(1, 100), w_dtype=synth.BF16, kv_dtype=synth.BF16,
                                           seed=307),
    # dim > 8192 with int8 wires
    "wide_q8_b2": synth.small_llama(name="wide_q8", dim=8448, n_heads=4, n_kv_heads=4,
                                    head_dim=32, ffn_hidden=256, tp=2, batch=2, past=(2, 40),
                                    w_dtype=synth.BF16, kv_dtype=synth.BF16,
                                    quant=synth.Q_PARTIALS, seed=304),
}


@pytest.mark.parametrize("case", list(CASES))
def test_fused_merge_equals_step_then_merge(case):
    import torch
    w = CASES[case]
    B = w.batch
    d = synth.llama_inputs(w)
    say(f"decode_merge_step {case} dim={w.dim} B={B} T={w.tp} quant={w.quant}")
    L = Layer(w, d)
    x = dev_tensor(d["x"])
    lens = dev_tensor(d["lens"])
    ranks = L.ranks

    # attention stage; rank 0's wire is the first of the merge
    wa, _ = L.stage(tp.TP_STAGE_ATTN, x, lens, B, with_taps=False)
    h_ref = L.merge(tp.TP_STAGE_ATTN, wa, x, B)
    sh = L.shards[ranks[0]]
    own = sh.new_wire()
    h2 = torch.full_like(x, float("nan"))
    sh.step_merge(tp.TP_STAGE_ATTN, x, lens, B, own, [own] + [wa[r] for r in ranks[1:]], h2)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(h2), _bits(h_ref))
    assert np.array_equal(_wire_bytes(w, own, B), _wire_bytes(w, wa[ranks[0]], B))

    # FFN stage; the last rank's wire is the last of the merge
    wf, _ = L.stage(tp.TP_STAGE_FFN, h_ref, None, B, with_taps=False)
    x_ref = L.merge(tp.TP_STAGE_FFN, wf, h_ref, B)
    shl = L.shards[ranks[-1]]
    own = shl.new_wire()
    x2 = torch.full_like(x, float("nan"))
    shl.step_merge(tp.TP_STAGE_FFN, h_ref, None, B, own, [wf[r] for r in ranks[:-1]] + [own], x2)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(x2), _bits(x_ref))
    assert np.array_equal(_wire_bytes(w, own, B), _wire_bytes(w, wf[ranks[-1]], B))

    # in place: x_out is the stage input
    y = h_ref.clone()
    own = shl.new_wire()
    shl.step_merge(tp.TP_STAGE_FFN, y, None, B, own, [wf[r] for r in ranks[:-1]] + [own], y)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), _bits(x_ref))
    assert tp.read_error_word(sh.handle) == 0


@pytest.mark.parametrize("case", ["tiny_fp32_b1", "micro_q8_b3", "micro_bf16_b16", "micro_fp32_b8"])
def test_fused_merge_of_many_wires(case):
    """11 wires, the own one tenth: past the 8 requested ahead of time."""
    import torch
    w = CASES[case]
    B = w.batch
    d = synth.llama_inputs(w)
    say(f"decode_merge_step 11 wires {case}")
    L = Layer(w, d)
    x = dev_tensor(d["x"])
    wa, _ = L.stage(tp.TP_STAGE_ATTN, x, dev_tensor(d["lens"]), B, with_taps=False)
    h = L.merge(tp.TP_STAGE_ATTN, wa, x, B)
    wf, _ = L.stage(tp.TP_STAGE_FFN, h, None, B, with_taps=False)
    sh = L.shards[1]
    others = [wf[r] for r in L.ranks] * 5
    ref_list = others[:9] + [wf[1]] + others[9:10]
    ref = torch.empty_like(h)
    sh.merge(tp.TP_STAGE_FFN, ref_list, h, ref, B)
    own = sh.new_wire()
    out = torch.full_like(h, float("nan"))
    sh.step_merge(tp.TP_STAGE_FFN, h, None, B, own, others[:9] + [own] + others[9:10], out)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), _bits(ref))


@pytest.mark.parametrize("case", ["fused_qkv_attn_b3", "micro_q8_b3", "splitk_bf16_b16"])
def test_merge_step_graph_replays(case):
    """Rank 0's whole layer step as the benchmark replays it: decode_merge_step
    for the attention stage (one launch of QKV + attention at batch 3, its
    W_O merging) and for the FFN stage, the other ranks' wires computed once
    beforehand; captured once, replayed three times with new inputs copied in
    between and the program's own eager work after each, every replay bitwise
    equal to an eager step on the same inputs."""
    import torch
    w = CASES[case]
    B = w.batch
    d = synth.llama_inputs(w)
    say(f"decode_merge_step graph replays {case}")
    L = Layer(w, d)
    ranks = L.ranks
    x = dev_tensor(d["x"])
    lens = dev_tensor(d["lens"])
    wa, _ = L.stage(tp.TP_STAGE_ATTN, x, lens, B, with_taps=False)
    h_ref = L.merge(tp.TP_STAGE_ATTN, wa, x, B)
    wf, _ = L.stage(tp.TP_STAGE_FFN, h_ref, None, B, with_taps=False)
    sh = L.shards[ranks[0]]
    own_a, own_f = sh.new_wire(), sh.new_wire()
    h, out = torch.empty_like(x), torch.empty_like(x)

    def step(h, out):
        sh.step_merge(tp.TP_STAGE_ATTN, x, lens, B, own_a, [own_a] + [wa[r] for r in ranks[1:]], h)
        sh.step_merge(tp.TP_STAGE_FFN, h, None, B, own_f, [own_f] + [wf[r] for r in ranks[1:]], out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(h, out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(h, out)
    rng = np.random.default_rng(308)
    h_e, out_e = torch.empty_like(x), torch.empty_like(x)
    for rep in range(3):
        x.copy_(torch.from_numpy(rng.standard_normal(d["x"].shape).astype(np.float32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_h, got_out = _bits(h).copy(), _bits(out).copy()
        step(h_e, out_e)
        torch.cuda.synchronize()
        assert np.array_equal(got_h, _bits(h_e)), f"replay {rep}: h"
        assert np.array_equal(got_out, _bits(out_e)), f"replay {rep}: out"
        torch.zeros(1000, device="cuda").sum().item()  # eager work between replays
    assert tp.read_error_word(sh.handle) == 0
