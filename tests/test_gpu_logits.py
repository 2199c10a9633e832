"""GPU parity of the final stage (final RMSNorm, vocabulary-split logits, their
int8 wire and merge) and of a whole decode step (layers chained, then the
final stage) against the fp64 oracle, through the C ABI.

Bars: int8 codes and scales of a wire bit-exact against the oracle's codec
of the GPU's own fp32 logits; the merge bit-exact against the placement of
the GPU's own (dequantised) wires; fp32 values within rel-L2 1e-4 (fp32
weights) or 1e-3 (bf16 or int8 weights, fp32 accumulation), and the merged
rows within 2e-2 when they went through the int8 wire (its rounding).
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import synth
from conftest import rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from gpu_harness import Layer, Logits, split_logits_wire  # noqa: E402


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _tol(w):
    return 1e-4 if w.w_dtype == synth.F32 and not w.quant & synth.Q_WEIGHTS else 1e-3


def check_logits(w, B=None, d=None, max_batch=None):
    B = w.batch if B is None else B
    d = d or synth.logits_inputs(w, B)
    say(f"{w.name} D={w.dim} V={w.vocab} T={w.tp} B={B} max_batch={max_batch or B} quant={w.quant}")
    g = Logits(w, d, max_batch=max_batch or B).run(d["x"])
    o = oracle.logits(d["w_cls"], d["g_final"], d["x"], w.tp, w.quant, w.norm_eps, w.w_dtype,
                      bool(w.quant & synth.Q_WEIGHTS))
    tol, Vs = _tol(w), w.vocab // w.tp
    placed = []
    for r in range(w.tp):
        t = g["taps"][r]
        assert np.all(np.isfinite(t["p_pre"])), f"logits[{r}] not finite"
        e_xn, e_z = rel_l2(t["xn"], o["xn"]), rel_l2(t["p_pre"], o["z"][r])
        assert e_xn <= tol and e_z <= tol, f"shard {r}: xn {e_xn:.3e} logits {e_z:.3e} > {tol}"
        if w.quant & synth.Q_PARTIALS:
            codes, scales = split_logits_wire(w, g["wires"][r], B)
            oc, os_ = oracle.q8_quantize(t["p_pre"].reshape(-1))
            assert np.array_equal(codes.reshape(-1), oc), f"wire {r}: codes differ"
            assert np.array_equal(scales.reshape(-1).view(np.uint32), os_.view(np.uint32))
            placed.append(oracle.q8_dequantize(codes, scales).reshape(B, Vs))
        else:
            wire = g["wires"][r][:B * Vs * 4].view(np.float32).reshape(B, Vs)
            assert np.array_equal(wire.view(np.uint32), t["p_pre"].view(np.uint32))
            placed.append(wire)
    want = np.concatenate(placed, axis=1)
    assert np.array_equal(g["out"].view(np.uint32), want.view(np.uint32)), "merge is not placement"
    e = rel_l2(g["out"], o["out"])
    assert e <= (2e-2 if w.quant & synth.Q_PARTIALS else tol), f"merged logits rel-L2 {e:.3e}"
    say(f"{w.name} B={B} logits rel-L2 {e:.3e}")
    return g, o


def _small(name, dim, vocab, tp_, batch, w_dtype=synth.BF16, quant=0, seed=2001):
    return synth.LlamaLogits(name, dim=dim, vocab=vocab, tp=tp_, batch=batch, w_dtype=w_dtype,
                             quant=quant, seed=seed)


@pytest.mark.parametrize("case", [
    # (dim, vocab, T, batch, dtype, quant): the GEMV paths (LDS-fused norm below
    # batch 5, MFMA tiles from 5, split-K with the norm folded in for long K
    # and V/T a multiple of 128), ragged V/T, the int8 wire and int8 weights
    (256, 1024, 4, 1, synth.F32, 0),
    (256, 1024, 4, 3, synth.F32, synth.Q_PARTIALS),
    (288, 400, 2, 2, synth.BF16, 0),            # V/T = 200: not a multiple of 16
    (288, 400, 2, 7, synth.F32, 0),             # fp32 weights beyond batch 4
    (256, 1024, 4, 5, synth.BF16, 0),
    (256, 1024, 4, 16, synth.BF16, synth.Q_PARTIALS),
    (4096, 8192, 4, 16, synth.BF16, 0),         # split-K, folded norm
    (256, 1024, 2, 2, synth.BF16, synth.Q_WEIGHTS),
    (256, 1024, 2, 16, synth.BF16, synth.Q_WEIGHTS | synth.Q_PARTIALS),
    (256, 512, 1, 3, synth.BF16, synth.Q_PARTIALS),   # one shard: the merge is a dequantised copy
], ids=lambda c: f"D{c[0]}_V{c[1]}_T{c[2]}_B{c[3]}_{c[4]}_q{c[5]}")
def test_logits_shapes(case):
    D, V, T, B, dt, q = case
    check_logits(_small(f"logits_D{D}_V{V}", D, V, T, B, dt, q))


@pytest.mark.parametrize("B", [1, 5, 13])
def test_logits_batch_below_max_batch(B):
    """A handle planned for batch 16 run at a smaller batch: the int8 wire's
    scales sit right after that batch's codes (tp_wire_scales_offset of the
    batch run), in the step and in the merge alike."""
    check_logits(_small("logits_maxb16", 256, 2048, 4, B, synth.BF16, synth.Q_PARTIALS, seed=2002),
                 max_batch=16)


def test_llama7b_logits_b1():
    check_logits(synth.L7B_LOGITS)


def test_llama7b_logits_b1_q8():
    check_logits(synth.L7B_LOGITS_Q8)


def test_llama7b_logits_b16():
    check_logits(dataclasses.replace(synth.L7B_LOGITS, batch=16))


def test_llama70b_logits_b16():
    check_logits(synth.L70B_LOGITS)


def test_llama7b_logits_b1_int8_classifier():
    check_logits(dataclasses.replace(synth.L7B_LOGITS, name="llama2_7b_tp4_logits_b1_w8",
                                     quant=synth.Q_WEIGHTS))


def test_llama70b_logits_b16_int8_wire():
    check_logits(dataclasses.replace(synth.L70B_LOGITS, name="llama2_70b_tp8_logits_b16_q8",
                                     quant=synth.Q_PARTIALS))


def test_decode_step_int8_wires_then_logits():
    """The two-layer decode step with int8 wires in the layers and on the
    logits: the layer deltas and the logits within the int8 bound, every
    wire's codes checked against the codec of the GPU's own partial by the
    layer and logits checks."""
    layers = []
    for i in range(2):
        w = synth.small_llama(name=f"decode_q8_l{i}", dim=256, n_heads=8, n_kv_heads=4, head_dim=32,
                              ffn_hidden=512, tp=2, batch=2, past=(3, 40), w_dtype=synth.BF16,
                              kv_dtype=synth.BF16, quant=synth.Q_PARTIALS, seed=2120 + i)
        layers.append((w, synth.llama_weights(w)))
    w0 = layers[0][0]
    lens = synth.llama_lens(w0)
    kcs = [synth.llama_kv_cache(w, lens, "kcache") for w, _ in layers]
    vcs = [synth.llama_kv_cache(w, lens, "vcache") for w, _ in layers]
    lw = _small("decode_q8_logits", 256, 2048, 2, 2, quant=synth.Q_PARTIALS, seed=2130)
    ld = synth.logits_inputs(lw)
    x = synth.llama_x(w0)
    say(f"decode step with int8 wires: 2 layers x T=2, B=2, lens={lens.tolist()}")
    h = x
    for (w, wts), kc, vc in zip(layers, kcs, vcs):
        h = Layer(w, dict(wts, kcache=kc, vcache=vc)).run(h, lens, with_taps=False)["out"]
    g = Logits(lw, ld).run(h, with_taps=False)
    o = oracle.llama_decode(layers, ld["w_cls"], ld["g_final"], x, lens, [k.copy() for k in kcs],
                            [v.copy() for v in vcs], quant_logits=synth.Q_PARTIALS,
                            cls_dtype=lw.w_dtype)
    e_h = rel_l2(h.astype(np.float64) - x, o["h"][-1] - x)
    e = rel_l2(g["out"], o["out"])
    say(f"decode step with int8 wires: last layer delta rel-L2 {e_h:.3e}, logits rel-L2 {e:.3e}")
    assert e_h <= 2e-2 and e <= 2e-2


def test_decode_step_two_layers_then_logits():
    """A whole decode step: two layers of every shard in turn, each fed the
    previous layer's merged output, then the final stage, against the
    oracle's decode loop."""
    layers = []
    for i in range(2):
        w = synth.small_llama(name=f"decode_l{i}", dim=256, n_heads=8, n_kv_heads=4, head_dim=32,
                              ffn_hidden=512, tp=2, batch=3, past=(3, 40), w_dtype=synth.BF16,
                              kv_dtype=synth.BF16, seed=2100 + i)
        layers.append((w, synth.llama_weights(w)))
    w0 = layers[0][0]
    lens = synth.llama_lens(w0)
    kcs = [synth.llama_kv_cache(w, lens, "kcache") for w, _ in layers]
    vcs = [synth.llama_kv_cache(w, lens, "vcache") for w, _ in layers]
    lw = _small("decode_logits", 256, 2048, 2, 3, seed=2110)
    ld = synth.logits_inputs(lw)
    x = synth.llama_x(w0)
    say(f"decode step: 2 layers x T=2, B=3, lens={lens.tolist()}, V=2048")
    h = x
    for (w, wts), kc, vc in zip(layers, kcs, vcs):
        dd = dict(wts, kcache=kc, vcache=vc)
        h = Layer(w, dd).run(h, lens, with_taps=False)["out"]
    g = Logits(lw, ld).run(h, with_taps=False)
    o = oracle.llama_decode(layers, ld["w_cls"], ld["g_final"], x, lens, [k.copy() for k in kcs],
                            [v.copy() for v in vcs], cls_dtype=lw.w_dtype)
    e_h = rel_l2(h.astype(np.float64) - x, o["h"][-1] - x)
    e = rel_l2(g["out"], o["out"])
    say(f"decode step: last layer delta rel-L2 {e_h:.3e}, logits rel-L2 {e:.3e}")
    assert e_h <= 1e-3 and e <= 1e-3
    # the token each row would pick: the GPU's argmax is a maximum of the
    # oracle's logits up to the tolerance (exact ties may pick either)
    top = o["out"][np.arange(lw.batch), np.argmax(g["out"], axis=1)]
    assert np.all(top >= o["out"].max(axis=1) - 1e-3 * np.abs(o["out"]).max())


def test_graph_replay_of_the_final_stage():
    """Every shard's final stage and the merge captured in a HIP graph (int8
    wire, batch 16: split-K with the folded norm): every replay, with eager
    work between them, is bitwise the eager result."""
    w = _small("logits_graph", 4096, 8192, 4, 16, synth.BF16, synth.Q_PARTIALS, seed=2003)
    d = synth.logits_inputs(w)
    say("final stage: graph replay")
    L = Logits(w, d)
    from gpu_harness import dev_tensor, to_np
    import tensor_tp_shard_amd as tp
    x = dev_tensor(d["x"])
    wires = [sh.new_wire() for sh in L.shards]
    out = torch.empty((w.batch, w.vocab), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def step():
        for sh, wr in zip(L.shards, wires):
            sh.step(tp.TP_STAGE_LOGITS, x, None, w.batch, wr)
        L.shards[0].merge_logits(wires, out, w.batch)

    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    eager = to_np(out).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_np(out).view(np.uint32), eager.view(np.uint32))
        torch.zeros(1000, device="cuda").sum().item()  # eager work between replays
