"""decode_step_noalloc, the entry point for callers that cannot allocate:
the same kernels as decode_step with the workspace regions in the library's
static scratch. Checked through the C ABI against decode_step on twin
shards: wires, taps and cache appends bitwise equal, on two calls in a row,
the second with a smaller batch (the scratch keeps the first call's
contents); a handle loaded without a workspace; the caller's error word; the
size limit, rejected before anything is enqueued."""
import numpy as np
import pytest

import synth
import tensor_tp_shard_amd as tp
from gpu_harness import config_of, dev_tensor, shard_cache, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    tp.lib()


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


CASES = {
    # batch 16 then 5: MFMA projections, MFMA attention (4 q heads per kv head)
    "mfma_b16_then_b5": (dict(dim=256, n_heads=8, n_kv_heads=2, head_dim=64, ffn_hidden=512,
                              batch=16, past=(5, 200)), 0, 16, 5),
    # batch 7 then 2 at dim 4096: split-K up-projections with the folded norm,
    # then the LDS-staged GEMVs with the norm in their prologue
    "splitk_b7_then_b2": (dict(dim=4096, n_heads=8, n_kv_heads=2, head_dim=128, ffn_hidden=4096,
                               batch=7, past=(1, 100)), 0, 7, 2),
    # int8 wires and int8 inputs, batch 3 then 1
    "q8_b3_then_b1": (dict(dim=256, n_heads=8, n_kv_heads=8, head_dim=32, ffn_hidden=512, batch=3,
                           past=(30, 70)), synth.Q_PARTIALS | synth.Q_INPUTS, 3, 1),
}


def _twins(w, d, rank):
    """Two identically loaded shards: one with a workspace, one without."""
    dw = {k: dev_tensor(d[k]) for k in ("wq", "wk", "wv", "wo", "w1", "w3", "w2", "g_att", "g_ffn")}
    out = []
    for ws in (True, False):
        sh = tp.Shard(config_of(w, rank), caches=False, workspace=ws)
        sh.load(dw, k_cache=dev_tensor(shard_cache(w, d["kcache"], rank)).reshape(-1),
                v_cache=dev_tensor(shard_cache(w, d["vcache"], rank)).reshape(-1))
        out.append(sh)
    return out


def _taps(w, B, stage):
    import torch
    f = lambda *s: torch.full(s, float("nan"), device="cuda")  # noqa: E731
    T, hd = w.tp, w.head_dim
    if stage == tp.TP_STAGE_ATTN:
        return {"xn": f(B, w.dim), "xq": f(B, w.dim), "q": f(B, w.n_heads // T * hd),
                "k": f(B, w.n_kv_heads // T * hd), "v": f(B, w.n_kv_heads // T * hd),
                "att": f(B, w.n_heads // T * hd), "p_pre": f(B, w.dim)}
    return {"xn": f(B, w.dim), "xq": f(B, w.dim), "a": f(B, w.ffn_hidden // T), "p_pre": f(B, w.dim)}


def _same(a, b):
    return np.array_equal(to_np(a).view(np.uint8), to_np(b).view(np.uint8))


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_equals_decode_step(case):
    import torch
    shape, quant, B1, B2 = CASES[case]
    w = synth.small_llama(name=f"noalloc_{case}", tp=2, w_dtype=synth.BF16, kv_dtype=synth.BF16,
                          quant=quant, seed=95, **shape)
    d = synth.llama_inputs(w)
    say(f"decode_step_noalloc {case}: batch {B1} then {B2}")
    A, Z = _twins(w, d, 1)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(96)
    for call, B in enumerate((B1, B2)):
        x = dev_tensor(rng.standard_normal((B, w.dim)).astype(np.float32))
        # the second call appends at the next slot (the last slot stays in range)
        lens = dev_tensor(np.minimum(d["lens"][:B] + call, w.max_ctx - 1).astype(np.int32))
        for stage in (tp.TP_STAGE_ATTN, tp.TP_STAGE_FFN):
            wa, wz = A.new_wire(), Z.new_wire()
            wa.fill_(0xA5)
            wz.fill_(0x5A)
            ta, tz = _taps(w, B, stage), _taps(w, B, stage)
            ln = lens if stage == tp.TP_STAGE_ATTN else None
            A.step(stage, x, ln, B, wa, ta)
            Z.step_noalloc(stage, x, ln, B, wz, tz, err_out=err)
            torch.cuda.synchronize()
            nbytes = (tp.wire_scales_offset(A.cfg, B) + B * (w.dim // 32) * 4
                      if quant & synth.Q_PARTIALS else B * w.dim * 4)
            assert _same(wa[:nbytes], wz[:nbytes]), f"call {call} stage {stage}: wires differ"
            for k in ta:
                assert _same(ta[k], tz[k]), f"call {call} stage {stage}: tap {k} differs"
        assert _same(A.k_cache, Z.k_cache) and _same(A.v_cache, Z.v_cache), f"call {call}: caches"
    assert int(err.item()) == 0
    assert tp.read_error_word(A.handle) == 0


def test_noalloc_without_workspace_and_error_word():
    import torch
    w = synth.small_llama(name="noalloc_err", dim=256, n_heads=8, n_kv_heads=8, head_dim=32,
                          ffn_hidden=512, tp=1, batch=3, past=(5, 9), w_dtype=synth.BF16,
                          kv_dtype=synth.BF16, seed=97)
    d = synth.llama_inputs(w)
    say("decode_step_noalloc: no workspace, error word")
    A, Z = _twins(w, d, 0)
    x = dev_tensor(d["x"])
    bad = d["lens"].copy()
    bad[1] = w.max_ctx
    lens = dev_tensor(bad)
    # a handle without a workspace runs only through decode_step_noalloc
    with pytest.raises(tp.TpError) as e:
        Z.step(tp.TP_STAGE_ATTN, x, lens, w.batch, Z.new_wire())
    assert e.value.status == tp.TP_ESTATE
    with pytest.raises(tp.TpError):
        tp.read_error_word(Z.handle)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ta, tz = _taps(w, w.batch, tp.TP_STAGE_ATTN), _taps(w, w.batch, tp.TP_STAGE_ATTN)
    A.step(tp.TP_STAGE_ATTN, x, lens, w.batch, A.new_wire(), ta)
    Z.step_noalloc(tp.TP_STAGE_ATTN, x, lens, w.batch, Z.new_wire(), tz, err_out=err)
    torch.cuda.synchronize()
    assert tp.read_error_word(A.handle) == tp.TP_DERR_LEN
    assert int(err.item()) == tp.TP_DERR_LEN
    assert _same(ta["att"], tz["att"]) and np.all(to_np(tz["att"])[1] == 0)
    # no error word given: the step still runs (its bits go to an unread word)
    wz = Z.new_wire()
    Z.step_noalloc(tp.TP_STAGE_ATTN, x, dev_tensor(d["lens"]), w.batch, wz)
    torch.cuda.synchronize()


def test_noalloc_rejects_a_shard_beyond_the_scratch():
    """A shape whose workspace exceeds the 16 MiB scratch (chunk records of a
    65536-position cache at batch 16) is refused before anything is enqueued;
    the handle's caches are never touched, so stand-ins of 16 bytes serve."""
    import torch
    cfg = tp.make_config(dim=256, n_heads=8, n_kv_heads=8, head_dim=32, ffn_hidden=512, tp_size=1,
                         tp_rank=0, max_batch=16, max_ctx=65536, w_dtype=tp.TP_BF16,
                         kv_dtype=tp.TP_BF16)
    sh = tp.Shard(cfg, caches=False, workspace=False)
    assert sh.sizes.workspace > 16 << 20
    rng = np.random.default_rng(98)
    f = lambda *s: torch.from_numpy((0.02 * rng.standard_normal(s)).astype(np.float32)).cuda().to(torch.bfloat16)  # noqa: E731
    W = {"wq": f(256, 256), "wk": f(256, 256), "wv": f(256, 256), "wo": f(256, 256), "w1": f(512, 256),
         "w3": f(512, 256), "w2": f(256, 512), "g_att": torch.ones(256, device="cuda"),
         "g_ffn": torch.ones(256, device="cuda")}
    stand_in = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    sh.load(W, k_cache=stand_in, v_cache=stand_in)
    torch.cuda.synchronize()
    with pytest.raises(tp.TpError) as e:
        sh.step_noalloc(tp.TP_STAGE_ATTN, torch.zeros(1, 256, device="cuda"),
                        torch.zeros(1, dtype=torch.int32, device="cuda"), 1, sh.new_wire())
    assert e.value.status == tp.TP_EINVAL and "scratch" in str(e.value)
