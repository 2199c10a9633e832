"""The one-launch QKV projection + attention (batch <= 4, bf16 cache of head
dim 128, at most 2 q heads per kv head), checked through the C ABI against
the separate launches that decode_step_noalloc always takes, on twin shards
loaded identically: wires, taps and cache appends bitwise equal, over three
calls in a row with new inputs each time (each call's attention must take
that call's queries, not the previous call's hand-off words), at ragged
lengths (the new token alone, chunk edges, the owner of position lens[b] in
every wave slot); and under HIP graph replay, each replay fed new inputs and
checked against the separate launches. Parity of the same path with the
oracle is in test_gpu_parity (test_fused_qkv_attention_ragged_batch)."""
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
    # MHA (one q head per kv head), bf16 weights, batch 4 then 1 then 3
    "mha_bf16": (dict(dim=512, n_heads=8, n_kv_heads=8, head_dim=128, ffn_hidden=512,
                      past=(0, 200)), 0, (4, 1, 3)),
    # GQA with 2 q heads per kv head, int8 weights, batch 3 then 2 then 1
    "gqa2_w8": (dict(dim=512, n_heads=8, n_kv_heads=4, head_dim=128, ffn_hidden=512,
                     past=(0, 200)), synth.Q_WEIGHTS, (3, 2, 1)),
    # int8 wires and int8 inputs (the norm's round trip in the prologue), batch 2 then 4
    "mha_q8": (dict(dim=512, n_heads=4, n_kv_heads=4, head_dim=128, ffn_hidden=512,
                    past=(60, 140)), synth.Q_PARTIALS | synth.Q_INPUTS, (2, 4, 2)),
}
LENS = np.array([0, 64, 130, 63], np.int32)  # the new token alone, chunk edges


def _twins(w, d, rank):
    """Two identically loaded shards: decode_step (fused launch) and
    decode_step_noalloc (separate launches)."""
    dw = {k: dev_tensor(d[k]) for k in ("wq", "wk", "wv", "wo", "w1", "w3", "w2", "g_att", "g_ffn")}
    out = []
    for ws in (True, False):
        sh = tp.Shard(config_of(w, rank), caches=False, workspace=ws)
        sh.load(dw, k_cache=dev_tensor(shard_cache(w, d["kcache"], rank)).reshape(-1),
                v_cache=dev_tensor(shard_cache(w, d["vcache"], rank)).reshape(-1))
        out.append(sh)
    return out


def _taps(w, B):
    import torch
    f = lambda *s: torch.full(s, float("nan"), device="cuda")  # noqa: E731
    T, hd = w.tp, w.head_dim
    return {"xn": f(B, w.dim), "xq": f(B, w.dim), "q": f(B, w.n_heads // T * hd),
            "k": f(B, w.n_kv_heads // T * hd), "v": f(B, w.n_kv_heads // T * hd),
            "att": f(B, w.n_heads // T * hd), "p_pre": f(B, w.dim)}


def _same(a, b):
    return np.array_equal(to_np(a).view(np.uint8), to_np(b).view(np.uint8))


def _wire_bytes(w, cfg, B):
    if w.quant & synth.Q_PARTIALS:
        return tp.wire_scales_offset(cfg, B) + B * (w.dim // 32) * 4
    return B * w.dim * 4


def _layer(case):
    shape, quant, batches = CASES[case]
    w = synth.small_llama(name=f"qkv_attn_{case}", tp=2, batch=max(batches), w_dtype=synth.BF16,
                          kv_dtype=synth.BF16, quant=quant, seed=101, **shape)
    d = synth.llama_inputs(w)
    d["lens"] = np.minimum(LENS[:w.batch], w.max_ctx - 4).astype(np.int32)
    d["kcache"] = synth.llama_kv_cache(w, d["lens"] + 3, "kcache")
    d["vcache"] = synth.llama_kv_cache(w, d["lens"] + 3, "vcache")
    return w, d, batches


@pytest.mark.parametrize("case", list(CASES))
def test_fused_equals_separate_launches(case):
    import torch
    w, d, batches = _layer(case)
    rng = np.random.default_rng(102)
    for rank in range(w.tp):
        say(f"qkv + attention {case} rank {rank}: batches {batches}")
        A, Z = _twins(w, d, rank)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        for call, B in enumerate(batches):
            x = dev_tensor(rng.standard_normal((B, w.dim)).astype(np.float32))
            lens = dev_tensor((d["lens"][:B] + call).astype(np.int32))
            wa, wz = A.new_wire(), Z.new_wire()
            wa.fill_(0xA5)
            wz.fill_(0x5A)
            ta, tz = _taps(w, B), _taps(w, B)
            A.step(tp.TP_STAGE_ATTN, x, lens, B, wa, ta)
            Z.step_noalloc(tp.TP_STAGE_ATTN, x, lens, B, wz, tz, err_out=err)
            torch.cuda.synchronize()
            n = _wire_bytes(w, A.cfg, B)
            assert _same(wa[:n], wz[:n]), f"rank {rank} call {call}: wires differ"
            for k in ta:
                assert _same(ta[k], tz[k]), f"rank {rank} call {call}: tap {k} differs"
            assert _same(A.k_cache, Z.k_cache) and _same(A.v_cache, Z.v_cache), f"call {call}: caches"
        assert int(err.item()) == 0
        assert tp.read_error_word(A.handle) == 0


def test_fused_graph_replays_take_each_replays_inputs():
    """The attention stage captured once and replayed with new inputs copied
    in between: every replay equals the separate launches on those inputs
    (the stage's W_O kernel advances the epoch that each replay's tags come
    from, so no replay can take the previous one's hand-off words)."""
    import torch
    w, d, _ = _layer("mha_bf16")
    B = 3
    A, Z = _twins(w, d, 0)
    rng = np.random.default_rng(103)
    x = torch.zeros(B, w.dim, device="cuda")
    lens = dev_tensor(d["lens"][:B])
    wa = A.new_wire()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("qkv + attention graph replays")
    with torch.cuda.stream(s):
        A.step(tp.TP_STAGE_ATTN, x, lens, B, wa)  # eager pass before capture
    torch.cuda.synchronize()
    wz = Z.new_wire()
    Z.step_noalloc(tp.TP_STAGE_ATTN, x, lens, B, wz)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        A.step(tp.TP_STAGE_ATTN, x, lens, B, wa)
    n = _wire_bytes(w, A.cfg, B)
    for rep in range(4):
        x.copy_(torch.from_numpy(rng.standard_normal((B, w.dim)).astype(np.float32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        Z.step_noalloc(tp.TP_STAGE_ATTN, x, lens, B, wz)
        torch.cuda.synchronize()
        assert _same(wa[:n], wz[:n]), f"replay {rep}: wire differs from the separate launches"
        assert _same(A.k_cache, Z.k_cache) and _same(A.v_cache, Z.v_cache), f"replay {rep}: caches"
        torch.zeros(1000, device="cuda").sum().item()  # eager work between replays
    assert tp.read_error_word(A.handle) == 0


def test_handoff_wait_runs_out_sets_the_error_word():
    """The bounded wait's error path, forced from the host (tp_handoff_test):
    the waiting workgroups look for a tag no word carries, with a 20 us limit.
    The launch ends, TP_DERR_HANDOFF is set; with the normal settings back, the
    next call equals the separate launches again (the same cache slot is
    written by both shards)."""
    import torch
    w, d, _ = _layer("mha_bf16")
    A, Z = _twins(w, d, 0)
    B = 2
    x = dev_tensor(np.random.default_rng(105).standard_normal((B, w.dim)).astype(np.float32))
    lens = dev_tensor(d["lens"][:B])
    say("qkv + attention: hand-off waits forced to run out")
    tp.handoff_test(A.handle, 2000, 0x40000000)
    A.step(tp.TP_STAGE_ATTN, x, lens, B, A.new_wire())
    torch.cuda.synchronize()
    assert tp.read_error_word(A.handle) == tp.TP_DERR_HANDOFF
    tp.handoff_test(A.handle, 0, 0)
    wa, wz = A.new_wire(), Z.new_wire()
    A.step(tp.TP_STAGE_ATTN, x, lens, B, wa)
    Z.step_noalloc(tp.TP_STAGE_ATTN, x, lens, B, wz)
    torch.cuda.synchronize()
    n = _wire_bytes(w, A.cfg, B)
    assert _same(wa[:n], wz[:n])
    assert _same(A.k_cache, Z.k_cache) and _same(A.v_cache, Z.v_cache)
    assert tp.read_error_word(A.handle) == 0


def test_fused_at_the_7b_shape_batch4_grid_beyond_residency():
    """The 7B shard's shape (dim 4096, 8 of 32 heads, 2048 cached positions)
    at batch 4: the one-launch grid (768 projection, 1056 attention and 32
    combine workgroups) no longer fits on the GPU at once, so waiting
    workgroups are resident while later producers wait for slots. Rank 0,
    three calls in a row, bitwise against the separate launches."""
    import dataclasses
    import torch
    w = dataclasses.replace(synth.L7B, name="qkv_attn_7b_b4", batch=4, past=(1500, 2048), seed=106)
    d = synth.llama_inputs(w)
    d["lens"] = np.array([2047, 1500, 1983, 1600], np.int32)
    d["kcache"] = synth.llama_kv_cache(w, d["lens"] + 1, "kcache")
    d["vcache"] = synth.llama_kv_cache(w, d["lens"] + 1, "vcache")
    A, Z = _twins(w, d, 0)
    rng = np.random.default_rng(107)
    say("qkv + attention at the 7B shape, batch 4")
    for call in range(3):
        B = 4
        x = dev_tensor(rng.standard_normal((B, w.dim)).astype(np.float32))
        lens = dev_tensor(np.minimum(d["lens"] + call, w.max_ctx - 1).astype(np.int32))
        wa, wz = A.new_wire(), Z.new_wire()
        ta, tz = _taps(w, B), _taps(w, B)
        A.step(tp.TP_STAGE_ATTN, x, lens, B, wa, ta)
        Z.step_noalloc(tp.TP_STAGE_ATTN, x, lens, B, wz, tz)
        torch.cuda.synchronize()
        n = _wire_bytes(w, A.cfg, B)
        assert _same(wa[:n], wz[:n]), f"call {call}: wires differ"
        for k in ta:
            assert _same(ta[k], tz[k]), f"call {call}: tap {k} differs"
        assert _same(A.k_cache, Z.k_cache) and _same(A.v_cache, Z.v_cache), f"call {call}: caches"
    assert tp.read_error_word(A.handle) == 0
