"""GPU parity of batch-sharded attention (every head of a shard's sequences)
and of the all-to-alls around it, against the fp64 oracle, through the C ABI.

Bars: the all-to-alls and the cache slots other than the appended one
bit-exact; attention outputs within rel-L2 1e-4 (fp32 cache) or 1e-3 (bf16
cache); the appended K/V within the same bound (bf16: the same rounding of
values that differ only by the fp32-vs-fp64 RoPE)."""
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

import tensor_tp_shard_amd as tp  # noqa: E402
from gpu_harness import AttnBatchShard, dev_tensor, to_np  # noqa: E402


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _tol(w):
    return 1e-4 if w.kv_dtype == synth.F32 else 1e-3


def _widen(w, a):
    return synth.bf16_bits_to_f32(a) if w.kv_dtype == synth.BF16 else a


def check_shard(w, d, r, batch=None):
    nb = w.batch // w.tp
    B = nb if batch is None else batch
    rows = slice(r * nb, r * nb + B)
    say(f"{w.name} shard {r}/{w.tp}: {B} of {nb} sequences, Hq={w.n_heads} Hkv={w.n_kv_heads} "
        f"hd={w.head_dim} kv={w.kv_dtype} lens={d['lens'][rows].tolist()[:4]}")
    sh = AttnBatchShard(w, d, r)
    qkv = dev_tensor(np.ascontiguousarray(d["qkv"][r * nb:(r + 1) * nb]))
    att, taps = sh.run(qkv, B)
    torch.cuda.synchronize()
    kc = np.ascontiguousarray(d["kcache"][rows]).copy()
    vc = np.ascontiguousarray(d["vcache"][rows]).copy()
    ref = oracle.attn_batch_shard(d["qkv"][rows], d["lens"][rows], kc, vc, w.n_heads, w.n_kv_heads,
                                  w.head_dim, w.kv_dtype, w.rope_theta)
    got = to_np(att)
    assert np.all(np.isfinite(got))
    e = rel_l2(got, ref)
    assert e <= _tol(w), f"attention rel-L2 {e:.3e}"
    assert np.array_equal(to_np(taps["att"]).view(np.uint32), got.view(np.uint32))
    gk, gv = sh.cache()
    init_k, init_v = d["kcache"][r * nb:(r + 1) * nb], d["vcache"][r * nb:(r + 1) * nb]
    mask = np.zeros(gk.shape, bool)
    for b in range(B):
        mask[b, :, d["lens"][r * nb + b]] = True
    for got_c, ref_c, init in ((gk, kc, init_k), (gv, vc, init_v)):
        assert np.array_equal(got_c[~mask].view(np.uint8), init[~mask].view(np.uint8))
        ek = rel_l2(_widen(w, got_c[:B][mask[:B]]), _widen(w, ref_c[mask[:B]]))
        assert ek <= _tol(w), f"appended cache rel-L2 {ek:.3e}"
    say(f"{w.name} shard {r}: attention rel-L2 {e:.3e}")


def _small(kv, T=2, B=4, hd=64, Hq=8, Hkv=2, past=(0, 64), seed=2201):
    return synth.AttnBatch(f"attn_batch_T{T}_B{B}_{kv}", n_heads=Hq, n_kv_heads=Hkv, head_dim=hd, tp=T,
                           batch=B, past=past, kv_dtype=kv, seed=seed)


@pytest.mark.parametrize("kv", [synth.F32, synth.BF16])
def test_batch_shards_small(kv):
    w = _small(kv)
    d = synth.attn_batch_inputs(w)
    for r in range(w.tp):
        check_shard(w, d, r)


def test_batch_shard_fewer_rows_than_planned():
    w = _small(synth.BF16, T=2, B=8, seed=2202)
    check_shard(w, synth.attn_batch_inputs(w), 1, batch=2)


def test_llama70b_tp16_batch_shards():
    """Llama-2-70B attention at TP = 16: one sequence per shard with all 64 q
    and 8 kv heads, up to 4096 cached positions (bf16 cache)."""
    w = synth.L70B_ATTN_BATCH
    d = synth.attn_batch_inputs(w)
    for r in (0, 9, 15):
        check_shard(w, d, r)


@pytest.mark.parametrize("kv", [synth.BF16])   # an fp32 K/V chunk of hd 128 exceeds the LDS rule
def test_llama7b_mha_batch_shard(kv):
    """Llama-2-7B attention (MHA: one q head per kv head, the vector-FMA
    attention kernel) sharded by sequence at TP = 4: one sequence per shard
    with all 32 heads, 2048 cached positions."""
    w = synth.AttnBatch(f"llama2_7b_tp4_attn_batch_b4_{kv}", n_heads=32, n_kv_heads=32, head_dim=128,
                        tp=4, batch=4, past=(2048, 2048), kv_dtype=kv, seed=2207)
    d = synth.attn_batch_inputs(w)
    for r in (0, 3):
        check_shard(w, d, r)


@pytest.mark.parametrize("T", [2, 4])
def test_all_to_all_both_directions(T):
    """Heads -> batch into the first columns of wider rows (the attention
    input rows), batch -> heads into padded rows: bitwise placement, other
    columns untouched."""
    Hq, Hkv, hd, B = 8, 2, 32, 8
    w = _small(synth.F32, T=T, B=B, hd=hd, Hq=Hq, Hkv=Hkv, seed=2203)
    C, nb = Hq // T * hd, B // T
    rng = np.random.default_rng(7)
    ld_src = C + 4
    heads = rng.standard_normal((T, B, ld_src)).astype(np.float32)   # head-sharded q rows, padded
    ld_q = (Hq + 2 * Hkv) * hd
    bsrc = rng.standard_normal((T, nb, Hq * hd + 8)).astype(np.float32)  # batch-sharded outputs, padded
    for r in range(T):
        say(f"all-to-all T={T} r={r}")
        sh = tp.Shard(__import__("gpu_harness").attn_batch_config(w, r), caches=False)
        srcs = [dev_tensor(heads[i]) for i in range(T)]
        dst = torch.full((nb, ld_q), -7.0, device="cuda")
        tp.all_to_all(sh.handle, tp.TP_A2A_HEADS_TO_BATCH, srcs, ld_src, dst, ld_q)
        got = to_np(dst)
        want = oracle.a2a_heads_to_batch(heads[:, :, :C], r)
        assert np.array_equal(got[:, :T * C], want.astype(np.float32))
        assert np.all(got[:, T * C:] == -7.0)
        srcs2 = [dev_tensor(bsrc[i]) for i in range(T)]
        dst2 = torch.full((B, C + 8), -7.0, device="cuda")
        tp.all_to_all(sh.handle, tp.TP_A2A_BATCH_TO_HEADS, srcs2, Hq * hd + 8, dst2, C + 8)
        got2 = to_np(dst2)
        want2 = oracle.a2a_batch_to_heads(bsrc[:, :, :Hq * hd], r)
        assert np.array_equal(got2[:, :C], want2.astype(np.float32))
        assert np.all(got2[:, C:] == -7.0)
        sh.close()


def test_heads_to_batch_attention_and_back():
    """The whole re-sharded attention on T = 2: each head shard's raw q rows
    go through the all-to-all into the batch shards' input rows (their k / v
    columns filled with the shard's own rows), every batch shard attends, and
    the outputs come back to head-sharded rows; against the oracle's
    batch-shard attention and all-to-alls."""
    w = _small(synth.BF16, T=2, B=4, seed=2204)
    d = synth.attn_batch_inputs(w)
    T, nb, hd = w.tp, w.batch // w.tp, w.head_dim
    C, Hq, Hkv = w.n_heads // T * hd, w.n_heads, w.n_kv_heads
    qh = [dev_tensor(np.ascontiguousarray(d["qkv"][:, i * C:(i + 1) * C])) for i in range(T)]
    shards = [AttnBatchShard(w, d, r) for r in range(T)]
    outs = []
    for r, sh in enumerate(shards):
        rows = d["qkv"][r * nb:(r + 1) * nb].copy()
        rows[:, :Hq * hd] = -7.0   # the queries must come from the all-to-all
        x = dev_tensor(rows)
        tp.all_to_all(sh.sh.handle, tp.TP_A2A_HEADS_TO_BATCH, qh, C, x, (Hq + 2 * Hkv) * hd)
        att, _ = sh.run(x, taps=False)
        outs.append(att)
    back = []
    for r, sh in enumerate(shards):
        dst = torch.empty((w.batch, C), device="cuda")
        tp.all_to_all(sh.sh.handle, tp.TP_A2A_BATCH_TO_HEADS, outs, Hq * hd, dst, C)
        back.append(to_np(dst))
    ref_b = []
    for r in range(T):
        rows = slice(r * nb, (r + 1) * nb)
        ref_b.append(oracle.attn_batch_shard(d["qkv"][rows], d["lens"][rows], d["kcache"][rows].copy(),
                                             d["vcache"][rows].copy(), Hq, Hkv, hd, w.kv_dtype))
    for r in range(T):
        want = oracle.a2a_batch_to_heads(np.stack(ref_b), r)
        e = rel_l2(back[r], want)
        say(f"re-sharded attention, head shard {r}: rel-L2 {e:.3e}")
        assert e <= 1e-3


def test_bad_length_sets_error_word_and_skips_sequence():
    w = _small(synth.BF16, T=2, B=4, seed=2205)
    d = synth.attn_batch_inputs(w)
    say("batch-sharded attention: error word")
    d["lens"] = d["lens"].copy()
    d["lens"][3] = w.max_ctx          # shard 1's second sequence
    sh = AttnBatchShard(w, d, 1)
    att, _ = sh.run(dev_tensor(np.ascontiguousarray(d["qkv"][2:4])), taps=False)
    torch.cuda.synchronize()
    assert tp.read_error_word(sh.sh.handle) == tp.TP_DERR_LEN
    got = to_np(att)
    assert np.all(got[1] == 0)
    kc = d["kcache"][2:3].copy()
    vc = d["vcache"][2:3].copy()
    ref = oracle.attn_batch_shard(d["qkv"][2:3], d["lens"][2:3], kc, vc, w.n_heads, w.n_kv_heads,
                                  w.head_dim, w.kv_dtype)
    assert rel_l2(got[0], ref[0]) <= 1e-3
    assert tp.read_error_word(sh.sh.handle) == 0   # read clears


def test_graph_replay_of_the_resharded_attention():
    """All-to-all in, attention, all-to-all out captured in a HIP graph:
    every replay (with eager work between them) is bitwise the eager result."""
    w = _small(synth.BF16, T=2, B=4, seed=2206)
    d = synth.attn_batch_inputs(w)
    T, nb, hd = w.tp, w.batch // w.tp, w.head_dim
    C, Hq, Hkv = w.n_heads // T * hd, w.n_heads, w.n_kv_heads
    say("batch-sharded attention: graph replay")
    qh = [dev_tensor(np.ascontiguousarray(d["qkv"][:, i * C:(i + 1) * C])) for i in range(T)]
    shards = [AttnBatchShard(w, d, r) for r in range(T)]
    xs = [dev_tensor(np.ascontiguousarray(d["qkv"][r * nb:(r + 1) * nb])) for r in range(T)]
    atts = [torch.empty((nb, Hq * hd), device="cuda") for _ in range(T)]
    back = torch.empty((w.batch, C), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def step():
        for r, sh in enumerate(shards):
            tp.all_to_all(sh.sh.handle, tp.TP_A2A_HEADS_TO_BATCH, qh, C, xs[r], (Hq + 2 * Hkv) * hd)
            sh.sh.step(tp.TP_STAGE_ATTN, xs[r], sh.lens, nb, atts[r])
        tp.all_to_all(shards[0].sh.handle, tp.TP_A2A_BATCH_TO_HEADS, atts, Hq * hd, back, C)

    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    eager = to_np(back).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_np(back).view(np.uint32), eager.view(np.uint32))
        torch.zeros(1000, device="cuda").sum().item()  # eager work between replays
