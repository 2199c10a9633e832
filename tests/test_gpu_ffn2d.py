"""Parity of the MFMA FFN block (2D weight-stationary PaLM shape) with the
fp64 oracle. The product stores H = silu(X Wg^T) * (X Win^T) in bf16 between
the two GEMMs; the contract tolerance for bf16 paths is relative L2 2e-2 and
these tests hold 5e-3 (bf16 rounding of H alone gives about 1e-3)."""
import sys

import numpy as np
import pytest

import oracle
import synth
import tensor_tp_shard_amd as tp
from conftest import rel_l2

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    tp.lib()


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def run_ffn2d(d, max_batch, batches):
    import torch
    B0, E = d["x"].shape
    F = d["w_gate"].shape[0]
    cfg = tp.make_config(kind=tp.TP_FFN_2D, dim=E, ffn_hidden=F, tp_size=1, tp_rank=0,
                         max_batch=max_batch, w_dtype=tp.TP_BF16)
    sh = tp.Shard(cfg, caches=False)
    W = {"w1": dev(d["w_gate"]), "w3": dev(d["w_in"]), "w2": dev(d["w_out"])}
    sh.load(W)
    x = dev(d["x"])
    outs = []
    for B in batches:
        y = torch.full((B, E), float("nan"), dtype=torch.float32, device="cuda")
        sh.step(tp.TP_STAGE_FFN, x, None, B, y)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    return outs


def test_ffn2d_small_ragged():
    """E = 576, F = 576, 200 rows (one full and one partial 128-row tile), and
    a 5-row call on the same handle."""
    w = synth.Ffn2D("ffn2d_small", e_blk=576, f_blk=576, batch=200, seed=91)
    d = synth.ffn2d_inputs(w)
    say("ffn2d small ragged")
    y200, y5 = run_ffn2d(d, 200, [200, 5])
    ref = oracle.ffn2d(d["x"], d["w_gate"], d["w_in"], d["w_out"])
    assert np.all(np.isfinite(y200))
    e = rel_l2(y200, ref)
    say(f"ffn2d small rel-L2 {e:.3e}")
    assert e <= TOL
    assert rel_l2(y5, ref[:5]) <= TOL


def _sampled_rows_check(w, rows):
    d = synth.ffn2d_inputs(w)
    say(f"{w.name} B={w.batch}")
    (y,) = run_ffn2d(d, w.batch, [w.batch])
    assert np.all(np.isfinite(y))
    for r in rows:
        ref = oracle.ffn2d(d["x"], d["w_gate"], d["w_in"], d["w_out"], row0=r, nrows=1)
        e = rel_l2(y[r], ref[0])
        assert e <= TOL, f"row {r} rel-L2 {e:.3e}"
    return y


def test_palm_ffn2d_decode_512_sampled_rows():
    """512 tokens: the down-projection splits K 4 ways and maps one split and
    half the N-tiles to each XCD; 128 rows (one in every 4, at every residue
    mod 16, so every lane row of the 16-row MFMA tiles and every 64-row M-tile;
    each row covers every N-tile and split) plus tile edges."""
    rows = sorted({0, 1, 63, 64, 127, 128, 300, 511} | {64 * t + 17 for t in range(8)}
                  | {4 * i + (i // 4) % 4 for i in range(128)})
    y = _sampled_rows_check(synth.PALM_DEC, rows)
    # deterministic: a second run is bitwise equal
    d = synth.ffn2d_inputs(synth.PALM_DEC)
    (y2,) = run_ffn2d(d, 512, [512])
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_palm_ffn2d_prefill_8192_sampled_rows():
    """8192 tokens: the one-split down-projection gives each XCD 1/8 of the
    256-row M-tiles with every N-tile; a row in every M-tile, and 128 rows
    spread over every 64-row quarter of them at varying offsets."""
    _sampled_rows_check(synth.PALM_PRE, sorted({0, 4095, 8191} | {256 * t + 101 for t in range(32)}
                                               | {64 * i + (5 * i) % 64 for i in range(128)}))


def test_palm_ffn2d_weight_gathered_sampled_rows():
    """The weight-gathered prefill share (E = F' = 18432, 18432 tokens): the
    same kernels at a 37.6 TFLOP shape; rows at 256-row tile edges and four
    more inside tiles across the batch."""
    _sampled_rows_check(synth.PALM_GATHERED, [0, 255, 256, 4711, 9300, 13057, 16421, 18431])


@pytest.mark.parametrize("B,tile", [(2100, 128), (4100, 256)])
def test_ffn2d_large_batch_tiles_and_ragged_tail(B, tile):
    """Large batches: 2100 rows on the 128-row tiles with 32 K values per
    stage, 4100 rows on the 256-row tiles of 8 waves; rows at tile edges and
    the whole ragged tail against the oracle."""
    w = synth.Ffn2D(f"ffn2d_big{B}", e_blk=576, f_blk=1152, batch=B, seed=92)
    full = B // tile * tile
    rows = sorted({0, 1, tile - 1, tile, 2 * tile - 1, full - tile, full - 1} | set(range(full, B)))
    _sampled_rows_check(w, rows)


def test_palm_ffn2d_split_k_across_calls():
    """The split-K down-projection on one handle over calls of 512, 130, 512
    and 64 rows (4, 8, 4 and 8 splits sharing the partials buffer), each on
    new inputs (the token rows rolled): every call's sampled rows against the
    oracle (a partial left from an earlier call would show), the two 512-row
    calls on the same inputs bitwise equal."""
    import torch
    w = synth.PALM_DEC
    d = synth.ffn2d_inputs(w)
    E = d["x"].shape[1]
    F = d["w_gate"].shape[0]
    cfg = tp.make_config(kind=tp.TP_FFN_2D, dim=E, ffn_hidden=F, tp_size=1, tp_rank=0,
                         max_batch=w.batch, w_dtype=tp.TP_BF16)
    sh = tp.Shard(cfg, caches=False)
    sh.load({"w1": dev(d["w_gate"]), "w3": dev(d["w_in"]), "w2": dev(d["w_out"])})
    outs = {}
    for call, (B, shift) in enumerate([(512, 0), (130, 37), (512, 0), (64, 301)]):
        xs = np.roll(d["x"], shift, axis=0)[:B]
        say(f"ffn2d split-K: call {call}, {B} rows, roll {shift}")
        y = torch.full((B, E), float("nan"), dtype=torch.float32, device="cuda")
        sh.step(tp.TP_STAGE_FFN, dev(xs), None, B, y)
        torch.cuda.synchronize()
        y = y.cpu().numpy()
        assert np.all(np.isfinite(y))
        for r in sorted({0, 1, 63, B - 1} | {64 * t + 17 for t in range(B // 64)}):
            ref = oracle.ffn2d(xs, d["w_gate"], d["w_in"], d["w_out"], row0=r, nrows=1)
            e = rel_l2(y[r], ref[0])
            assert e <= TOL, f"call {call} row {r} rel-L2 {e:.3e}"
        outs.setdefault(B, []).append(y)
    assert np.array_equal(outs[512][0].view(np.uint32), outs[512][1].view(np.uint32))


def test_palm_ffn2d_graph_replays_match_eager():
    """The 512-token block (up-projection, 4-way split-K down-projection and
    its reduce) captured once and replayed three times with new inputs copied
    in between and the program's own eager work after each: every replay
    bitwise equal to an eager step on the same inputs."""
    import torch
    w = synth.PALM_DEC
    d = synth.ffn2d_inputs(w)
    B, E = d["x"].shape
    F = d["w_gate"].shape[0]
    cfg = tp.make_config(kind=tp.TP_FFN_2D, dim=E, ffn_hidden=F, tp_size=1, tp_rank=0,
                         max_batch=B, w_dtype=tp.TP_BF16)
    sh = tp.Shard(cfg, caches=False)
    sh.load({"w1": dev(d["w_gate"]), "w3": dev(d["w_in"]), "w2": dev(d["w_out"])})
    x = dev(d["x"])
    y = torch.empty((B, E), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("ffn2d graph replays")
    with torch.cuda.stream(s):
        sh.step(tp.TP_STAGE_FFN, x, None, B, y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        sh.step(tp.TP_STAGE_FFN, x, None, B, y)
    for rep, shift in enumerate((0, 101, 333)):
        x.copy_(dev(np.roll(d["x"], shift, axis=0)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.cpu().numpy().copy()
        ref = torch.empty_like(y)
        sh.step(tp.TP_STAGE_FFN, x, None, B, ref)
        torch.cuda.synchronize()
        assert np.array_equal(got.view(np.uint32), ref.cpu().numpy().view(np.uint32)), f"replay {rep}"
        torch.zeros(1000, device="cuda").sum().item()  # eager work between replays
