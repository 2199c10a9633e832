"""Drives the HIP library through its C ABI (via the ctypes binding) for the
GPU parity tests and the benchmark: uploads seeded synthetic inputs, runs
every shard of a layer in turn on one GPU, merges on the device and brings
the results back as numpy arrays. Imports nothing from oracle/."""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

import synth
import tensor_tp_shard_amd as tp


def torch():
    import torch as _t
    return _t


def dev_tensor(a: np.ndarray, bf16: bool = False):
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16)).view(t.bfloat16).cuda()
    return t.from_numpy(a).cuda()


def to_np(t) -> np.ndarray:
    tt = torch()
    t = t.detach()
    if t.dtype == tt.bfloat16:
        return t.view(tt.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def config_of(w, rank: int = 0, max_batch: Optional[int] = None) -> tp.TpConfig:
    dt = {synth.F32: tp.TP_F32, synth.BF16: tp.TP_BF16}
    return tp.make_config(kind=tp.TP_LLAMA_BLOCK, dim=w.dim, n_heads=w.n_heads,
                          n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn_hidden=w.ffn_hidden,
                          tp_size=w.tp, tp_rank=rank, max_batch=max_batch or w.batch,
                          max_ctx=w.max_ctx, w_dtype=dt[w.w_dtype], kv_dtype=dt[w.kv_dtype],
                          quant=w.quant, quant_block=32, rope_theta=w.rope_theta,
                          norm_eps=w.norm_eps)


def shard_cache(w, full_cache: np.ndarray, rank: int) -> np.ndarray:
    """The shard's slice [B][Hkv_s][max_ctx][hd] of a full cache."""
    hs = w.n_kv_heads // w.tp
    return np.ascontiguousarray(full_cache[:, rank * hs:(rank + 1) * hs])


class Layer:
    """All T shards of one layer on the GPU, with their caches."""

    def __init__(self, w, d: Dict[str, np.ndarray], ranks: Optional[List[int]] = None):
        self.w = w
        self.ranks = list(range(w.tp)) if ranks is None else ranks
        self.dw = {k: dev_tensor(d[k]) for k in ("wq", "wk", "wv", "wo", "w1", "w3", "w2",
                                                 "g_att", "g_ffn")}
        self.shards = {}
        for r in self.ranks:
            sh = tp.Shard(config_of(w, r), caches=False)
            kc = dev_tensor(shard_cache(w, d["kcache"], r)).reshape(-1)
            vc = dev_tensor(shard_cache(w, d["vcache"], r)).reshape(-1)
            sh.load(self.dw, k_cache=kc, v_cache=vc)
            self.shards[r] = sh
        torch().cuda.synchronize()

    def taps(self, stage: int, B: int) -> Dict[str, object]:
        t = torch()
        w = self.w
        hd, T = w.head_dim, w.tp
        f = lambda *s: t.full(s, float("nan"), dtype=t.float32, device="cuda")  # noqa: E731
        if stage == tp.TP_STAGE_ATTN:
            return {"xn": f(B, w.dim), "xq": f(B, w.dim), "q": f(B, w.n_heads // T * hd),
                    "k": f(B, w.n_kv_heads // T * hd), "v": f(B, w.n_kv_heads // T * hd),
                    "att": f(B, w.n_heads // T * hd), "p_pre": f(B, w.dim)}
        return {"xn": f(B, w.dim), "xq": f(B, w.dim), "a": f(B, w.ffn_hidden // T),
                "p_pre": f(B, w.dim)}

    def stage(self, stage: int, x, lens, B: int, with_taps: bool = True):
        """Runs `stage` on every rank; returns (wires, taps) per rank."""
        wires, taps = {}, {}
        for r in self.ranks:
            sh = self.shards[r]
            wires[r] = sh.new_wire()
            taps[r] = self.taps(stage, B) if with_taps else None
            sh.step(stage, x, lens, B, wires[r], taps[r])
        return wires, taps

    def merge(self, stage: int, wires, residual, B: int):
        out = torch().empty_like(residual)
        self.shards[self.ranks[0]].merge(stage, [wires[r] for r in self.ranks], residual, out, B)
        return out

    def run(self, x_np: np.ndarray, lens_np: np.ndarray, with_taps: bool = True):
        """The whole layer step: every shard's attention stage, merge, every
        shard's FFN stage, merge. Returns numpy results."""
        t = torch()
        B = x_np.shape[0]
        x = dev_tensor(np.ascontiguousarray(x_np, dtype=np.float32))
        lens = dev_tensor(np.ascontiguousarray(lens_np, dtype=np.int32))
        wa, ta = self.stage(tp.TP_STAGE_ATTN, x, lens, B, with_taps)
        h = self.merge(tp.TP_STAGE_ATTN, wa, x, B)
        wf, tf = self.stage(tp.TP_STAGE_FFN, h, None, B, with_taps)
        out = self.merge(tp.TP_STAGE_FFN, wf, h, B)
        t.cuda.synchronize()
        res = {"h": to_np(h), "out": to_np(out),
               "wire_att": {r: to_np(v) for r, v in wa.items()},
               "wire_ffn": {r: to_np(v) for r, v in wf.items()}}
        if with_taps:
            res["taps_att"] = {r: {k: to_np(v) for k, v in ta[r].items()} for r in self.ranks}
            res["taps_ffn"] = {r: {k: to_np(v) for k, v in tf[r].items()} for r in self.ranks}
        return res

    def cache(self, rank: int):
        sh = self.shards[rank]
        w = self.w
        shape = (w.batch, w.n_kv_heads // w.tp, w.max_ctx, w.head_dim)
        return to_np(sh.k_cache).reshape(shape), to_np(sh.v_cache).reshape(shape)

    def error_word(self, rank: int) -> int:
        return tp.read_error_word(self.shards[rank].handle)


def split_wire(w, wire: np.ndarray, B: int):
    """(codes int8 [B][D], scales fp32 [B][D/32]) of a quantised wire."""
    D = w.dim
    off = tp.wire_scales_offset(config_of(w), B)
    codes = wire[:B * D].view(np.int8).reshape(B, D)
    scales = wire[off:off + B * (D // 32) * 4].view(np.float32).reshape(B, D // 32)
    return codes, scales


def fp32_wire(w, wire: np.ndarray, B: int) -> np.ndarray:
    return wire[:B * w.dim * 4].view(np.float32).reshape(B, w.dim)


def with_batch(w, B: int):
    return dataclasses.replace(w, batch=B)


def logits_config(w, rank: int = 0, max_batch: Optional[int] = None) -> tp.TpConfig:
    dt = {synth.F32: tp.TP_F32, synth.BF16: tp.TP_BF16}
    return tp.make_config(kind=tp.TP_LOGITS, dim=w.dim, ffn_hidden=w.vocab, tp_size=w.tp,
                          tp_rank=rank, max_batch=max_batch or w.batch, w_dtype=dt[w.w_dtype],
                          quant=w.quant, quant_block=32, norm_eps=w.norm_eps)


class Logits:
    """All T shards of the final stage (final norm + vocabulary-split logits)."""

    def __init__(self, w, d: Dict[str, np.ndarray], max_batch: Optional[int] = None):
        self.w = w
        self.dw = {"w1": dev_tensor(d["w_cls"]), "g_att": dev_tensor(d["g_final"])}
        self.shards = [tp.Shard(logits_config(w, r, max_batch), caches=False) for r in range(w.tp)]
        for sh in self.shards:
            sh.load(self.dw)
        torch().cuda.synchronize()

    def run(self, x_np: np.ndarray, with_taps: bool = True):
        """Every shard's logits stage, then the merge: wires, taps and the
        full logits rows as numpy arrays."""
        t = torch()
        w = self.w
        B, Vs = x_np.shape[0], w.vocab // w.tp
        x = dev_tensor(np.ascontiguousarray(x_np, dtype=np.float32))
        wires, taps = [], []
        for sh in self.shards:
            wires.append(sh.new_wire())
            tap = None
            if with_taps:
                tap = {"xn": t.full((B, w.dim), float("nan"), device="cuda"),
                       "p_pre": t.full((B, Vs), float("nan"), device="cuda")}
            taps.append(tap)
            sh.step(tp.TP_STAGE_LOGITS, x, None, B, wires[-1], tap)
        out = t.full((B, w.vocab), float("nan"), device="cuda")
        self.shards[0].merge_logits(wires, out, B)
        t.cuda.synchronize()
        res = {"out": to_np(out), "wires": [to_np(v) for v in wires]}
        if with_taps:
            res["taps"] = [{k: to_np(v) for k, v in tap.items()} for tap in taps]
        return res


def split_logits_wire(w, wire: np.ndarray, B: int):
    """(codes int8 [B][V/T], scales fp32 [B][V/T/32]) of a quantised logits wire."""
    Vs = w.vocab // w.tp
    off = tp.wire_scales_offset(logits_config(w), B)
    codes = wire[:B * Vs].view(np.int8).reshape(B, Vs)
    scales = wire[off:off + B * (Vs // 32) * 4].view(np.float32).reshape(B, Vs // 32)
    return codes, scales


def attn_batch_config(w, rank: int = 0) -> tp.TpConfig:
    dt = {synth.F32: tp.TP_F32, synth.BF16: tp.TP_BF16}
    return tp.make_config(kind=tp.TP_ATTN_BATCH, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads,
                          head_dim=w.head_dim, tp_size=w.tp, tp_rank=rank, max_batch=w.batch,
                          max_ctx=w.max_ctx, kv_dtype=dt[w.kv_dtype], rope_theta=w.rope_theta)


class AttnBatchShard:
    """One batch shard of sequence-sharded attention with its caches (rows
    [r*B/T, (r+1)*B/T) of the full caches)."""

    def __init__(self, w, d: Dict[str, np.ndarray], rank: int):
        self.w, self.r = w, rank
        self.nb = w.batch // w.tp
        rows = slice(rank * self.nb, (rank + 1) * self.nb)
        self.sh = tp.Shard(attn_batch_config(w, rank), caches=False)
        kc = dev_tensor(np.ascontiguousarray(d["kcache"][rows])).reshape(-1)
        vc = dev_tensor(np.ascontiguousarray(d["vcache"][rows])).reshape(-1)
        self.sh.load({}, k_cache=kc, v_cache=vc)
        self.lens = dev_tensor(np.ascontiguousarray(d["lens"][rows], dtype=np.int32))
        torch().cuda.synchronize()

    def run(self, qkv, batch: Optional[int] = None, taps: bool = True):
        """qkv: device fp32 [nb][(Hq + 2 Hkv) hd] -> (att [batch][Hq hd], taps)."""
        t = torch()
        w = self.w
        B = self.nb if batch is None else batch
        att = t.full((B, w.n_heads * w.head_dim), float("nan"), device="cuda")
        tap = None
        if taps:
            f = lambda *s: t.full(s, float("nan"), device="cuda")  # noqa: E731
            tap = {"q": f(B, w.n_heads * w.head_dim), "k": f(B, w.n_kv_heads * w.head_dim),
                   "v": f(B, w.n_kv_heads * w.head_dim), "att": f(B, w.n_heads * w.head_dim)}
        self.sh.step(tp.TP_STAGE_ATTN, qkv, self.lens, B, att, tap)
        return att, tap

    def cache(self):
        w = self.w
        shape = (self.nb, w.n_kv_heads, w.max_ctx, w.head_dim)
        return to_np(self.sh.k_cache).reshape(shape), to_np(self.sh.v_cache).reshape(shape)


def wire_values(w, wire: np.ndarray, B: int) -> np.ndarray:
    """The values a merge adds for one wire, float32 [B][D]: the fp32 partial,
    or float32(code) * scale per element of an int8 wire (one float32
    multiply, numpy's IEEE rounding)."""
    if not w.quant & synth.Q_PARTIALS:
        return fp32_wire(w, wire, B)
    codes, scales = split_wire(w, wire, B)
    c = codes.reshape(B, -1, 32).astype(np.float32)
    return (c * scales[:, :, None]).reshape(B, w.dim)


def host_merge(residual: np.ndarray, parts) -> np.ndarray:
    """residual + parts[0] + parts[1] + ... in float32, one add per part in
    order: what the merge is defined to produce, bit for bit."""
    acc = np.ascontiguousarray(residual, dtype=np.float32).copy()
    for p in parts:
        acc = acc + np.asarray(p, dtype=np.float32)
    return acc
