"""fp64 CPU oracle for the tensor-parallel shard decode step (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``. The product path (the HIP library
and its binding in ``tensor_tp_shard_amd``) never imports it, and this package
imports nothing from the product.

The arithmetic lives in ``oracle.c`` (plain C, fp64, no FMA contraction);
this wrapper only converts numpy arrays to pointers. Each function's page
citation is in ``oracle.c``.

Parity pins: every function here is checked by ``tests/test_oracle_pins.py``
against closed forms, invariants, special cases, hand-worked int8 blocks
(``tests/golden/``) or float64 library routines. The whole layer as a
composition is pinned by identity-weight closed forms and by the sharding
invariance (sum of row-split partials == unsharded block). No page prints a
numeric output for any step, so no value is compared against the pages
themselves.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.environ.get("TP_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

F32, BF16 = 0, 1
Q_PARTIALS, Q_INPUTS, Q_WEIGHTS = 1, 2, 4
QBLOCK = 32

# The same source built with -fopenmp: independent output rows, features and
# heads spread over the host's threads, every sum in the same order (same bits).
LIB_OMP = os.path.join(HERE, "liboracle_omp.so")

_lib = None
_loaded: Dict[str, ctypes.CDLL] = {}


def build(force: bool = False, omp: bool = False) -> str:
    """Compile oracle.c into liboracle.so (liboracle_omp.so with omp) with gcc
    (always when force)."""
    out = LIB_OMP if omp else LIB
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(SRC):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, *(["-fopenmp"] if omp else []), "-o", tmp, SRC, "-lm"])
        os.replace(tmp, out)
    return out


def _load(path: str) -> ctypes.CDLL:
    if path not in _loaded:
        L = ctypes.CDLL(path)
        _declare(L)
        _loaded[path] = L
    return _loaded[path]


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = _load(LIB)
    return _lib


def use_threads(omp: bool) -> int:
    """Route the functions below to the OpenMP build (omp) or the plain one;
    returns the number of threads the chosen build uses."""
    global _lib
    if omp:
        build(omp=True)
    elif not os.path.exists(LIB):
        build()
    _lib = _load(LIB_OMP if omp else LIB)
    return int(_lib.orc_threads())


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_D = ctypes.c_double


class LlamaCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "dim", "n_heads", "n_kv_heads", "head_dim", "ffn_hidden", "tp_size", "batch", "max_ctx",
        "w_dtype", "kv_dtype", "quant", "pad_")] + [("rope_theta", _D), ("norm_eps", _D)]


class LlamaWeights(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("wq", "wk", "wv", "wo", "w1", "w3", "w2", "g_att", "g_ffn")]


class LayerOut(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("xn", "q", "k", "v", "att", "p_att", "codes_att", "scales_att",
                                  "h", "hn", "a", "p_ffn", "codes_ffn", "scales_ffn", "out")]


def _declare(L):
    L.orc_rmsnorm.argtypes = [_I64, _P, _P, _D, _P]
    L.orc_q8_quantize.argtypes = [_I64, _P, _P, _P]
    L.orc_q8_dequantize.argtypes = [_I64, _P, _P, _P]
    L.orc_matvec.argtypes = [_I64, _I64, _P, ctypes.c_int, _I64, _I64, _P, _P]
    L.orc_rope.argtypes = [_I64, _I64, _D, _P]
    L.orc_softmax.argtypes = [_I64, _P, _P]
    L.orc_attend.argtypes = [_I64, _I64, _P, _P, _P, ctypes.c_int, _I64, _P]
    L.orc_silu.argtypes = [_D]
    L.orc_silu.restype = _D
    L.orc_attn_shard.argtypes = [_P, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    L.orc_attn_shard.restype = ctypes.c_int
    L.orc_ffn_shard.argtypes = [_P, _P, _I32, _P, _P, _P, _P]
    L.orc_ffn_shard.restype = ctypes.c_int
    L.orc_wire.argtypes = [_I64, _I64, _I32, _P, _P, _P, _P]
    L.orc_merge.argtypes = [_I64, _I32, _P, _P, _P]
    L.orc_llama_layer.argtypes = [_P, _P, _P, _P, _P, _P, _P]
    L.orc_llama_layer.restype = ctypes.c_int
    L.orc_ffn2d.argtypes = [_I64, _I64, _P, _P, _P, _P, _I64, _I64, _P]
    L.orc_logits_shard.argtypes = [_I64, _I64, _I64, _I32, _I32, _P, ctypes.c_int, _P, _D, _P, _P,
                                   _P]
    L.orc_logits_shard.restype = ctypes.c_int
    L.orc_merge_logits.argtypes = [_I64, _I64, _I32, _P, _P]
    L.orc_attn_batch_shard.argtypes = [_I64, _I64, _I64, _I64, _I64, _D, ctypes.c_int, _P, _P, _P, _P,
                                       _P]
    L.orc_attn_batch_shard.restype = ctypes.c_int
    L.orc_a2a_heads_to_batch.argtypes = [_I64, _I32, _I32, _I64, _P, _P]
    L.orc_a2a_batch_to_heads.argtypes = [_I64, _I32, _I32, _I64, _P, _P]


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _dt(name) -> int:
    return {"f32": F32, "bf16": BF16, F32: F32, BF16: BF16}[name]


def _typed(a: np.ndarray, dt: int) -> np.ndarray:
    want = np.float32 if dt == F32 else np.uint16
    a = np.ascontiguousarray(a)
    assert a.dtype == want, f"expected {want}, got {a.dtype}"
    return a


# ---------------------------------------------------------------- single steps

def rmsnorm(x, g, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float32)
    y = np.empty_like(x)
    lib().orc_rmsnorm(x.size, _ptr(x), _ptr(g), eps, _ptr(y))
    return y


def q8_quantize(x):
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    assert x.size % QBLOCK == 0
    codes = np.empty(x.size, dtype=np.int8)
    scales = np.empty(x.size // QBLOCK, dtype=np.float32)
    lib().orc_q8_quantize(x.size, _ptr(x), _ptr(codes), _ptr(scales))
    return codes, scales


def q8_dequantize(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8).reshape(-1)
    scales = np.ascontiguousarray(scales, dtype=np.float32).reshape(-1)
    assert codes.size == scales.size * QBLOCK
    y = np.empty(codes.size, dtype=np.float32)
    lib().orc_q8_dequantize(codes.size, _ptr(codes), _ptr(scales), _ptr(y))
    return y


def q8_weights(W, dtype="bf16"):
    """Weight-only int8 (CS349E lecture 4, 03_pope_partitioning.py, demo 4:
    int8 weights for the weight-bound small-batch decode). The pages give no
    weight format; the reading taken here: each row of W [N][K] is cut into
    blocks of 32 consecutive k and every block goes through the exchange
    codec above (one fp32 scale, 32 int8 codes). Returns (codes [N][K] int8,
    scales [N][K/32] fp32, dequantised weights [N][K] fp32); the layer stages
    with TP_Q_WEIGHTS use the dequantised weights."""
    dt = _dt(dtype)
    W = _typed(W, dt)
    N, K = W.shape
    assert K % QBLOCK == 0
    f = W if dt == F32 else (W.astype(np.uint32) << 16).view(np.float32)
    codes, scales = q8_quantize(f.reshape(-1))
    deq = q8_dequantize(codes, scales)
    return codes.reshape(N, K), scales.reshape(N, K // QBLOCK), deq.reshape(N, K)


def matvec(W, x, dtype="f32", col0: int = 0, K: Optional[int] = None) -> np.ndarray:
    dt = _dt(dtype)
    W = _typed(W, dt)
    N, ldw = W.shape
    K = ldw - col0 if K is None else K
    x = np.ascontiguousarray(x, dtype=np.float64)
    assert x.size == K
    y = np.empty(N, dtype=np.float64)
    lib().orc_matvec(N, K, _ptr(W), dt, ldw, col0, _ptr(x), _ptr(y))
    return y


def rope(u, pos: int, theta: float = 10000.0) -> np.ndarray:
    u = np.array(u, dtype=np.float64, copy=True)
    lib().orc_rope(u.size, pos, theta, _ptr(u))
    return u


def softmax(s) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float64)
    w = np.empty_like(s)
    lib().orc_softmax(s.size, _ptr(s), _ptr(w))
    return w


def attend(q, K, V, kv_dtype="f32") -> np.ndarray:
    dt = _dt(kv_dtype)
    K, V = _typed(K, dt), _typed(V, dt)
    q = np.ascontiguousarray(q, dtype=np.float64)
    n_pos, hd = K.shape
    assert V.shape == K.shape and q.size == hd
    o = np.empty(hd, dtype=np.float64)
    lib().orc_attend(hd, n_pos, _ptr(q), _ptr(K), _ptr(V), dt, hd, _ptr(o))
    return o


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


# ---------------------------------------------------------------- block stages

def _cfg(w) -> LlamaCfg:
    # int8 weights: the stages see the dequantised fp32 weights (_Weights)
    w8 = bool(w.quant & Q_WEIGHTS)
    return LlamaCfg(dim=w.dim, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                    ffn_hidden=w.ffn_hidden, tp_size=w.tp, batch=w.batch, max_ctx=w.max_ctx,
                    w_dtype=F32 if w8 else _dt(w.w_dtype), kv_dtype=_dt(w.kv_dtype),
                    quant=w.quant & ~Q_WEIGHTS, pad_=0, rope_theta=w.rope_theta, norm_eps=w.norm_eps)


class _Weights:
    def __init__(self, w, weights: Dict[str, np.ndarray]):
        dt = _dt(w.w_dtype)
        names = ("wq", "wk", "wv", "wo", "w1", "w3", "w2")
        if w.quant & Q_WEIGHTS:
            self.keep = {k: q8_weights(weights[k], w.w_dtype)[2] for k in names}
        else:
            self.keep = {k: _typed(weights[k], dt) for k in names}
        self.keep["g_att"] = np.ascontiguousarray(weights["g_att"], dtype=np.float32)
        self.keep["g_ffn"] = np.ascontiguousarray(weights["g_ffn"], dtype=np.float32)
        self.s = LlamaWeights(**{k: _ptr(v) for k, v in self.keep.items()})


def attn_shard(w, weights, s: int, x, lens, kcache, vcache) -> Dict[str, np.ndarray]:
    """Attention stage of shard s. kcache/vcache (full [B][Hkv][max_ctx][hd])
    are updated in place at slot lens[b] of the shard's kv heads."""
    B, D, hd = w.batch, w.dim, w.head_dim
    Hq_s, Hkv_s = w.n_heads // w.tp, w.n_kv_heads // w.tp
    cfg, W = _cfg(w), _Weights(w, weights)
    x = np.ascontiguousarray(x, dtype=np.float64).reshape(B, D)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    kdt = _dt(w.kv_dtype)
    kcache, vcache = _typed(kcache, kdt), _typed(vcache, kdt)
    out = {"xn": np.empty((B, D)), "q": np.empty((B, Hq_s * hd)), "k": np.empty((B, Hkv_s * hd)),
           "v": np.empty((B, Hkv_s * hd)), "att": np.empty((B, Hq_s * hd)), "p": np.empty((B, D))}
    rc = lib().orc_attn_shard(ctypes.byref(cfg), ctypes.byref(W.s), s, _ptr(x), _ptr(lens),
                              _ptr(kcache), _ptr(vcache), *[_ptr(out[k]) for k in
                                                            ("xn", "q", "k", "v", "att", "p")])
    if rc:
        raise ValueError(f"orc_attn_shard rejected the input ({rc})")
    return out


def ffn_shard(w, weights, s: int, h) -> Dict[str, np.ndarray]:
    B, D = w.batch, w.dim
    Fs = w.ffn_hidden // w.tp
    cfg, W = _cfg(w), _Weights(w, weights)
    h = np.ascontiguousarray(h, dtype=np.float64).reshape(B, D)
    out = {"hn": np.empty((B, D)), "a": np.empty((B, Fs)), "p": np.empty((B, D))}
    rc = lib().orc_ffn_shard(ctypes.byref(cfg), ctypes.byref(W.s), s, _ptr(h), _ptr(out["hn"]),
                             _ptr(out["a"]), _ptr(out["p"]))
    if rc:
        raise ValueError(f"orc_ffn_shard rejected the input ({rc})")
    return out


def wire(p, quant: int):
    """-> (d, codes, scales); codes/scales are None without partial quantisation."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    B, D = p.shape
    d = np.empty_like(p)
    codes = np.zeros((B, D), dtype=np.int8)
    scales = np.zeros((B, D // QBLOCK), dtype=np.float32) if D % QBLOCK == 0 else None
    lib().orc_wire(B, D, quant, _ptr(p), _ptr(d), _ptr(codes), _ptr(scales))
    if not quant & Q_PARTIALS:
        return d, None, None
    return d, codes, scales


def merge(residual, parts) -> np.ndarray:
    residual = np.ascontiguousarray(residual, dtype=np.float64)
    parts = np.ascontiguousarray(parts, dtype=np.float64)
    T = parts.shape[0]
    assert parts.shape[1:] == residual.shape
    out = np.empty_like(residual)
    lib().orc_merge(residual.size, T, _ptr(residual), _ptr(parts), _ptr(out))
    return out


def llama_layer(w, weights, x, lens, kcache, vcache) -> Dict[str, np.ndarray]:
    """Whole layer step, every shard in turn. kcache/vcache are updated in place."""
    B, D, hd, T = w.batch, w.dim, w.head_dim, w.tp
    Hq_s, Hkv_s, Fs = w.n_heads // T, w.n_kv_heads // T, w.ffn_hidden // T
    cfg, W = _cfg(w), _Weights(w, weights)
    x = np.ascontiguousarray(x, dtype=np.float64).reshape(B, D)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    kdt = _dt(w.kv_dtype)
    kcache, vcache = _typed(kcache, kdt), _typed(vcache, kdt)
    qz = w.quant & Q_PARTIALS
    o = {
        "xn": np.empty((T, B, D)), "q": np.empty((T, B, Hq_s * hd)),
        "k": np.empty((T, B, Hkv_s * hd)), "v": np.empty((T, B, Hkv_s * hd)),
        "att": np.empty((T, B, Hq_s * hd)), "p_att": np.empty((T, B, D)),
        "codes_att": np.zeros((T, B, D), np.int8) if qz else None,
        "scales_att": np.zeros((T, B, D // QBLOCK), np.float32) if qz else None,
        "h": np.empty((B, D)), "hn": np.empty((T, B, D)), "a": np.empty((T, B, Fs)),
        "p_ffn": np.empty((T, B, D)),
        "codes_ffn": np.zeros((T, B, D), np.int8) if qz else None,
        "scales_ffn": np.zeros((T, B, D // QBLOCK), np.float32) if qz else None,
        "out": np.empty((B, D)),
    }
    lo = LayerOut(**{k: _ptr(v) for k, v in o.items()})
    rc = lib().orc_llama_layer(ctypes.byref(cfg), ctypes.byref(W.s), _ptr(x), _ptr(lens),
                               _ptr(kcache), _ptr(vcache), ctypes.byref(lo))
    if rc:
        raise ValueError(f"orc_llama_layer rejected the input ({rc})")
    return o


def ffn2d(x, w_gate, w_in, w_out, row0: int = 0, nrows: Optional[int] = None) -> np.ndarray:
    """Y[r] for rows [row0, row0+nrows) of X (bf16 bit patterns everywhere)."""
    x, w_gate, w_in, w_out = (_typed(a, BF16) for a in (x, w_gate, w_in, w_out))
    B, E = x.shape
    F = w_gate.shape[0]
    assert w_in.shape == (F, E) and w_out.shape == (E, F)
    nrows = B - row0 if nrows is None else nrows
    assert 0 <= row0 and row0 + nrows <= B
    y = np.empty((nrows, E), dtype=np.float64)
    lib().orc_ffn2d(E, F, _ptr(x), _ptr(w_gate), _ptr(w_in), _ptr(w_out), row0, nrows, _ptr(y))
    return y


# ---------------------------------------------------------------- final stage

def logits_shard(w_cls, g, x, tp: int, s: int, eps: float = 1e-5, dtype="bf16",
                 w8: bool = False) -> Dict[str, np.ndarray]:
    """Final RMSNorm + shard s's vocabulary slice of the logits.
    w_cls [V][D] in dtype (f32 array or bf16 bit patterns), g fp32 [D],
    x [B][D]. With w8 the classifier goes through the int8 weight codec
    first (q8_weights). -> {"xn": [B][D], "z": [B][V/tp]} fp64."""
    dt = _dt(dtype)
    W = _typed(w_cls, dt)
    if w8:
        W, dt = np.ascontiguousarray(q8_weights(W, dtype)[2]), F32
    V, D = W.shape
    g = np.ascontiguousarray(g, dtype=np.float32)
    x = np.ascontiguousarray(x, dtype=np.float64).reshape(-1, D)
    B = x.shape[0]
    assert V % tp == 0
    out = {"xn": np.empty((B, D)), "z": np.empty((B, V // tp))}
    rc = lib().orc_logits_shard(B, D, V, tp, s, _ptr(W), dt, _ptr(g), eps, _ptr(x), _ptr(out["xn"]),
                                _ptr(out["z"]))
    if rc:
        raise ValueError(f"orc_logits_shard rejected the input ({rc})")
    return out


def merge_logits(slices) -> np.ndarray:
    """slices [T][B][Vs] (dequantised wires in shard order) -> [B][T*Vs]."""
    d = np.ascontiguousarray(slices, dtype=np.float64)
    T, B, Vs = d.shape
    out = np.empty((B, T * Vs))
    lib().orc_merge_logits(B, Vs, T, _ptr(d), _ptr(out))
    return out


def logits(w_cls, g, x, tp: int, quant: int = 0, eps: float = 1e-5, dtype="bf16",
           w8: bool = False) -> Dict[str, np.ndarray]:
    """Every shard's logits stage in turn, its wire (int8 with Q_PARTIALS)
    and the merge into full rows. -> {"xn", "z" [T][B][Vs] (before the wire),
    "codes" / "scales" [T][B][...] (None without Q_PARTIALS), "out" [B][V]}."""
    zs, ds, cs, ss, xn = [], [], [], [], None
    for s in range(tp):
        o = logits_shard(w_cls, g, x, tp, s, eps, dtype, w8)
        xn = o["xn"]
        d, c, sc = wire(o["z"], quant)
        zs.append(o["z"]), ds.append(d), cs.append(c), ss.append(sc)
    q = bool(quant & Q_PARTIALS)
    return {"xn": xn, "z": np.stack(zs), "codes": np.stack(cs) if q else None,
            "scales": np.stack(ss) if q else None, "out": merge_logits(np.stack(ds))}


def llama_decode(layers, w_cls, g_final, x, lens, kcaches, vcaches, quant_logits: int = 0,
                 eps: float = 1e-5, cls_dtype="bf16", cls_w8: bool = False) -> Dict[str, np.ndarray]:
    """One decode step of a whole model ([DL] buildLlama2Arch: the layer task
    list once per layer, llamaNextBlock passing each layer's merged output to
    the next, then the final norm, logits and their merge). layers: a list of
    (block description, weights) pairs; kcaches / vcaches: one cache pair per
    layer, updated in place. -> {"h": [L][B][D] layer outputs, "out": [B][V]}."""
    hs = []
    h = np.ascontiguousarray(x, dtype=np.float64)
    for (w, weights), kc, vc in zip(layers, kcaches, vcaches):
        h = llama_layer(w, weights, h, lens, kc, vc)["out"]
        hs.append(h)
    tp = layers[0][0].tp
    lo = logits(w_cls, g_final, h, tp, quant_logits, eps, cls_dtype, cls_w8)
    return {"h": np.stack(hs), "out": lo["out"], "z": lo["z"]}


# ---------------------------------------------------------------- batch-sharded attention

def attn_batch_shard(qkv, lens, kcache, vcache, n_heads: int, n_kv_heads: int, head_dim: int,
                     kv_dtype="bf16", rope_theta: float = 10000.0) -> np.ndarray:
    """One batch shard's attention: qkv [nb][(Hq + 2 Hkv) hd] raw rows of its
    sequences, caches [nb][Hkv][max_ctx][hd] (updated in place at slot
    lens[b]). -> att [nb][Hq hd] fp64."""
    dt = _dt(kv_dtype)
    kcache, vcache = _typed(kcache, dt), _typed(vcache, dt)
    nb, Hkv, C, hd = kcache.shape
    assert Hkv == n_kv_heads and hd == head_dim and vcache.shape == kcache.shape
    qkv = np.ascontiguousarray(qkv, dtype=np.float64).reshape(nb, (n_heads + 2 * Hkv) * hd)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    att = np.empty((nb, n_heads * hd))
    rc = lib().orc_attn_batch_shard(nb, n_heads, Hkv, hd, C, rope_theta, dt, _ptr(qkv), _ptr(lens),
                                    _ptr(kcache), _ptr(vcache), _ptr(att))
    if rc:
        raise ValueError(f"orc_attn_batch_shard rejected the input ({rc})")
    return att


def a2a_heads_to_batch(src, r: int) -> np.ndarray:
    """src [T][B][C] head-sharded rows of every shard -> shard r's [B/T][T C]."""
    src = np.ascontiguousarray(src, dtype=np.float64)
    T, B, C = src.shape
    assert B % T == 0
    dst = np.empty((B // T, T * C))
    lib().orc_a2a_heads_to_batch(B, T, r, C, _ptr(src), _ptr(dst))
    return dst


def a2a_batch_to_heads(src, r: int) -> np.ndarray:
    """src [T][B/T][T C] batch-sharded rows of every shard -> shard r's [B][C]."""
    src = np.ascontiguousarray(src, dtype=np.float64)
    T, nb, TC = src.shape
    assert TC % T == 0
    dst = np.empty((T * nb, TC // T))
    lib().orc_a2a_batch_to_heads(T * nb, T, r, TC // T, _ptr(src), _ptr(dst))
    return dst
