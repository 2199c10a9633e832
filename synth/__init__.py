"""Seeded synthetic inputs for the tensor-parallel shard decode step.

This module is shared by the HIP path's tests/bench and by the fp64 oracle.
It holds NO arithmetic of the method itself: it only draws random numbers,
rounds them to the storage types the workloads use (fp32, bf16 bit patterns,
int32 lengths) and fills unused KV-cache slots with NaN canaries.

Recipe (same on every machine that has this numpy):
  * every tensor has its own stream: numpy ``Generator(PCG64(SeedSequence(
    [seed, stream_id])))``; normals are ``standard_normal(dtype=float32)``
    scaled by sigma (and shifted by the mean) in fp32;
  * bf16 tensors are the fp32 draws rounded to nearest-even on the upper
    16 bits (stored as uint16 bit patterns);
  * projection weights ~ N(0, 0.02); RMSNorm gains ~ 1 + N(0, 0.02);
    decode inputs ~ N(0, 1); cached K/V entries ~ N(0, 0.02);
  * per-sequence cached lengths are fixed, or uniform integers in an
    inclusive range [lo, hi] drawn as lo + floor(u * (hi - lo + 1));
  * KV-cache slots at positions > lens[b] hold a quiet-NaN canary, so a read
    beyond the valid range poisons the result; slot lens[b] (where the new
    token is appended) is also a canary before the step.

The workloads are the Llama-style block shapes on the pages' subject
(tensor-parallel decode of Llama-2-7B / 70B, a tiny Llama) and the PaLM-540B
FFN block under 2D weight-stationary partitioning.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

F32 = "f32"
BF16 = "bf16"

Q_NONE = 0
Q_PARTIALS = 1
Q_INPUTS = 2
Q_WEIGHTS = 4

BF16_NAN = np.uint16(0x7FC0)

# stream ids of the tensors (one independent stream per tensor)
STREAMS = {
    "wq": 1, "wk": 2, "wv": 3, "wo": 4, "w1": 5, "w3": 6, "w2": 7,
    "g_att": 8, "g_ffn": 9, "x": 10, "lens": 11, "kcache": 12, "vcache": 13,
    "ffn_x": 20, "ffn_win": 21, "ffn_wgate": 22, "ffn_wout": 23,
    "w_cls": 30, "g_final": 31, "final_x": 32,
    "attn_qkv": 40,
}


@dataclasses.dataclass(frozen=True)
class LlamaBlock:
    """Shape of one Llama-style decoder block split over ``tp`` shards."""
    name: str
    dim: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_hidden: int
    tp: int
    batch: int
    past: Tuple[int, int]          # cached positions per sequence: fixed (a, a) or uniform [lo, hi]
    w_dtype: str
    kv_dtype: str
    quant: int
    seed: int
    rope_theta: float = 10000.0
    norm_eps: float = 1e-5
    kind: str = "llama"

    @property
    def max_ctx(self) -> int:
        return self.past[1] + 1


@dataclasses.dataclass(frozen=True)
class Ffn2D:
    """A PaLM-style FFN block held by one chip under 2D weight-stationary
    partitioning: E_blk x F_blk slices of W_in / W_gate and the transposed
    slice of W_out."""
    name: str
    e_blk: int
    f_blk: int
    batch: int
    seed: int
    kind: str = "ffn2d"


@dataclasses.dataclass(frozen=True)
class LlamaLogits:
    """The final stage of a Llama-style decode step split over ``tp`` shards:
    final RMSNorm and the vocabulary slice V/tp of the classifier per shard."""
    name: str
    dim: int
    vocab: int
    tp: int
    batch: int
    w_dtype: str
    quant: int
    seed: int
    norm_eps: float = 1e-5
    kind: str = "logits"


@dataclasses.dataclass(frozen=True)
class AttnBatch:
    """Attention of one decoder layer sharded by sequence over ``tp`` shards
    (each shard: batch / tp sequences, every head)."""
    name: str
    n_heads: int
    n_kv_heads: int
    head_dim: int
    tp: int
    batch: int
    past: Tuple[int, int]
    kv_dtype: str
    seed: int
    rope_theta: float = 10000.0
    kind: str = "attn_batch"

    @property
    def max_ctx(self) -> int:
        return self.past[1] + 1


@dataclasses.dataclass(frozen=True)
class LlamaDecode:
    """A whole decode step of one TP shard: ``n_layers`` blocks of shape
    ``block`` (each with its own weights and KV cache), then the final stage
    ``logits``."""
    name: str
    block: "LlamaBlock"
    logits: "LlamaLogits"
    n_layers: int
    kind: str = "decode"


WORKLOADS: Dict[str, object] = {}


def _add(w):
    WORKLOADS[w.name] = w
    return w


# tiny Llama block, fp32, 2 shards, 64 cached positions
TINY = _add(LlamaBlock("tiny_llama_tp2_b1", dim=288, n_heads=6, n_kv_heads=6, head_dim=48,
                       ffn_hidden=768, tp=2, batch=1, past=(64, 64), w_dtype=F32, kv_dtype=F32,
                       quant=Q_NONE, seed=1001))
# Llama-2-7B layer, one of 4 shards, bf16 weights/cache, batch 1, 2048 cached positions
L7B = _add(LlamaBlock("llama2_7b_tp4_b1", dim=4096, n_heads=32, n_kv_heads=32, head_dim=128,
                      ffn_hidden=11008, tp=4, batch=1, past=(2048, 2048), w_dtype=BF16,
                      kv_dtype=BF16, quant=Q_NONE, seed=1002))
# same with block-32 int8 exchange of the partials and the normalised inputs
L7B_Q8 = _add(dataclasses.replace(L7B, name="llama2_7b_tp4_b1_q8", quant=Q_PARTIALS | Q_INPUTS,
                                  seed=1003))
# Llama-2-70B GQA layer, one of 8 shards, batch 16, lengths uniform in [1024, 4096]
L70B = _add(LlamaBlock("llama2_70b_tp8_b16", dim=8192, n_heads=64, n_kv_heads=8, head_dim=128,
                       ffn_hidden=28672, tp=8, batch=16, past=(1024, 4096), w_dtype=BF16,
                       kv_dtype=BF16, quant=Q_NONE, seed=1004))
# the 7B and 70B shards with weight-only int8 projections (block-32 codes and
# scales made from the same seeded bf16 weights at load time)
L7B_W8 = _add(dataclasses.replace(L7B, name="llama2_7b_tp4_b1_w8", quant=Q_WEIGHTS, seed=1006))
L70B_W8 = _add(dataclasses.replace(L70B, name="llama2_70b_tp8_b16_w8", quant=Q_WEIGHTS, seed=1007))
# PaLM-540B FFN block of an 8x8 2D weight-stationary grid: E=18432/8, F=73728/8
PALM_DEC = _add(Ffn2D("palm540b_ffn2d_b512", e_blk=2304, f_blk=9216, batch=512, seed=1005))
PALM_PRE = _add(Ffn2D("palm540b_ffn2d_prefill8192", e_blk=2304, f_blk=9216, batch=8192, seed=1005))
# weight-gathered prefill on the same 64 chips: with the weights all-gathered over
# N chips each chip holds an E x (F N / n) block and takes BL / N tokens; at
# BL = F N^2 / n = 294,912 tokens the optimal N = sqrt(BL n / F) is 16, so one
# chip's share is E = 18432, F' = 18432, 18432 tokens
PALM_GATHERED = _add(Ffn2D("palm540b_ffn2d_gathered", e_blk=18432, f_blk=18432, batch=18432, seed=1008))


# final norm + logits of Llama-2 (vocabulary 32000) at the two block shapes
L7B_LOGITS = _add(LlamaLogits("llama2_7b_tp4_logits_b1", dim=4096, vocab=32000, tp=4, batch=1,
                              w_dtype=BF16, quant=Q_NONE, seed=1009))
L7B_LOGITS_Q8 = _add(dataclasses.replace(L7B_LOGITS, name="llama2_7b_tp4_logits_b1_q8",
                                         quant=Q_PARTIALS, seed=1010))
L70B_LOGITS = _add(LlamaLogits("llama2_70b_tp8_logits_b16", dim=8192, vocab=32000, tp=8, batch=16,
                               w_dtype=BF16, quant=Q_NONE, seed=1011))


# Llama-2-70B attention at TP = 16 (more shards than its 8 kv heads), sharded
# by sequence: one sequence of the batch of 16 per shard, all 64 / 8 heads
L70B_ATTN_BATCH = _add(AttnBatch("llama2_70b_tp16_attn_batch_b16", n_heads=64, n_kv_heads=8,
                                 head_dim=128, tp=16, batch=16, past=(1024, 4096), kv_dtype=BF16,
                                 seed=1012))

# whole decode steps: Llama-2 7B (32 layers) and 70B (80 layers)
L7B_DECODE = _add(LlamaDecode("llama2_7b_tp4_decode_b1", L7B, L7B_LOGITS, 32))
L70B_DECODE = _add(LlamaDecode("llama2_70b_tp8_decode_b16", L70B, L70B_LOGITS, 80))


def get(name: str):
    return WORKLOADS[name]


# ---------------------------------------------------------------- primitives

def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def normal_f32(seed: int, stream: int, shape, sigma: float = 1.0, mean: float = 0.0) -> np.ndarray:
    g = _rng(seed, stream)
    a = g.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(sigma)
    if mean:
        a += np.float32(mean)
    return a


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns.
    Finite inputs only (the generator never produces NaN/Inf)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_in = a.reshape(-1).view(np.uint32)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat_in.size, step):
        u = flat_in[i:i + step]
        bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        flat_out[i:i + step] = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (for inspection in tests)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniform_int(seed: int, stream: int, n: int, lo: int, hi: int) -> np.ndarray:
    g = _rng(seed, stream)
    u = g.random(n)
    return (lo + np.floor(u * (hi - lo + 1))).astype(np.int32)


def _typed(a_f32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a_f32) if dtype == BF16 else a_f32


def weight(w, key: str, shape, sigma: float = 0.02, dtype: Optional[str] = None) -> np.ndarray:
    return _typed(normal_f32(w.seed, STREAMS[key], shape, sigma), dtype or w.w_dtype)


# ---------------------------------------------------------------- Llama block inputs

def llama_weights(w: LlamaBlock) -> Dict[str, np.ndarray]:
    """Full (unsharded) layer weights, stored (out, in) row-major."""
    D, hd = w.dim, w.head_dim
    return {
        "wq": weight(w, "wq", (w.n_heads * hd, D)),
        "wk": weight(w, "wk", (w.n_kv_heads * hd, D)),
        "wv": weight(w, "wv", (w.n_kv_heads * hd, D)),
        "wo": weight(w, "wo", (D, w.n_heads * hd)),
        "w1": weight(w, "w1", (w.ffn_hidden, D)),
        "w3": weight(w, "w3", (w.ffn_hidden, D)),
        "w2": weight(w, "w2", (D, w.ffn_hidden)),
        "g_att": normal_f32(w.seed, STREAMS["g_att"], (D,), 0.02, 1.0),
        "g_ffn": normal_f32(w.seed, STREAMS["g_ffn"], (D,), 0.02, 1.0),
    }


def llama_lens(w: LlamaBlock) -> np.ndarray:
    lo, hi = w.past
    if lo == hi:
        return np.full(w.batch, lo, dtype=np.int32)
    return uniform_int(w.seed, STREAMS["lens"], w.batch, lo, hi)


def llama_x(w: LlamaBlock, stream_offset: int = 0) -> np.ndarray:
    return normal_f32(w.seed, STREAMS["x"] + 1000 * stream_offset, (w.batch, w.dim), 1.0)


def llama_kv_cache(w: LlamaBlock, lens: np.ndarray, which: str) -> np.ndarray:
    """Full cache [B][Hkv][max_ctx][hd] in the cache dtype; positions < lens[b]
    hold N(0, 0.02) entries (taken as already rotated), the rest NaN canaries."""
    B, H, C, hd = w.batch, w.n_kv_heads, w.max_ctx, w.head_dim
    vals = normal_f32(w.seed, STREAMS[which], (B, H, C, hd), 0.02)
    pos = np.arange(C)[None, None, :, None]
    dead = pos >= np.asarray(lens).reshape(B, 1, 1, 1)
    if w.kv_dtype == BF16:
        c = f32_to_bf16_bits(vals)
        c[np.broadcast_to(dead, c.shape)] = BF16_NAN
    else:
        c = vals
        c[np.broadcast_to(dead, c.shape)] = np.float32("nan")
    return c


def llama_inputs(w: LlamaBlock) -> Dict[str, np.ndarray]:
    lens = llama_lens(w)
    d = llama_weights(w)
    d["x"] = llama_x(w)
    d["lens"] = lens
    d["kcache"] = llama_kv_cache(w, lens, "kcache")
    d["vcache"] = llama_kv_cache(w, lens, "vcache")
    return d


def logits_inputs(w: LlamaLogits, batch: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Full classifier W_cls [V][D] (N(0, 0.02), w_dtype), final gain g
    (N(1, 0.02)) and the last layer's merged output x [B][D] (N(0, 1))."""
    B = w.batch if batch is None else batch
    return {
        "w_cls": weight(w, "w_cls", (w.vocab, w.dim)),
        "g_final": normal_f32(w.seed, STREAMS["g_final"], (w.dim,), 0.02, 1.0),
        "x": normal_f32(w.seed, STREAMS["final_x"], (B, w.dim), 1.0),
    }


def attn_batch_inputs(w: AttnBatch) -> Dict[str, np.ndarray]:
    """Raw q / k / v rows [B][(Hq + 2 Hkv) hd] of every sequence (N(0, 1)),
    lens and full caches [B][Hkv][max_ctx][hd] as for a Llama block."""
    lens = llama_lens(w)
    return {"qkv": normal_f32(w.seed, STREAMS["attn_qkv"],
                              (w.batch, (w.n_heads + 2 * w.n_kv_heads) * w.head_dim), 1.0),
            "lens": lens, "kcache": llama_kv_cache(w, lens, "kcache"),
            "vcache": llama_kv_cache(w, lens, "vcache")}


# ---------------------------------------------------------------- 2D FFN block inputs

def ffn2d_inputs(w: Ffn2D, batch: Optional[int] = None) -> Dict[str, np.ndarray]:
    """X bf16 [B][E]; W_in, W_gate bf16 [F][E]; W_out bf16 [E][F]."""
    B = w.batch if batch is None else batch
    E, F = w.e_blk, w.f_blk
    return {
        "x": f32_to_bf16_bits(normal_f32(w.seed, STREAMS["ffn_x"] + 17 * B, (B, E), 1.0)),
        "w_in": weight(w, "ffn_win", (F, E), dtype=BF16),
        "w_gate": weight(w, "ffn_wgate", (F, E), dtype=BF16),
        "w_out": weight(w, "ffn_wout", (E, F), dtype=BF16),
    }


def small_llama(name="micro", dim=64, n_heads=4, n_kv_heads=4, head_dim=16, ffn_hidden=128, tp=2,
                batch=1, past=(5, 5), w_dtype=F32, kv_dtype=F32, quant=Q_NONE, seed=7,
                rope_theta=10000.0, norm_eps=1e-5) -> LlamaBlock:
    """Helper for small test shapes."""
    return LlamaBlock(name, dim, n_heads, n_kv_heads, head_dim, ffn_hidden, tp, batch, past,
                      w_dtype, kv_dtype, quant, seed, rope_theta, norm_eps)
