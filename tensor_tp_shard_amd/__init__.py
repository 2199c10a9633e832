"""Python binding of libtpshard (ctypes over include/tpshard.h).

Argument marshalling only: every step of the shard's decode step runs in the
library's HIP kernels. PyTorch supplies device memory (``torch.empty``) and
the stream (``torch.cuda.current_stream()``). The names mirror the C ABI:
``init_shard``, ``load_weights``, ``decode_step``, ``merge_partials``,
``decode_merge_step``, ``merge_logits``, ``destroy_shard``; ``Shard`` bundles a handle with torch-allocated buffers.

There is no fallback: if ``libtpshard.so`` is missing or fails to load,
every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtpshard.so")

TP_F32, TP_BF16 = 0, 1
TP_LLAMA_BLOCK, TP_FFN_2D, TP_LOGITS, TP_ATTN_BATCH = 0, 1, 2, 3
TP_A2A_HEADS_TO_BATCH, TP_A2A_BATCH_TO_HEADS = 0, 1
TP_STAGE_ATTN, TP_STAGE_FFN, TP_STAGE_LOGITS = 0, 1, 2
TP_Q_NONE, TP_Q_PARTIALS, TP_Q_INPUTS, TP_Q_WEIGHTS = 0, 1, 2, 4
TP_OK, TP_EINVAL, TP_EALIGN, TP_ESTATE, TP_ENODEV, TP_EHIP, TP_ENOTIMPL = 0, -1, -2, -3, -4, -5, -6
TP_DERR_LEN = 1
TP_DERR_HANDOFF = 2

# every symbol include/tpshard.h declares
EXPORTS = ("init_shard", "load_weights", "decode_step", "decode_step_noalloc", "merge_partials",
           "decode_merge_step",
           "merge_logits", "tp_all_to_all", "tp_wire_scales_offset",
           "tp_packed_int8_view",
           "tp_read_error_word", "tp_kernel_timing_arm", "tp_kernel_timing_read",
           "tp_kernel_name", "tp_probe_read", "tp_probe_mfma", "destroy_shard", "tp_status_str",
           "tp_last_error", "tp_handoff_test")


class TpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class TpConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kind", "dim", "n_heads", "n_kv_heads", "head_dim", "ffn_hidden", "tp_size", "tp_rank",
        "max_batch", "max_ctx", "w_dtype", "kv_dtype", "quant", "quant_block")] + [
        ("rope_theta", ctypes.c_float), ("norm_eps", ctypes.c_float)]


class TpSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("packed_weights", "kv_cache_each", "workspace",
                                                "wire")]


class TpLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("wq", "wk", "wv", "wo", "w1", "w3", "w2", "g_att",
                                                "g_ffn")]


class TpTaps(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("xn", "q", "k", "v", "att", "a", "p_pre", "xq")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
        L.init_shard.argtypes = [P, P, P]
        L.load_weights.argtypes = [P, P, P, P, P, P, P]
        L.decode_step.argtypes = [P, I32, P, P, I32, P, P, P]
        L.decode_step_noalloc.argtypes = [P, I32, P, P, I32, P, P, P, P]
        L.merge_partials.argtypes = [P, I32, P, I32, P, P, I32, P]
        L.decode_merge_step.argtypes = [P, I32, P, P, I32, P, P, I32, P, P, P]
        L.merge_logits.argtypes = [P, P, I32, P, I32, P]
        L.tp_all_to_all.argtypes = [P, I32, P, I32, ctypes.c_int64, P, ctypes.c_int64, P]
        L.tp_wire_scales_offset.argtypes = [P, I32]
        L.tp_wire_scales_offset.restype = U64
        L.tp_read_error_word.argtypes = [P, P, I32, P]
        L.tp_packed_int8_view.argtypes = [P, I32, P, P, P, P]
        L.tp_kernel_timing_arm.argtypes = [P, I32]
        L.tp_kernel_timing_read.argtypes = [P, P, P]
        L.tp_probe_read.argtypes = [P, U64, P, I32, P]
        L.tp_probe_mfma.argtypes = [I32, I32, P, P]
        L.tp_kernel_name.argtypes = [I32]
        L.tp_handoff_test.argtypes = [P, ctypes.c_uint32, ctypes.c_uint32]
        L.tp_kernel_name.restype = ctypes.c_char_p
        L.destroy_shard.argtypes = [P]
        L.destroy_shard.restype = None
        L.tp_status_str.argtypes = [I32]
        L.tp_status_str.restype = ctypes.c_char_p
        L.tp_last_error.restype = ctypes.c_char_p
        for f in ("init_shard", "load_weights", "decode_step", "decode_step_noalloc", "merge_partials",
                  "decode_merge_step", "merge_logits", "tp_all_to_all", "tp_read_error_word", "tp_kernel_timing_arm", "tp_kernel_timing_read",
                  "tp_packed_int8_view", "tp_probe_read", "tp_probe_mfma"):
            getattr(L, f).restype = I32
        _lib = L
    return _lib


def _check(st: int, what: str):
    if st != TP_OK:
        L = lib()
        raise TpError(st, f"{what}: {L.tp_status_str(st).decode()}: {L.tp_last_error().decode()}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def make_config(kind=TP_LLAMA_BLOCK, dim=0, n_heads=0, n_kv_heads=0, head_dim=0, ffn_hidden=0,
                tp_size=1, tp_rank=0, max_batch=1, max_ctx=1, w_dtype=TP_BF16, kv_dtype=TP_BF16,
                quant=TP_Q_NONE, quant_block=32, rope_theta=10000.0, norm_eps=1e-5) -> TpConfig:
    return TpConfig(kind, dim, n_heads, n_kv_heads, head_dim, ffn_hidden, tp_size, tp_rank,
                    max_batch, max_ctx, w_dtype, kv_dtype, quant, quant_block, rope_theta,
                    norm_eps)


# ---------------------------------------------------------------- C ABI, same names

def init_shard(cfg: TpConfig):
    """-> (handle, TpSizes)."""
    h = ctypes.c_void_p()
    sizes = TpSizes()
    _check(lib().init_shard(ctypes.byref(cfg), ctypes.byref(h), ctypes.byref(sizes)), "init_shard")
    return h, sizes


def load_weights(handle, weights: Dict[str, object], packed, k_cache, v_cache, workspace,
                 stream=None):
    w = TpLayerWeights(**{f: _ptr(weights.get(f)) for f, _ in TpLayerWeights._fields_})
    _check(lib().load_weights(handle, ctypes.byref(w), _ptr(packed), _ptr(k_cache), _ptr(v_cache),
                              _ptr(workspace), _stream(stream)), "load_weights")



def decode_step(handle, stage: int, x, lens, batch: int, wire_out, taps: Optional[dict] = None,
                stream=None):
    t = None
    if taps:
        t = TpTaps(**{k: _ptr(v) for k, v in taps.items()})
    _check(lib().decode_step(handle, stage, _ptr(x), _ptr(lens), batch, _ptr(wire_out),
                             ctypes.byref(t) if t is not None else None, _stream(stream)),
           "decode_step")


def decode_step_noalloc(handle, stage: int, x, lens, batch: int, wire_out,
                        taps: Optional[dict] = None, err_out=None, stream=None):
    t = None
    if taps:
        t = TpTaps(**{k: _ptr(v) for k, v in taps.items()})
    _check(lib().decode_step_noalloc(handle, stage, _ptr(x), _ptr(lens), batch, _ptr(wire_out),
                                     ctypes.byref(t) if t is not None else None, _ptr(err_out),
                                     _stream(stream)), "decode_step_noalloc")


def merge_partials(handle, stage: int, wires: Sequence, residual, out, batch: int, stream=None):
    arr = (ctypes.c_void_p * len(wires))(*[_ptr(w) for w in wires])
    _check(lib().merge_partials(handle, stage, arr, len(wires), _ptr(residual), _ptr(out), batch,
                                _stream(stream)), "merge_partials")


def decode_merge_step(handle, stage: int, x, lens, batch: int, wire_out, wires: Sequence,
                      x_out, taps: Optional[dict] = None, stream=None):
    arr = (ctypes.c_void_p * len(wires))(*[_ptr(w) for w in wires])
    t = None
    if taps:
        t = TpTaps(**{k: _ptr(v) for k, v in taps.items()})
    _check(lib().decode_merge_step(handle, stage, _ptr(x), _ptr(lens), batch, _ptr(wire_out), arr,
                                   len(wires), _ptr(x_out),
                                   ctypes.byref(t) if t is not None else None, _stream(stream)),
           "decode_merge_step")


def merge_logits(handle, wires: Sequence, out, batch: int, stream=None):
    arr = (ctypes.c_void_p * len(wires))(*[_ptr(w) for w in wires])
    _check(lib().merge_logits(handle, arr, len(wires), _ptr(out), batch, _stream(stream)),
           "merge_logits")


def all_to_all(handle, direction: int, srcs: Sequence, ld_src: int, dst, ld_dst: int, stream=None):
    arr = (ctypes.c_void_p * len(srcs))(*[_ptr(w) for w in srcs])
    _check(lib().tp_all_to_all(handle, direction, arr, len(srcs), ld_src, _ptr(dst), ld_dst,
                               _stream(stream)), "tp_all_to_all")


def wire_scales_offset(cfg: TpConfig, batch: int) -> int:
    return int(lib().tp_wire_scales_offset(ctypes.byref(cfg), batch))


def read_error_word(handle, clear: bool = True, stream=None) -> int:
    w = ctypes.c_uint32()
    _check(lib().tp_read_error_word(handle, ctypes.byref(w), 1 if clear else 0, _stream(stream)),
           "tp_read_error_word")
    return w.value


def packed_int8_view(handle, proj: int):
    """(codes byte offset, scales byte offset, rows, cols) of projection proj
    (0 Wqkv, 1 Wo, 2 W13 interleaved, 3 W2) inside the packed weights of a
    shard with int8 weights."""
    co, so = ctypes.c_uint64(), ctypes.c_uint64()
    r, c = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().tp_packed_int8_view(handle, proj, ctypes.byref(co), ctypes.byref(so), ctypes.byref(r),
                                     ctypes.byref(c)), "tp_packed_int8_view")
    return co.value, so.value, r.value, c.value


def kernel_timing_arm(handle, kernel_id: int):
    _check(lib().tp_kernel_timing_arm(handle, kernel_id), "tp_kernel_timing_arm")


def kernel_timing_read(handle):
    """-> (total_ms, launches)"""
    ms, n = ctypes.c_double(), ctypes.c_int32()
    _check(lib().tp_kernel_timing_read(handle, ctypes.byref(ms), ctypes.byref(n)),
           "tp_kernel_timing_read")
    return ms.value, n.value


def handoff_test(handle, wait_ticks: int, tag_xor: int) -> None:
    """Test hook of the one-launch attention's bounded waits (tp_handoff_test)."""
    _check(lib().tp_handoff_test(handle, wait_ticks, tag_xor), "tp_handoff_test")


def kernel_names():
    out, i = [], 0
    while True:
        n = lib().tp_kernel_name(i)
        if n is None:
            return out
        out.append(n.decode())
        i += 1


def probe_read(buf, nbytes: int, out, blocks: int, stream=None):
    """Enqueues the read-stream probe over nbytes of buf (measurement only)."""
    _check(lib().tp_probe_read(_ptr(buf), nbytes, _ptr(out), blocks, _stream(stream)), "tp_probe_read")


def probe_mfma(blocks: int, iters: int, out, stream=None):
    """Enqueues the bf16 MFMA-loop probe (measurement only)."""
    _check(lib().tp_probe_mfma(blocks, iters, _ptr(out), _stream(stream)), "tp_probe_mfma")


def destroy_shard(handle):
    if handle:
        lib().destroy_shard(handle)


# ---------------------------------------------------------------- convenience

class Shard:
    """A shard handle plus torch-allocated device buffers of the sizes
    init_shard asks for (packed weights, K/V caches, workspace)."""

    def __init__(self, cfg: TpConfig, device="cuda", caches: bool = True, workspace: bool = True):
        import torch
        self.cfg = cfg
        self.handle, self.sizes = init_shard(cfg)
        dev = torch.device(device)
        self.packed = torch.empty(self.sizes.packed_weights, dtype=torch.uint8, device=dev)
        # no workspace: the stages run only through decode_step_noalloc
        self.workspace = (torch.empty(self.sizes.workspace, dtype=torch.uint8, device=dev)
                          if workspace else None)
        kvt = torch.bfloat16 if cfg.kv_dtype == TP_BF16 else torch.float32
        self.k_cache = self.v_cache = None
        if caches and self.sizes.kv_cache_each:
            n = self.sizes.kv_cache_each // (2 if cfg.kv_dtype == TP_BF16 else 4)
            self.k_cache = torch.empty(n, dtype=kvt, device=dev)
            self.v_cache = torch.empty(n, dtype=kvt, device=dev)

    def new_wire(self, batch=None):
        import torch
        return torch.empty(self.sizes.wire, dtype=torch.uint8, device=self.packed.device)

    def load(self, weights: Dict[str, object], stream=None, k_cache=None, v_cache=None):
        if k_cache is not None:
            self.k_cache, self.v_cache = k_cache, v_cache
        load_weights(self.handle, weights, self.packed, self.k_cache, self.v_cache, self.workspace,
                     stream)

    def step(self, stage, x, lens, batch, wire_out, taps=None, stream=None):
        decode_step(self.handle, stage, x, lens, batch, wire_out, taps, stream)

    def step_noalloc(self, stage, x, lens, batch, wire_out, taps=None, err_out=None, stream=None):
        decode_step_noalloc(self.handle, stage, x, lens, batch, wire_out, taps, err_out, stream)

    def merge(self, stage, wires, residual, out, batch, stream=None):
        merge_partials(self.handle, stage, wires, residual, out, batch, stream)

    def merge_logits(self, wires, out, batch, stream=None):
        merge_logits(self.handle, wires, out, batch, stream)

    def step_merge(self, stage, x, lens, batch, wire_out, wires, x_out, taps=None, stream=None):
        decode_merge_step(self.handle, stage, x, lens, batch, wire_out, wires, x_out, taps, stream)

    def close(self):
        destroy_shard(self.handle)
        self.handle = None

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                destroy_shard(self.handle)
        except Exception:
            pass
