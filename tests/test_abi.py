"""Host-side checks of the C ABI (no GPU needed, no compute calls): the
library loads, exports every function include/tpshard.h declares, and
rejects bad arguments with the documented status before touching a device."""
import ctypes
import os
import re

import pytest

import tensor_tp_shard_amd as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpshard.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[a-z_][\w \*]*?\b(\w+)\s*\([^;{]*\)\s*;", src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12, names
    L = tp.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing
    assert set(names) == set(tp.EXPORTS)


def cfg7b(**kw):
    base = dict(dim=4096, n_heads=32, n_kv_heads=32, head_dim=128, ffn_hidden=11008, tp_size=4,
                tp_rank=0, max_batch=1, max_ctx=2049)
    base.update(kw)
    return tp.make_config(**base)


def test_sizes_of_the_7b_shard():
    h, s = tp.init_shard(cfg7b())
    D, hd = 4096, 128
    weights = (3 * 8 * hd * D + D * 8 * hd + 2 * 2752 * D + D * 2752) * 2
    assert s.packed_weights >= weights and s.packed_weights < weights + 2 * 2049 * 64 * 8 + 8192
    assert s.kv_cache_each == 1 * 8 * 2049 * 128 * 2
    assert s.wire == D * 4
    tp.destroy_shard(h)
    h, s = tp.init_shard(cfg7b(quant=tp.TP_Q_PARTIALS | tp.TP_Q_INPUTS))
    assert s.wire == D + (D // 32) * 4
    assert tp.wire_scales_offset(cfg7b(), 3) == 3 * D
    tp.destroy_shard(h)
    # int8 weights: one byte per weight plus an fp32 scale per 32
    h, s = tp.init_shard(cfg7b(quant=tp.TP_Q_WEIGHTS))
    n_w = weights // 2
    w8 = n_w + n_w // 32 * 4
    assert s.packed_weights >= w8 and s.packed_weights < w8 + 2 * 2049 * 64 * 8 + 8192
    tp.destroy_shard(h)


def test_packed_int8_view():
    h, _ = tp.init_shard(cfg7b())
    with pytest.raises(tp.TpError):
        tp.packed_int8_view(h, 0)  # no int8 weights
    tp.destroy_shard(h)
    h, s = tp.init_shard(cfg7b(quant=tp.TP_Q_WEIGHTS))
    views = [tp.packed_int8_view(h, p) for p in range(4)]
    assert [v[2:] for v in views] == [(3072, 4096), (4096, 1024), (5504, 4096), (4096, 2752)]
    ends = sorted((co, co + r * c) for co, _, r, c in views) + \
        sorted((so, so + r * c // 8) for _, so, r, c in views)
    for (a0, a1), (b0, _) in zip(ends, ends[1:]):
        assert a1 <= b0 and a0 % 256 == 0  # disjoint, 256-byte aligned, codes before scales
    assert ends[-1][1] <= s.packed_weights
    with pytest.raises(tp.TpError):
        tp.packed_int8_view(h, 4)
    tp.destroy_shard(h)


@pytest.mark.parametrize("kw", [
    dict(n_heads=30),                # n_heads % n_kv_heads
    dict(tp_size=3),                 # T does not divide heads
    dict(tp_rank=4),                 # rank outside [0, T)
    dict(head_dim=120),              # not a multiple of 16
    dict(max_batch=0),
    dict(max_batch=17),
    dict(quant=8),                   # unknown bit
    dict(quant=4, ffn_hidden=11072),  # int8 weights: F/T = 2768 not a multiple of 32
    dict(quant=1, quant_block=16),   # block must be 32
    dict(w_dtype=7),
    dict(kind=5),
    dict(n_kv_heads=2, n_heads=32, tp_size=2),  # 16 q heads per kv head
    dict(dim=4100, n_heads=32, quant=1),  # dim % 32 when quantising
])
def test_init_rejects_bad_config(kw):
    with pytest.raises(tp.TpError) as e:
        tp.init_shard(cfg7b(**kw))
    assert e.value.status == tp.TP_EINVAL


def test_order_alignment_and_device_errors():
    h, s = tp.init_shard(tp.make_config(dim=288, n_heads=6, n_kv_heads=6, head_dim=48,
                                        ffn_hidden=768, tp_size=2, max_batch=1, max_ctx=65,
                                        w_dtype=tp.TP_F32, kv_dtype=tp.TP_F32))
    fake = 0x10000  # never dereferenced: every call below fails on the host
    W = {k: fake for k in ("wq", "wk", "wv", "wo", "w1", "w3", "w2", "g_att", "g_ffn")}
    with pytest.raises(tp.TpError) as e:
        tp.decode_step(h, tp.TP_STAGE_ATTN, fake, fake, 1, fake, stream=0)
    assert e.value.status == tp.TP_ESTATE
    with pytest.raises(tp.TpError) as e:
        tp.load_weights(h, W, fake + 4, fake, fake, fake, stream=0)
    assert e.value.status == tp.TP_EALIGN
    W2 = dict(W)
    W2["wo"] = None
    with pytest.raises(tp.TpError) as e:
        tp.load_weights(h, W2, fake, fake, fake, fake, stream=0)
    assert e.value.status == tp.TP_EINVAL
    import torch
    if not torch.cuda.is_available():
        with pytest.raises(tp.TpError) as e:
            tp.load_weights(h, W, fake, fake, fake, fake, stream=0)
        assert e.value.status == tp.TP_ENODEV
    with pytest.raises(tp.TpError) as e:
        tp.merge_partials(h, tp.TP_STAGE_FFN, [], fake, fake, 1, stream=0)
    assert e.value.status == tp.TP_EINVAL
    with pytest.raises(tp.TpError) as e:
        tp.merge_partials(h, tp.TP_STAGE_FFN, [fake] * 65, fake, fake, 1, stream=0)
    assert e.value.status == tp.TP_EINVAL
    with pytest.raises(tp.TpError) as e:
        tp.kernel_timing_arm(h, 99)
    assert e.value.status == tp.TP_EINVAL
    # decode_merge_step: the merge's checks, wire_out exactly once among the
    # wires, x_out not a wire; then the stage's (no weights loaded yet)
    other, own = fake + 0x100000, fake + 0x200000
    dms = tp.decode_merge_step
    with pytest.raises(tp.TpError) as e:
        dms(h, tp.TP_STAGE_FFN, fake, None, 1, own, [], other, stream=0)
    assert e.value.status == tp.TP_EINVAL
    with pytest.raises(tp.TpError) as e:
        dms(h, tp.TP_STAGE_FFN, fake, None, 1, own, [own, fake + 8], other, stream=0)
    assert e.value.status == tp.TP_EALIGN
    with pytest.raises(tp.TpError) as e:
        dms(h, tp.TP_STAGE_FFN, fake, None, 1, own, [other, fake], fake + 0x300000, stream=0)
    assert e.value.status == tp.TP_EINVAL and "not one of the wires" in str(e.value)
    with pytest.raises(tp.TpError) as e:
        dms(h, tp.TP_STAGE_FFN, fake, None, 1, own, [own, other, own], fake, stream=0)
    assert e.value.status == tp.TP_EINVAL and "twice" in str(e.value)
    with pytest.raises(tp.TpError) as e:
        dms(h, tp.TP_STAGE_FFN, fake, None, 1, own, [own, other], other, stream=0)
    assert e.value.status == tp.TP_EINVAL and "aliases wire 1" in str(e.value)
    with pytest.raises(tp.TpError) as e:
        dms(h, tp.TP_STAGE_FFN, fake, None, 2, own, [own, other], fake, stream=0)
    assert e.value.status == tp.TP_EINVAL  # batch above max_batch
    with pytest.raises(tp.TpError) as e:  # x_out may alias x; then: no weights yet
        dms(h, tp.TP_STAGE_FFN, fake, None, 1, own, [own, other], fake, stream=0)
    assert e.value.status == tp.TP_ESTATE
    tp.destroy_shard(h)
    h2, _ = tp.init_shard(tp.make_config(kind=tp.TP_FFN_2D, dim=576, ffn_hidden=576,
                                         max_batch=8, w_dtype=tp.TP_BF16))
    with pytest.raises(tp.TpError) as e:
        dms(h2, tp.TP_STAGE_FFN, fake, None, 1, own, [own], other, stream=0)
    assert e.value.status == tp.TP_EINVAL and "TP_LLAMA_BLOCK" in str(e.value)
    tp.destroy_shard(h2)


def test_null_arguments_and_status_strings():
    L = tp.lib()
    assert L.init_shard(None, None, None) == tp.TP_EINVAL
    assert b"null" in L.tp_last_error()
    assert L.tp_status_str(tp.TP_EALIGN) == b"TP_EALIGN"
    names = tp.kernel_names()
    assert "gemv_w13_swiglu" in names and len(names) == len(set(names))
    L.destroy_shard(None)


def cfg_logits(**kw):
    base = dict(kind=tp.TP_LOGITS, dim=4096, ffn_hidden=32000, tp_size=4, tp_rank=1, max_batch=16,
                w_dtype=tp.TP_BF16, quant=0, quant_block=32)
    base.update(kw)
    return tp.make_config(**base)


def test_logits_shard_sizes_and_wire_layout():
    h, s = tp.init_shard(cfg_logits())
    assert s.kv_cache_each == 0
    assert s.packed_weights >= 8000 * 4096 * 2 + 4096 * 4
    assert s.wire == 16 * 8000 * 4
    tp.destroy_shard(h)
    c = cfg_logits(quant=tp.TP_Q_PARTIALS)
    h, s = tp.init_shard(c)
    assert tp.wire_scales_offset(c, 3) == 3 * 8000  # rows of V/T codes, 16-byte aligned
    assert tp.wire_scales_offset(c, 1) == 8000
    assert s.wire == 16 * 8000 + 16 * 250 * 4
    tp.destroy_shard(h)
    h, s = tp.init_shard(cfg_logits(quant=tp.TP_Q_WEIGHTS))
    co, so, r, cols = tp.packed_int8_view(h, 0)
    assert (r, cols) == (8000, 4096) and co + r * cols <= so and so + r * cols // 8 <= s.packed_weights
    with pytest.raises(tp.TpError):
        tp.packed_int8_view(h, 1)
    tp.destroy_shard(h)


@pytest.mark.parametrize("kw", [
    dict(tp_size=3),                        # T does not divide the vocabulary
    dict(tp_rank=4),
    dict(max_batch=17),
    dict(quant=tp.TP_Q_INPUTS),             # no round trip of the final norm's output
    dict(dim=4100),                         # not a multiple of 8
    dict(ffn_hidden=4 * 8004),              # V/T not a multiple of 8
    dict(ffn_hidden=4 * 8008, quant=tp.TP_Q_PARTIALS),   # V/T not a multiple of 32
    dict(dim=4104, quant=tp.TP_Q_WEIGHTS),  # int8 weights need dim % 32
])
def test_logits_init_rejects_bad_config(kw):
    with pytest.raises(tp.TpError) as e:
        tp.init_shard(cfg_logits(**kw))
    assert e.value.status == tp.TP_EINVAL


def test_logits_stage_and_merge_host_errors():
    h, s = tp.init_shard(cfg_logits(max_batch=2))
    fake = 0x10000  # never dereferenced: every call below fails on the host
    with pytest.raises(tp.TpError) as e:
        tp.decode_step(h, tp.TP_STAGE_LOGITS, fake, None, 1, fake, stream=0)
    assert e.value.status == tp.TP_ESTATE
    with pytest.raises(tp.TpError) as e:
        tp.load_weights(h, {"w1": fake, "g_att": None}, fake, None, None, fake, stream=0)
    assert e.value.status == tp.TP_EINVAL
    with pytest.raises(tp.TpError) as e:
        tp.load_weights(h, {"w1": fake + 8, "g_att": fake}, fake, None, None, fake, stream=0)
    assert e.value.status == tp.TP_EALIGN
    for wires, out, B, st in (([fake] * 3, fake + 4096, 1, tp.TP_EINVAL),   # n_wires != T
                              ([fake] * 4, fake + 4096, 3, tp.TP_EINVAL),   # batch > max_batch
                              ([fake] * 4, fake + 4, 1, tp.TP_EALIGN),
                              ([fake, fake, fake, fake + 4096], fake + 4096, 1, tp.TP_EINVAL),
                              ([fake, None, fake, fake], fake + 4096, 1, tp.TP_EINVAL)):
        with pytest.raises(tp.TpError) as e:
            tp.merge_logits(h, wires, out, B, stream=0)
        assert e.value.status == st
    # the logits stage belongs to TP_LOGITS handles only, and they have no other
    hb, _ = tp.init_shard(cfg7b())
    with pytest.raises(tp.TpError) as e:
        tp.merge_logits(hb, [fake] * 4, fake + 4096, 1, stream=0)
    assert e.value.status == tp.TP_EINVAL
    tp.destroy_shard(hb)
    tp.destroy_shard(h)


def cfg_attn_batch(**kw):
    base = dict(kind=tp.TP_ATTN_BATCH, n_heads=64, n_kv_heads=8, head_dim=128, tp_size=16, tp_rank=3,
                max_batch=16, max_ctx=4097, kv_dtype=tp.TP_BF16)
    base.update(kw)
    return tp.make_config(**base)


def test_attn_batch_shard_sizes():
    h, s = tp.init_shard(cfg_attn_batch())
    assert s.kv_cache_each == 1 * 8 * 4097 * 128 * 2   # one sequence, every kv head
    assert s.wire == 1 * 64 * 128 * 4
    assert s.packed_weights >= 4097 * 64 * 8           # the RoPE table only
    tp.destroy_shard(h)
    h, s = tp.init_shard(cfg_attn_batch(tp_size=4, max_batch=16))
    assert s.kv_cache_each == 4 * 8 * 4097 * 128 * 2
    assert s.wire == 4 * 64 * 128 * 4
    tp.destroy_shard(h)


@pytest.mark.parametrize("kw", [
    dict(max_batch=24),                    # T does not divide the batch
    dict(tp_size=4, max_batch=68),         # more than 16 sequences a shard
    dict(tp_size=128, max_batch=128),      # T does not divide the q heads
    dict(n_heads=60),                      # n_kv_heads does not divide n_heads
    dict(n_kv_heads=4),                    # 16 q heads per kv head
    dict(head_dim=96),
    dict(quant=tp.TP_Q_PARTIALS),
    dict(kv_dtype=7),
])
def test_attn_batch_init_rejects_bad_config(kw):
    with pytest.raises(tp.TpError) as e:
        tp.init_shard(cfg_attn_batch(**kw))
    assert e.value.status == tp.TP_EINVAL


def test_attn_batch_host_errors():
    h, _ = tp.init_shard(cfg_attn_batch(tp_size=2, tp_rank=1, max_batch=4, n_heads=8, n_kv_heads=2, head_dim=64,
                                        max_ctx=65))
    fake = 0x10000  # never dereferenced: every call below fails on the host
    with pytest.raises(tp.TpError) as e:
        tp.decode_step(h, tp.TP_STAGE_ATTN, fake, fake, 1, fake, stream=0)
    assert e.value.status == tp.TP_ESTATE
    with pytest.raises(tp.TpError) as e:
        tp.load_weights(h, {}, fake, None, fake, fake, stream=0)
    assert e.value.status == tp.TP_EINVAL
    C = 4 * 64  # Hq / T * hd
    for d, srcs, ld_s, dst, ld_d, st in (
            (2, [fake] * 2, C, fake + 4096, 2 * C, tp.TP_EINVAL),                      # direction
            (tp.TP_A2A_HEADS_TO_BATCH, [fake] * 3, C, fake + 4096, 2 * C, tp.TP_EINVAL),  # n_srcs != T
            (tp.TP_A2A_HEADS_TO_BATCH, [fake] * 2, C - 4, fake + 4096, 2 * C, tp.TP_EINVAL),
            (tp.TP_A2A_HEADS_TO_BATCH, [fake] * 2, C, fake + 4096, C, tp.TP_EINVAL),   # dst too narrow
            (tp.TP_A2A_BATCH_TO_HEADS, [fake] * 2, C, fake + 4096, C, tp.TP_EINVAL),   # src too narrow
            (tp.TP_A2A_HEADS_TO_BATCH, [fake] * 2, C + 2, fake + 4096, 2 * C, tp.TP_EINVAL),
            (tp.TP_A2A_HEADS_TO_BATCH, [fake] * 2, C, fake + 4100, 2 * C, tp.TP_EALIGN),
            (tp.TP_A2A_HEADS_TO_BATCH, [fake, fake + 4096], C, fake + 4096, 2 * C, tp.TP_EINVAL)):
        with pytest.raises(tp.TpError) as e:
            tp.all_to_all(h, d, srcs, ld_s, dst, ld_d, stream=0)
        assert e.value.status == st
    hl, _ = tp.init_shard(cfg_logits())
    with pytest.raises(tp.TpError) as e:
        tp.all_to_all(hl, tp.TP_A2A_HEADS_TO_BATCH, [fake] * 4, 4096, fake + 4096, 4096, stream=0)
    assert e.value.status == tp.TP_EINVAL
    tp.destroy_shard(hl)
    tp.destroy_shard(h)
