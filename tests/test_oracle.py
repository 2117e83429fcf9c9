"""Pins of the CPU oracle to things other than itself (no GPU).

The oracle follows the definition on the docs.rs source page "onnxruntime-ep-mlx
0.31.1: src/ops/paged_attention.rs" (VECTOR_BODY: head mapping h / (H/KV),
visible window past + (causal ? r + 1 : NQ), block-table address; VECTOR_REDUCE
and PARTIALS_REDUCE: merge of partial states). The pins are:
  * brute force: a dense float64 formulation and torch's SDPA on tiny inputs,
  * closed forms: one key returns v exactly; equal scores return the mean of the
    visible values; two keys give the logistic mix,
  * invariants: physical block order, block size, partitioning and causality
    do not change the result,
  * exact widening of stored binary16 / bfloat16 bit patterns,
  * slot patching: rows stored by the append come back through the block
    table at their logical positions, nothing else in the pools changes, and
    a cached position whose slot is re-written reads the new row (the highest
    j pointing at it) -- against SDPA on the dense problem with that position
    replaced directly,
  * dense GQA forward with masks: torch's SDPA on heads-expanded K/V with the
    mask broadcast, right-padded and causal-limited by the test itself; fully
    masked rows are zero; one visible key returns its value; a per-row additive
    constant changes nothing and an additive -inf equals a boolean False,
  * mutation check: plausible mistakes planted in a copy of the oracle's C
    source each make at least one of these pins fail.
"""
import math
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from tests import problems as P

ORACLE_DIR = os.path.dirname(os.path.abspath(oracle.__file__))


def _ora(w, lib=None, **kw):
    return oracle.paged_decode(*P.args(w), causal=w.spec.causal, lib=lib, **kw)


SWEEP = [
    # (B, H, KV, D, BS, NQ, causal, dtype, lens)
    (1, 4, 2, 64, 16, 1, True, "f32", (100,)),
    (2, 4, 4, 64, 16, 1, True, "f32", (0, 1)),          # MHA, empty and one-token past
    (3, 8, 1, 64, 16, 3, True, "f32", (15, 16, 17)),     # MQA, page boundaries
    (2, 8, 2, 128, 32, 3, False, "f16", (31, 64)),       # non-causal multi-row
    (2, 16, 2, 128, 16, 8, True, "bf16", (0, 33)),       # G = 8, NQ = 8
    (1, 2, 1, 64, 32, 2, True, "bf16", (100,)),
    (2, 4, 2, 128, 16, 1, True, "f16", (1, 48)),
]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: "-".join(map(str, c[:8])))
def test_oracle_matches_dense_and_sdpa(case):
    B, H, KV, D, BS, NQ, causal, dtype, lens = case
    w = P.small(B=B, H=H, KV=KV, D=D, BS=BS, NQ=NQ, causal=causal, dtype=dtype, lens=lens,
                seed=11 + B + NQ)
    ref = _ora(w)
    dense = oracle.dense_reference(*P.args(w), causal=causal)
    sdpa = oracle.sdpa_reference(*P.args(w), causal=causal)
    assert np.abs(ref - dense).max() < 1e-12
    assert np.abs(ref - sdpa).max() < 1e-12


def test_single_key_returns_new_v_exactly():
    # No past and one new row: the only visible key has weight exactly 1.
    w = P.small(B=2, H=8, KV=2, D=64, NQ=1, lens=(0, 0), dtype="bf16")
    out = _ora(w)
    G = w.spec.H // w.spec.KV
    nv = w.new_v.double().numpy()
    for b in range(2):
        for h in range(w.spec.H):
            assert np.array_equal(out[b, h, 0], nv[b, h // G, 0])


def test_causal_row0_without_past_is_new_v0():
    w = P.small(B=1, H=4, KV=2, D=64, NQ=4, causal=True, lens=(0,), dtype="f16")
    out = _ora(w)
    nv = w.new_v.double().numpy()
    for h in range(4):
        assert np.array_equal(out[0, h, 0], nv[0, h // 2, 0])


@pytest.mark.parametrize("causal", [True, False])
def test_equal_scores_give_mean_of_visible_values(causal):
    w = P.small(B=2, H=4, KV=2, D=64, NQ=3, causal=causal, lens=(21, 7), dtype="f32")
    w.q.zero_()
    out = _ora(w)
    for b in range(2):
        for h in range(4):
            for r in range(3):
                _, vs = P.logical_rows(w, b, h // 2, r)
                mean = [sum(col) / len(vs) for col in zip(*vs)]
                assert np.allclose(out[b, h, r], mean, rtol=0, atol=1e-14)


def test_zero_scale_gives_mean():
    w = P.small(B=1, H=2, KV=1, D=64, NQ=2, causal=True, lens=(9,), dtype="f32")
    w.scale = 0.0
    out = _ora(w)
    for r in range(2):
        _, vs = P.logical_rows(w, 0, 0, r)
        mean = [sum(col) / len(vs) for col in zip(*vs)]
        assert np.allclose(out[0, 0, r], mean, rtol=0, atol=1e-14)


def test_two_keys_logistic_mix():
    # One cached key (through the table) and one new key.
    w = P.small(B=1, H=2, KV=1, D=64, NQ=1, lens=(1,), dtype="f32", pool_extra=5)
    out = _ora(w)
    (k0, k1), (v0, v1) = P.logical_rows(w, 0, 0, 0)
    for h in range(2):
        qv = [float(x) for x in w.q[0, h, 0].double()]
        s0 = w.scale * sum(a * b for a, b in zip(qv, k0))
        s1 = w.scale * sum(a * b for a, b in zip(qv, k1))
        a0 = 1.0 / (1.0 + math.exp(s1 - s0))
        a1 = 1.0 / (1.0 + math.exp(s0 - s1))
        expect = [a0 * x + a1 * y for x, y in zip(v0, v1)]
        assert np.allclose(out[0, h, 0], expect, rtol=0, atol=1e-13)


def test_argmax_probe_selects_each_logical_position():
    # Make logical key t dominate: out must equal v_t.
    w = P.small(B=1, H=2, KV=1, D=64, NQ=1, lens=(40,), dtype="f32", pool_extra=4)
    for t in (0, 15, 16, 39):
        w2 = P.relayout(w, shuffle_seed=3 + t)
        phys = int(w2.block_table[0, t // 16])
        q = w2.q[0, 0, 0].clone()
        w2.k_pool[phys, t % 16, 0] = q * 40.0
        out = _ora(w2)
        expect = w2.v_pool[phys, t % 16, 0].double().numpy()
        assert np.allclose(out[0, 0, 0], expect, atol=1e-9)


def test_block_order_and_block_size_do_not_change_the_result():
    w = P.small(B=3, H=8, KV=2, D=64, BS=16, NQ=2, causal=True, lens=(70, 16, 33), dtype="f16")
    base = _ora(w)
    for kw in (dict(shuffle_seed=1), dict(shuffle_seed=2, extra_blocks=5),
               dict(new_bs=32, shuffle_seed=4)):
        w2 = P.relayout(w, **kw)
        assert np.array_equal(_ora(w2), base), kw


def test_unused_pool_space_is_never_read():
    w = P.small(B=2, H=4, KV=2, D=64, BS=16, NQ=1, lens=(45, 3), dtype="bf16")
    w2 = P.relayout(w, shuffle_seed=9, extra_blocks=4, fill=float("nan"))
    out = _ora(w2)
    assert np.isfinite(out).all()
    assert np.array_equal(out, _ora(w))


@pytest.mark.parametrize("chunk", [1, 5, 16, 64, 1000])
def test_partitioned_equals_single_pass(chunk):
    w = P.small(B=2, H=8, KV=2, D=128, BS=16, NQ=3, causal=True, lens=(130, 17), dtype="bf16")
    single = _ora(w)
    part, m, z, o = oracle.paged_decode_partitioned(*P.args(w), chunk=chunk, causal=True,
                                                    want_parts=True)
    assert np.abs(part - single).max() < 1e-12
    # chunk states, merged by hand with weights exp(m_c - M), give the same rows
    for b, h, r in ((0, 0, 0), (1, 7, 2)):
        ok = np.isfinite(m[b, h, r])
        M = m[b, h, r][ok].max()
        wts = np.exp(m[b, h, r][ok] - M)
        merged = (wts[:, None] * o[b, h, r][ok]).sum(0) / (wts * z[b, h, r][ok]).sum()
        assert np.abs(merged - single[b, h, r]).max() < 1e-12


def test_causality_new_rows_after_r_do_not_matter():
    w = P.small(B=1, H=4, KV=2, D=64, NQ=4, causal=True, lens=(10,), dtype="f32")
    base = _ora(w)
    for j in range(1, 4):
        w2 = P.small(B=1, H=4, KV=2, D=64, NQ=4, causal=True, lens=(10,), dtype="f32")
        w2.new_k[0, :, j] += 3.0
        w2.new_v[0, :, j] -= 2.0
        out = _ora(w2)
        assert np.array_equal(out[:, :, :j], base[:, :, :j])
        assert not np.allclose(out[:, :, j:], base[:, :, j:])


def test_non_causal_rows_all_see_every_new_row():
    w = P.small(B=1, H=2, KV=1, D=64, NQ=3, causal=False, lens=(4,), dtype="f32")
    base = _ora(w)
    w.new_v[0, 0, 2] += 1.0
    out = _ora(w)
    assert (np.abs(out - base).reshape(2, 3, -1).max(-1) > 0).all()


def test_widen_is_exact():
    f16 = torch.from_numpy(np.array([0x3C00, 0x0001, 0x7BFF, 0x8400, 0x7C00, 0x3555],
                                    dtype=np.uint16).view(np.int16).copy())
    expect = [1.0, 2.0 ** -24, 65504.0, -(2.0 ** -14), math.inf, 0.333251953125]
    for i, e in enumerate(expect):
        assert oracle.widen(f16.view(torch.float16), i) == e
    u = np.array([0x3F80, 0x0001, 0xC2F7, 0x7F80], dtype=np.uint16).view(np.int16)
    bf = torch.from_numpy(u.copy()).view(torch.bfloat16)
    expect = [1.0, 2.0 ** -133, -123.5, math.inf]
    for i, e in enumerate(expect):
        assert oracle.widen(bf, i) == e
    f32 = torch.tensor([1.5, -2.0 ** -149], dtype=torch.float32)
    assert oracle.widen(f32, 0) == 1.5 and oracle.widen(f32, 1) == -(2.0 ** -149)


def test_rejects_malformed_arguments():
    w = P.small(B=1, H=4, KV=2, D=64, lens=(20,))
    bad = w.context_lens.copy()
    bad[0] = 10 ** 6  # beyond max_blocks * BS
    with pytest.raises(ValueError):
        oracle.paged_decode(w.q, w.k_pool, w.v_pool, w.block_table, bad, w.new_k, w.new_v,
                            w.scale)


# --------------------------------------------------------------------------
# Slot patching: the step's new rows stored into their pool slots
# --------------------------------------------------------------------------
APPEND_CASES = [
    # (B, H, KV, D, BS, NQ, causal, dtype, lens)
    (3, 8, 2, 64, 16, 1, True, "f16", (0, 15, 40)),
    (2, 16, 2, 128, 16, 8, True, "bf16", (5, 33)),
    (2, 4, 1, 64, 32, 3, False, "f32", (31, 64)),
    (2, 6, 3, 64, 16, 4, True, "f32", (16, 47)),
]


def _bits(t: torch.Tensor) -> torch.Tensor:
    """Bit patterns of a tensor (NaN-safe exact comparison)."""
    return t.contiguous().view(torch.int32 if t.element_size() == 4 else torch.int16)


def _dense_with_reads(w, reads, causal):
    """Brute force of the patched step: the dense problem of the cache as
    stored, with cached position p of sequence b replaced by new row j for each
    reads[(b, p)] = j, through torch's SDPA in float64."""
    qd, Kh, Vh, vis = oracle._dense_problem(*P.args(w)[:7], causal)
    G = w.spec.H // w.spec.KV
    nk, nv = w.new_k.cpu().double(), w.new_v.cpu().double()
    for (b, p), j in reads.items():
        Kh[b, :, p] = nk[b, :, j].repeat_interleave(G, dim=0)
        Vh[b, :, p] = nv[b, :, j].repeat_interleave(G, dim=0)
    out = torch.nn.functional.scaled_dot_product_attention(
        qd, Kh, Vh, attn_mask=vis, scale=float(np.float32(w.scale)))
    return out.numpy()


def _append_case(case, **kw):
    B, H, KV, D, BS, NQ, causal, dtype, lens = case
    w = P.small(B=B, H=H, KV=KV, D=D, BS=BS, NQ=NQ, causal=causal, dtype=dtype, lens=lens,
                seed=13 + NQ)
    return P.append_problem(w, **kw)


def _append(w, slots, lib=None):
    return oracle.paged_decode_append(*P.args(w)[:7], slots, w.scale, causal=w.spec.causal,
                                      lib=lib)


@pytest.mark.parametrize("case", APPEND_CASES, ids=lambda c: "-".join(map(str, c[:8])))
def test_append_rows_come_back_through_the_block_table(case):
    w, slots, reads = _append_case(case, seed=3)
    assert not reads
    out, kp, vp = _append(w, slots)
    s = w.spec
    written = np.zeros((w.num_blocks, s.BS), dtype=bool)
    for b, L in enumerate(w.context_lens):
        for j in range(s.NQ):
            i = int(L) + j  # logical position of new row j, read through the table
            phys = int(w.block_table[b, i // s.BS])
            assert torch.equal(_bits(kp[phys, i % s.BS]), _bits(w.new_k[b, :, j]))
            assert torch.equal(_bits(vp[phys, i % s.BS]), _bits(w.new_v[b, :, j]))
            written[phys, i % s.BS] = True
    keep = torch.from_numpy(~written)
    assert torch.equal(_bits(kp)[keep], _bits(w.k_pool)[keep])
    assert torch.equal(_bits(vp)[keep], _bits(w.v_pool)[keep])
    # nothing cached was re-written, so the attention is the plain step's
    assert np.array_equal(out, _ora(w))


@pytest.mark.parametrize("case", APPEND_CASES, ids=lambda c: "-".join(map(str, c[:8])))
def test_overwritten_cached_positions_read_the_new_row(case):
    w, slots, reads = _append_case(case, overwrite=3, duplicate=True, seed=4)
    assert reads
    out, _, _ = _append(w, slots)
    assert np.abs(out - _dense_with_reads(w, reads, w.spec.causal)).max() < 1e-12
    # and differs from the unpatched step
    assert np.abs(out - _ora(w)).max() > 1e-6


def test_negative_and_out_of_range_slots_are_neither_stored_nor_read():
    case = APPEND_CASES[1]
    w, slots, reads = _append_case(case, overwrite=2, negative=3, out_of_range=3, seed=6)
    out, kp, vp = _append(w, slots)
    s = w.spec
    n_slots = w.num_blocks * s.BS
    changed = (_bits(kp) != _bits(w.k_pool)).reshape(n_slots, -1).any(dim=1)
    expect = torch.zeros(n_slots, dtype=torch.bool)
    for b in range(s.B):
        for j in range(s.NQ):
            if 0 <= slots[b, j] < n_slots:
                expect[int(slots[b, j])] = True
    assert torch.equal(changed, expect)
    assert np.abs(out - _dense_with_reads(w, reads, s.causal)).max() < 1e-12


# --------------------------------------------------------------------------
# Dense GQA forward with masks
# --------------------------------------------------------------------------
def _dense_inputs(B, HQ, HK, SQ, SK, D, dtype="f32", seed=0):
    g = torch.Generator().manual_seed(seed)
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    q = torch.randn(B, HQ, SQ, D, generator=g).to(dt)
    k = torch.randn(B, HK, SK, D, generator=g).to(dt)
    v = torch.randn(B, HK, SK, D, generator=g).to(dt)
    return q, k, v


def _sdpa_dense(q, k, v, scale, mask=None, causal=False):
    """torch SDPA (float64) on K/V repeated to every query head, with the mask
    turned into a full [B, HQ, SQ, SK] bias here; rows with no visible key are
    returned as NaN by SDPA and reported in `empty`."""
    B, HQ, SQ, D = q.shape
    HK, SK = k.shape[1], k.shape[2]
    G = HQ // HK
    bias = torch.zeros(B, HQ, SQ, SK, dtype=torch.float64)
    if mask is not None:
        mw = mask.shape[3]
        m = mask if mask.dtype != torch.bool else torch.where(
            mask, torch.tensor(0.0), torch.tensor(float("-inf")))
        m = m.double()
        if mw != 1 and mw < SK:  # keys past the mask's width are hidden
            m = torch.cat([m, torch.full(m.shape[:3] + (SK - mw,), float("-inf"),
                                         dtype=torch.float64)], dim=3)
        bias = bias + m.expand(B, HQ, SQ, SK)
    if causal:
        hide = torch.arange(SK)[None, :] > torch.arange(SQ)[:, None]
        bias = bias.masked_fill(hide, float("-inf"))
    empty = torch.isinf(bias).all(dim=-1) & (bias.amax(dim=-1) < 0)
    kh = k.double().repeat_interleave(G, dim=1)
    vh = v.double().repeat_interleave(G, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(
        q.double(), kh, vh, attn_mask=bias, scale=float(np.float32(scale)))
    return out.numpy(), empty.numpy()


def _mask(kind, dims, seed=0, p=0.7):
    g = torch.Generator().manual_seed(seed)
    if kind == "bool":
        return torch.rand(dims, generator=g) < p
    return torch.randn(dims, generator=g).float() * 2.0


DENSE_CASES = [
    # (B, HQ, HK, SQ, SK, D, dtype, mask kind, mask dims, causal)
    (2, 4, 2, 5, 9, 64, "f32", None, None, False),
    (2, 4, 2, 9, 9, 64, "f16", None, None, True),           # square causal
    (1, 8, 2, 12, 7, 64, "bf16", None, None, True),         # SQ > SK: top-left
    (2, 4, 1, 6, 11, 32, "f32", "bool", (2, 4, 6, 11), False),
    (2, 4, 2, 6, 11, 64, "f32", "bool", (1, 1, 6, 11), True),
    (2, 6, 3, 5, 13, 64, "f16", "add", (2, 1, 1, 13), False),
    (1, 4, 2, 7, 16, 64, "f32", "add", (1, 4, 7, 10), False),   # padded past width 10
    (2, 4, 2, 4, 8, 64, "bf16", "bool", (2, 1, 4, 1), True),    # width 1: broadcast over keys
]


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: "-".join(map(str, c[:8])) + ("-c" if c[9] else ""))
def test_dense_matches_sdpa(case):
    B, HQ, HK, SQ, SK, D, dtype, kind, dims, causal = case
    q, k, v = _dense_inputs(B, HQ, HK, SQ, SK, D, dtype, seed=SQ + SK)
    mask = _mask(kind, dims, seed=3) if kind else None
    ref = oracle.dense_attention(q, k, v, 0.2, mask=mask, causal=causal)
    exp, empty = _sdpa_dense(q, k, v, 0.2, mask=mask, causal=causal)
    assert np.abs(ref[~empty] - exp[~empty]).max() < 1e-12
    assert (ref[empty] == 0).all()


def test_dense_fully_masked_rows_are_zero():
    q, k, v = _dense_inputs(2, 4, 2, 6, 8, 64, seed=1)
    mask = torch.ones(2, 1, 6, 8, dtype=torch.bool)
    mask[1, 0, 2] = False          # row 2 of batch 1 sees nothing
    mask[0, 0, :, 5:] = False      # batch 0: only keys 0..4
    out = oracle.dense_attention(q, k, v, 0.3, mask=mask, causal=False)
    assert (out[1, :, 2] == 0).all() and np.abs(out[1, :, 3]).max() > 0
    exp, empty = _sdpa_dense(q, k, v, 0.3, mask=mask)
    assert empty[1, :, 2].all() and not empty[0].any()
    assert np.abs(out[~empty] - exp[~empty]).max() < 1e-12


def test_dense_single_visible_key_returns_its_value():
    B, HQ, HK, SQ, SK, D = 1, 4, 2, 5, 9, 64
    q, k, v = _dense_inputs(B, HQ, HK, SQ, SK, D, seed=2)
    pick = [3, 0, 8, 5, 1]
    mask = torch.zeros(1, 1, SQ, SK, dtype=torch.bool)
    for i, j in enumerate(pick):
        mask[0, 0, i, j] = True
    out = oracle.dense_attention(q, k, v, 0.5, mask=mask)
    for h in range(HQ):
        for i, j in enumerate(pick):
            assert np.array_equal(out[0, h, i], v[0, h // (HQ // HK), j].double().numpy())


def test_dense_additive_bias_semantics():
    q, k, v = _dense_inputs(2, 4, 2, 6, 10, 64, seed=4)
    base = torch.round(_mask("add", (2, 4, 6, 10), seed=5) * 64) / 64  # exact in float32
    shifted = base + torch.arange(6, dtype=torch.float32)[None, None, :, None] * 3.0
    a = oracle.dense_attention(q, k, v, 0.25, mask=base)
    b = oracle.dense_attention(q, k, v, 0.25, mask=shifted)   # a constant per row: no change
    assert np.abs(a - b).max() < 1e-12
    vis = _mask("bool", (2, 1, 6, 10), seed=6)
    add = torch.where(vis, torch.tensor(0.0), torch.tensor(float("-inf"))).float()
    assert np.array_equal(oracle.dense_attention(q, k, v, 0.25, mask=vis),
                          oracle.dense_attention(q, k, v, 0.25, mask=add))


# --------------------------------------------------------------------------
# Dense GQA backward
# --------------------------------------------------------------------------
def _full_bias(B, HQ, SQ, SK, mask, causal):
    """[B, HQ, SQ, SK] float64 bias of the dense problem, built independently of
    the oracle: bool -> 0/-inf, additive as is, -inf past a short width, -inf
    above the top-left diagonal when causal."""
    bias = torch.zeros(B, HQ, SQ, SK, dtype=torch.float64)
    if mask is not None:
        mw = mask.shape[3]
        m = mask if mask.dtype != torch.bool else torch.where(
            mask, torch.tensor(0.0), torch.tensor(float("-inf")))
        m = m.double()
        if mw != 1 and mw < SK:
            m = torch.cat([m, torch.full(m.shape[:3] + (SK - mw,), float("-inf"),
                                         dtype=torch.float64)], dim=3)
        bias = bias + m.expand(B, HQ, SQ, SK)
    if causal:
        hide = torch.arange(SK)[None, :] > torch.arange(SQ)[:, None]
        bias = bias.masked_fill(hide, float("-inf"))
    return bias


def _autograd_dense(q, k, v, dout, scale, mask=None, causal=False):
    """Gradients of sum(Y * dout) by torch float64 autograd of a separate
    formulation: K/V repeated to every query head, scores scale * Q K^T + bias,
    softmax with rows of no visible key set to zero, Y = P V."""
    B, HQ, SQ, D = q.shape
    HK, SK = k.shape[1], k.shape[2]
    G = HQ // HK
    bias = _full_bias(B, HQ, SQ, SK, mask, causal)
    empty = torch.isinf(bias).all(dim=-1) & (bias.amax(dim=-1) < 0)
    qd = q.double().requires_grad_()
    kd = k.double().requires_grad_()
    vd = v.double().requires_grad_()
    s = float(np.float32(scale)) * (qd @ kd.repeat_interleave(G, dim=1).transpose(-1, -2)) + bias
    s = s.masked_fill(empty[..., None], 0.0)
    p = torch.softmax(s, dim=-1).masked_fill(empty[..., None], 0.0)
    y = p @ vd.repeat_interleave(G, dim=1)
    (y * dout.double()).sum().backward()
    return qd.grad.numpy(), kd.grad.numpy(), vd.grad.numpy()


def _bwd_case(case, seed=0):
    B, HQ, HK, SQ, SK, D, dtype, kind, dims, causal = case
    q, k, v = _dense_inputs(B, HQ, HK, SQ, SK, D, dtype, seed=SQ + SK + seed)
    g = torch.Generator().manual_seed(100 + seed)
    dout = torch.randn(B, HQ, SQ, D, generator=g).to(q.dtype)
    mask = _mask(kind, dims, seed=3) if kind else None
    return q, k, v, dout, mask, causal


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: "-".join(map(str, c[:8])) + ("-c" if c[9] else ""))
def test_dense_backward_matches_autograd(case):
    q, k, v, dout, mask, causal = _bwd_case(case)
    got = oracle.dense_attention_backward(q, k, v, dout, 0.2, mask=mask, causal=causal)
    exp = _autograd_dense(q, k, v, dout, 0.2, mask=mask, causal=causal)
    for a, b in zip(got, exp):
        assert np.abs(a - b).max() < 1e-11


def test_dense_backward_finite_differences():
    # central differences of the forward oracle's loss sum(Y * dout), inputs in
    # float32 moved by 2^-12 (exact in float32 for these magnitudes)
    B, HQ, HK, SQ, SK, D = 1, 4, 2, 5, 7, 16
    q, k, v = _dense_inputs(B, HQ, HK, SQ, SK, D, "f32", seed=9)
    dout = torch.randn(B, HQ, SQ, D, generator=torch.Generator().manual_seed(10))
    mask = _mask("add", (1, 1, SQ, SK), seed=11)
    scale, h = 0.3, 2.0 ** -12
    dq, dk, dv = oracle.dense_attention_backward(q, k, v, dout, scale, mask=mask, causal=True)

    def loss(qq, kk, vv):
        y = oracle.dense_attention(qq, kk, vv, scale, mask=mask, causal=True)
        return float((y * dout.double().numpy()).sum())

    rng = np.random.default_rng(12)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        base = [q, k, v][which]
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in base.shape)
            plus, minus = base.clone(), base.clone()
            plus[idx] += h
            minus[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = plus, minus
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(grad[idx])), (which, idx, fd, grad[idx])


def test_dense_backward_invariants():
    # Every row's dS sums to 0 over its keys, so the key-gradients of a KV head
    # sum to 0; rows of P sum to 1, so its value-gradients sum to the dout rows
    # of its G query heads (rows that see at least one key)
    case = (2, 6, 2, 9, 13, 32, "f32", "bool", (2, 1, 9, 13), True)
    q, k, v, dout, mask, causal = _bwd_case(case, seed=1)
    mask[1, 0, 4] = False  # one row of batch 1 sees nothing
    dq, dk, dv = oracle.dense_attention_backward(q, k, v, dout, 0.25, mask=mask, causal=causal)
    assert np.abs(dk.sum(axis=2)).max() < 1e-12
    bias = _full_bias(2, 6, 9, 13, mask, causal)
    seen = ~(torch.isinf(bias).all(dim=-1))  # [B, HQ, SQ]
    want = (dout.double() * seen[..., None]).reshape(2, 2, 3, 9, 32).sum(dim=(2, 3)).numpy()
    assert np.abs(dv.sum(axis=2) - want).max() < 1e-12
    assert (dq[1, :, 4] == 0).all()


# --------------------------------------------------------------------------
# Mutation check: each planted mistake must trip at least one pin.
# --------------------------------------------------------------------------
def _pins(lib):
    """Compact pin suite; returns the names of the pins that fail with `lib`."""
    failed = []
    try:
        for case in (SWEEP[2], SWEEP[4], SWEEP[3]):
            B, H, KV, D, BS, NQ, causal, dtype, lens = case
            w = P.small(B=B, H=H, KV=KV, D=D, BS=BS, NQ=NQ, causal=causal, dtype=dtype,
                        lens=lens, seed=5)
            if np.abs(_ora(w, lib) - oracle.sdpa_reference(*P.args(w), causal=causal)).max() > 1e-12:
                failed.append("sdpa")
                break
        w = P.small(B=2, H=4, KV=2, D=64, NQ=3, causal=True, lens=(21, 7), dtype="f32")
        w.q.zero_()
        out = _ora(w, lib)
        _, vs = P.logical_rows(w, 1, 1, 2)
        mean = np.array([sum(c) / len(vs) for c in zip(*vs)])
        if np.abs(out[1, 3, 2] - mean).max() > 1e-13:
            failed.append("mean")
        w = P.small(B=2, H=8, KV=2, D=128, BS=16, NQ=3, causal=True, lens=(130, 17), dtype="bf16")
        single = _ora(w, lib)
        part = oracle.paged_decode_partitioned(*P.args(w), chunk=7, causal=True, lib=lib)
        if np.abs(part - single).max() > 1e-12:
            failed.append("partition")
        bf = torch.from_numpy(np.array([0x3F80, 0xC2F7], dtype=np.uint16).view(np.int16).copy())
        h16 = torch.tensor([0x3C00, 0x0001], dtype=torch.int16)
        if (oracle.widen(bf.view(torch.bfloat16), 1, lib) != -123.5
                or oracle.widen(h16.view(torch.float16), 1, lib) != 2.0 ** -24
                or oracle.widen(h16.view(torch.float16), 0, lib) != 1.0):
            failed.append("widen")
        w, slots, _ = _append_case(APPEND_CASES[1], seed=3)
        _, kp, _ = _append(w, slots, lib)
        L = int(w.context_lens[1])
        phys = int(w.block_table[1, (L + 2) // w.spec.BS])
        if not torch.equal(_bits(kp[phys, (L + 2) % w.spec.BS]), _bits(w.new_k[1, :, 2])):
            failed.append("append_round_trip")
        w, slots, reads = _append_case(APPEND_CASES[1], overwrite=3, duplicate=True, seed=4)
        out, _, _ = _append(w, slots, lib)
        if np.abs(out - _dense_with_reads(w, reads, True)).max() > 1e-12:
            failed.append("append_overwrite")
        for case in (DENSE_CASES[2], DENSE_CASES[4], DENSE_CASES[6], DENSE_CASES[7]):
            B, HQ, HK, SQ, SK, D, dtype, kind, dims, causal = case
            q, k, v = _dense_inputs(B, HQ, HK, SQ, SK, D, dtype, seed=SQ + SK)
            mask = _mask(kind, dims, seed=3) if kind else None
            ref = oracle.dense_attention(q, k, v, 0.2, mask=mask, causal=causal, lib=lib)
            exp, empty = _sdpa_dense(q, k, v, 0.2, mask=mask, causal=causal)
            if np.abs(ref[~empty] - exp[~empty]).max() > 1e-12 or (ref[empty] != 0).any():
                failed.append("dense")
                break
        for case in (DENSE_CASES[2], DENSE_CASES[4], DENSE_CASES[5], DENSE_CASES[6]):
            q, k, v, dout, mask, causal = _bwd_case(case)
            got = oracle.dense_attention_backward(q, k, v, dout, 0.2, mask=mask, causal=causal,
                                                  lib=lib)
            exp = _autograd_dense(q, k, v, dout, 0.2, mask=mask, causal=causal)
            if any(np.abs(a - b).max() > 1e-11 for a, b in zip(got, exp)):
                failed.append("dense_backward")
                break
    except ValueError:
        failed.append("rejected")
    return failed


MUTATIONS = {
    "gqa_head_mapping": ("const int h = kh * G + g;", "const int h = g * KV + kh;"),
    "drop_causal_window": ("(causal ? r + 1 : NQ)", "(causal ? NQ : NQ)"),
    "table_index_uses_slot": ("block_table[(int64_t)b * max_blocks + i / BS]",
                              "block_table[(int64_t)b * max_blocks + i % BS]"),
    "slot_off_by_one": ("((physical * BS + i % BS) * KV + kh)", "((physical * BS + (i + 1) % BS) * KV + kh)"),
    "drop_kv_head_offset": ("((physical * BS + i % BS) * KV + kh)", "((physical * BS + i % BS) * KV)"),
    "drop_scale": ("s[i] = scale * dot;", "s[i] = dot;"),
    "flip_exponent_sign": ("double w = exp(s[i] - m);", "double w = exp(m - s[i]);"),
    "drop_normalisation": ("o[d] = Z != 0.0 ? acc[d] / Z : 0.0;\n                } else {",
                           "o[d] = acc[d];\n                } else {"),
    "values_from_keys": ("acc[d] += w * V[(int64_t)i * D + d];", "acc[d] += w * K[(int64_t)i * D + d];"),
    "merge_weight_sign": ("const double weight = exp(mc - M);", "const double weight = exp(M - mc);"),
    "bf16_shift": ("(uint32_t)b << 16", "(uint32_t)b << 15"),
    "half_exponent_bias": ("exponent - 25", "exponent - 24"),
    "new_rows_from_wrong_head": ("(((int64_t)b * KV + kh) * NQ + j) * D", "(((int64_t)b * KV) * NQ + j) * D"),
    "append_rows_in_reverse": ("for (int j = 0; j < NQ; ++j) {\n            const int64_t slot",
                               "for (int j = NQ - 1; j >= 0; --j) {\n            const int64_t slot"),
    "append_slot_as_block": ("const int64_t dst = slot * row_bytes",
                             "const int64_t dst = (slot / BS) * row_bytes"),
    "append_first_head_only": ("for (int kh = 0; kh < KV; ++kh) {\n                const int64_t row",
                               "for (int kh = 0; kh < 1; ++kh) {\n                const int64_t row"),
    "append_rows_of_head_0": ("const int64_t row = ((int64_t)b * KV + kh) * NQ + j;",
                              "const int64_t row = ((int64_t)b * KV) * NQ + j;"),
    "dense_causal_shifted_diagonal": ("if (causal && j > i)", "if (causal && j > i - 2)"),
    "dense_head_mapping": ("const int kh = h / G; /* query head h = kh*G + g */",
                           "const int kh = h % HK; /* query head h = kh*G + g */"),
    "dense_pad_off_by_one": ("if (mw != 1 && j >= mw) {", "if (mw != 1 && j > mw) {"),
    "dense_mask_head_index": ("(mh == 1 ? 0 : h)) * mq", "(mh == 1 ? 0 : h / 2)) * mq"),
    "dense_bias_scaled": ("\n            s[j] = sc * dot + dense_bias(",
                          "\n            s[j] = sc * 2.0 * dot + dense_bias("),
    "dense_bias_doubled": ("bias = (double)((const float*)mask)[mi];",
                           "bias = 2.0 * (double)((const float*)mask)[mi];"),
    "bwd_head_mapping": ("const int h = g + kh * G;", "const int h = g * HK + kh;"),
    "bwd_drop_delta": ("dp[j] = s[j] * (dot - delta);", "dp[j] = s[j] * dot;"),
    "bwd_dk_first_head_only": ("dk[(kv0 + j) * D + d] += sc * dp[j] * qr[d];",
                               "if (g == 0) dk[(kv0 + j) * D + d] += sc * dp[j] * qr[d];"),
    "bwd_dq_without_scale": ("dq[row * D + d] += sc * dp[j] *", "dq[row * D + d] += dp[j] *"),
    "bwd_dv_from_y": ("dv[(kv0 + j) * D + d] += s[j] * gy[d];",
                      "dv[(kv0 + j) * D + d] += s[j] * y[d];"),
    "bwd_dp_from_keys": ("dot += gy[d] * oracle_widen(v,", "dot += gy[d] * oracle_widen(k,"),
    "bwd_dk_from_dout": ("dk[(kv0 + j) * D + d] += sc * dp[j] * qr[d];",
                         "dk[(kv0 + j) * D + d] += sc * dp[j] * gy[d];"),
    "bwd_unnormalised_p": ("                    s[j] /= z;\n", "                    s[j] /= 1.0;\n"),
}


def test_pins_pass_on_the_oracle():
    assert _pins(None) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(ORACLE_DIR, "oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    (tmp_path / "oracle.c").write_text(src.replace(old, new))
    shutil.copy(os.path.join(ORACLE_DIR, "oracle.h"), tmp_path / "oracle.h")
    so = tmp_path / f"liboracle_{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", str(tmp_path / "oracle.c"),
                    "-o", str(so), "-lm"], check=True)
    # The mutant may read out of bounds, so its pins run in a child process; a
    # crash of that process also counts as caught.
    root = os.path.dirname(ORACLE_DIR)
    code = ("import sys, oracle; from tests.test_oracle import _pins; "
            f"sys.exit(3 if _pins(oracle.load_library({str(so)!r})) else 0)")
    res = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode != 0, f"no pin caught the planted mistake {name}: {res.stderr[-500:]}"
