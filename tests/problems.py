"""Small seeded problems for the tests (inputs only; no attention arithmetic)."""
from __future__ import annotations

import numpy as np
import torch

from paged_kv_gqa_decode_amd import workloads as W


def small_spec(B=2, H=4, KV=2, D=64, BS=16, NQ=1, causal=True, dtype="f32", lens=(37, 5),
               pool_extra=3, seed=7, max_blocks=None) -> W.Spec:
    lens = tuple(int(x) for x in lens)
    assert len(lens) == B
    pages = sum((L + BS - 1) // BS for L in lens)
    if max_blocks is None:
        max_blocks = max(1, max((L + BS - 1) // BS for L in lens) if lens else 1)
    return W.Spec(f"small_b{B}_h{H}_kv{KV}_d{D}_bs{BS}_nq{NQ}", B=B, H=H, KV=KV, D=D, BS=BS,
                  NQ=NQ, causal=causal, dtype=dtype, lengths=("list", lens),
                  pool=("fixed", max(1, pages + pool_extra)), max_blocks=max_blocks, seed=seed)


def small(device="cpu", **kw) -> W.Workload:
    return W.make_workload(small_spec(**kw), device=device)


def args(w: W.Workload):
    return (w.q, w.k_pool, w.v_pool, w.block_table, w.context_lens, w.new_k, w.new_v, w.scale)


def relayout(w: W.Workload, new_bs: int = None, shuffle_seed: int = None, extra_blocks: int = 0,
             fill=0.0) -> W.Workload:
    """Store the same logical cache in a fresh pool: other block size and/or other
    physical block order. Unused pool space is filled with `fill` (NaN to poison)."""
    s = w.spec
    BS = new_bs or s.BS
    lens = [int(L) for L in w.context_lens]
    pages = [(L + BS - 1) // BS for L in lens]
    nblocks = max(1, sum(pages) + extra_blocks)
    order = np.arange(nblocks)
    if shuffle_seed is not None:
        order = np.random.default_rng(shuffle_seed).permutation(nblocks)
    max_blocks = max(1, max(pages, default=1))
    table = np.zeros((s.B, max_blocks), dtype=np.int32)
    kp = torch.full((nblocks, BS, s.KV, s.D), fill, dtype=w.k_pool.dtype)
    vp = torch.full_like(kp, fill)
    src_k, src_v = w.k_pool.cpu(), w.v_pool.cpu()
    nxt = 0
    for b, L in enumerate(lens):
        for n in range(pages[b]):
            phys = int(order[nxt])
            nxt += 1
            table[b, n] = phys
            for t in range(BS):
                i = n * BS + t
                if i >= L:
                    break
                sp = int(w.block_table[b, i // s.BS])
                kp[phys, t] = src_k[sp, i % s.BS]
                vp[phys, t] = src_v[sp, i % s.BS]
    spec = s.replace(BS=BS, max_blocks=max_blocks)
    return W.Workload(spec, w.context_lens.copy(), table, nblocks, w.q.cpu(), kp, vp,
                      w.new_k.cpu(), w.new_v.cpu(), w.scale)


def logical_rows(w: W.Workload, b: int, kh: int, r: int):
    """Visible (k, v) rows of (b, kh) for new row r, as Python float lists (loops)."""
    s = w.spec
    L = int(w.context_lens[b])
    ks, vs = [], []
    kp, vp = w.k_pool.cpu().double(), w.v_pool.cpu().double()
    for i in range(L):
        phys = int(w.block_table[b][i // s.BS])
        ks.append([float(x) for x in kp[phys, i % s.BS, kh]])
        vs.append([float(x) for x in vp[phys, i % s.BS, kh]])
    n_new = r + 1 if s.causal else s.NQ
    nk, nv = w.new_k.cpu().double(), w.new_v.cpu().double()
    for j in range(n_new):
        ks.append([float(x) for x in nk[b, kh, j]])
        vs.append([float(x) for x in nv[b, kh, j]])
    return ks, vs


def split_single_piece_units(context_lens, KV, NQ, n_grp, min_seg, max_tokens):
    """Units (b, kh) that the balanced split leaves in one group.

    Integer model of the split: sequence b spans ceil(L_b/16) + ceil(NQ/16)
    positions of 16 keys along one axis of W positions; n = min(n_grp,
    max(1, W // min_seg)) groups start at floor(g*W/n), and every KV head of a
    sequence shares its groups."""
    nnew = (NQ + 15) // 16
    nsub = [(min(max(int(L), 0), max_tokens) + 15) // 16 + nnew for L in context_lens]
    W = sum(nsub)
    n = min(n_grp, max(1, W // min_seg if min_seg > 1 else W))

    def group_of(x):
        return ((x + 1) * n - 1) // W

    out, start = set(), 0
    for b, m in enumerate(nsub):
        if group_of(start) == group_of(start + m - 1):
            out.update((b, kh) for kh in range(KV))
        start += m
    return out
