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


def split_single_piece_units(context_lens, KV, NQ, n_grp, min_seg, max_tokens, seq_pad=0):
    """Units (b, kh) that the balanced split leaves in one group.

    Integer model of the split: sequence b spans n_b = ceil(L_b/16) +
    ceil(NQ/16) positions of 16 keys along one axis, and costs n_b + seq_pad
    units of a cost axis of C units (seq_pad = 0 for plans with an explicit
    number of partitions); n = min(n_grp, max(1, C // min_seg)) groups start at
    cost unit floor(g*C/n), and every KV head of a sequence shares its groups.
    Position x of sequence b is cost unit x + seq_pad*b, in group
    floor(((x + seq_pad*b + 1)*n - 1) / C)."""
    nnew = (NQ + 15) // 16
    nsub = [(min(max(int(L), 0), max_tokens) + 15) // 16 + nnew for L in context_lens]
    C = sum(nsub) + seq_pad * len(nsub)
    n = min(n_grp, max(1, C // min_seg if min_seg > 1 else C))

    def group_of(x, b):
        return ((x + seq_pad * b + 1) * n - 1) // C

    out, start = set(), 0
    for b, m in enumerate(nsub):
        if group_of(start, b) == group_of(start + m - 1, b):
            out.update((b, kh) for kh in range(KV))
        start += m
    return out


def append_problem(w: W.Workload, *, overwrite: int = 0, duplicate: bool = False,
                   negative: int = 0, out_of_range: int = 0, seed: int = 0, fill=float("nan")):
    """The same logical cache re-stored with room for this step's new rows, and a
    slot mapping int32 [B, NQ] for them (inputs only, no attention arithmetic).

    New row j of sequence b is mapped to the token slot of logical position
    L_b + j: block table entry (L_b + j) // BS, offset (L_b + j) % BS; space past
    each cached length holds `fill`. Then, chosen with the seed: `overwrite`
    entries are re-pointed at the slot of a random cached position of the same
    sequence; `duplicate` makes the last new row of each sequence (NQ > 1) share
    the slot of its first; `negative` entries become -1 and `out_of_range`
    entries point past the pool (neither is stored nor read).
    Returns (workload, slot_mapping, reads) with reads[(b, p)] = j: cached
    position p of sequence b is overwritten this step, by new row j (the
    highest j that points at it)."""
    s = w.spec
    rng = np.random.default_rng(seed)
    BS, NQ = s.BS, s.NQ
    lens = [int(L) for L in w.context_lens]
    pages = [max(1, (L + NQ + BS - 1) // BS) for L in lens]
    nblocks = sum(pages) + 2
    order = rng.permutation(nblocks)
    max_blocks = max(pages)
    table = np.zeros((s.B, max_blocks), dtype=np.int32)
    kp = torch.full((nblocks, BS, s.KV, s.D), fill, dtype=w.k_pool.dtype)
    vp = torch.full_like(kp, fill)
    src_k, src_v = w.k_pool.cpu(), w.v_pool.cpu()
    nxt = 0
    for b, L in enumerate(lens):
        for n in range(pages[b]):
            table[b, n] = int(order[nxt])
            nxt += 1
        for i in range(L):
            sp = int(w.block_table[b, i // s.BS])
            kp[table[b, i // BS], i % BS] = src_k[sp, i % s.BS]
            vp[table[b, i // BS], i % BS] = src_v[sp, i % s.BS]

    def slot_of(b, i):
        return int(table[b, i // BS]) * BS + i % BS

    slots = np.array([[slot_of(b, lens[b] + j) for j in range(NQ)] for b in range(s.B)],
                     dtype=np.int32).reshape(s.B, NQ)
    entries = [(b, j) for b in range(s.B) for j in range(NQ)]
    with_past = [(b, j) for (b, j) in entries if lens[b] > 0]
    for k in rng.permutation(len(with_past))[:overwrite]:
        b, j = with_past[k]
        slots[b, j] = slot_of(b, int(rng.integers(0, lens[b])))
    if duplicate and NQ > 1:
        slots[:, NQ - 1] = slots[:, 0]
    for k in rng.permutation(len(entries))[:negative]:
        b, j = entries[k]
        slots[b, j] = -1
    for k in rng.permutation(len(entries))[:out_of_range]:
        b, j = entries[k]
        slots[b, j] = nblocks * BS + int(rng.integers(0, 3 * BS))
    reads = {}
    for b, L in enumerate(lens):
        where = {slot_of(b, p): p for p in range(L)}
        for j in range(NQ):
            p = where.get(int(slots[b, j]))
            if p is not None:
                reads[(b, p)] = j  # j ascending: the highest j stays
    spec = s.replace(max_blocks=max_blocks, pool=("fixed", nblocks))
    w2 = W.Workload(spec, w.context_lens.copy(), table, nblocks, w.q.cpu(), kp, vp,
                    w.new_k.cpu(), w.new_v.cpu(), w.scale)
    return w2, slots, reads


# ---------------------------------------------------------------------------
# Score staircases: inputs whose running maximum moves at chosen key positions
# ---------------------------------------------------------------------------
STAIR_STEP_LOG2 = 9.0  # one jump of the score, in log2 units (above a slack of 8)


def stair_levels(n_keys: int, jumps) -> np.ndarray:
    """Level of key j: the number of jump sub-pages J (of 16 keys) with 16*J <= j."""
    j = np.arange(n_keys)
    return np.array([sum(1 for J in jumps if 16 * J <= x) for x in j], dtype=np.float64)


def stair_direction(D: int, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0)


def staircase_dense(B, HQ, HK, S, D, dtype, jumps_per_seq, seed=0):
    """q [B, HQ, S, D] = s * u with u in {-1, 1}^D and s = 1 or 0.55 by (head,
    16-position block) parity; k = level * step * u / sqrt(D) + 0.05 noise, so
    with scale 1/sqrt(D) the scores of sequence b rise by step * s natural-log
    units at every jump sub-page of jumps_per_seq[b]. v is N(0, 1). Returns
    (q, k, v, scale) as CPU tensors of the dtype."""
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    g = torch.Generator().manual_seed(seed)
    u = stair_direction(D, seed + 1)
    step = STAIR_STEP_LOG2 / np.log2(np.e)
    h = torch.arange(HQ)[:, None]
    i = torch.arange(S)[None, :]
    s = torch.where((h + i // 16) % 2 == 0, 1.0, 0.55)            # [HQ, S]
    q = (s[None, :, :, None] * u).expand(B, HQ, S, D).contiguous()
    lev = torch.stack([torch.from_numpy(stair_levels(S, jumps_per_seq[b])).float()
                       for b in range(B)])                          # [B, S]
    k = (lev[:, None, :, None] * (step / np.sqrt(D)) * u).expand(B, HK, S, D)
    k = k + 0.05 * torch.randn(B, HK, S, D, generator=g)
    v = torch.randn(B, HK, S, D, generator=g)
    return q.to(dt), k.to(dt), v.to(dt), float(np.float32(1.0 / np.sqrt(D)))


def staircase_decode(w: W.Workload, jumps_per_seq, seed=0) -> W.Workload:
    """The same staircase on a paged workload: q[b, h, r] = s_h * u (s_h = 1 or
    0.55 by head parity); the key at logical position p of sequence b gets
    level(p) * step * u / sqrt(D) + 0.05 noise through the block table, and the
    new rows take the level of the last cached key plus one jump. Values and the
    layout are unchanged; the scale becomes 1/sqrt(D)."""
    s = w.spec
    g = torch.Generator().manual_seed(seed)
    u = stair_direction(s.D, seed + 1)
    step = STAIR_STEP_LOG2 / np.log2(np.e)
    dt = w.q.dtype
    sh = torch.where(torch.arange(s.H) % 2 == 0, 1.0, 0.55)
    q = (sh[None, :, None, None] * u).expand(s.B, s.H, s.NQ, s.D).to(dt).contiguous()
    kp = w.k_pool.clone()
    nk = w.new_k.clone()
    for b in range(s.B):
        L = int(w.context_lens[b])
        lev = stair_levels(L, jumps_per_seq[b])
        for p in range(L):
            blk = int(w.block_table[b, p // s.BS])
            row = lev[p] * (step / np.sqrt(s.D)) * u + 0.05 * torch.randn(s.KV, s.D, generator=g)
            kp[blk, p % s.BS] = row.to(dt)
        top = (lev[-1] if L else 0.0) + 1.0
        nk[b] = (top * (step / np.sqrt(s.D)) * u
                 + 0.05 * torch.randn(s.KV, s.NQ, s.D, generator=g)).to(dt)
    return W.Workload(s, w.context_lens, w.block_table, w.num_blocks, q, kp, w.v_pool, nk,
                      w.new_v, float(np.float32(1.0 / np.sqrt(s.D))))


# ---------------------------------------------------------------------------
# Argmax probe: one cached key per sequence dominates every query row
# ---------------------------------------------------------------------------
def argmax_probe(w: W.Workload, ts, lead: float = 12.0, seed: int = 0):
    """Inputs where logical position ts[b] of sequence b wins every row by far.

    Each KV head kh gets a direction u_kh in {-1, 1}^D; every query row of the
    heads that read kh is u_kh, and the key at position ts[b] of head kh is
    lead * u_kh, so its score is lead * D * scale (D = 128, scale 1/sqrt(D):
    about 136 natural-log units for lead 12, 196 in log2 units) while the other
    keys, N(0, 1), score a few units: every other softmax weight is below
    2^-150, which is 0 in binary32. Returns (workload, expect) with expect[b]
    [H, NQ, D] = the stored v row of position ts[b] for each head's KV head,
    in the I/O dtype (what an exact argmax returns)."""
    s = w.spec
    G = s.H // s.KV
    g = torch.Generator().manual_seed(seed)
    u = torch.where(torch.rand(s.KV, s.D, generator=g) < 0.5, -1.0, 1.0)
    q = u.repeat_interleave(G, dim=0)[None, :, None, :].expand(s.B, s.H, s.NQ, s.D)
    q = q.to(w.q.dtype).contiguous()
    kp = w.k_pool.clone()
    expect = []
    for b, t in enumerate(ts):
        assert 0 <= t < int(w.context_lens[b])
        phys = int(w.block_table[b, t // s.BS])
        kp[phys, t % s.BS] = (lead * u).to(kp.dtype)
        vrow = w.v_pool[phys, t % s.BS]                       # [KV, D]
        expect.append(vrow.repeat_interleave(G, dim=0)[:, None, :].expand(s.H, s.NQ, s.D).clone())
    w2 = W.Workload(s, w.context_lens, w.block_table, w.num_blocks, q, kp, w.v_pool, w.new_k,
                    w.new_v, float(np.float32(1.0 / np.sqrt(s.D))))
    return w2, expect
