"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances (max-abs against the fp64 oracle): 1e-5 for fp32 I/O, 4e-3 for
fp16/bf16 I/O. Where half a unit in the last place of the output dtype at the
expected value already exceeds the 16-bit bar (bf16 outputs of magnitude >= 1,
fp16 >= 8: possible with only a few visible keys), rounding the exact result
to the output dtype alone can use it up; there the bar per element is that
half unit plus 1e-3 for the arithmetic. Block-table indexing must be
bit-exact: outputs for the same logical cache stored in another physical block
order are compared with torch.equal, and poisoned (NaN) unused pool space must
not change a bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_decode_amd as pa
from paged_kv_gqa_decode_amd import workloads as W
from tests import problems as P

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 4e-3, "bf16": 4e-3}
DEV = "cuda:0"


def to_device(w: W.Workload) -> W.Workload:
    return W.Workload(w.spec, w.context_lens, w.block_table, w.num_blocks, w.q.to(DEV),
                      w.k_pool.to(DEV), w.v_pool.to(DEV), w.new_k.to(DEV), w.new_v.to(DEV),
                      w.scale)


def gpu_decode(w: W.Workload, num_partitions=0, kernel=0, max_context_len=None):
    assert w.q.is_cuda
    table = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(DEV)
    lens = torch.from_numpy(np.ascontiguousarray(w.context_lens)).to(DEV)
    mcl = w.max_context_len if max_context_len is None else max_context_len
    print(f"[gpu] {w.spec.name} B={w.spec.B} dtype={w.spec.dtype} parts={num_partitions} "
          f"kernel={kernel} max_ctx={mcl}", flush=True)
    out = pa.decode(w.q, w.k_pool, w.v_pool, table, lens, w.new_k, w.new_v, w.scale,
                    max_context_len=mcl, causal=w.spec.causal,
                    num_partitions=num_partitions, kernel=kernel)
    torch.cuda.synchronize()
    return out


def ref(w: W.Workload) -> np.ndarray:
    return oracle.paged_decode(*P.args(w), causal=w.spec.causal)


MANTISSA_BITS = {"f16": 10, "bf16": 7}


def allowed(expect: np.ndarray, dtype: str) -> np.ndarray:
    """Per-element bar: TOL, or half an ulp of the output dtype at the expected
    value plus 1e-3 where that half ulp is the larger."""
    tol = np.full(expect.shape, TOL[dtype])
    if dtype in MANTISSA_BITS:
        mag = np.maximum(np.abs(expect), np.finfo(np.float64).tiny)
        half_ulp = np.exp2(np.floor(np.log2(mag)) - MANTISSA_BITS[dtype] - 1)
        tol = np.where(half_ulp > TOL[dtype] / 4 * 3, np.maximum(tol, half_ulp + 1e-3), tol)
    return tol


def max_err(out: torch.Tensor, expect: np.ndarray) -> float:
    return float(np.abs(out.detach().cpu().double().numpy() - expect).max()) if expect.size else 0.0


def check(w, out, expect=None):
    expect = ref(w) if expect is None else expect
    got = out.detach().cpu().double().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - expect)
    bar = allowed(expect, w.spec.dtype)
    worst = np.unravel_index(np.argmax(err - bar), err.shape) if err.size else None
    assert (err <= bar).all(), (f"error {err[worst]} > {bar[worst]} at {worst} "
                                f"(expected {expect[worst]})")
    return float(err.max()) if err.size else 0.0


# ---------------------------------------------------------------------------
# The five workloads at full size (every output compared)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", range(len(W.CONFIGS)), ids=[c.name for c in W.CONFIGS])
def test_config_full_size(cfg):
    w = W.make_workload(W.CONFIGS[cfg], device=DEV)
    out = gpu_decode(w)
    err = check(w, out)
    print(f"[gpu] {W.CONFIGS[cfg].name}: max-abs error {err:.3e}", flush=True)


@pytest.mark.parametrize("cfg", [1, 4], ids=["llama3_8b_decode", "ragged_serving"])
def test_repeated_calls_reuse_the_workspace(cfg):
    # One Decoder (problem, workspace, output) called again and again, as a
    # serving loop does: every call must match the oracle.
    w = W.make_workload(W.CONFIGS[cfg], device=DEV)
    table = torch.from_numpy(w.block_table).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    dec = pa.Decoder(w.q, w.k_pool, table, max_context_len=w.max_context_len,
                     causal=w.spec.causal)
    assert dec.partitions > 1
    expect = ref(w)
    for rep in range(4):
        print(f"[gpu] {w.spec.name} repeat {rep}", flush=True)
        out = dec(w.q, w.k_pool, w.v_pool, table, lens, w.new_k, w.new_v, w.scale)
        torch.cuda.synchronize()
        check(w, out, expect)


# ---------------------------------------------------------------------------
# Shrunken variants: several pages per wave, ragged tails, several partitions
# ---------------------------------------------------------------------------
SMALL = [
    W.shrink(W.CONFIGS[1], B=5, lengths=("list", (0, 1, 17, 700, 1999)), max_blocks=125),
    W.shrink(W.CONFIGS[2], B=2, lengths=("list", (5000, 9001)), max_blocks=600),
    W.shrink(W.CONFIGS[3], B=3, lengths=("list", (0, 35, 300)), max_blocks=20),
    W.shrink(W.CONFIGS[4], B=9, lengths=("lognormal", 200, 1.0, 16, 3000), max_blocks=100),
]


@pytest.mark.parametrize("spec", SMALL, ids=[s.name for s in SMALL])
@pytest.mark.parametrize("parts", [0, 1, 2, 3, 7])
def test_small_variants_all_partitions(spec, parts):
    w = W.make_workload(spec, device=DEV)
    check(w, gpu_decode(w, num_partitions=parts))


GEOMETRIES = [
    # B, H, KV, D, BS, NQ, causal, dtype, lens
    (2, 4, 4, 64, 16, 1, True, "f32", (0, 77)),        # MHA
    (3, 8, 1, 64, 32, 3, True, "f16", (15, 16, 33)),   # MQA, multi-row
    (2, 8, 2, 128, 32, 3, False, "bf16", (31, 64)),    # non-causal multi-row
    (2, 16, 2, 128, 16, 8, True, "f16", (0, 333)),     # 64 rows per KV head: four row tiles
    (2, 16, 2, 64, 16, 5, True, "bf16", (40, 250)),    # 40 rows, D=64: a padded fourth tile
    (2, 16, 1, 128, 32, 3, True, "f16", (100, 1)),     # 48 rows: one padded tile
    (3, 16, 2, 128, 16, 4, True, "bf16", (17, 0, 400)),  # 32 rows: two row tiles
    (2, 12, 2, 64, 32, 4, False, "f16", (90, 33)),     # 24 rows: a half-filled second tile
    (3, 12, 3, 128, 16, 1, True, "f16", (50, 300, 7)),   # KV=3: groups straddle workgroups
    (2, 32, 16, 64, 16, 2, True, "bf16", (260, 19)),   # KV=16: a group spans 4 workgroups
    (1, 32, 2, 128, 16, 8, True, "bf16", (500,)),      # 128 rows per KV head
    (2, 4, 2, 64, 16, 2, True, "f32", (129, 1)),
    (2, 4, 2, 128, 32, 1, True, "f32", (700, 64)),
    # more than 16 new rows: the new rows span two sub-pages, and rows below
    # the second one's first row see none of its keys (causal limit <= 0)
    (2, 4, 4, 128, 16, 32, True, "f16", (0, 77)),      # MHA, NQ = 32: two row tiles
    (2, 8, 4, 64, 32, 20, True, "bf16", (45, 300)),    # G = 2, NQ = 20: cooperative kernel
    (2, 4, 2, 128, 16, 24, False, "f16", (19, 130)),   # G = 2, NQ = 24, non-causal
    # 36 and 33 rows: the merge's last tile of 8 rows (two per wave) is short
    (2, 8, 2, 64, 16, 9, True, "f16", (33, 210)),
    (3, 6, 2, 128, 32, 11, True, "bf16", (0, 140, 77)),
]


@pytest.mark.parametrize("case", GEOMETRIES, ids=lambda c: "-".join(map(str, c[:8])))
def test_geometries(case):
    B, H, KV, D, BS, NQ, causal, dtype, lens = case
    w = to_device(P.small(B=B, H=H, KV=KV, D=D, BS=BS, NQ=NQ, causal=causal, dtype=dtype,
                          lens=lens, seed=31))
    expect = ref(w)
    for parts in (0, 1, 3):
        check(w, gpu_decode(w, num_partitions=parts), expect)


@pytest.mark.parametrize("B,dtype", [(1, "f16"), (64, "bf16"), (65, "f16"), (130, "bf16")])
@pytest.mark.parametrize("rows", [4, 24, 64])
@pytest.mark.parametrize("D,BS", [(128, 16), (64, 32)])
def test_sequence_tables(B, dtype, rows, D, BS):
    # batches of up to 64 sequences keep the sequence table in registers,
    # larger ones in LDS; 4 rows per KV head: the one-wave kernel with one row
    # tile, 24: with two, 64: the cooperative kernel; D = 64 slots are half as
    # large, so those kernels hold twice as many
    H, NQ = {4: (8, 1), 24: (16, 3), 64: (16, 8)}[rows]
    lens = tuple(int(x) for x in np.random.default_rng(B).integers(0, 200, size=B))
    w = to_device(P.small(B=B, H=H, KV=2, D=D, BS=BS, NQ=NQ, causal=True, dtype=dtype,
                          lens=lens, seed=23))
    expect = ref(w)
    for parts in (0, 1, 3, 40):
        check(w, gpu_decode(w, num_partitions=parts), expect)


# The batch limits of the balanced split: 8192 sequences (the largest batch the
# matrix-core kernels take; the sequence table then fills 64 KiB of LDS beside
# the slots), for the one-wave and the cooperative kernel, and 8193 (the plan
# moves to the vector kernel)
@pytest.mark.parametrize("B,H,NQ,dtype", [(8192, 8, 1, "f16"), (8192, 16, 8, "bf16"),
                                          (8193, 8, 1, "bf16")])
def test_batch_limits(B, H, NQ, dtype):
    lens = np.random.default_rng(B + NQ).integers(0, 41, size=B)
    w = P.small(B=B, H=H, KV=2, D=128, NQ=NQ, causal=True, lens=tuple(lens), dtype=dtype,
                seed=23)
    wd = to_device(w)
    expect = ref(w)
    for parts in (0, 3):
        check(wd, gpu_decode(wd, num_partitions=parts), expect)


@pytest.mark.parametrize("B,parts,dtype", [(9, 40, "bf16"), (20, 150, "f16"), (9, 100, "f16")])
def test_merge_of_many_pieces(B, parts, dtype):
    # one long sequence among short ones: the merge picks its batch of pieces
    # from groups / sequences + 1 (here 5, 8 and 12), while the long sequence
    # has about `parts` pieces: several batches per run, and runs of 64 pieces
    lens = (5000,) + tuple(range(3, 3 + 2 * (B - 1), 2))
    w = to_device(P.small(B=B, H=8, KV=2, D=128, BS=16, NQ=1, causal=True, dtype=dtype,
                          lens=lens, seed=41))
    check(w, gpu_decode(w, num_partitions=parts))


def test_many_short_sequences():
    # 4200 sequences of 0..39 cached keys: an LDS prefix of 33 KiB beside the
    # slots, most sequences inside one group, several per wave
    B = 4200
    lens = tuple(int(x) for x in np.random.default_rng(21).integers(0, 40, size=B))
    w = to_device(P.small(B=B, H=4, KV=2, D=64, BS=16, NQ=1, causal=True, dtype="f16",
                          lens=lens, seed=22))
    expect = ref(w)
    for parts in (0, 5):
        check(w, gpu_decode(w, num_partitions=parts), expect)


# ---------------------------------------------------------------------------
# Slot-patched step (paged_attn_decode_append): out against the oracle, and
# the pools afterwards bit for bit against the oracle's stored rows
# ---------------------------------------------------------------------------
_LENS70 = tuple(int(x) for x in np.random.default_rng(70).integers(0, 60, size=70))
APPEND_GPU = [
    # B, H, KV, D, BS, NQ, causal, dtype, lens, kernel
    (3, 8, 2, 128, 16, 1, True, "f16", (0, 15, 300), pa.PA_KERNEL_MFMA),    # one row tile
    (2, 32, 8, 128, 16, 1, True, "bf16", (700, 33), pa.PA_KERNEL_MFMA),     # Llama-3-8B heads
    (2, 16, 2, 128, 16, 8, True, "f16", (5, 333), pa.PA_KERNEL_MFMA),       # 64 rows: cooperative
    (2, 16, 2, 64, 32, 3, True, "bf16", (40, 250), pa.PA_KERNEL_MFMA),      # 24 rows, D=64, BS=32
    (2, 4, 2, 64, 16, 2, True, "f32", (129, 1), pa.PA_KERNEL_AUTO),         # fp32: vector ALU
    (2, 8, 2, 128, 32, 3, False, "f16", (31, 64), pa.PA_KERNEL_VALU),       # forced vector ALU
    (2, 4, 4, 128, 16, 32, True, "f16", (3, 77), pa.PA_KERNEL_MFMA),       # NQ = 32: two sub-pages
    (2, 8, 4, 64, 32, 20, True, "bf16", (45, 300), pa.PA_KERNEL_MFMA),     # NQ = 20, cooperative
    # 70 sequences: the sequence table in LDS (one tile, two tiles, cooperative)
    (70, 8, 2, 128, 16, 1, True, "f16", _LENS70, pa.PA_KERNEL_MFMA),
    (70, 16, 2, 128, 16, 3, True, "bf16", _LENS70, pa.PA_KERNEL_MFMA),
    (70, 16, 2, 64, 32, 8, True, "f16", _LENS70, pa.PA_KERNEL_MFMA),
]
APPEND_SCENARIOS = {
    "natural": dict(seed=3),
    "overwrite": dict(overwrite=3, duplicate=True, seed=4),
    "ignored": dict(overwrite=1, negative=2, out_of_range=2, seed=6),
}


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16)


def gpu_decode_append(w, slots, num_partitions=0, kernel=0):
    table = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(DEV)
    lens = torch.from_numpy(np.ascontiguousarray(w.context_lens)).to(DEV)
    kp, vp = w.k_pool.to(DEV).clone(), w.v_pool.to(DEV).clone()
    print(f"[gpu] append {w.spec.name} B={w.spec.B} dtype={w.spec.dtype} parts={num_partitions} "
          f"kernel={kernel}", flush=True)
    out = pa.decode_append(w.q.to(DEV), kp, vp, table, lens, w.new_k.to(DEV), w.new_v.to(DEV),
                           torch.from_numpy(slots).to(DEV), w.scale,
                           max_context_len=w.max_context_len, causal=w.spec.causal,
                           num_partitions=num_partitions, kernel=kernel)
    torch.cuda.synchronize()
    return out, kp, vp


@pytest.mark.parametrize("scenario", sorted(APPEND_SCENARIOS))
@pytest.mark.parametrize("case", APPEND_GPU, ids=lambda c: "-".join(map(str, c[:8])) + f"-k{c[9]}")
def test_append_matches_the_oracle(case, scenario):
    B, H, KV, D, BS, NQ, causal, dtype, lens, kernel = case
    w = P.small(B=B, H=H, KV=KV, D=D, BS=BS, NQ=NQ, causal=causal, dtype=dtype, lens=lens,
                seed=41)
    w, slots, reads = P.append_problem(w, **APPEND_SCENARIOS[scenario])
    if scenario == "overwrite":
        assert reads
    expect, kp_ref, vp_ref = oracle.paged_decode_append(*P.args(w)[:7], slots, w.scale,
                                                        causal=causal)
    for parts in (0, 1, 3):
        out, kp, vp = gpu_decode_append(w, slots, num_partitions=parts, kernel=kernel)
        check(w, out, expect)
        assert torch.equal(_bits(kp), _bits(kp_ref)) and torch.equal(_bits(vp), _bits(vp_ref))


def test_append_with_every_slot_negative_is_the_plain_step():
    w = P.small(B=3, H=8, KV=2, D=128, BS=16, NQ=2, causal=True, dtype="bf16", lens=(20, 0, 90),
                seed=42)
    w, slots, _ = P.append_problem(w, seed=7)
    slots[:] = -1
    for kernel in (pa.PA_KERNEL_MFMA, pa.PA_KERNEL_VALU):
        out, kp, vp = gpu_decode_append(w, slots, num_partitions=3, kernel=kernel)
        assert torch.equal(out, gpu_decode(to_device(w), num_partitions=3, kernel=kernel))
        assert torch.equal(_bits(kp), _bits(w.k_pool)) and torch.equal(_bits(vp), _bits(w.v_pool))


def test_plain_step_leaves_the_pools_alone():
    w = to_device(P.small(B=2, H=8, KV=2, D=128, BS=16, NQ=1, dtype="f16", lens=(70, 5), seed=43))
    k0, v0 = w.k_pool.clone(), w.v_pool.clone()
    gpu_decode(w, num_partitions=2)
    assert torch.equal(w.k_pool, k0) and torch.equal(w.v_pool, v0)


# ---------------------------------------------------------------------------
# Dense GQA attention forward (pa_dense_attention) against the oracle
# ---------------------------------------------------------------------------
DENSE_GPU = [
    # B, HQ, HK, SQ, SK, D, dtype, mask kind, mask dims, causal
    (2, 4, 4, 70, 70, 64, "f16", None, None, True),                 # G = 1: 64 positions a block
    (1, 8, 2, 37, 53, 128, "bf16", None, None, False),               # G = 4, ragged tails
    (2, 16, 2, 29, 29, 128, "f16", None, None, True),                # G = 8: 8 positions a block
    (1, 12, 4, 45, 33, 64, "bf16", None, None, True),                # G = 3: 21 positions (R = 63)
    (1, 8, 2, 80, 24, 128, "f16", None, None, True),                 # SQ > SK: top-left limit
    (1, 4, 2, 5, 7, 128, "f16", None, None, False),                  # fewer keys than a sub-page
    (2, 8, 2, 33, 47, 128, "f16", "bool", (2, 8, 33, 47), False),   # full boolean mask
    (2, 8, 2, 33, 47, 64, "bf16", "bool", (1, 1, 33, 30), True),    # width 30 < SK: padded
    (1, 8, 4, 40, 40, 128, "bf16", "add", (1, 8, 1, 40), False),    # additive, per head
    (2, 4, 2, 18, 50, 64, "f16", "add", (2, 1, 18, 1), True),       # width 1: one bias per row
]


def _dense_case_inputs(case, seed=61):
    B, HQ, HK, SQ, SK, D, dtype, kind, dims, causal = case
    g = torch.Generator().manual_seed(seed + SQ + SK)
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    q = torch.randn(B, HQ, SQ, D, generator=g).to(dt)
    k = torch.randn(B, HK, SK, D, generator=g).to(dt)
    v = torch.randn(B, HK, SK, D, generator=g).to(dt)
    mask = None
    if kind == "bool":
        mask = torch.rand(dims, generator=g) < 0.7
        mask[0, 0, 0] = False  # a fully masked row (every key hidden)
    elif kind == "add":
        mask = torch.randn(dims, generator=g).float() * 2.0
    return q, k, v, mask, causal, dtype


def check_dense(out, expect, dtype):
    got = out.detach().cpu().double().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - expect)
    bar = allowed(expect, dtype)
    worst = np.unravel_index(np.argmax(err - bar), err.shape)
    assert (err <= bar).all(), f"error {err[worst]} > {bar[worst]} at {worst}"


@pytest.mark.parametrize("case", DENSE_GPU, ids=lambda c: "-".join(map(str, c[:8])) + ("-c" if c[9] else ""))
def test_dense_matches_the_oracle(case):
    q, k, v, mask, causal, dtype = _dense_case_inputs(case)
    expect = oracle.dense_attention(q, k, v, 0.09, mask=mask, causal=causal)
    print(f"[gpu] dense {case[:8]}", flush=True)
    out = pa.dense_attention(q.to(DEV), k.to(DEV), v.to(DEV), 0.09,
                             mask=mask.to(DEV) if mask is not None else None, causal=causal)
    torch.cuda.synchronize()
    check_dense(out, expect, dtype)
    if mask is not None and mask.dtype == torch.bool:
        assert (out[0, 0, 0] == 0).all()  # the fully masked row (batch 0, head 0, query 0)


def test_dense_long_causal_rows_sampled():
    # 1 x 32 query heads over 8 KV heads, 1024 positions: three blocks of rows
    # compared with the oracle on the same rows (causal limit given as a mask)
    B, HQ, HK, S, D = 1, 32, 8, 1024, 128
    g = torch.Generator().manual_seed(71)
    q = torch.randn(B, HQ, S, D, generator=g).half()
    k = torch.randn(B, HK, S, D, generator=g).half()
    v = torch.randn(B, HK, S, D, generator=g).half()
    print("[gpu] dense long causal", flush=True)
    out = pa.dense_attention(q.to(DEV), k.to(DEV), v.to(DEV), 0.088, causal=True).cpu()
    for a, n in ((0, 24), (500, 24), (S - 24, 24)):
        vis = (torch.arange(a + n)[None, :] <= torch.arange(a, a + n)[:, None])[None, None]
        expect = oracle.dense_attention(q[:, :, a:a + n], k[:, :, :a + n], v[:, :, :a + n],
                                        0.088, mask=vis, causal=False)
        check_dense(out[:, :, a:a + n], expect, "f16")


# ---------------------------------------------------------------------------
# Dense GQA attention backward (pa_dense_attention_backward) against the oracle
# ---------------------------------------------------------------------------
DENSE_BWD_GPU = DENSE_GPU + [
    (1, 8, 2, 24, 80, 128, "bf16", None, None, True),              # SK > SQ: keys no query sees
    (1, 8, 2, 130, 150, 128, "f16", None, None, False),            # several key blocks and tiles
    (2, 8, 1, 70, 90, 64, "bf16", "bool", (2, 8, 70, 90), True),   # G = 8, D = 64, masked
    (1, 8, 2, 150, 150, 128, "f16", None, None, True),             # 3 key blocks: the middle alone
    (1, 6, 2, 40, 200, 64, "f16", "add", (1, 6, 40, 200), True),   # G = 3 halves, 4 key blocks
]


def _bwd_inputs(case, seed=61):
    q, k, v, mask, causal, dtype = _dense_case_inputs(case, seed)
    g = torch.Generator().manual_seed(seed + 7)
    dout = torch.randn(q.shape, generator=g).to(q.dtype)
    return q, k, v, dout, mask, causal, dtype


def check_grad(name, got, expect, dtype):
    got = got.detach().cpu().double().numpy()
    assert np.isfinite(got).all(), name
    err = np.abs(got - expect)
    bar = allowed(expect, dtype)
    worst = np.unravel_index(np.argmax(err - bar), err.shape) if err.size else None
    print(f"[gpu]   {name}: max err {err.max() if err.size else 0:.3e}, max |ref| "
          f"{np.abs(expect).max() if err.size else 0:.3e}", flush=True)
    assert (err <= bar).all(), f"{name}: error {err[worst]} > {bar[worst]} at {worst}"


@pytest.mark.parametrize("case", DENSE_BWD_GPU,
                         ids=lambda c: "-".join(map(str, c[:8])) + ("-c" if c[9] else ""))
def test_dense_backward_matches_the_oracle(case):
    q, k, v, dout, mask, causal, dtype = _bwd_inputs(case)
    edq, edk, edv = oracle.dense_attention_backward(q, k, v, dout, 0.09, mask=mask, causal=causal)
    print(f"[gpu] dense backward {case[:8]} causal={causal}", flush=True)
    dq, dk, dv = pa.dense_attention_backward(
        q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV), 0.09,
        mask=mask.to(DEV) if mask is not None else None, causal=causal)
    torch.cuda.synchronize()
    check_grad("dq", dq, edq, dtype)
    check_grad("dk", dk, edk, dtype)
    check_grad("dv", dv, edv, dtype)


@pytest.mark.parametrize("causal", [False, True])
def test_dense_backward_empty_sides(causal):
    # no queries: dk and dv are written as zeros; no keys: dq is
    g = torch.Generator().manual_seed(81)
    k = torch.randn(1, 2, 50, 64, generator=g).half().to(DEV)
    v = torch.randn(1, 2, 50, 64, generator=g).half().to(DEV)
    q0 = torch.empty(1, 8, 0, 64, dtype=torch.float16, device=DEV)
    print(f"[gpu] dense backward without queries causal={causal}", flush=True)
    _, dk, dv = pa.dense_attention_backward(q0, k, v, q0, 0.1, causal=causal)
    torch.cuda.synchronize()
    assert (dk == 0).all() and (dv == 0).all()
    q = torch.randn(1, 8, 20, 64, generator=g).half().to(DEV)
    k0 = torch.empty(1, 2, 0, 64, dtype=torch.float16, device=DEV)
    print(f"[gpu] dense backward without keys causal={causal}", flush=True)
    dq, _, _ = pa.dense_attention_backward(q, k0, k0, q, 0.1, causal=causal)
    torch.cuda.synchronize()
    assert (dq == 0).all()


def _oracle_backward_by_head(q, k, v, dout, scale, causal):
    """The oracle's gradients of a one-KV-head problem, one query head per call
    (calls run in parallel threads: the library releases the interpreter lock),
    dk and dv of the group summed over its query heads in float64 (a KV head's
    gradient is the sum of its query heads' contributions)."""
    from concurrent.futures import ThreadPoolExecutor
    assert k.shape[1] == 1
    HQ = q.shape[1]

    def one(h):
        return oracle.dense_attention_backward(q[:, h:h + 1].contiguous(), k, v,
                                               dout[:, h:h + 1].contiguous(), scale,
                                               causal=causal)

    with ThreadPoolExecutor(max_workers=HQ) as ex:
        parts = list(ex.map(one, range(HQ)))
    dq = np.concatenate([p[0] for p in parts], axis=1)
    dk = sum(p[1] for p in parts)
    dv = sum(p[2] for p in parts)
    return dq, dk, dv


def test_dense_prefill_one_group_every_element():
    # One KV head of the prefill the bench times (2048 positions, 4 query heads
    # per KV head, D = 128, causal, fp16): every element of the forward output
    # and of dq, dk and dv against the oracle
    B, HQ, HK, S, D = 1, 4, 1, 2048, 128
    g = torch.Generator().manual_seed(75)
    q = torch.randn(B, HQ, S, D, generator=g).half()
    k = torch.randn(B, HK, S, D, generator=g).half()
    v = torch.randn(B, HK, S, D, generator=g).half()
    dout = torch.randn(B, HQ, S, D, generator=g).half()
    scale = 0.088
    print("[gpu] dense prefill, one group: forward", flush=True)
    out = pa.dense_attention(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal=True)
    print("[gpu] dense prefill, one group: backward", flush=True)
    dq, dk, dv = pa.dense_attention_backward(q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV),
                                             scale, causal=True)
    torch.cuda.synchronize()
    print("[gpu] dense prefill, one group: oracle forward", flush=True)
    check_dense(out, oracle.dense_attention(q, k, v, scale, causal=True), "f16")
    print("[gpu] dense prefill, one group: oracle backward", flush=True)
    edq, edk, edv = _oracle_backward_by_head(q, k, v, dout, scale, True)
    check_grad("dq", dq, edq, "f16")
    check_grad("dk", dk, edk, "f16")
    check_grad("dv", dv, edv, "f16")


def test_dense_backward_prefill_sampled():
    # 1 x 32 query heads over 8 KV heads, 2048 positions, causal, fp16 (the
    # prefill the bench times): dq of three blocks of rows against the oracle on
    # those rows (their keys, the causal limit as a mask); dk and dv through the
    # sums that hold at any size (keys: 0; values: the dout rows of the group)
    B, HQ, HK, S, D = 1, 32, 8, 2048, 128
    g = torch.Generator().manual_seed(73)
    q = torch.randn(B, HQ, S, D, generator=g).half()
    k = torch.randn(B, HK, S, D, generator=g).half()
    v = torch.randn(B, HK, S, D, generator=g).half()
    dout = torch.randn(B, HQ, S, D, generator=g).half()
    scale = 0.088
    print("[gpu] dense backward prefill", flush=True)
    dq, dk, dv = pa.dense_attention_backward(q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV),
                                             scale, causal=True)
    dq, dk, dv = dq.cpu(), dk.cpu().double(), dv.cpu().double()
    for a, n in ((0, 24), (1000, 24), (S - 24, 24)):
        vis = (torch.arange(a + n)[None, :] <= torch.arange(a, a + n)[:, None])[None, None]
        edq, _, _ = oracle.dense_attention_backward(
            q[:, :, a:a + n], k[:, :, :a + n], v[:, :, :a + n], dout[:, :, a:a + n], scale,
            mask=vis, causal=False)
        check_grad(f"dq rows {a}..{a + n - 1}", dq[:, :, a:a + n], edq, "f16")
    G = HQ // HK
    ksum = dk.sum(dim=2).numpy()
    kbar = 2.0 ** -9 * dk.abs().sum(dim=2).numpy() + 1e-2
    assert (np.abs(ksum) <= kbar).all(), np.abs(ksum).max()
    want = dout.double().reshape(B, HK, G, S, D).sum(dim=(2, 3)).numpy()
    vsum = dv.sum(dim=2).numpy()
    vbar = 2.0 ** -9 * dv.abs().sum(dim=2).numpy() + 1e-2
    print(f"[gpu]   sum dk max {np.abs(ksum).max():.3e}, sum dv err "
          f"{np.abs(vsum - want).max():.3e}", flush=True)
    assert (np.abs(vsum - want) <= vbar).all(), np.abs(vsum - want).max()


# ---------------------------------------------------------------------------
# Score staircases: the running maximum moves mid-stream, at odd and even
# sub-pages, and in some row tiles of a wave but not the others (fp16 sums two
# sub-pages' PV products at once, so a move can find one of them waiting)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_dense_score_staircase(dtype, causal):
    q, k, v, scale = P.staircase_dense(2, 8, 2, 200, 128, dtype, [(2, 5), (4, 8)], seed=5)
    expect = oracle.dense_attention(q, k, v, scale, causal=causal)
    print(f"[gpu] dense staircase {dtype} causal={causal}", flush=True)
    out = pa.dense_attention(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal=causal)
    torch.cuda.synchronize()
    check_dense(out, expect, dtype)


@pytest.mark.parametrize("case", [
    (3, 16, 2, 128, 16, 8, "f16", (333, 200, 517)),   # 64 rows per KV head
    (2, 16, 2, 64, 32, 4, "f16", (260, 150)),         # 32 rows, pages of 32 keys
    (2, 16, 2, 128, 16, 8, "bf16", (333, 200)),
], ids=lambda c: "-".join(map(str, c[:7])))
def test_decode_score_staircase(case):
    B, H, KV, D, BS, NQ, dtype, lens = case
    w = P.small(B=B, H=H, KV=KV, D=D, BS=BS, NQ=NQ, causal=True, dtype=dtype, lens=lens, seed=37)
    w = to_device(P.staircase_decode(w, [(3, 9, 15), (2, 7), (11, 20, 26)][:B], seed=9))
    expect = ref(w)
    for parts in (0, 1, 3):
        check(w, gpu_decode(w, num_partitions=parts), expect)


# ---------------------------------------------------------------------------
# Block-table indexing: bit-exact invariants, on every pass-1 kernel family
# ---------------------------------------------------------------------------
# (H, KV, NQ, dtype): R = (H/KV)*NQ query rows per KV head selects the kernel:
# R <= 16 one matrix-core row tile, 17..32 two tiles, 33..64 the cooperative
# two-wave kernel, > 64 the 16-bit vector-ALU kernel; fp32 the vector-ALU one.
BITEXACT = [
    (8, 2, 1, "f16"), (8, 2, 1, "bf16"),     # R = 4
    (16, 2, 3, "f16"), (16, 2, 3, "bf16"),   # R = 24
    (16, 2, 8, "f16"), (16, 2, 8, "bf16"),   # R = 64
    (32, 2, 8, "f16"), (32, 2, 8, "bf16"),   # R = 128
    (8, 2, 1, "f32"),                        # R = 4, fp32
]
BITEXACT_IDS = [f"h{h}-kv{kv}-nq{nq}-{dt}" for h, kv, nq, dt in BITEXACT]


@pytest.mark.parametrize("case", BITEXACT, ids=BITEXACT_IDS)
def test_block_order_is_bit_exact(case):
    H, KV, NQ, dtype = case
    w = P.small(B=3, H=H, KV=KV, D=128, BS=16, NQ=NQ, causal=True, dtype=dtype,
                lens=(70, 16, 333), seed=3)
    expect = ref(w)
    for parts in (0, 3):
        base = gpu_decode(to_device(w), num_partitions=parts)
        check(w, base, expect)
        for seed in (1, 2):
            w2 = to_device(P.relayout(w, shuffle_seed=seed, extra_blocks=7))
            assert torch.equal(gpu_decode(w2, num_partitions=parts), base), (parts, seed)


@pytest.mark.parametrize("case", BITEXACT, ids=BITEXACT_IDS)
def test_unused_pool_space_and_table_entries_are_never_read(case):
    H, KV, NQ, dtype = case
    w = P.small(B=3, H=H, KV=KV, D=128, BS=16, NQ=NQ, dtype=dtype, lens=(45, 3, 160), seed=4)
    clean = to_device(P.relayout(w, shuffle_seed=5, extra_blocks=6))
    poisoned = P.relayout(w, shuffle_seed=5, extra_blocks=6, fill=float("nan"))
    # table entries past each sequence's last page point at poisoned blocks
    spare = sorted(set(range(poisoned.num_blocks)) - set(
        int(poisoned.block_table[b, n]) for b in range(3)
        for n in range((int(poisoned.context_lens[b]) + 15) // 16)))
    wide = np.zeros((3, poisoned.block_table.shape[1] + 4), dtype=np.int32)
    wide[:, :poisoned.block_table.shape[1]] = poisoned.block_table
    for b in range(3):
        used = (int(poisoned.context_lens[b]) + 15) // 16
        wide[b, used:] = spare[b % len(spare)]
    poisoned.block_table = wide
    poisoned.spec = poisoned.spec.replace(max_blocks=wide.shape[1])
    for parts in (0, 3):
        base = gpu_decode(clean, num_partitions=parts)
        out = gpu_decode(to_device(poisoned), num_partitions=parts)
        assert torch.isfinite(out.float()).all()
        assert torch.equal(out, base), parts


@pytest.mark.parametrize("case", BITEXACT, ids=BITEXACT_IDS)
def test_argmax_probe_maps_every_position(case):
    # Every query row of sequence b scores logical position t_b above all other
    # visible keys by more than 150 in log2 units, so every other weight is 0
    # in fp32 and the output is v_t bit for bit, whichever page holds it.
    H, KV, NQ, dtype = case
    ts = [0, 1, 15, 16, 17, 31, 63, 100, 255]
    w = P.small(B=len(ts), H=H, KV=KV, D=128, BS=16, NQ=NQ, dtype=dtype, lens=[256] * len(ts),
                seed=8)
    w = P.relayout(w, shuffle_seed=12, extra_blocks=3, fill=float("nan"))
    w, expect = P.argmax_probe(w, ts)
    wd = to_device(w)
    for parts in (0, 1, 3):
        out = gpu_decode(wd, num_partitions=parts).cpu()
        for b, t in enumerate(ts):
            assert torch.equal(out[b], expect[b]), (parts, b, t)


# ---------------------------------------------------------------------------
# Closed forms and special cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_single_key_returns_new_v_exactly(dtype):
    w = to_device(P.small(B=3, H=8, KV=2, D=128, BS=16, NQ=1, dtype=dtype, lens=(0, 0, 0)))
    out = gpu_decode(w)
    G = 4
    for h in range(8):
        assert torch.equal(out[:, h, 0], w.new_v[:, h // G, 0])


def test_equal_scores_give_the_mean():
    w = P.small(B=2, H=4, KV=2, D=64, NQ=3, causal=True, lens=(21, 300), dtype="f32", seed=9)
    w.q.zero_()
    wd = to_device(w)
    expect = ref(w)
    for parts in (1, 4):
        check(wd, gpu_decode(wd, num_partitions=parts), expect)


# scale 0 (every visible key weighted equally: the mean of V), a negative scale
# (the row max is the most negative q.k) and a sharp one, on every decode family:
# one-wave matrix-core kernel (R = 4), its two-tile form (R = 24), the
# cooperative kernel (R = 64), the 16-bit vector kernel (R = 128), fp32 vector
@pytest.mark.parametrize("H,KV,NQ,dtype", [(8, 2, 1, "f16"), (16, 2, 3, "bf16"), (16, 2, 8, "f16"),
                                           (32, 2, 8, "bf16"), (8, 2, 1, "f32")])
@pytest.mark.parametrize("scale", [0.0, -0.09, 0.6])
def test_scale_edge_cases(H, KV, NQ, dtype, scale):
    w = P.small(B=3, H=H, KV=KV, D=128, NQ=NQ, causal=True, lens=(0, 77, 300), dtype=dtype,
                seed=21)
    w = dataclasses.replace(w, scale=float(np.float32(scale)))
    wd = to_device(w)
    expect = ref(w)
    for parts in (0, 5):
        check(wd, gpu_decode(wd, num_partitions=parts), expect)


def test_causality_is_bit_exact():
    w = P.small(B=2, H=4, KV=2, D=128, NQ=4, causal=True, lens=(10, 90), dtype="bf16", seed=10)
    base = gpu_decode(to_device(w))
    for j in range(1, 4):
        w2 = P.small(B=2, H=4, KV=2, D=128, NQ=4, causal=True, lens=(10, 90), dtype="bf16", seed=10)
        w2.new_k[:, :, j] += 3.0
        w2.new_v[:, :, j] -= 2.0
        out = gpu_decode(to_device(w2))
        assert torch.equal(out[:, :, :j], base[:, :, :j])


@pytest.mark.parametrize("kernel", [pa.PA_KERNEL_MFMA, pa.PA_KERNEL_VALU])
def test_combine_remerges_the_workspace(kernel):
    w = to_device(W.make_workload(SMALL[0], device="cpu"))
    table = torch.from_numpy(w.block_table).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    # VALU: 5 key partitions per sequence; matrix-core: 20 groups, so the
    # longer sequences straddle groups (combine) and the short ones are
    # finished in pass 1
    parts = 20 if kernel == pa.PA_KERNEL_MFMA else 5
    dec = pa.Decoder(w.q, w.k_pool, table, max_context_len=w.max_context_len,
                     num_partitions=parts, kernel=kernel)
    assert dec.partitions > 1 and dec.kernel == kernel
    out = dec(w.q, w.k_pool, w.v_pool, table, lens, w.new_k, w.new_v, w.scale).clone()
    torch.cuda.synchronize()
    check(w, out)
    # rows that went through the workspace are rebuilt from it alone
    s = w.spec
    G = s.H // s.KV
    merged = torch.zeros(s.B, s.H, dtype=torch.bool)
    if kernel == pa.PA_KERNEL_MFMA:
        whole = P.split_single_piece_units(w.context_lens, s.KV, s.NQ, dec.partitions,
                                           dec.chunk_tokens // 16, s.max_blocks * s.BS)
        for b in range(s.B):
            for h in range(s.H):
                merged[b, h] = (b, h // G) not in whole
    else:
        for b in range(s.B):
            merged[b, :] = int(w.context_lens[b]) > dec.chunk_tokens
    assert merged.any() and not merged.all()
    again = out.clone()
    again[merged.to(DEV)] = 0
    pa.paged_attn_combine(dec.problem, lens, dec.workspace, dec.workspace_bytes, again,
                          stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(again, out)


def test_combine_remerges_the_workspace_cooperative_auto_plan():
    # 64 rows per KV head (the cooperative kernel) and the plan's own group
    # count: each sequence also costs 3 positions of the cut (the
    # cooperative family's fixed cost per sequence), which the model follows
    lens = tuple(int(x) for x in np.random.default_rng(31).integers(0, 700, size=12))
    w = to_device(P.small(B=12, H=16, KV=2, D=128, BS=16, NQ=8, causal=True, dtype="f16",
                          lens=lens, seed=32))
    table = torch.from_numpy(w.block_table).to(DEV)
    lens_t = torch.from_numpy(w.context_lens).to(DEV)
    dec = pa.Decoder(w.q, w.k_pool, table, max_context_len=w.max_context_len, causal=True,
                     kernel=pa.PA_KERNEL_MFMA)
    assert dec.partitions > 1
    out = dec(w.q, w.k_pool, w.v_pool, table, lens_t, w.new_k, w.new_v, w.scale).clone()
    torch.cuda.synchronize()
    check(w, out)
    s = w.spec
    G = s.H // s.KV
    whole = P.split_single_piece_units(w.context_lens, s.KV, s.NQ, dec.partitions,
                                       dec.chunk_tokens // 16, s.max_blocks * s.BS, seq_pad=3)
    merged = torch.zeros(s.B, s.H, dtype=torch.bool)
    for b in range(s.B):
        for h in range(s.H):
            merged[b, h] = (b, h // G) not in whole
    assert merged.any() and not merged.all()
    again = out.clone()
    again[merged.to(DEV)] = 0
    pa.paged_attn_combine(dec.problem, lens_t, dec.workspace, dec.workspace_bytes, again,
                          stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(again, out)


def test_workspace_too_small_is_rejected():
    w = to_device(W.make_workload(SMALL[1], device="cpu"))
    table = torch.from_numpy(w.block_table).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    prob = pa.make_problem(w.q, w.k_pool, table, max_context_len=w.max_context_len,
                           num_partitions=4)
    assert pa.pa_plan(prob)[1] == 4
    _, need = pa.pa_workspace_size(prob)
    assert need > 0
    ws = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(w.q)
    rc = pa.paged_attn_decode(prob, w.q, w.k_pool, w.v_pool, table, lens, w.new_k, w.new_v,
                              w.scale, out, ws, need - 16, raise_on_error=False)
    assert rc == pa.PA_ERR_WORKSPACE


def test_plan_on_device_matches_pure_host_plan():
    w = W.make_workload(SMALL[0], device="cpu")
    prob = pa.make_problem(w.q, w.k_pool, torch.from_numpy(w.block_table),
                           max_context_len=w.max_context_len)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert pa.pa_plan(prob)[1:] == pa.pa_plan_ex(prob, cus)[1:]


@pytest.mark.parametrize("spec", [SMALL[1], SMALL[0]], ids=["bf16", "f16"])
@pytest.mark.parametrize("kernel", [pa.PA_KERNEL_MFMA, pa.PA_KERNEL_VALU])
def test_deferred_combine_matches_one_call(kernel, spec):
    # fp16 on the matrix-core family keeps its partial outputs as fp16 o / l
    w = to_device(W.make_workload(spec, device="cpu"))
    table = torch.from_numpy(w.block_table).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    args = (w.q, w.k_pool, w.v_pool, table, lens, w.new_k, w.new_v, w.scale)
    one = pa.Decoder(w.q, w.k_pool, table, max_context_len=w.max_context_len, num_partitions=6,
                     kernel=kernel)
    two = pa.Decoder(w.q, w.k_pool, table, max_context_len=w.max_context_len, num_partitions=6,
                     kernel=kernel, flags=pa.PA_FLAG_DEFER_COMBINE)
    a = one(*args).clone()
    two(*args)
    pa.paged_attn_combine(two.problem, lens, two.workspace, two.workspace_bytes, two.out,
                          stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(a, two.out)
    check(w, a)
