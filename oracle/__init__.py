"""Reference oracle for paged-KV GQA decode attention (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this package. The product path (the HIP library and its binding) never imports
it, and this package never imports the product path.

Two independent implementations live here:
  * `paged_decode` / `paged_decode_partitioned`: ctypes calls into the plain C
    oracle (liboracle.so, double precision): block-table gather in logical
    order, then a textbook max-subtracted softmax. `paged_decode_append`: the
    slot-patched step (new rows stored into their pool slots, then the same
    gather).
  * `dense_reference` / `sdpa_reference`: brute force in torch float64 on the
    CPU. The paged cache is first materialised into a dense [B, KV, S, D]
    tensor by fancy indexing, query heads are expanded with repeat_interleave,
    and a boolean visibility mask is applied; `sdpa_reference` hands the same
    dense problem to torch.nn.functional.scaled_dot_product_attention.
Both follow the docs.rs source page "onnxruntime-ep-mlx 0.31.1:
src/ops/paged_attention.rs" (VECTOR_BODY for the head mapping, visible window
and address; VECTOR_REDUCE for the all-masked row -> 0 convention).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# PAGED_ATTN_ORACLE_LIB selects another build of oracle.c (the sanitizer test's)
_LIB_PATH = os.environ.get("PAGED_ATTN_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
_lib = None

_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


def load_library(path: str):
    """Open an oracle shared library (the built one, or a test's variant of it)."""
    lib = ctypes.CDLL(path)
    i, p, f = ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    lib.oracle_paged_decode.argtypes = [i] * 9 + [p] * 7 + [f, p]
    lib.oracle_paged_decode.restype = i
    lib.oracle_paged_decode_partitioned.argtypes = [i] * 9 + [p] * 7 + [f, i, i, p, p, p, p]
    lib.oracle_paged_decode_partitioned.restype = i
    lib.oracle_kv_append.argtypes = [i] * 7 + [p] * 5
    lib.oracle_kv_append.restype = i
    lib.oracle_dense_attention.argtypes = [i] * 7 + [p] * 3 + [i, p, p, i, f, p]
    lib.oracle_dense_attention.restype = i
    lib.oracle_dense_attention_backward.argtypes = [i] * 7 + [p] * 4 + [i, p, p, i, f, p, p, p]
    lib.oracle_dense_attention_backward.restype = i
    lib.oracle_widen.argtypes = [p, ctypes.c_int64, i]
    lib.oracle_widen.restype = ctypes.c_double
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i
    return lib


def _load(lib=None):
    global _lib
    if lib is not None:
        return lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = load_library(_LIB_PATH)
    return _lib


def num_threads() -> int:
    return _load().oracle_num_threads()


def widen(t: torch.Tensor, index: int, lib=None) -> float:
    t = t.detach().cpu().contiguous()
    return _load(lib).oracle_widen(ctypes.c_void_p(t.data_ptr()), index, _DT[t.dtype])


def _host(t: torch.Tensor) -> torch.Tensor:
    return t.detach().cpu().contiguous()


def _common(q, k_pool, v_pool, block_table, context_lens, new_k, new_v):
    q, k_pool, v_pool, new_k, new_v = (_host(x) for x in (q, k_pool, v_pool, new_k, new_v))
    dt = q.dtype
    assert all(x.dtype == dt for x in (k_pool, v_pool, new_k, new_v))
    table = np.ascontiguousarray(block_table, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, H, NQ, D = q.shape
    _, BS, KV, _ = k_pool.shape
    keep = (q, k_pool, v_pool, new_k, new_v, table, lens)
    dims = (B, H, KV, D, BS, table.shape[1] if table.ndim == 2 else 0, NQ)
    ptrs = [ctypes.c_void_p(x.data_ptr()) for x in (q, k_pool, v_pool)]
    ptrs += [table.ctypes.data_as(ctypes.c_void_p), lens.ctypes.data_as(ctypes.c_void_p)]
    ptrs += [ctypes.c_void_p(x.data_ptr()) for x in (new_k, new_v)]
    return keep, dims, _DT[dt], ptrs


def paged_decode(q, k_pool, v_pool, block_table, context_lens, new_k, new_v, scale: float,
                 causal: bool = True, lib=None) -> np.ndarray:
    """Double-precision output [B, H, NQ, D] of the plain C oracle."""
    keep, dims, dt, ptrs = _common(q, k_pool, v_pool, block_table, context_lens, new_k, new_v)
    B, H, KV, D, BS, MB, NQ = dims
    out = np.zeros((B, H, NQ, D), dtype=np.float64)
    rc = _load(lib).oracle_paged_decode(B, H, KV, D, BS, MB, NQ, int(causal), dt, *ptrs,
                                     ctypes.c_float(scale),
                                     out.ctypes.data_as(ctypes.c_void_p))
    del keep
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return out


def paged_decode_partitioned(q, k_pool, v_pool, block_table, context_lens, new_k, new_v,
                             scale: float, chunk: int, causal: bool = True,
                             max_chunks: Optional[int] = None,
                             want_parts: bool = False, lib=None):
    """Partitioned oracle. Returns out, or (out, m, Z, o) with per-chunk states."""
    keep, dims, dt, ptrs = _common(q, k_pool, v_pool, block_table, context_lens, new_k, new_v)
    B, H, KV, D, BS, MB, NQ = dims
    if max_chunks is None:
        longest = int(np.max(context_lens, initial=0)) + NQ
        max_chunks = max(1, -(-longest // chunk))
    out = np.zeros((B, H, NQ, D), dtype=np.float64)
    pm = pz = po = None
    pp = [None, None, None]
    if want_parts:
        pm = np.zeros((B, H, NQ, max_chunks), dtype=np.float64)
        pz = np.zeros_like(pm)
        po = np.zeros((B, H, NQ, max_chunks, D), dtype=np.float64)
        pp = [x.ctypes.data_as(ctypes.c_void_p) for x in (pm, pz, po)]
    rc = _load(lib).oracle_paged_decode_partitioned(B, H, KV, D, BS, MB, NQ, int(causal), dt,
                                                 *ptrs, ctypes.c_float(scale), chunk,
                                                 max_chunks, *pp,
                                                 out.ctypes.data_as(ctypes.c_void_p))
    del keep
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return (out, pm, pz, po) if want_parts else out


def kv_append(k_pool, v_pool, new_k, new_v, slot_mapping, lib=None):
    """Host copies of the pools with this step's new rows stored into their
    slots (C oracle_kv_append); the inputs are not modified."""
    kp, vp = _host(k_pool).clone(), _host(v_pool).clone()
    nk, nv = _host(new_k), _host(new_v)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    NB, BS, KV, D = kp.shape
    B, _, NQ, _ = nk.shape
    assert slots.shape == (B, NQ), "slot_mapping must be [B, NQ]"
    rc = _load(lib).oracle_kv_append(B, KV, D, BS, NB, NQ, _DT[kp.dtype],
                                     ctypes.c_void_p(kp.data_ptr()), ctypes.c_void_p(vp.data_ptr()),
                                     ctypes.c_void_p(nk.data_ptr()), ctypes.c_void_p(nv.data_ptr()),
                                     slots.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return kp, vp


def paged_decode_append(q, k_pool, v_pool, block_table, context_lens, new_k, new_v,
                        slot_mapping, scale: float, causal: bool = True, lib=None):
    """The slot-patched step: (out double [B, H, NQ, D], k_pool after, v_pool after).
    New rows are stored into their slots first; the decode then reads the
    updated pools (a cached position whose slot was written reads the new row)."""
    kp, vp = kv_append(k_pool, v_pool, new_k, new_v, slot_mapping, lib=lib)
    out = paged_decode(q, kp, vp, block_table, context_lens, new_k, new_v, scale,
                       causal=causal, lib=lib)
    return out, kp, vp


MASK_NONE, MASK_BOOL, MASK_ADD = 0, 1, 2


def dense_attention(q, k, v, scale: float, mask=None, causal: bool = False,
                    lib=None) -> np.ndarray:
    """Dense GQA forward (C oracle_dense_attention): q [B, HQ, SQ, D], k/v
    [B, HK, SK, D]; `mask` a 4-D tensor [mb, mh, mq, mw] (bool: visible where
    True; float32: additive bias), each dim 1 or full size, mw <= SK. Returns
    double [B, HQ, SQ, D]."""
    q, k, v = _host(q), _host(k), _host(v)
    B, HQ, SQ, D = q.shape
    _, HK, SK, _ = k.shape
    kind, mptr, dims, keep = MASK_NONE, None, None, None
    if mask is not None:
        m = _host(mask)
        assert m.dim() == 4, "mask must be 4-D [mb, mh, mq, mw]"
        if m.dtype == torch.bool:
            kind, keep = MASK_BOOL, m.to(torch.uint8).contiguous()
        else:
            kind, keep = MASK_ADD, m.to(torch.float32).contiguous()
        mptr = ctypes.c_void_p(keep.data_ptr())
        dims = np.ascontiguousarray(list(m.shape), dtype=np.int32)
    out = np.zeros((B, HQ, SQ, D), dtype=np.float64)
    rc = _load(lib).oracle_dense_attention(
        B, HQ, HK, SQ, SK, D, _DT[q.dtype], ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()), kind, mptr,
        dims.ctypes.data_as(ctypes.c_void_p) if dims is not None else None, int(causal),
        ctypes.c_float(scale), out.ctypes.data_as(ctypes.c_void_p))
    del keep
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return out


def _dense_mask(mask):
    """(kind, pointer, dims, kept tensor) of a 4-D dense-attention mask or None."""
    if mask is None:
        return MASK_NONE, None, None, None
    m = _host(mask)
    assert m.dim() == 4, "mask must be 4-D [mb, mh, mq, mw]"
    if m.dtype == torch.bool:
        kind, keep = MASK_BOOL, m.to(torch.uint8).contiguous()
    else:
        kind, keep = MASK_ADD, m.to(torch.float32).contiguous()
    dims = np.ascontiguousarray(list(m.shape), dtype=np.int32)
    return kind, ctypes.c_void_p(keep.data_ptr()), dims, keep


def dense_attention_backward(q, k, v, dout, scale: float, mask=None, causal: bool = False,
                             lib=None):
    """Dense GQA backward (C oracle_dense_attention_backward): the gradients
    (dq [B, HQ, SQ, D], dk [B, HK, SK, D], dv [B, HK, SK, D]) in double of the
    forward `dense_attention(q, k, v, scale, mask, causal)` for the output
    gradient `dout` [B, HQ, SQ, D] (same dtype as q)."""
    q, k, v, dout = _host(q), _host(k), _host(v), _host(dout)
    B, HQ, SQ, D = q.shape
    _, HK, SK, _ = k.shape
    assert dout.shape == q.shape and dout.dtype == q.dtype
    kind, mptr, dims, keep = _dense_mask(mask)
    dq = np.zeros((B, HQ, SQ, D), dtype=np.float64)
    dk = np.zeros((B, HK, SK, D), dtype=np.float64)
    dv = np.zeros((B, HK, SK, D), dtype=np.float64)
    rc = _load(lib).oracle_dense_attention_backward(
        B, HQ, HK, SQ, SK, D, _DT[q.dtype], ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(dout.data_ptr()), kind, mptr,
        dims.ctypes.data_as(ctypes.c_void_p) if dims is not None else None, int(causal),
        ctypes.c_float(scale), dq.ctypes.data_as(ctypes.c_void_p),
        dk.ctypes.data_as(ctypes.c_void_p), dv.ctypes.data_as(ctypes.c_void_p))
    del keep
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return dq, dk, dv


# ----------------------------------------------------------------------------
# Brute force (torch float64, CPU): an independent dense formulation.
# ----------------------------------------------------------------------------
def _dense_problem(q, k_pool, v_pool, block_table, context_lens, new_k, new_v, causal):
    q = _host(q).double()
    kp, vp = _host(k_pool).double(), _host(v_pool).double()
    nk, nv = _host(new_k).double(), _host(new_v).double()
    table = torch.as_tensor(np.asarray(block_table, dtype=np.int64))
    lens = [int(x) for x in np.asarray(context_lens)]
    B, H, NQ, D = q.shape
    _, BS, KV, _ = kp.shape
    S = max(lens, default=0) + NQ
    K = torch.zeros(B, KV, S, D, dtype=torch.float64)
    V = torch.zeros_like(K)
    visible = torch.zeros(B, NQ, S, dtype=torch.bool)
    for b, L in enumerate(lens):
        pos = torch.arange(L)
        phys = table[b, pos // BS] if L else pos
        # kp[phys, slot] has shape [L, KV, D]; move KV first.
        K[b, :, :L] = kp[phys, pos % BS].permute(1, 0, 2)
        V[b, :, :L] = vp[phys, pos % BS].permute(1, 0, 2)
        K[b, :, L:L + NQ] = nk[b]
        V[b, :, L:L + NQ] = nv[b]
        for r in range(NQ):
            visible[b, r, :L + (r + 1 if causal else NQ)] = True
    G = H // KV
    Kh = K.repeat_interleave(G, dim=1)  # [B, H, S, D]: head h reads KV head h // G
    Vh = V.repeat_interleave(G, dim=1)
    return q, Kh, Vh, visible[:, None, :, :].expand(B, H, NQ, S)


def dense_reference(q, k_pool, v_pool, block_table, context_lens, new_k, new_v, scale: float,
                    causal: bool = True) -> np.ndarray:
    """softmax(scale * q K^T + mask) V with explicit masking; empty rows give 0."""
    qd, Kh, Vh, vis = _dense_problem(q, k_pool, v_pool, block_table, context_lens, new_k,
                                     new_v, causal)
    s = torch.matmul(qd, Kh.transpose(-1, -2)) * float(np.float32(scale))
    s = s.masked_fill(~vis, float("-inf"))
    m = s.amax(dim=-1, keepdim=True)
    empty = torch.isinf(m) & (m < 0)
    w = torch.exp(s - torch.where(empty, torch.zeros_like(m), m))
    w = w.masked_fill(~vis, 0.0)
    z = w.sum(dim=-1, keepdim=True)
    out = torch.matmul(w, Vh) / torch.where(z == 0, torch.ones_like(z), z)
    return out.numpy()


def sdpa_reference(q, k_pool, v_pool, block_table, context_lens, new_k, new_v, scale: float,
                   causal: bool = True) -> np.ndarray:
    """The same dense problem through torch's scaled_dot_product_attention (float64, CPU)."""
    qd, Kh, Vh, vis = _dense_problem(q, k_pool, v_pool, block_table, context_lens, new_k,
                                     new_v, causal)
    out = torch.nn.functional.scaled_dot_product_attention(
        qd, Kh, Vh, attn_mask=vis, scale=float(np.float32(scale)))
    return out.numpy()


def workload_args(w) -> Tuple:
    """(q, k_pool, v_pool, block_table, context_lens, new_k, new_v, scale) of a Workload."""
    return (w.q, w.k_pool, w.v_pool, w.block_table, w.context_lens, w.new_k, w.new_v, w.scale)
