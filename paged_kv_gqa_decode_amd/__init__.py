"""MI355X-native paged-KV grouped-query decode attention.

Thin ctypes binding of libpaged_attn.so (built from csrc/ with hipcc for
gfx950). Every step of the computation runs in the library's HIP kernels; this
module only marshals arguments: torch tensors -> device pointers, the current
HIP stream, and the pa_problem struct. The entry points keep the C names
declared in include/paged_attn.h.

There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# PAGED_ATTN_LIBRARY selects another build of the library (e.g. a sanitizer build
# of the host code for CPU tests)
LIB_PATH = os.environ.get("PAGED_ATTN_LIBRARY") or os.path.join(HERE, "libpaged_attn.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_DEVICE, PA_ERR_LAUNCH = range(6)
PA_F32, PA_F16, PA_BF16 = 0, 1, 2
PA_KERNEL_AUTO, PA_KERNEL_VALU, PA_KERNEL_MFMA = 0, 1, 2
PA_FLAG_DEFER_COMBINE = 1
PA_MASK_NONE, PA_MASK_BOOL, PA_MASK_ADD = 0, 1, 2

PA_STATIC_WORKSPACE_BYTES = 32 << 20

EXPORTED = ("pa_plan_ex", "pa_plan", "pa_workspace_size", "pa_workspace_size_ex",
            "paged_attn_decode", "paged_attn_decode_append", "paged_attn_decode_static",
            "paged_attn_combine",
            "pa_dense_attention", "pa_dense_backward_workspace_size",
            "pa_dense_attention_backward", "paged_attn_last_error", "paged_attn_version")


class PaProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_heads", "num_kv_heads", "head_dim", "block_size", "num_blocks",
        "max_blocks_per_seq", "nq", "causal", "dtype", "max_context_len", "num_partitions",
        "kernel", "flags")]


class PaDenseProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_heads", "num_kv_heads", "head_dim", "q_len", "kv_len", "causal", "dtype",
        "mask_kind")] + [("mask_dims", ctypes.c_int32 * 4)]


class PagedAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[pa_status {code}] {message}")
        self.code = code


_lib = None


def library(path: Optional[str] = None):
    """Load libpaged_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    # torch ships its own libamdhip64.so.7; whichever copy is loaded first serves
    # the whole process, so let torch load it before this library binds to it.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built: run `python -m paged_kv_gqa_decode_amd.build` "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(p)
    P, vp, i32p = ctypes.POINTER(PaProblem), ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
    szp = ctypes.POINTER(ctypes.c_size_t)
    lib.pa_plan_ex.argtypes = [P, ctypes.c_int32, i32p, i32p, i32p]
    lib.pa_plan.argtypes = [P, i32p, i32p, i32p]
    lib.pa_workspace_size.argtypes = [P, szp]
    lib.pa_workspace_size_ex.argtypes = [P, ctypes.c_int32, szp]
    lib.paged_attn_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp,
                                      ctypes.c_size_t, vp]
    lib.paged_attn_decode_append.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                             vp, vp, ctypes.c_size_t, vp]
    lib.paged_attn_decode_append.restype = ctypes.c_int
    lib.paged_attn_decode_static.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                             vp, vp]
    lib.paged_attn_decode_static.restype = ctypes.c_int
    lib.paged_attn_combine.argtypes = [P, vp, vp, ctypes.c_size_t, vp, vp]
    lib.pa_dense_attention.argtypes = [ctypes.POINTER(PaDenseProblem), vp, vp, vp, vp,
                                       ctypes.c_float, vp, vp]
    lib.pa_dense_attention.restype = ctypes.c_int
    lib.pa_dense_backward_workspace_size.argtypes = [ctypes.POINTER(PaDenseProblem),
                                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.pa_dense_backward_workspace_size.restype = ctypes.c_int
    lib.pa_dense_attention_backward.argtypes = [ctypes.POINTER(PaDenseProblem), vp, vp, vp, vp,
                                                vp, ctypes.c_float, vp, vp, vp, vp,
                                                ctypes.c_size_t, vp]
    lib.pa_dense_attention_backward.restype = ctypes.c_int
    lib.paged_attn_last_error.argtypes = []
    lib.paged_attn_last_error.restype = ctypes.c_char_p
    lib.paged_attn_version.argtypes = []
    for name in ("pa_plan_ex", "pa_plan", "pa_workspace_size", "pa_workspace_size_ex",
                 "paged_attn_decode", "paged_attn_combine", "paged_attn_version"):
        getattr(lib, name).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def paged_attn_last_error() -> str:
    return library().paged_attn_last_error().decode()


def _check(rc: int):
    if rc != PA_OK:
        raise PagedAttnError(rc, paged_attn_last_error())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _stream(stream) -> Optional[int]:
    """None -> the null stream; a torch stream -> its HIP handle; an int -> itself."""
    if stream is None:
        return None
    return getattr(stream, "cuda_stream", stream)


# ---------------------------------------------------------------------------
# C entry points, same names (return the pa_status; raise=True turns errors
# into PagedAttnError).
# ---------------------------------------------------------------------------
def pa_plan_ex(problem: PaProblem, num_cus: int, raise_on_error: bool = True):
    parts, chunk, kern = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    rc = library().pa_plan_ex(ctypes.byref(problem), num_cus, ctypes.byref(parts),
                              ctypes.byref(chunk), ctypes.byref(kern))
    if raise_on_error:
        _check(rc)
    return rc, parts.value, chunk.value, kern.value


def pa_plan(problem: PaProblem, raise_on_error: bool = True):
    parts, chunk, kern = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    rc = library().pa_plan(ctypes.byref(problem), ctypes.byref(parts), ctypes.byref(chunk),
                           ctypes.byref(kern))
    if raise_on_error:
        _check(rc)
    return rc, parts.value, chunk.value, kern.value


def pa_workspace_size(problem: PaProblem, raise_on_error: bool = True):
    n = ctypes.c_size_t()
    rc = library().pa_workspace_size(ctypes.byref(problem), ctypes.byref(n))
    if raise_on_error:
        _check(rc)
    return rc, n.value


def pa_workspace_size_ex(problem: PaProblem, num_cus: int, raise_on_error: bool = True):
    n = ctypes.c_size_t()
    rc = library().pa_workspace_size_ex(ctypes.byref(problem), num_cus, ctypes.byref(n))
    if raise_on_error:
        _check(rc)
    return rc, n.value


def paged_attn_decode(problem: PaProblem, q, k_pool, v_pool, block_table, context_lens, new_k,
                      new_v, scale: float, out, workspace=None, workspace_bytes: int = 0,
                      stream=None, raise_on_error: bool = True) -> int:
    rc = library().paged_attn_decode(
        ctypes.byref(problem), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
        _ptr(context_lens), _ptr(new_k), _ptr(new_v), ctypes.c_float(scale), _ptr(out),
        _ptr(workspace), ctypes.c_size_t(workspace_bytes), _stream(stream))
    if raise_on_error:
        _check(rc)
    return rc


def paged_attn_decode_append(problem: PaProblem, q, k_pool, v_pool, block_table, context_lens,
                             new_k, new_v, slot_mapping, scale: float, out, workspace=None,
                             workspace_bytes: int = 0, stream=None,
                             raise_on_error: bool = True) -> int:
    rc = library().paged_attn_decode_append(
        ctypes.byref(problem), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
        _ptr(context_lens), _ptr(new_k), _ptr(new_v), _ptr(slot_mapping), ctypes.c_float(scale),
        _ptr(out), _ptr(workspace), ctypes.c_size_t(workspace_bytes), _stream(stream))
    if raise_on_error:
        _check(rc)
    return rc


def paged_attn_decode_static(problem: PaProblem, q, k_pool, v_pool, block_table, context_lens,
                             new_k, new_v, scale: float, out, stream=None,
                             raise_on_error: bool = True) -> int:
    rc = library().paged_attn_decode_static(
        ctypes.byref(problem), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
        _ptr(context_lens), _ptr(new_k), _ptr(new_v), ctypes.c_float(scale), _ptr(out),
        _stream(stream))
    if raise_on_error:
        _check(rc)
    return rc


def paged_attn_combine(problem: PaProblem, context_lens, workspace, workspace_bytes: int, out,
                       stream=None, raise_on_error: bool = True) -> int:
    rc = library().paged_attn_combine(ctypes.byref(problem), _ptr(context_lens), _ptr(workspace),
                                      ctypes.c_size_t(workspace_bytes), _ptr(out),
                                      _stream(stream))
    if raise_on_error:
        _check(rc)
    return rc


def pa_dense_attention(problem: PaDenseProblem, q, k, v, mask, scale: float, out, stream=None,
                       raise_on_error: bool = True) -> int:
    rc = library().pa_dense_attention(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(mask), ctypes.c_float(scale), _ptr(out),
                                      _stream(stream))
    if raise_on_error:
        _check(rc)
    return rc


def pa_dense_backward_workspace_size(problem: PaDenseProblem, raise_on_error: bool = True):
    n = ctypes.c_size_t()
    rc = library().pa_dense_backward_workspace_size(ctypes.byref(problem), ctypes.byref(n))
    if raise_on_error:
        _check(rc)
    return rc, n.value


def pa_dense_attention_backward(problem: PaDenseProblem, q, k, v, mask, dout, scale: float, dq,
                                dk, dv, workspace, workspace_bytes: int, stream=None,
                                raise_on_error: bool = True) -> int:
    rc = library().pa_dense_attention_backward(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(dout),
        ctypes.c_float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
        ctypes.c_size_t(workspace_bytes), _stream(stream))
    if raise_on_error:
        _check(rc)
    return rc


def paged_attn_version() -> int:
    return library().paged_attn_version()


# ---------------------------------------------------------------------------
# Torch convenience layer: builds the problem from tensor shapes, allocates
# out/workspace with torch, launches on the current stream.
# ---------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch
    code = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}.get(t.dtype)
    if code is None:
        raise TypeError(f"dtype {t.dtype} is not supported (float32, float16 or bfloat16)")
    return code


def _expect(t, name: str, shape, dtype, device):
    """Raise unless t is a contiguous tensor of that shape, dtype and device (the
    C ABI reads raw pointers, so a wrong dtype, a strided view or a host tensor
    would be read as something else without any error)."""
    if t is None:
        raise ValueError(f"{name} is missing")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device} (the other tensors' device)")
    if not t.is_contiguous():
        raise ValueError(f"{name} is not contiguous (strides {t.stride()}); pass .contiguous()")


def check_decode_args(q, k_pool, v_pool, block_table, context_lens, new_k, new_v, out=None,
                      slot_mapping=None):
    """Shapes, dtypes, devices and contiguity of one decode step's tensors:
    q, out [B, H, NQ, D]; k_pool, v_pool [num_blocks, BS, KV, D] (q's dtype);
    block_table int32 [B, max_blocks_per_seq]; context_lens int32 [B]; new_k,
    new_v [B, KV, NQ, D]; slot_mapping int32 [B, NQ]; all on q's device."""
    import torch
    if q is None or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B, H, NQ, D]")
    if k_pool is None or k_pool.dim() != 4:
        raise ValueError("k_pool must be a 4-D tensor [num_blocks, BS, KV, D]")
    B, H, NQ, D = q.shape
    dt, dev = q.dtype, q.device
    _dtype_code(q)
    KV = k_pool.shape[2]
    _expect(q, "q", (B, H, NQ, D), dt, dev)
    _expect(k_pool, "k_pool", (k_pool.shape[0], k_pool.shape[1], KV, D), dt, dev)
    _expect(v_pool, "v_pool", tuple(k_pool.shape), dt, dev)
    if block_table is None or block_table.dim() != 2:
        raise ValueError("block_table must be a 2-D int32 tensor [B, max_blocks_per_seq]")
    _expect(block_table, "block_table", (B, block_table.shape[1]), torch.int32, dev)
    _expect(context_lens, "context_lens", (B,), torch.int32, dev)
    _expect(new_k, "new_k", (B, KV, NQ, D), dt, dev)
    _expect(new_v, "new_v", (B, KV, NQ, D), dt, dev)
    if out is not None:
        _expect(out, "out", (B, H, NQ, D), dt, dev)
    if slot_mapping is not None:
        _expect(slot_mapping, "slot_mapping", (B, NQ), torch.int32, dev)


def make_problem(q, k_pool, block_table, *, max_context_len: int, causal: bool = True,
                 num_partitions: int = 0, kernel: int = PA_KERNEL_AUTO,
                 flags: int = 0) -> PaProblem:
    if q.dim() != 4 or k_pool.dim() != 4 or block_table.dim() != 2:
        raise ValueError("q [B, H, NQ, D], k_pool [num_blocks, BS, KV, D] and block_table "
                         "[B, max_blocks_per_seq] must be 4-, 4- and 2-D")
    B, H, NQ, D = q.shape
    NB, BS, KV, D2 = k_pool.shape
    if D != D2 or k_pool.dtype != q.dtype:
        raise ValueError(f"q ({q.dtype}, head_dim {D}) and k_pool ({k_pool.dtype}, head_dim "
                         f"{D2}) differ")
    if block_table.shape[0] != B:
        raise ValueError(f"block_table has {block_table.shape[0]} rows for a batch of {B}")
    return PaProblem(batch=B, num_heads=H, num_kv_heads=KV, head_dim=D, block_size=BS,
                     num_blocks=NB, max_blocks_per_seq=block_table.shape[1], nq=NQ,
                     causal=int(causal), dtype=_dtype_code(q),
                     max_context_len=int(max_context_len), num_partitions=int(num_partitions),
                     kernel=int(kernel), flags=int(flags))


class Decoder:
    """Holds the problem, workspace and output of one decode shape for repeated calls."""

    def __init__(self, q, k_pool, block_table, *, max_context_len: int, causal: bool = True,
                 num_partitions: int = 0, kernel: int = PA_KERNEL_AUTO, flags: int = 0):
        import torch
        self.problem = make_problem(q, k_pool, block_table, max_context_len=max_context_len,
                                    causal=causal, num_partitions=num_partitions, kernel=kernel,
                                    flags=flags)
        _, self.partitions, self.chunk_tokens, self.kernel = pa_plan(self.problem)
        _, self.workspace_bytes = pa_workspace_size(self.problem)
        dev = q.device
        # no initial contents are required (zero-filled for reproducible dumps)
        self.workspace = (torch.zeros(self.workspace_bytes, dtype=torch.uint8, device=dev)
                          if self.workspace_bytes else None)
        self.out = torch.empty_like(q)

    def _check_problem(self, q, k_pool, block_table):
        p = self.problem
        if (tuple(q.shape) != (p.batch, p.num_heads, p.nq, p.head_dim)
                or tuple(k_pool.shape) != (p.num_blocks, p.block_size, p.num_kv_heads, p.head_dim)
                or tuple(block_table.shape) != (p.batch, p.max_blocks_per_seq)):
            raise ValueError("the tensors' shapes differ from the ones this Decoder was built for")

    def __call__(self, q, k_pool, v_pool, block_table, context_lens, new_k, new_v, scale,
                 out=None, stream=None, slot_mapping=None, check: bool = True):
        """One step; with slot_mapping (int32 [B, NQ]) the slot-patched step that
        also stores the new rows into the pools. check=False skips the tensor
        checks (for a loop over tensors already checked once)."""
        import torch
        out = self.out if out is None else out
        if check:
            check_decode_args(q, k_pool, v_pool, block_table, context_lens, new_k, new_v, out,
                              slot_mapping)
            self._check_problem(q, k_pool, block_table)
        if stream is None:
            stream = torch.cuda.current_stream()
        if slot_mapping is None:
            paged_attn_decode(self.problem, q, k_pool, v_pool, block_table, context_lens, new_k,
                              new_v, scale, out, self.workspace, self.workspace_bytes, stream)
        else:
            paged_attn_decode_append(self.problem, q, k_pool, v_pool, block_table, context_lens,
                                     new_k, new_v, slot_mapping, scale, out, self.workspace,
                                     self.workspace_bytes, stream)
        return out


def decode(q, k_pool, v_pool, block_table, context_lens, new_k, new_v, scale: float, *,
           max_context_len: int, causal: bool = True, num_partitions: int = 0,
           kernel: int = PA_KERNEL_AUTO, out=None, stream=None):
    """One decode-attention step; returns out [B, H, NQ, D] in q's dtype."""
    check_decode_args(q, k_pool, v_pool, block_table, context_lens, new_k, new_v, out)
    dec = Decoder(q, k_pool, block_table, max_context_len=max_context_len, causal=causal,
                  num_partitions=num_partitions, kernel=kernel)
    return dec(q, k_pool, v_pool, block_table, context_lens, new_k, new_v, scale, out=out,
               stream=stream, check=False)


def decode_append(q, k_pool, v_pool, block_table, context_lens, new_k, new_v, slot_mapping,
                  scale: float, *, max_context_len: int, causal: bool = True,
                  num_partitions: int = 0, kernel: int = PA_KERNEL_AUTO, out=None, stream=None):
    """The slot-patched step: returns out and stores the new rows into k_pool/v_pool."""
    check_decode_args(q, k_pool, v_pool, block_table, context_lens, new_k, new_v, out,
                      slot_mapping)
    dec = Decoder(q, k_pool, block_table, max_context_len=max_context_len, causal=causal,
                  num_partitions=num_partitions, kernel=kernel)
    return dec(q, k_pool, v_pool, block_table, context_lens, new_k, new_v, scale, out=out,
               stream=stream, slot_mapping=slot_mapping, check=False)


def check_dense_args(q, k, v, mask=None, dout=None, out=None):
    """q, out, dout [B, HQ, SQ, D]; k, v [B, HK, SK, D]; same dtype (fp16 or bf16)
    and device, contiguous; mask 4-D [mb, mh, mq, mw] on that device, each dim 1
    or the full size (mw up to SK), uint8/bool or float32, contiguous."""
    import torch
    if q is None or k is None or q.dim() != 4 or k.dim() != 4:
        raise ValueError("q [B, HQ, SQ, D] and k [B, HK, SK, D] must be 4-D tensors")
    B, HQ, SQ, D = q.shape
    _, HK, SK, _ = k.shape
    dt, dev = q.dtype, q.device
    if dt not in (torch.float16, torch.bfloat16):
        raise TypeError(f"dense attention takes float16 or bfloat16, not {dt}")
    _expect(q, "q", (B, HQ, SQ, D), dt, dev)
    _expect(k, "k", (B, HK, SK, D), dt, dev)
    _expect(v, "v", (B, HK, SK, D), dt, dev)
    if dout is not None:
        _expect(dout, "dout", (B, HQ, SQ, D), dt, dev)
    if out is not None:
        _expect(out, "out", (B, HQ, SQ, D), dt, dev)
    if mask is not None:
        if mask.dim() != 4:
            raise ValueError("mask must be 4-D [mb, mh, mq, mw]")
        if mask.dtype not in (torch.bool, torch.uint8, torch.float32):
            raise TypeError(f"mask dtype {mask.dtype}: bool/uint8 (visible) or float32 (bias)")
        if mask.device != dev or not mask.is_contiguous():
            raise ValueError("mask must be contiguous and on q's device")


def make_dense_problem(q, k, *, causal: bool = False, mask=None) -> PaDenseProblem:
    B, HQ, SQ, D = q.shape
    _, HK, SK, _ = k.shape
    p = PaDenseProblem(batch=B, num_heads=HQ, num_kv_heads=HK, head_dim=D, q_len=SQ, kv_len=SK,
                       causal=int(causal), dtype=_dtype_code(q), mask_kind=PA_MASK_NONE)
    if mask is not None:
        import torch
        assert mask.dim() == 4, "mask must be 4-D [mb, mh, mq, mw]"
        p.mask_kind = PA_MASK_BOOL if mask.dtype in (torch.bool, torch.uint8) else PA_MASK_ADD
        for i in range(4):
            p.mask_dims[i] = mask.shape[i]
    return p


def dense_attention(q, k, v, scale: float, *, mask=None, causal: bool = False, out=None,
                    stream=None):
    """Dense GQA attention forward; q [B, HQ, SQ, D], k/v [B, HK, SK, D]; mask 4-D
    [mb, mh, mq, mw], bool (True = visible) or float32 additive. Returns out."""
    import torch
    if mask is not None:
        mask = mask.to(torch.uint8) if mask.dtype == torch.bool else mask.to(torch.float32)
        mask = mask.contiguous()
    check_dense_args(q, k, v, mask, out=out)
    prob = make_dense_problem(q, k, causal=causal, mask=mask)
    out = torch.empty_like(q) if out is None else out
    if stream is None:
        stream = torch.cuda.current_stream()
    pa_dense_attention(prob, q, k, v, mask, scale, out, stream)
    return out


def dense_attention_backward(q, k, v, dout, scale: float, *, mask=None, causal: bool = False,
                             stream=None, workspace=None):
    """Dense GQA attention backward for the forward dense_attention(q, k, v,
    scale, mask=mask, causal=causal) and the output gradient dout (same shape
    and dtype as q). Returns (dq, dk, dv), with dk and dv summed over the query
    heads of each KV head."""
    import torch
    if mask is not None:
        mask = mask.to(torch.uint8) if mask.dtype == torch.bool else mask.to(torch.float32)
        mask = mask.contiguous()
    check_dense_args(q, k, v, mask, dout=dout)
    prob = make_dense_problem(q, k, causal=causal, mask=mask)
    _, need = pa_dense_backward_workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if stream is None:
        stream = torch.cuda.current_stream()
    pa_dense_attention_backward(prob, q, k, v, mask, dout, scale, dq, dk, dv, workspace,
                                workspace.numel(), stream)
    return dq, dk, dv
