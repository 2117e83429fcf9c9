"""paged_attn_decode_static (the entry point that allocates nothing) against
paged_attn_decode with a caller workspace: the same kernels, so the outputs
must agree bit for bit, and both must meet the oracle bar. Two calls in a row
on one device share the static array; the second is smaller than the first.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_decode_amd as pa
from paged_kv_gqa_decode_amd import workloads as W
from tests import problems as P
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(w):
    table = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(DEV)
    lens = torch.from_numpy(np.ascontiguousarray(w.context_lens)).to(DEV)
    return (w.q.to(DEV), w.k_pool.to(DEV), w.v_pool.to(DEV), table, lens, w.new_k.to(DEV),
            w.new_v.to(DEV))


def _both(w, num_partitions=0):
    q, kp, vp, table, lens, nk, nv = _inputs(w)
    prob = pa.make_problem(q, kp, table, max_context_len=w.max_context_len,
                           causal=w.spec.causal, num_partitions=num_partitions)
    _, need = pa.pa_workspace_size(prob)
    stream = torch.cuda.current_stream()
    print(f"[gpu] static workspace: {w.spec.name} B={w.spec.B} parts={num_partitions} "
          f"needs {need} B", flush=True)
    # the output is pre-filled with NaN so that an unwritten row shows
    out_static = torch.full_like(q, float("nan"))
    pa.paged_attn_decode_static(prob, q, kp, vp, table, lens, nk, nv, w.scale, out_static,
                                stream=stream)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    out = torch.full_like(q, float("nan"))
    pa.paged_attn_decode(prob, q, kp, vp, table, lens, nk, nv, w.scale, out, ws, need,
                         stream=stream)
    torch.cuda.synchronize()
    return out_static, out, need


@pytest.mark.parametrize("first,second", [
    # a large split plan, then a smaller problem of another geometry
    (W.CONFIGS[4], W.shrink(W.CONFIGS[1], B=5, lengths=("list", (0, 1, 17, 700, 1999)),
                            max_blocks=125)),
    # 64 rows per KV head (fp16 partials), then fp32 on the vector-ALU family
    (W.shrink(W.CONFIGS[3], B=3, lengths=("list", (0, 35, 300)), max_blocks=20),
     W.CONFIGS[0]),
], ids=["ragged_then_llama_small", "multirow_small_then_tiny"])
def test_static_workspace_matches_the_caller_workspace(first, second):
    for i, spec in enumerate((first, second)):
        w = W.make_workload(spec, device=DEV)
        parts = 0 if i == 0 else 3
        out_static, out, need = _both(w, num_partitions=parts)
        assert need <= pa.PA_STATIC_WORKSPACE_BYTES
        assert torch.equal(out_static, out)
        expect = oracle.paged_decode(*P.args(w), causal=spec.causal)
        check(w, out_static, expect)


def test_static_workspace_repeated_calls_keep_matching():
    # the array keeps the previous call's contents: nothing may depend on them
    w = W.make_workload(W.shrink(W.CONFIGS[2], B=2, lengths=("list", (5000, 9001)),
                                 max_blocks=600), device=DEV)
    expect = oracle.paged_decode(*P.args(w), causal=w.spec.causal)
    for parts in (7, 2, 7):
        out_static, out, need = _both(w, num_partitions=parts)
        assert need > 0
        assert torch.equal(out_static, out)
        check(w, out_static, expect)


def test_static_workspace_rejects_what_does_not_fit():
    w = W.make_workload(W.shrink(W.CONFIGS[4], B=64, lengths=("lognormal", 400, 1.0, 16, 3000),
                                 max_blocks=100), device=DEV)
    q, kp, vp, table, lens, nk, nv = _inputs(w)
    out = torch.zeros_like(q)
    # a forced group count whose partial states exceed the static array
    prob = pa.make_problem(q, kp, table, max_context_len=w.max_context_len, num_partitions=40000)
    _, need = pa.pa_workspace_size(prob)
    assert need > pa.PA_STATIC_WORKSPACE_BYTES
    print(f"[gpu] static workspace: rejecting a plan of {need} B", flush=True)
    rc = pa.paged_attn_decode_static(prob, q, kp, vp, table, lens, nk, nv, w.scale, out,
                                     stream=torch.cuda.current_stream(), raise_on_error=False)
    assert rc == pa.PA_ERR_WORKSPACE
    assert "static workspace" in pa.paged_attn_last_error()
    # the deferred merge cannot be used with it
    prob = pa.make_problem(q, kp, table, max_context_len=w.max_context_len,
                           flags=pa.PA_FLAG_DEFER_COMBINE)
    rc = pa.paged_attn_decode_static(prob, q, kp, vp, table, lens, nk, nv, w.scale, out,
                                     stream=torch.cuda.current_stream(), raise_on_error=False)
    assert rc == pa.PA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert (out == 0).all()  # nothing was launched
