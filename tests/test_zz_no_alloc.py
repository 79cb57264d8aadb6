"""pa_paged_decode_static (the decode entry point that allocates nothing: its workspace is a
device array inside the library) against pa_paged_decode with a caller-owned workspace, on
the same plan and inputs: two calls in a row, the second with a smaller batch, each equal
bit for bit to the workspace path and within the oracle's tolerance."""

import numpy as np
import pytest
import torch

from synth import make_decode_case
from parity import say, compare, oracle_decode, out_to_np
import paged_attention_hd512_amd.pa as pa

pytestmark = pytest.mark.gpu


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return "cuda"


def static_decode(plan, plan_buf, q, cache, table, params, out, lse, stream):
    pa.pa_paged_decode_static(plan, plan_buf, q, cache, table, params, out, lse, stream)


def run_both(c):
    from paged_attention_hd512_amd import PagedDecode
    run = PagedDecode(c.k_pool, c.v_pool, c.kv_indptr, c.kv_indices, c.kv_last_page_len,
                      c.num_qo_heads, kv_dtype=c.kv_dtype, k_scale=c.k_scale,
                      v_scale=c.v_scale, sm_scale=c.sm_scale, window=c.window,
                      num_splits=c.num_splits, out_dtype=c.out_dtype, k_sf=c.k_sf, v_sf=c.v_sf)
    assert run.plan.num_merges > 0  # partials go through the workspace
    o_ref, l_ref = run.run(c.q)
    o = torch.full_like(o_ref, float("nan"))
    l = torch.full_like(l_ref, float("nan"))
    before = pa.pa_launch_count()
    static_decode(run.plan, run.plan_buf, c.q.data_ptr(), run.cache, run.table, run.params,
                  o.data_ptr(), l.data_ptr(), pa.current_stream_handle())
    torch.cuda.synchronize()
    assert pa.pa_launch_count() == before + 2  # partial and merge kernels ran
    return o_ref, l_ref, o, l


def test_static_workspace_decode_equals_the_workspace_path_on_two_calls():
    first = make_decode_case([37, 3000, 12000, 500, 64, 8000], 24, 4, 512, 16, num_splits=8,
                             out_dtype="fp32", seed=71, device=dev())
    second = make_decode_case([900, 33], 12, 4, 512, 64, kv_dtype="fp8", num_splits=3,
                              out_dtype="bf16", seed=72, device=dev())
    for name, c in (("first, 6 requests", first), ("second, 2 requests", second)):
        say(f"static-workspace decode: {name}")
        o_ref, l_ref, o, l = run_both(c)
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref), name
        ref, ref_lse = oracle_decode(c)
        compare(f"static workspace {name}", out_to_np(o), ref, l.cpu().numpy(), ref_lse,
                out_dtype=c.out_dtype)


def test_static_workspace_rejects_a_plan_larger_than_it():
    say("static-workspace decode: oversized plan")
    c = make_decode_case([2048] * 16, 64, 8, 512, 16, num_splits=64, seed=73, device=dev())
    from paged_attention_hd512_amd import PagedDecode
    run = PagedDecode(c.k_pool, c.v_pool, c.kv_indptr, c.kv_indices, c.kv_last_page_len,
                      c.num_qo_heads, num_splits=64, sm_scale=c.sm_scale)
    assert run.plan.workspace_bytes > 64 << 20
    out = torch.empty((c.batch, c.num_qo_heads, 512), dtype=torch.bfloat16, device=dev())
    with pytest.raises(pa.PaError) as e:
        static_decode(run.plan, run.plan_buf, c.q.data_ptr(), run.cache, run.table, run.params,
                      out.data_ptr(), None, pa.current_stream_handle())
    assert e.value.status == pa.PA_ERR_WORKSPACE_TOO_SMALL and "static" in e.value.message
