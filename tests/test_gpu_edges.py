"""GPU parity at the edges of the boundary: score scales of either sign (and zero), runs that
ask for no lse, and K and V pools in separate allocations with different paddings.

The FlashInfer page's commit that adds the (qk, vo) = (512, 512) 16-bit configuration
builds K and V as views of differently padded parent tensors, so that a kernel reading V
through K's strides fails; the combined HND cache alone gives K and V equal strides, so
these cases do the same here for bf16 and FP8 at 512/512 (and the other widths)."""

import numpy as np
import pytest
import torch

from synth import make_decode_case, make_prefill_case
from parity import (say, compare, oracle_decode, oracle_prefill, gpu_decode, gpu_prefill,
                    out_to_np, repad)
import paged_attention_hd512_amd.pa as pa

pytestmark = pytest.mark.gpu


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return "cuda"


@pytest.mark.parametrize("sm_scale", [0.0, -0.04, -1.0 / 512 ** 0.5])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_prefill_and_decode_with_zero_and_negative_scales(sm_scale, kv_dtype):
    """The scale is a free parameter of the definition: zero gives uniform weights over the
    visible keys, a negative one reverses the order of the scores.  Causal rows and
    windows mask keys, which must stay masked whatever the sign."""
    say(f"sm_scale={sm_scale} {kv_dtype}")
    p = make_prefill_case([40, 7, 3], [100, 7, 2000], 8, 2, 512, 16, head_dim_vo=512,
                          kv_dtype=kv_dtype, out_dtype="fp32", sm_scale=sm_scale, seed=61,
                          device=dev())
    _, o, lse = gpu_prefill(p)
    ref, ref_lse = oracle_prefill(p)
    assert np.isfinite(out_to_np(o)).all()
    compare(f"prefill sm_scale={sm_scale} {kv_dtype}", out_to_np(o), ref, lse.cpu().numpy(),
            ref_lse)
    w = make_prefill_case([50], [300], 4, 1, 256, 3, window=17, kv_dtype=kv_dtype,
                          out_dtype="fp32", sm_scale=sm_scale, seed=62, device=dev())
    _, o, lse = gpu_prefill(w)
    ref, ref_lse = oracle_prefill(w)
    compare(f"windowed prefill sm_scale={sm_scale} {kv_dtype}", out_to_np(o), ref,
            lse.cpu().numpy(), ref_lse)
    d = make_decode_case([37, 64, 1000], 12, 4, 512, 16, kv_dtype=kv_dtype, window=100,
                         num_splits=3, out_dtype="fp32", sm_scale=sm_scale, seed=63,
                         device=dev())
    _, o, lse = gpu_decode(d)
    ref, ref_lse = oracle_decode(d)
    compare(f"decode sm_scale={sm_scale} {kv_dtype}", out_to_np(o), ref, lse.cpu().numpy(),
            ref_lse)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "nvfp4"])
def test_runs_without_lse_write_the_same_output(kv_dtype):
    """lse is optional (NULL) in both run calls; the output must not depend on it, split
    and merged requests included."""
    say(f"lse = NULL, {kv_dtype}")
    d = make_decode_case([37, 64, 3000, 0], 12, 4, 512, 16, kv_dtype=kv_dtype, num_splits=4,
                         seed=64, device=dev())
    _, o1, _ = gpu_decode(d)
    _, o2, l2 = gpu_decode(d, with_lse=False)
    assert l2 is None and torch.equal(o1, o2)
    p = make_prefill_case([40, 3, 1], [100, 3000, 5000], 8, 2, 512, 16, head_dim_vo=256,
                          kv_dtype=kv_dtype, seed=65, device=dev())
    from paged_attention_hd512_amd import PagedPrefill
    run = PagedPrefill(p.k_pool, p.v_pool, p.qo_indptr, p.kv_indptr, p.kv_indices,
                       p.kv_last_page_len, p.num_qo_heads, kv_dtype=kv_dtype,
                       k_scale=p.k_scale, v_scale=p.v_scale, sm_scale=p.sm_scale,
                       out_dtype=p.out_dtype, k_sf=p.k_sf, v_sf=p.v_sf)
    assert run.plan.num_merges > 0  # the split path runs too
    o1, _ = run.run(p.q)
    o2, l2 = run.run(p.q, with_lse=False)
    torch.cuda.synchronize()
    assert l2 is None and torch.equal(o1, o2)
    ref, _ = oracle_prefill(p)
    compare(f"prefill without lse {kv_dtype}", out_to_np(o2), ref, out_dtype=p.out_dtype)


@pytest.mark.parametrize("kv_dtype,dqk,dvo,page", [
    ("bf16", 512, 512, 16), ("bf16", 512, 512, 64), ("fp8", 512, 512, 64), ("fp8", 512, 512, 1),
    ("bf16", 512, 256, 3), ("fp8", 256, 256, 32)])
def test_k_and_v_pools_with_different_paddings(kv_dtype, dqk, dvo, page):
    """K and V in two allocations whose rows carry different paddings (so their token,
    head and page strides all differ): decode and prefill must read each pool through its
    own strides."""
    say(f"padded pools {kv_dtype} dims={dqk}/{dvo} page={page}")
    d = make_decode_case([37, 300, 1000, 5], 8, 2, dqk, page, head_dim_vo=dvo,
                         kv_dtype=kv_dtype, out_dtype="fp32", num_splits=2, seed=66,
                         device=dev())
    d.k_pool, d.v_pool = repad(d.k_pool, 16), repad(d.v_pool, 48)
    d.cache = None
    assert d.k_pool.stride()[:3] != d.v_pool.stride()[:3]
    _, o, lse = gpu_decode(d)
    ref, ref_lse = oracle_decode(d)
    compare(f"padded decode {kv_dtype} {dqk}/{dvo}", out_to_np(o), ref, lse.cpu().numpy(),
            ref_lse)
    p = make_prefill_case([40, 3, 70], [300, 900, 70], 8, 2, dqk, page, head_dim_vo=dvo,
                          kv_dtype=kv_dtype, out_dtype="fp32", seed=67, device=dev())
    p.k_pool, p.v_pool = repad(p.k_pool, 48), repad(p.v_pool, 16)
    p.cache = None
    _, o, lse = gpu_prefill(p)
    ref, ref_lse = oracle_prefill(p)
    compare(f"padded prefill {kv_dtype} {dqk}/{dvo}", out_to_np(o), ref, lse.cpu().numpy(),
            ref_lse)


def test_debug_gather_copies_nvfp4_data_and_block_scales_bit_exactly():
    """NVFP4 page-table handling: the debug gather copies each row's packed bytes followed by
    its block-scale codes, through the kernels' address path; the oracle's gather of the
    data and of the scale tensor must equal them byte for byte."""
    import oracle
    for dim, dvo, page in ((512, 512, 16), (512, 256, 1), (256, 256, 64)):
        say(f"nvfp4 gather dims={dim}/{dvo} page={page}")
        c = make_decode_case([37, 64, 1, 100], 4, 2, dim, page, head_dim_vo=dvo,
                             kv_dtype="nvfp4", seed=68, device=dev())
        c.k_pool, c.v_pool = repad(c.k_pool, 16), repad(c.v_pool, 32)
        c.k_sf, c.v_sf = repad(c.k_sf, 32), repad(c.v_sf, 16)
        cache = pa.cache_from_pools(c.k_pool, c.v_pool, "nvfp4", c.k_scale, c.v_scale,
                                    c.k_sf, c.v_sf)
        ip = torch.as_tensor(c.kv_indptr).to(dev())
        ix = torch.as_tensor(c.kv_indices).to(dev())
        la = torch.as_tensor(c.kv_last_page_len).to(dev())
        table = pa.pa_page_table(ip.data_ptr(), ix.data_ptr(), la.data_ptr(), c.batch)
        np_ = lambda t: t.contiguous().cpu().numpy()
        kp, vp, ks, vs = np_(c.k_pool), np_(c.v_pool), np_(c.k_sf), np_(c.v_sf)
        for b in range(c.batch):
            L = int(c.kv_lens[b])
            for h in range(c.num_kv_heads):
                ko = torch.empty((L, dim // 2 + dim // 16), dtype=torch.uint8, device=dev())
                vo = torch.empty((L, dvo // 2 + dvo // 16), dtype=torch.uint8, device=dev())
                pa.pa_debug_gather_kv(cache, table, b, L, h, ko.data_ptr(), vo.data_ptr(),
                                      pa.current_stream_handle())
                torch.cuda.synchronize()
                g = lambda pool: oracle.gather_request_kv(pool, c.kv_indptr, c.kv_indices,
                                                          c.kv_last_page_len, page, b)[:, h]
                assert np.array_equal(np_(ko), np.concatenate([g(kp), g(ks)], axis=1))
                assert np.array_equal(np_(vo), np.concatenate([g(vp), g(vs)], axis=1))
