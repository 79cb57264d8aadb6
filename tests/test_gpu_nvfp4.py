"""GPU parity of NVFP4 decode (packed E2M1 K/V with one E4M3 block scale per 16 head_dim
elements, dequantised on load) with the oracle, through the C ABI.

The FlashInfer NVFP4 page (section "NVFP4 split-KV correctness (added)") reports output
drift when a short query over long KV is split across the key axis; here the split and
unsplit decodes of the same inputs are both held to the oracle's tolerance, and to each
other."""

import numpy as np
import pytest
import torch

import oracle
from synth import make_decode_case, decode_workload
from parity import say, compare, oracle_decode, gpu_decode, out_to_np, pool_to_np, repad

pytestmark = pytest.mark.gpu


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return "cuda"


def test_single_key_requests_return_the_dequantised_v_row_exactly():
    """With one visible key the softmax weight is 1, so the fp32 output is the key's V row
    dequantised (e2m1 x block scale, exact) times v_scale, one rounding: bit for bit the
    oracle's value rounded to fp32.  The lse is sm_scale * k_scale * q.k of that key."""
    for dim, dvo, page in ((512, 512, 16), (256, 256, 1), (512, 256, 3)):
        say(f"nvfp4 single-key rows dims={dim}/{dvo} page={page}")
        c = make_decode_case([1] * 96, 8, 2, dim, page, head_dim_vo=dvo, kv_dtype="nvfp4",
                             out_dtype="fp32", seed=21, device=dev())
        _, o, lse = gpu_decode(c)
        ref, ref_lse = oracle_decode(c)
        got = o.cpu().numpy()
        assert np.array_equal(got, ref.astype(np.float32)), "V dequantisation is not exact"
        assert np.abs(lse.cpu().numpy() - ref_lse).max() < 1e-4


NVFP4_SWEEP = [
    # lens, hq, hkv, dim, dvo, page, window, splits, out
    ([37, 64, 1, 16, 17, 300], 8, 1, 512, 512, 16, 0, 0, "fp32"),
    ([37, 64, 1, 16, 17, 300], 24, 4, 512, 512, 16, 0, 8, "bf16"),
    ([5, 130, 777, 64], 12, 4, 512, 512, 64, 0, 0, "bf16"),
    ([5, 130, 777, 64], 12, 4, 512, 512, 64, 0, 3, "fp32"),
    ([600, 1500, 33, 2048], 16, 8, 512, 512, 1, 100, 0, "bf16"),
    ([600, 1500, 33, 2048], 16, 8, 256, 256, 32, 1024, 0, "fp32"),
    ([600, 1500, 33, 2048], 16, 8, 256, 256, 1, 100, 4, "bf16"),
    ([45, 46, 47, 200], 6, 2, 512, 256, 3, 0, 2, "fp32"),
    ([45, 46, 47, 200], 6, 2, 512, 256, 16, 17, 0, "fp32"),
    ([100, 200, 300], 4, 1, 256, 256, 8, 0, 0, "bf16"),
    ([64, 128, 192], 40, 8, 512, 512, 16, 0, 64, "bf16"),
    ([0, 20, 0, 3], 8, 1, 512, 512, 16, 0, 2, "fp32"),
    # one query head per KV head, and full groups of 8 at the narrower value widths: the
    # value MFMA holds heads 0..7 of its output columns and discards those past the group
    ([37, 64, 1, 16, 17, 300], 4, 4, 512, 512, 16, 0, 0, "bf16"),
    ([100, 200, 300], 2, 2, 256, 256, 16, 0, 0, "fp32"),
    ([45, 46, 47, 200], 16, 2, 512, 256, 16, 0, 0, "bf16"),
    ([100, 200, 300], 8, 1, 256, 256, 8, 0, 3, "bf16"),
]


@pytest.mark.parametrize("lens,hq,hkv,dim,dvo,page,window,splits,out", NVFP4_SWEEP)
def test_nvfp4_decode_sweep(lens, hq, hkv, dim, dvo, page, window, splits, out):
    name = (f"nvfp4 lens={lens} heads={hq}/{hkv} dims={dim}/{dvo} page={page} "
            f"window={window} splits={splits} out={out}")
    say(name)
    c = make_decode_case(lens, hq, hkv, dim, page, head_dim_vo=dvo, kv_dtype="nvfp4",
                         window=window, num_splits=splits, out_dtype=out,
                         seed=len(lens) + hq + 100, device=dev())
    _, o, lse = gpu_decode(c)
    ref, ref_lse = oracle_decode(c)
    compare(name, out_to_np(o), ref, lse.cpu().numpy(), ref_lse, out_dtype=out)


def test_split_and_unsplit_nvfp4_decode_agree_on_long_kv():
    """One query over long NVFP4 KV, unsplit (balanced pieces), and cut into 1, 8 and 64
    key chunks: every result meets the oracle's tolerance and they agree with each other
    to fp32 rounding of the merge."""
    lens = [9000, 12000, 700, 16384]
    c = make_decode_case(lens, 16, 8, 512, 64, head_dim_vo=512, kv_dtype="nvfp4",
                         out_dtype="fp32", seed=33, device=dev())
    ref, ref_lse = oracle_decode(c)
    outs = {}
    for splits in (0, 1, 8, 64):
        say(f"nvfp4 long KV splits={splits}")
        _, o, lse = gpu_decode(c, num_splits=splits)
        compare(f"nvfp4 long KV splits={splits}", out_to_np(o), ref, lse.cpu().numpy(), ref_lse)
        outs[splits] = (out_to_np(o), lse.cpu().numpy())
    for splits in (0, 8, 64):
        assert np.abs(outs[splits][0] - outs[1][0]).max() < 1e-4
        assert np.abs(outs[splits][1] - outs[1][1]).max() < 1e-4


@pytest.mark.slow
def test_full_size_nvfp4_workload_on_every_request():
    say("full-size nvfp4_decode")
    c = decode_workload("nvfp4_decode", device=dev())
    _, o, lse = gpu_decode(c)
    _, o32, lse32 = gpu_decode(c, out_dtype="fp32")
    everyone = list(range(c.batch))
    ref, ref_lse = oracle_decode(c, requests=everyone)
    compare(f"nvfp4_decode all {c.batch} requests, bf16 out", out_to_np(o), ref,
            lse.cpu().numpy(), ref_lse, out_dtype=c.out_dtype)
    compare(f"nvfp4_decode all {c.batch} requests, fp32 out", out_to_np(o32), ref,
            lse32.cpu().numpy(), ref_lse, out_dtype="fp32")


# --------------------------------------------------------------------------- prefill

from synth import make_prefill_case, prefill_workload  # noqa: E402
from parity import oracle_prefill, gpu_prefill  # noqa: E402

NVFP4_PREFILL_SWEEP = [
    # qo_lens, kv_lens, hq, hkv, dqk, dvo, page, causal, window, out
    ([40, 7], [100, 7], 4, 2, 512, 256, 16, True, 0, "fp32"),
    ([130, 64, 1], [300, 64, 1], 16, 8, 512, 256, 1, True, 0, "bf16"),
    ([200, 33], [1100, 40], 6, 2, 512, 256, 3, True, 100, "fp32"),
    ([130, 64], [300, 64], 16, 8, 256, 256, 64, True, 0, "bf16"),
    ([77, 5], [77, 9], 8, 1, 512, 512, 16, False, 0, "fp32"),
    ([64, 0, 65], [64, 10, 200], 3, 1, 512, 512, 64, True, 0, "fp32"),
    # short queries over long KV: the split-K prefill (key chunks merged per tile)
    ([3, 1, 16], [3000, 5000, 2100], 4, 2, 512, 256, 64, True, 0, "fp32"),
    ([16] * 4, [6000] * 4, 16, 8, 512, 256, 16, True, 0, "bf16"),
    ([8, 8], [9000, 9000], 4, 2, 512, 256, 32, True, 3000, "fp32"),
    # 512/512 runs as two passes over the halves of the value head_dim: with the split-K
    # merge, a window and bf16 output too
    ([3, 1, 16], [3000, 5000, 2100], 4, 2, 512, 512, 64, True, 0, "fp32"),
    ([8, 8], [9000, 9000], 4, 2, 512, 512, 16, True, 3000, "bf16"),
    ([130, 64, 1], [300, 64, 1], 16, 8, 512, 512, 1, True, 0, "bf16"),
]


@pytest.mark.parametrize("qo,kv,hq,hkv,dqk,dvo,page,causal,window,out", NVFP4_PREFILL_SWEEP)
def test_nvfp4_prefill_sweep(qo, kv, hq, hkv, dqk, dvo, page, causal, window, out):
    name = (f"nvfp4 prefill qo={qo} kv={kv} heads={hq}/{hkv} dims={dqk}/{dvo} page={page} "
            f"causal={causal} window={window} out={out}")
    say(name)
    c = make_prefill_case(qo, kv, hq, hkv, dqk, page, head_dim_vo=dvo, causal=causal,
                          window=window, out_dtype=out, kv_dtype="nvfp4", seed=sum(qo) + hq + 7,
                          device=dev())
    _, o, lse = gpu_prefill(c)
    ref, ref_lse = oracle_prefill(c)
    compare(name, out_to_np(o), ref, lse.cpu().numpy(), ref_lse, out_dtype=out)


def test_split_nvfp4_prefill_of_one_token_equals_unsplit_decode():
    """The geometry of the page's split-KV report (a short query over a long NVFP4 cache):
    the prefill splits each tile's keys into chunks and merges them; the decode of the
    same query token over the same cache, unsplit, must agree with it and with the oracle."""
    from synth import make_decode_case
    lens = [6000, 9000, 700]
    d = make_decode_case(lens, 8, 2, 512, 64, head_dim_vo=256, kv_dtype="nvfp4", num_splits=1,
                         out_dtype="fp32", seed=44, device=dev())
    say("nvfp4 split prefill (q_len 1) vs unsplit decode")
    from paged_attention_hd512_amd import PagedPrefill
    qo_indptr = np.arange(len(lens) + 1, dtype=np.int32)
    pre = PagedPrefill(d.k_pool, d.v_pool, qo_indptr, d.kv_indptr, d.kv_indices,
                       d.kv_last_page_len, d.num_qo_heads, kv_dtype="nvfp4", k_scale=d.k_scale,
                       v_scale=d.v_scale, sm_scale=d.sm_scale, causal=True, out_dtype="fp32",
                       k_sf=d.k_sf, v_sf=d.v_sf)
    assert pre.plan.num_merges > 0  # the split path runs
    po, pl = pre.run(d.q.contiguous())
    _, do, dl = gpu_decode(d)
    ref, ref_lse = oracle_decode(d)
    compare("nvfp4 split prefill", out_to_np(po), ref, pl.cpu().numpy(), ref_lse)
    compare("nvfp4 unsplit decode", out_to_np(do), ref, dl.cpu().numpy(), ref_lse)
    assert np.abs(out_to_np(po) - out_to_np(do)).max() < 2e-3


@pytest.mark.slow
def test_full_size_nvfp4_prefill_on_256_rows_per_request():
    say("full-size nvfp4_prefill (qk 512, vo 256)")
    from test_gpu_prefill import full_size_rows
    c = prefill_workload("nvfp4_prefill", device=dev(), head_dim_vo=256)
    _, o, lse = gpu_prefill(c)
    toks = full_size_rows(c, 256, 7)
    ref, ref_lse = oracle_prefill(c, tokens=toks)
    idx = torch.as_tensor(toks).to(o.device)
    compare(f"nvfp4_prefill {len(toks)} rows", out_to_np(o.index_select(0, idx)), ref,
            lse.index_select(0, idx).cpu().numpy(), ref_lse, out_dtype=c.out_dtype)


@pytest.mark.parametrize("dqk,dvo,page", [(512, 256, 16), (512, 512, 1), (256, 256, 64)])
def test_nvfp4_pools_with_different_stride_families(dqk, dvo, page):
    """K, V and their block-scale tensors in separate allocations with different row
    paddings (the FlashInfer page's test of separately allocated K/V pools and scale
    tensors with different strides): decode and prefill read each through its own
    strides."""
    say(f"nvfp4 padded pools dims={dqk}/{dvo} page={page}")
    from synth import make_decode_case
    d = make_decode_case([37, 300, 1000, 5], 8, 2, dqk, page, head_dim_vo=dvo, kv_dtype="nvfp4",
                         out_dtype="fp32", num_splits=2, seed=51, device=dev())
    d.k_pool, d.v_pool = repad(d.k_pool, 16), repad(d.v_pool, 48)
    d.k_sf, d.v_sf = repad(d.k_sf, 16), repad(d.v_sf, 48)
    d.cache = None
    assert d.k_pool.stride(2) != d.v_pool.stride(2) and d.k_sf.stride(2) != d.v_sf.stride(2)
    _, o, lse = gpu_decode(d)
    ref, ref_lse = oracle_decode(d)
    compare(f"nvfp4 padded decode {dqk}/{dvo}", out_to_np(o), ref, lse.cpu().numpy(), ref_lse)
    p = make_prefill_case([40, 3], [300, 900], 8, 2, dqk, page, head_dim_vo=dvo,
                          kv_dtype="nvfp4", out_dtype="fp32", seed=52, device=dev())
    p.k_pool, p.v_pool = repad(p.k_pool, 48), repad(p.v_pool, 16)
    p.k_sf, p.v_sf = repad(p.k_sf, 32), repad(p.v_sf, 16)
    p.cache = None
    _, o, lse = gpu_prefill(p)
    ref, ref_lse = oracle_prefill(p)
    compare(f"nvfp4 padded prefill {dqk}/{dvo}", out_to_np(o), ref, lse.cpu().numpy(), ref_lse)


def test_nvfp4_decode_replays_from_a_graph():
    say("nvfp4 decode in a captured graph")
    from synth import make_decode_case
    from paged_attention_hd512_amd import PagedDecode
    c = make_decode_case([37, 300, 1024, 5000], 12, 4, 512, 64, kv_dtype="nvfp4", num_splits=0,
                         seed=53, device=dev())
    run = PagedDecode(c.k_pool, c.v_pool, c.kv_indptr, c.kv_indices, c.kv_last_page_len,
                      c.num_qo_heads, kv_dtype="nvfp4", k_scale=c.k_scale, v_scale=c.v_scale,
                      sm_scale=c.sm_scale, out_dtype=c.out_dtype, k_sf=c.k_sf, v_sf=c.v_sf)
    q = c.q.clone()
    out_g, lse_g = run.run(q)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run.run(q, out=out_g, lse=lse_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.run(q, out=out_g, lse=lse_g)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(5)
    for i in range(3):
        q.copy_(torch.randn(c.q.shape, generator=gen).to(torch.bfloat16).to(q.device))
        out_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        out_e, lse_e = run.run(q)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e), f"replay {i}"


WIDENED_PREFILL = [
    # qo_lens, kv_lens, hq, hkv, dqk, dvo, page, window, out, padded pools
    ([2048, 2048], [2600, 2200], 16, 8, 512, 512, 16, 0, "bf16", False),
    ([2048, 2048], [2600, 2200], 16, 8, 512, 512, 16, 0, "fp32", True),
    ([2048, 2048], [2100, 3000], 16, 8, 512, 256, 1, 700, "fp32", False),
    ([8192], [8300], 8, 8, 256, 256, 64, 0, "bf16", True),
]


@pytest.mark.parametrize("qo,kv,hq,hkv,dqk,dvo,page,window,out,padded", WIDENED_PREFILL)
def test_nvfp4_prefill_over_widened_pages(qo, kv, hq, hkv, dqk, dvo, page, window, out, padded):
    """Causal prefills whose tiles read every key several times: the run widens the table's
    NVFP4 pages to bf16 once and runs the bf16 kernel over them (the plan says so); 64
    tokens of every request (all heads) match the oracle on the stored codes, also with K,
    V and their scales in separately padded allocations."""
    from test_gpu_prefill import full_size_rows
    name = f"nvfp4 widened prefill kv={kv} dims={dqk}/{dvo} page={page} window={window} {out}"
    say(name)
    c = make_prefill_case(qo, kv, hq, hkv, dqk, page, head_dim_vo=dvo, causal=True,
                          window=window, out_dtype=out, kv_dtype="nvfp4", seed=sum(kv) + page,
                          device=dev())
    if padded:
        c.k_pool, c.v_pool = repad(c.k_pool, 16), repad(c.v_pool, 48)
        c.k_sf, c.v_sf = repad(c.k_sf, 16), repad(c.v_sf, 32)
        c.cache = c.sf_cache = None
    runner, o, lse = gpu_prefill(c)
    assert runner.plan.staged_pages == int(c.kv_indptr[-1]) and runner.plan.num_merges == 0
    toks = full_size_rows(c, 64, 5)
    ref, ref_lse = oracle_prefill(c, tokens=toks)
    idx = torch.as_tensor(toks).to(o.device)
    compare(name, out_to_np(o.index_select(0, idx)), ref, lse.index_select(0, idx).cpu().numpy(),
            ref_lse, out_dtype=out)
    assert torch.isfinite(o.float()).all()
