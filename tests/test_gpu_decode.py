"""GPU parity of the decode path (libpa's HIP kernels through the C ABI) with the oracle."""

import numpy as np
import pytest
import torch

import oracle
from synth import make_decode_case, decode_workload
from parity import (say, compare, oracle_decode, gpu_decode, out_to_np, pool_to_np,
                    bf16_to_np, bf16_rne_bits)
import paged_attention_hd512_amd.pa as pa

pytestmark = pytest.mark.gpu


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return "cuda"


def test_fp8_conversion_matches_the_code_table():
    say("fp8 conversion, all 256 codes")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).to(dev())
    out = torch.empty(256, dtype=torch.float32, device=dev())
    pa.pa_debug_fp8_to_f32(codes.data_ptr(), out.data_ptr(), 256, pa.current_stream_handle())
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.E4M3FN_VALUES
    nan = np.isnan(ref)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("dim,dvo,page,kv_dtype", [(512, 512, 16, "bf16"), (256, 256, 1, "bf16"),
                                                   (512, 256, 3, "bf16"), (512, 512, 64, "fp8"),
                                                   (256, 256, 32, "fp8")])
def test_gather_is_bit_exact(dim, dvo, page, kv_dtype):
    say(f"gather dim={dim}/{dvo} page={page} {kv_dtype}")
    c = make_decode_case([37, 64, 1, 100], 4, 2, dim, page, head_dim_vo=dvo, kv_dtype=kv_dtype,
                         seed=3, device=dev())
    cache = pa.cache_from_pools(c.k_pool, c.v_pool, kv_dtype, c.k_scale, c.v_scale)
    ip = torch.as_tensor(c.kv_indptr).to(dev())
    ix = torch.as_tensor(c.kv_indices).to(dev())
    la = torch.as_tensor(c.kv_last_page_len).to(dev())
    table = pa.pa_page_table(ip.data_ptr(), ix.data_ptr(), la.data_ptr(), c.batch)
    kp, vp = pool_to_np(c.k_pool, kv_dtype), pool_to_np(c.v_pool, kv_dtype)
    edt = torch.bfloat16 if kv_dtype == "bf16" else torch.uint8
    for b in range(c.batch):
        L = int(c.kv_lens[b])
        for h in range(c.num_kv_heads):
            ko = torch.empty((L, dim), dtype=edt, device=dev())
            vo = torch.empty((L, dvo), dtype=edt, device=dev())
            pa.pa_debug_gather_kv(cache, table, b, L, h, ko.data_ptr(), vo.data_ptr(),
                                  pa.current_stream_handle())
            torch.cuda.synchronize()
            kr = oracle.gather_request_kv(kp, c.kv_indptr, c.kv_indices, c.kv_last_page_len,
                                          page, b)[:, h]
            vr = oracle.gather_request_kv(vp, c.kv_indptr, c.kv_indices, c.kv_last_page_len,
                                          page, b)[:, h]
            assert np.array_equal(pool_to_np(ko, kv_dtype), kr)
            assert np.array_equal(pool_to_np(vo, kv_dtype), vr)


def test_tiny_decode_workload_split_1_and_2():
    c = decode_workload("tiny_decode", device=dev())
    ref, ref_lse = oracle_decode(c)
    for splits in (1, 2):
        say(f"tiny decode split={splits}")
        before = pa.pa_launch_count()
        runner, out, lse = gpu_decode(c, num_splits=splits)
        launched = pa.pa_launch_count() - before
        assert launched == (1 if splits == 1 else 2)  # the HIP kernels actually ran
        assert out.dtype == torch.float32
        compare(f"tiny split={splits}", out_to_np(out), ref, lse.cpu().numpy(), ref_lse)


SWEEP = [
    # lens, hq, hkv, dim, dvo, page, kv_dtype, window, splits, out
    ([37, 64, 1, 16, 17, 300], 8, 1, 512, 512, 16, "bf16", 0, 0, "fp32"),
    ([37, 64, 1, 16, 17, 300], 24, 4, 512, 512, 16, "bf16", 0, 8, "bf16"),
    ([5, 130, 777, 64], 12, 4, 512, 512, 64, "fp8", 0, 0, "bf16"),
    ([5, 130, 777, 64], 12, 4, 512, 512, 64, "fp8", 0, 3, "fp32"),
    ([600, 1500, 33, 2048], 16, 8, 512, 512, 1, "bf16", 100, 0, "bf16"),
    ([600, 1500, 33, 2048], 16, 8, 512, 512, 32, "bf16", 1024, 0, "fp32"),
    ([600, 1500, 33, 2048], 16, 8, 256, 256, 1, "bf16", 1024, 0, "bf16"),
    ([600, 1500, 33, 2048], 16, 8, 256, 256, 32, "bf16", 100, 4, "bf16"),
    ([45, 46, 47, 200], 6, 2, 512, 256, 3, "bf16", 0, 2, "fp32"),
    ([45, 46, 47, 200], 6, 2, 512, 256, 16, "fp8", 17, 0, "fp32"),
    ([100, 200, 300], 2, 2, 512, 512, 16, "bf16", 0, 5, "fp32"),
    ([100, 200, 300], 4, 1, 256, 256, 8, "fp8", 0, 0, "bf16"),
    ([1, 2, 3, 1000], 16, 2, 512, 512, 16, "bf16", 1, 0, "fp32"),
    ([64, 128, 192], 40, 8, 512, 512, 16, "bf16", 0, 64, "bf16"),
    ([300, 1000, 129, 256], 8, 2, 512, 512, 128, "bf16", 0, 0, "bf16"),
    ([300, 1000, 129, 257], 12, 4, 512, 512, 256, "fp8", 500, 3, "fp32"),
    # groups of 7 and 5 query heads (the 8- and 6-wide instances with idle columns)
    ([700, 1300, 50], 14, 2, 512, 512, 16, "bf16", 0, 0, "fp32"),
    ([700, 1300, 50], 10, 2, 512, 256, 16, "fp8", 0, 3, "bf16"),
]


@pytest.mark.parametrize("lens,hq,hkv,dim,dvo,page,kv_dtype,window,splits,out", SWEEP)
def test_decode_sweep(lens, hq, hkv, dim, dvo, page, kv_dtype, window, splits, out):
    name = (f"lens={lens} heads={hq}/{hkv} dims={dim}/{dvo} page={page} {kv_dtype} "
            f"window={window} splits={splits} out={out}")
    say(name)
    c = make_decode_case(lens, hq, hkv, dim, page, head_dim_vo=dvo, kv_dtype=kv_dtype,
                         window=window, num_splits=splits, out_dtype=out, seed=len(lens) + hq,
                         device=dev())
    _, o, lse = gpu_decode(c)
    ref, ref_lse = oracle_decode(c)
    compare(name, out_to_np(o), ref, lse.cpu().numpy(), ref_lse, out_dtype=out)


def test_empty_requests_give_zero_output_and_minus_inf_lse():
    say("empty requests")
    c = make_decode_case([0, 20, 0], 8, 1, 512, 16, seed=5, device=dev(), out_dtype="fp32",
                         num_splits=2)
    _, o, lse = gpu_decode(c)
    o, lse = out_to_np(o), lse.cpu().numpy()
    assert np.array_equal(o[0], np.zeros_like(o[0])) and np.array_equal(o[2], np.zeros_like(o[2]))
    assert np.all(lse[[0, 2]] == -np.inf)
    ref, ref_lse = oracle_decode(c)
    compare("empty requests", o, ref, lse, ref_lse)


def test_page_relabeling_gives_bit_identical_output_and_runs_are_deterministic():
    say("page permutation invariance")
    c = make_decode_case([37, 64, 500, 1000], 24, 4, 512, 16, num_splits=3, seed=8, device=dev())
    _, o1, l1 = gpu_decode(c)
    _, o1b, l1b = gpu_decode(c)
    assert torch.equal(o1, o1b) and torch.equal(l1, l1b)
    perm = np.random.default_rng(2).permutation(c.num_pages)
    inv = torch.as_tensor(np.argsort(perm)).to(dev())
    cache2 = c.cache.index_select(0, inv)  # page p of the old pool is page perm[p] now
    c.cache, c.k_pool, c.v_pool = cache2, cache2[:, 0], cache2[:, 1]
    c.kv_indices = perm[c.kv_indices].astype(np.int32)
    _, o2, l2 = gpu_decode(c)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_waves_that_run_several_segments():
    """Many short requests: cutting each (request, KV head) on its own would take more
    waves than there are slots, so balanced pieces of 8 blocks span several pairs; waves run
    several segments, some pairs are merged and some are written directly."""
    say("waves with several segments")
    lens = list(np.random.default_rng(11).integers(1, 40, size=2500)) + [0, 700]
    c = make_decode_case(lens, 4, 1, 512, 16, num_splits=0, out_dtype="fp32", seed=12,
                         device=dev())
    runner, o, lse = gpu_decode(c)
    waves = pa.decode_waves(runner.plan, runner.plan_buf)
    assert max(len(w) for w in waves) >= 3
    slots = np.concatenate([w[:, 4] for w in waves])
    assert (slots < 0).any() and (slots >= 0).any()
    ref, ref_lse = oracle_decode(c)
    compare("several segments per wave", out_to_np(o), ref, lse.cpu().numpy(), ref_lse)


def test_fp8_single_key_requests_return_every_value_code_exactly():
    """With one visible key the softmax weight is 1, so the fp32 output is the key's V row
    decoded (E4M3FN, exact) times v_scale, one rounding: bit for bit the oracle's value
    rounded to fp32.  The keys' V rows are rewritten so that every finite E4M3FN code
    appears in every column position class: this checks the kernel's FP8 value decoding
    code by code."""
    for dim, dvo, page in ((512, 512, 16), (256, 256, 1), (512, 256, 3)):
        say(f"fp8 single-key rows, all codes, dims={dim}/{dvo} page={page}")
        c = make_decode_case([1] * 64, 8, 2, dim, page, head_dim_vo=dvo, kv_dtype="fp8",
                             out_dtype="fp32", seed=23, device=dev())
        for b in range(c.batch):
            pg = int(c.kv_indices[c.kv_indptr[b]])  # the request's only key: slot 0
            for h in range(c.num_kv_heads):
                row = (np.arange(dvo) + 7 * (b * c.num_kv_heads + h)) % 256
                row[(row & 0x7F) == 0x7F] = 0  # the NaN codes
                c.v_pool[pg, h, 0, :] = torch.as_tensor(row.astype(np.uint8)).to(dev())
        _, o, lse = gpu_decode(c)
        ref, ref_lse = oracle_decode(c)
        got = o.cpu().numpy()
        assert np.array_equal(got, ref.astype(np.float32)), "FP8 V decoding is not exact"
        assert np.abs(lse.cpu().numpy() - ref_lse).max() < 1e-4


def test_merges_of_more_than_64_segments():
    """Long requests cut into well over 64 balanced segments (129, 130 and 71 with the
    current planner): the merge reads the segments' log-sum-exps 64 at a time and their rows
    8 at a time, so these counts take every path (whole chunks of 64, a partial chunk, a
    tail shorter than 8 rows).  Eight query heads per KV head at 512/512 leave no LDS for
    grouped results, so every segment keeps a slot of its own."""
    say("merges of more than 64 segments")
    c = make_decode_case([16464, 9000], 16, 2, 512, 16, num_splits=0, out_dtype="fp32",
                         seed=21, device=dev())
    runner, o, lse = gpu_decode(c)
    assert runner.plan.grouped_partials == 0
    counts = pa.decode_merges(runner.plan, runner.plan_buf)[:, 3].tolist()
    assert max(counts) > 128 and any(64 < x < 128 for x in counts)
    assert any(x % 8 for x in counts)
    ref, ref_lse = oracle_decode(c)
    compare("more than 64 segments per merge", out_to_np(o), ref, lse.cpu().numpy(), ref_lse)


@pytest.mark.slow
@pytest.mark.parametrize("name,variant", [("gqa_decode", None), ("gqa_decode", "splitk8"),
                                          ("fp8_decode", None),
                                          ("window_decode", (512, 1)),
                                          ("window_decode", (512, 32)),
                                          ("window_decode", (256, 1)),
                                          ("window_decode", (256, 32))])
def test_full_size_workloads_on_every_request(name, variant):
    """The benchmark's workloads at full size, in its launch configuration (bf16 output),
    and the same inputs with fp32 output: the oracle checks every request of both, the
    fp32 output against the literal max-abs bound of 1e-2."""
    say(f"full-size {name} {variant}")
    c = decode_workload(name, device=dev(), variant=variant)
    _, o, lse = gpu_decode(c)
    _, o32, lse32 = gpu_decode(c, out_dtype="fp32")
    everyone = list(range(c.batch))
    ref, ref_lse = oracle_decode(c, requests=everyone)
    compare(f"{name} {variant} all {c.batch} requests, bf16 out", out_to_np(o), ref,
            lse.cpu().numpy(), ref_lse, out_dtype=c.out_dtype)
    compare(f"{name} {variant} all {c.batch} requests, fp32 out", out_to_np(o32), ref,
            lse32.cpu().numpy(), ref_lse, out_dtype="fp32")


@pytest.mark.parametrize("splits", [1, 3])
def test_bf16_output_is_the_rounded_fp32_output(splits):
    say(f"bf16 output = RNE(fp32 output), splits={splits}")
    c = make_decode_case([37, 64, 500], 24, 4, 512, 16, num_splits=splits, seed=4, device=dev())
    _, o32, l32 = gpu_decode(c, out_dtype="fp32")
    _, o16, l16 = gpu_decode(c, out_dtype="bf16")
    assert np.array_equal(bf16_to_np(o16), bf16_rne_bits(o32.cpu().numpy()))
    assert torch.equal(l32, l16)


@pytest.mark.parametrize("kv_dtype,hq,hkv,dim,dvo,page", [
    ("bf16", 24, 4, 512, 512, 16), ("fp8", 12, 4, 512, 512, 64), ("nvfp4", 12, 4, 512, 256, 16),
    ("bf16", 16, 2, 512, 512, 16), ("bf16", 16, 8, 256, 256, 1)])
def test_split_results_parked_in_lds_equal_results_stored_at_once(kv_dtype, hq, hkv, dim, dvo,
                                                                   page):
    """Fixed split-K 8 over short requests: most waves finish split segments before their
    last one, so the plan parks those results in LDS (deferred_partials = 1).  A wave parks
    the first of them and stores any further ones at once (waves here hold up to seven);
    the group of 8 at 512 wide has no LDS to spare and stores them all at once.  The output
    must match the oracle, and the same plan with parking cleared must give the same bits."""
    say(f"parked split results {kv_dtype} G={hq // hkv} dims={dim}/{dvo} page={page}")
    c = make_decode_case([700, 1500, 37, 3000, 900], hq, hkv, dim, page, head_dim_vo=dvo,
                         kv_dtype=kv_dtype, num_splits=8, out_dtype="fp32", seed=70,
                         device=dev())
    run, o, lse = gpu_decode(c)
    assert run.plan.deferred_partials == 1
    waves = pa.decode_waves(run.plan, run.plan_buf)
    assert max(sum(s[4] >= 0 for s in w[:-1]) for w in waves) >= 4
    ref, ref_lse = oracle_decode(c)
    compare(f"parked {kv_dtype} G={hq // hkv}", out_to_np(o), ref, lse.cpu().numpy(), ref_lse)
    run.plan.deferred_partials = 0
    o2, lse2 = run.run(c.q)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("lens,kv_dtype,hq,hkv,dim,dvo,page,window,splits", [
    ([5000, 2100, 64, 1, 3333, 800], "bf16", 24, 4, 512, 512, 16, 0, 0),
    ([5000, 2100, 64, 1, 3333, 800], "bf16", 24, 4, 512, 512, 16, 0, 8),
    ([1024], "bf16", 6, 1, 512, 512, 16, 0, 0),
    ([9000, 4100, 700], "fp8", 12, 4, 512, 512, 64, 0, 0),
    ([9000, 4100, 700], "nvfp4", 12, 4, 512, 256, 16, 0, 0),
    ([3000, 5000, 17, 2500], "bf16", 16, 8, 256, 256, 1, 1100, 0),
    ([6000, 33, 4000], "bf16", 4, 4, 512, 256, 16, 0, 3)])
def test_grouped_split_results(lens, kv_dtype, hq, hkv, dim, dvo, page, window, splits):
    """Consecutive waves of a workgroup whose last segments belong to one split (request,
    KV head) combine those results in LDS, the last to finish writing one slot: the output
    matches the oracle and repeated runs give the same bits (the group merges in wave
    order, whichever wave finishes last).  1024 keys on one KV head make one group of 8
    waves that covers the whole request (a merge of one slot)."""
    say(f"grouped split results {kv_dtype} lens={lens} G={hq // hkv} dims={dim}/{dvo} "
        f"page={page} window={window} splits={splits}")
    c = make_decode_case(lens, hq, hkv, dim, page, head_dim_vo=dvo, kv_dtype=kv_dtype,
                         window=window, num_splits=splits, out_dtype="fp32", seed=71,
                         device=dev())
    run, o, lse = gpu_decode(c)
    assert run.plan.grouped_partials == 1
    groups = pa.decode_groups(run.plan, run.plan_buf)
    assert max(n for n, _ in groups) >= 2
    if lens == [1024]:
        assert groups == [(8, 0)] * 8
        assert pa.decode_merges(run.plan, run.plan_buf)[:, 3].tolist() == [1]
    ref, ref_lse = oracle_decode(c)
    compare(f"grouped {kv_dtype} G={hq // hkv}", out_to_np(o), ref, lse.cpu().numpy(), ref_lse)
    o2, lse2 = run.run(c.q)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
