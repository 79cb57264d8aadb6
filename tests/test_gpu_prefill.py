"""GPU parity of the causal paged prefill (libpa's MFMA kernel through the C ABI)."""

import numpy as np
import pytest
import torch

from synth import make_prefill_case, prefill_workload
from parity import (say, compare, oracle_prefill, gpu_prefill, out_to_np, bf16_to_np,
                    bf16_rne_bits)
import paged_attention_hd512_amd.pa as pa

pytestmark = pytest.mark.gpu


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return "cuda"


SWEEP = [
    # qo_lens, kv_lens, hq, hkv, dqk, dvo, page, causal, window, out
    ([40, 7], [100, 7], 4, 2, 512, 256, 16, True, 0, "fp32"),
    ([40, 7], [100, 7], 4, 2, 512, 512, 16, True, 0, "fp32"),
    ([130, 64, 1], [300, 64, 1], 16, 8, 512, 512, 64, True, 0, "bf16"),
    ([130, 64, 1], [300, 64, 1], 16, 8, 256, 256, 1, True, 0, "bf16"),
    ([200, 33], [1100, 40], 6, 2, 512, 256, 3, True, 0, "fp32"),
    ([200, 33], [1100, 40], 6, 2, 512, 512, 32, True, 100, "fp32"),
    ([77, 5], [77, 9], 8, 1, 512, 512, 16, False, 0, "fp32"),
    ([150], [150], 16, 1, 256, 256, 16, True, 17, "bf16"),
    ([64, 0, 65], [64, 10, 200], 3, 1, 512, 512, 64, True, 0, "fp32"),
    ([300], [2000], 2, 2, 512, 512, 64, True, 0, "bf16"),
    # pages holding several 32-key stages (the one-lookup path steps within a page)
    ([260, 70], [1000, 300], 4, 2, 512, 512, 128, True, 0, "fp32"),
    ([129], [900], 8, 4, 512, 256, 256, True, 200, "bf16"),
    # short queries over long KV (split-K prefill: key chunks merged per tile)
    ([3, 1, 16], [3000, 5000, 2100], 4, 2, 512, 512, 64, True, 0, "fp32"),
    ([1, 40], [20000, 700], 8, 2, 512, 256, 16, False, 0, "bf16"),
    ([8, 8], [9000, 9000], 4, 2, 512, 512, 32, True, 3000, "fp32"),
    ([16] * 4, [6000] * 4, 16, 8, 512, 512, 64, True, 0, "bf16"),
    ([5, 2], [2500, 4000], 6, 2, 256, 256, 3, True, 0, "fp32"),
    # groups of 5, 6 and 7 query heads: tiles start and end inside a token's heads
    ([45, 9], [300, 9], 10, 2, 512, 512, 16, True, 0, "fp32"),
    ([45, 9], [300, 9], 12, 2, 512, 256, 16, True, 0, "fp32"),
    ([33], [200], 7, 1, 512, 256, 64, True, 40, "bf16"),
]


@pytest.mark.parametrize("qo,kv,hq,hkv,dqk,dvo,page,causal,window,out", SWEEP)
def test_prefill_sweep(qo, kv, hq, hkv, dqk, dvo, page, causal, window, out):
    name = (f"qo={qo} kv={kv} heads={hq}/{hkv} dims={dqk}/{dvo} page={page} causal={causal} "
            f"window={window} out={out}")
    say(name)
    c = make_prefill_case(qo, kv, hq, hkv, dqk, page, head_dim_vo=dvo, causal=causal,
                          window=window, out_dtype=out, seed=sum(qo) + hq, device=dev())
    before = pa.pa_launch_count()
    runner, o, lse = gpu_prefill(c)
    launches = (1 if sum(qo) > 0 else 0) + (1 if runner.plan.num_merges > 0 else 0)
    assert pa.pa_launch_count() == before + launches
    ref, ref_lse = oracle_prefill(c)
    compare(name, out_to_np(o), ref, lse.cpu().numpy(), ref_lse, out_dtype=out)


FP8_SWEEP = [
    # qo_lens, kv_lens, hq, hkv, dqk, dvo, page, causal, window, out
    ([130, 64, 1], [300, 64, 1], 16, 8, 512, 512, 64, True, 0, "fp32"),
    ([40, 7], [100, 7], 4, 2, 512, 256, 16, True, 0, "fp32"),
    ([130, 64, 1], [300, 64, 1], 16, 8, 256, 256, 1, True, 0, "bf16"),
    ([200, 33], [1100, 40], 6, 2, 512, 512, 1, True, 100, "fp32"),
    ([200, 33], [1100, 40], 6, 2, 512, 256, 64, True, 0, "bf16"),
    ([150], [150], 16, 1, 256, 256, 16, True, 17, "fp32"),
    ([77, 5], [77, 9], 8, 1, 512, 512, 16, False, 0, "fp32"),
    ([64, 0, 65], [64, 10, 200], 3, 1, 256, 256, 64, True, 0, "fp32"),
    ([260, 70], [1000, 300], 4, 2, 512, 512, 128, True, 0, "bf16"),
    # short queries over long KV (split-K prefill: key chunks merged per tile)
    ([3, 1, 16], [3000, 5000, 2100], 4, 2, 512, 512, 64, True, 0, "fp32"),
    ([16] * 4, [6000] * 4, 16, 8, 512, 256, 64, True, 0, "bf16"),
    ([5, 2], [2500, 4000], 6, 2, 256, 256, 3, True, 0, "fp32"),
    ([45, 9], [300, 9], 10, 2, 512, 256, 16, True, 0, "fp32"),
]


@pytest.mark.parametrize("qo,kv,hq,hkv,dqk,dvo,page,causal,window,out", FP8_SWEEP)
def test_fp8_prefill_sweep(qo, kv, hq, hkv, dqk, dvo, page, causal, window, out):
    """FP8 E4M3FN KV, cast on load (the Triton page, section "Approach"), against the
    oracle run on the stored codes, which it dequantises itself."""
    name = (f"fp8 prefill qo={qo} kv={kv} heads={hq}/{hkv} dims={dqk}/{dvo} page={page} "
            f"causal={causal} window={window} out={out}")
    say(name)
    c = make_prefill_case(qo, kv, hq, hkv, dqk, page, head_dim_vo=dvo, causal=causal,
                          window=window, out_dtype=out, kv_dtype="fp8",
                          seed=sum(qo) + hq + 3, device=dev())
    assert c.k_scale != 1.0 and c.v_scale != 1.0
    before = pa.pa_launch_count()
    runner, o, lse = gpu_prefill(c)
    assert pa.pa_launch_count() > before
    ref, ref_lse = oracle_prefill(c)
    compare(name, out_to_np(o), ref, lse.cpu().numpy(), ref_lse, out_dtype=out)


@pytest.mark.parametrize("dqk,dvo,page", [(512, 512, 64), (256, 256, 1), (512, 256, 3)])
def test_fp8_prefill_single_key_rows_return_every_value_code_exactly(dqk, dvo, page):
    """One new token over one key: its weight is 1, so the fp32 output is the key's V row
    widened (E4M3FN to bf16 is exact) times v_scale, one rounding -- bit for bit the
    oracle's value rounded to fp32.  The V rows are rewritten so that every finite code
    appears at many head_dim positions, which checks the stage conversion code by code."""
    say(f"fp8 prefill single-key rows, all codes, dims={dqk}/{dvo} page={page}")
    c = make_prefill_case([1] * 48, [1] * 48, 8, 2, dqk, page, head_dim_vo=dvo,
                          kv_dtype="fp8", out_dtype="fp32", seed=24, device=dev())
    for b in range(c.batch):
        pg = int(c.kv_indices[c.kv_indptr[b]])
        for h in range(c.num_kv_heads):
            row = (np.arange(dvo) + 5 * (b * c.num_kv_heads + h)) % 256
            row[(row & 0x7F) == 0x7F] = 0  # the NaN codes
            c.v_pool[pg, h, 0, :] = torch.as_tensor(row.astype(np.uint8)).to(dev())
    _, o, lse = gpu_prefill(c)
    ref, ref_lse = oracle_prefill(c)
    assert np.array_equal(o.cpu().numpy(), ref.astype(np.float32)), "FP8 V widening is not exact"
    assert np.abs(lse.cpu().numpy() - ref_lse).max() < 1e-4


def test_fp8_prefill_of_one_token_equals_fp8_decode():
    """Prefill with one new token per request and decode read the same FP8 cache; both
    cast on load, so they agree with each other and with the oracle.  Their outputs differ
    by the prefill's bf16-rounded weights in P V (up to 2^-9 relative each; decode applies
    fp32 weights), a few 1e-3 at most for these values, hence 5e-3."""
    say("fp8 prefill q_len 1 vs fp8 decode")
    from parity import gpu_decode, oracle_decode
    from synth import make_decode_case
    lens = [37, 3000, 64]
    d = make_decode_case(lens, 12, 4, 512, 64, kv_dtype="fp8", num_splits=1, out_dtype="fp32",
                         seed=25, device=dev())
    from paged_attention_hd512_amd import PagedPrefill
    pre = PagedPrefill(d.k_pool, d.v_pool, np.arange(len(lens) + 1, dtype=np.int32),
                       d.kv_indptr, d.kv_indices, d.kv_last_page_len, d.num_qo_heads,
                       kv_dtype="fp8", k_scale=d.k_scale, v_scale=d.v_scale,
                       sm_scale=d.sm_scale, out_dtype="fp32")
    po, pl = pre.run(d.q.contiguous())
    _, do, dl = gpu_decode(d)
    ref, ref_lse = oracle_decode(d)
    compare("fp8 prefill, one token", out_to_np(po), ref, pl.cpu().numpy(), ref_lse)
    assert np.abs(out_to_np(po) - out_to_np(do)).max() < 5e-3
    assert np.abs(pl.cpu().numpy() - dl.cpu().numpy()).max() < 1e-4


@pytest.mark.parametrize("dqk,dvo,page", [(512, 512, 64), (512, 256, 16), (256, 256, 3)])
def test_scores_far_above_the_first_stage_max(dqk, dvo, page):
    """Keys from position 100 on get 40x larger K rows, so their scores exceed every
    row's running max by far more than the kernel's rescale threshold: the accumulators
    must be rescaled and the result still match the oracle."""
    say(f"large later scores dims={dqk}/{dvo} page={page}")
    c = make_prefill_case([150, 40], [400, 40], 8, 2, dqk, page, head_dim_vo=dvo,
                          out_dtype="fp32", seed=31, device=dev())
    P = c.page_size
    for b in range(c.batch):
        for t in range(100, int(c.kv_lens[b])):
            pg = int(c.kv_indices[c.kv_indptr[b] + t // P])
            c.k_pool[pg, :, t % P, :] *= 40
    _, o, lse = gpu_prefill(c)
    ref, ref_lse = oracle_prefill(c)
    assert np.isfinite(ref).all()
    compare(f"large later scores {dqk}/{dvo}", out_to_np(o), ref, lse.cpu().numpy(), ref_lse)


def test_prefill_with_one_new_token_equals_decode():
    say("prefill q_len 1 vs decode")
    from parity import gpu_decode
    from synth import make_decode_case
    lens = [37, 300, 16]
    d = make_decode_case(lens, 8, 2, 512, 16, num_splits=1, out_dtype="fp32", seed=21,
                         device=dev())
    p = make_prefill_case([1, 1, 1], lens, 8, 2, 512, 16, out_dtype="fp32", seed=21,
                          device=dev())
    # Same cache and page table: use the decode case's tensors in the prefill run.
    p.k_pool, p.v_pool, p.q = d.k_pool, d.v_pool, d.q.reshape(3, 8, 512).contiguous()
    p.kv_indptr, p.kv_indices, p.kv_last_page_len = d.kv_indptr, d.kv_indices, d.kv_last_page_len
    _, od, ld = gpu_decode(d)
    _, op, lp = gpu_prefill(p)
    assert np.abs(out_to_np(od) - out_to_np(op)).max() < 2e-3
    assert np.abs(ld.cpu().numpy() - lp.cpu().numpy()).max() < 1e-4


def full_size_rows(c, per_request, seed):
    """Query tokens checked in a full-size prefill: per request its first and last two and
    random ones, `per_request` in all (every head of each)."""
    rng = np.random.default_rng(seed)
    toks = []
    for b in range(c.batch):
        q0, q1 = int(c.qo_indptr[b]), int(c.qo_indptr[b + 1])
        fixed = {q0, q0 + 1, q1 - 2, q1 - 1}
        rest = rng.choice(np.arange(q0 + 2, q1 - 2), size=per_request - len(fixed), replace=False)
        toks += sorted(fixed | set(int(x) for x in rest))
    return np.array(toks)


@pytest.mark.slow
@pytest.mark.parametrize("name,dvo", [("causal_prefill", 512), ("causal_prefill", 256),
                                      ("fp8_prefill", 512), ("fp8_prefill", 256)])
def test_full_size_causal_prefill_on_256_rows_per_request(name, dvo):
    """The benchmark's prefill (4 x 4096 new tokens over a 1024-token prefix, 16/8 heads,
    page 64) in its launch configuration (bf16 output) and with fp32 output: the oracle
    checks 256 query tokens (all heads) of every request, the fp32 output against the
    literal max-abs bound of 1e-2."""
    say(f"full-size {name} vo={dvo}")
    c = prefill_workload(name, device=dev(), head_dim_vo=dvo)
    _, o, lse = gpu_prefill(c)
    _, o32, lse32 = gpu_prefill(c, out_dtype="fp32")
    toks = full_size_rows(c, 256, dvo)
    ref, ref_lse = oracle_prefill(c, tokens=toks)
    idx = torch.as_tensor(toks).to(o.device)
    compare(f"{name} vo={dvo} {len(toks)} rows, bf16 out", out_to_np(o.index_select(0, idx)),
            ref, lse.index_select(0, idx).cpu().numpy(), ref_lse, out_dtype=c.out_dtype)
    compare(f"{name} vo={dvo} {len(toks)} rows, fp32 out", out_to_np(o32.index_select(0, idx)),
            ref, lse32.index_select(0, idx).cpu().numpy(), ref_lse, out_dtype="fp32")
    assert torch.isfinite(o.float()).all() and torch.isfinite(o32).all()


@pytest.mark.slow
def test_ragged_prefill_whose_keys_exceed_the_last_level_cache():
    """Three requests of different lengths (600, 1500 and 2500 new tokens over 9000, 6000 and
    2500 keys; 16/8 heads, 512/512 bf16, page 64): 273 MiB of K and V, above the 256 MiB
    last-level cache, so the tiles run request by request (the plan is checked), and 96
    tokens of every request (all heads) match the oracle."""
    say("ragged prefill above the last-level cache")
    c = make_prefill_case([600, 1500, 2500], [9000, 6000, 2500], 16, 8, 512, 64,
                          head_dim_vo=512, causal=True, out_dtype="bf16", seed=77, device=dev())
    runner, o, lse = gpu_prefill(c)
    assert runner.plan.num_merges == 0
    reqs = pa.prefill_items(runner.plan, runner.plan_buf)[:, 0].tolist()
    runs = [b for i, b in enumerate(reqs) if i == 0 or reqs[i - 1] != b]
    assert sorted(runs) == [0, 1, 2], runs  # each request's tiles are contiguous
    toks = full_size_rows(c, 96, 77)
    ref, ref_lse = oracle_prefill(c, tokens=toks)
    idx = torch.as_tensor(toks).to(o.device)
    compare(f"ragged prefill {len(toks)} rows", out_to_np(o.index_select(0, idx)), ref,
            lse.index_select(0, idx).cpu().numpy(), ref_lse, out_dtype=c.out_dtype)
    assert torch.isfinite(o.float()).all()


@pytest.mark.slow
def test_full_size_extend_prefill_is_split_and_matches():
    """The short-query extend workload (8 requests x 16 new tokens over 16368 cached keys,
    16/8 heads, page 64) in its launch configuration: the plan cuts every tile into key
    chunks, and every row of the first and last request matches the oracle."""
    say("full-size extend prefill")
    c = prefill_workload("extend_prefill", device=dev(), head_dim_vo=512)
    runner, o, lse = gpu_prefill(c)
    assert runner.plan.num_merges == c.batch and runner.plan.num_slots >= 2 * c.batch
    toks = []
    for b in (0, c.batch - 1):
        toks += list(range(int(c.qo_indptr[b]), int(c.qo_indptr[b + 1])))
    toks = np.array(toks)
    ref, ref_lse = oracle_prefill(c, tokens=toks)
    idx = torch.as_tensor(toks).to(o.device)
    compare(f"extend prefill rows {len(toks)}", out_to_np(o.index_select(0, idx)), ref,
            lse.index_select(0, idx).cpu().numpy(), ref_lse, out_dtype=c.out_dtype)
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("kv_dtype,dqk,dvo,page", [
    ("bf16", 512, 512, 64), ("bf16", 256, 256, 1), ("fp8", 512, 256, 16), ("fp8", 512, 512, 32),
    ("nvfp4", 512, 256, 16)])
def test_short_tile_form_equals_the_plain_form(kv_dtype, dqk, dvo, page):
    """Tiles of 32, 6 and 80 rows (group 2) keep 2, 1 and 5 of the 8 waves busy, so the
    plan picks the kernel form whose waves without rows only copy stages (short_tiles = 1).
    The output must match the oracle, and the same plan run by the plain form must give the
    same bits."""
    say(f"short-tile form {kv_dtype} dims={dqk}/{dvo} page={page}")
    c = make_prefill_case([16, 3, 40], [3000, 5000, 700], 8, 4, dqk, page, head_dim_vo=dvo,
                          kv_dtype=kv_dtype, causal=True, out_dtype="fp32", seed=71,
                          device=dev())
    run, o, lse = gpu_prefill(c)
    assert run.plan.short_tiles == 1
    ref, ref_lse = oracle_prefill(c)
    compare(f"short tiles {kv_dtype} {dqk}/{dvo}", out_to_np(o), ref, lse.cpu().numpy(), ref_lse,
            out_dtype="fp32")
    run.plan.short_tiles = 0
    o2, lse2 = run.run(c.q)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_bf16_output_is_the_rounded_fp32_output():
    say("prefill bf16 output = RNE(fp32 output)")
    c = make_prefill_case([130, 64], [300, 64], 16, 8, 512, 64, seed=6, device=dev())
    _, o32, l32 = gpu_prefill(c, out_dtype="fp32")
    _, o16, l16 = gpu_prefill(c, out_dtype="bf16")
    assert np.array_equal(bf16_to_np(o16), bf16_rne_bits(o32.cpu().numpy()))
    assert torch.equal(l32, l16)
