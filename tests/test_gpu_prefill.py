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


@pytest.mark.slow
@pytest.mark.parametrize("dvo", [512, 256])
def test_full_size_causal_prefill_on_sampled_rows(dvo):
    """The benchmark's prefill (4 x 4096 new tokens over a 1024-token prefix, 16/8 heads,
    page 64) in its launch configuration; the oracle checks 96 rows spread over the first
    and last request (first, last and random positions), all heads."""
    say(f"full-size causal prefill vo={dvo}")
    c = prefill_workload("causal_prefill", device=dev(), head_dim_vo=dvo)
    _, o, lse = gpu_prefill(c)
    rng = np.random.default_rng(dvo)
    toks = []
    for b in (0, c.batch - 1):
        q0, q1 = int(c.qo_indptr[b]), int(c.qo_indptr[b + 1])
        toks += [q0, q0 + 1, q1 - 1, q1 - 2] + list(rng.integers(q0, q1, size=44))
    toks = np.array(sorted(set(toks)))
    ref, ref_lse = oracle_prefill(c, tokens=toks)
    idx = torch.as_tensor(toks).to(o.device)
    compare(f"prefill vo={dvo} rows {len(toks)}", out_to_np(o.index_select(0, idx)), ref,
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


def test_bf16_output_is_the_rounded_fp32_output():
    say("prefill bf16 output = RNE(fp32 output)")
    c = make_prefill_case([130, 64], [300, 64], 16, 8, 512, 64, seed=6, device=dev())
    _, o32, l32 = gpu_prefill(c, out_dtype="fp32")
    _, o16, l16 = gpu_prefill(c, out_dtype="bf16")
    assert np.array_equal(bf16_to_np(o16), bf16_rne_bits(o32.cpu().numpy()))
    assert torch.equal(l32, l16)
