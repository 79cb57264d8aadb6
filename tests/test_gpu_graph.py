"""Decode and prefill run calls captured in a HIP graph (through torch.cuda.CUDAGraph) and
replayed: the run calls enqueue kernels only (no allocation, no memset, no copy), so a
captured step replays with preallocated workspaces.  Every replay is checked against the
eager result of the same inputs, with eager work and synchronisations between replays, and
with new query values written in place between replays (the graph reads the live inputs)."""

import pytest
import torch

from synth import make_decode_case, make_prefill_case
from parity import say
from paged_attention_hd512_amd import PagedDecode, PagedPrefill

pytestmark = pytest.mark.gpu


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return "cuda"


def capture(fn):
    """Captures fn() into a graph after one run on a side stream (torch's recipe)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_check(name, g, q, new_qs, eager, out_g, lse_g):
    for i, q_new in enumerate(new_qs):
        q.copy_(q_new)                     # eager work between replays
        out_g.zero_()
        lse_g.fill_(12345.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        out_e, lse_e = eager(q)
        torch.cuda.synchronize()
        say(f"{name}: replay {i}")
        assert torch.equal(out_g, out_e), f"{name}: replay {i} output differs from eager"
        assert torch.equal(lse_g, lse_e), f"{name}: replay {i} lse differs from eager"


@pytest.mark.parametrize("lens,splits,parked", [([37, 300, 1024, 5000, 16], 0, 0),
                                                 ([37, 300, 1024, 5000, 16], 8, 0),
                                                 ([700, 1500, 37, 3000, 900], 8, 1)])
def test_decode_step_replays_from_a_graph(lens, splits, parked):
    """The last case's plan parks split results in LDS (deferred_partials)."""
    name = f"graph decode splits={splits} parked={parked}"
    say(name)
    c = make_decode_case(lens, 24, 4, 512, 16, num_splits=splits, seed=41, device=dev())
    run = PagedDecode(c.k_pool, c.v_pool, c.kv_indptr, c.kv_indices, c.kv_last_page_len,
                      c.num_qo_heads, kv_dtype=c.kv_dtype, sm_scale=c.sm_scale,
                      window=c.window, num_splits=c.num_splits, out_dtype=c.out_dtype)
    assert run.plan.deferred_partials == parked
    q = c.q.clone()
    out_g, lse_g = run.run(q)
    torch.cuda.synchronize()
    g = capture(lambda: run.run(q, out=out_g, lse=lse_g))
    gen = torch.Generator(device="cpu").manual_seed(7)
    new_qs = [c.q] + [torch.randn(c.q.shape, generator=gen).to(torch.bfloat16).to(c.q.device)
                      for _ in range(3)]
    replay_and_check(name, g, q, new_qs, lambda x: run.run(x), out_g, lse_g)


@pytest.mark.parametrize("qo,kv", [([128, 64], [300, 64]), ([3, 16], [3000, 5000])])
def test_prefill_replays_from_a_graph(qo, kv):
    name = f"graph prefill qo={qo} kv={kv}"
    say(name)
    c = make_prefill_case(qo, kv, 8, 2, 512, 64, seed=43, device=dev())
    run = PagedPrefill(c.k_pool, c.v_pool, c.qo_indptr, c.kv_indptr, c.kv_indices,
                       c.kv_last_page_len, c.num_qo_heads, kv_dtype=c.kv_dtype,
                       sm_scale=c.sm_scale, window=c.window, causal=c.causal,
                       out_dtype=c.out_dtype)
    q = c.q.clone()
    out_g, lse_g = run.run(q)
    torch.cuda.synchronize()
    g = capture(lambda: run.run(q, out=out_g, lse=lse_g))
    gen = torch.Generator(device="cpu").manual_seed(9)
    new_qs = [c.q] + [torch.randn(c.q.shape, generator=gen).to(torch.bfloat16).to(c.q.device)
                      for _ in range(3)]
    replay_and_check(name, g, q, new_qs, lambda x: run.run(x), out_g, lse_g)
    if kv[0] > 1000:
        assert run.plan.num_merges > 0  # the split-K path (two kernels) is the one captured
    # Whole tiles run the plain kernel form, tiles of a few rows the short-tile form.
    assert run.plan.short_tiles == (1 if qo[0] < 16 else 0)
