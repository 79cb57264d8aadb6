"""CPU tests of libpa's host half: exports, descriptors, planners and argument checks.

Nothing here launches a kernel: the planners and validators never call HIP, and every
failing run-call case below is refused by the host checks before any HIP call.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle.partition import decode_partition_ref, prefill_plan_ref
import paged_attention_hd512_amd.pa as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) == 19
    out = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pa_[a-z0-9_]+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(names) == set(pa.SIGNATURES)  # the binding covers exactly the header


def test_version_and_counter():
    assert "gfx950" in pa.pa_version()
    assert pa.pa_launch_count() >= 0
    assert pa.pa_debug_launch_count() == pa.pa_launch_count()


def params(hq=8, window=0, causal=1, out=pa.PA_DTYPE_FP32, scale=0.05):
    return pa.pa_attn_params(hq, scale, window, causal, pa.PA_DTYPE_BF16, out)


def test_hnd_descriptor_layout():
    c = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_BF16, 10, 4, 16, 512)
    assert (c.k_stride_page, c.k_stride_head, c.k_stride_token) == (2 * 4 * 16 * 512, 16 * 512, 512)
    assert (c.v_stride_page, c.v_stride_head, c.v_stride_token) == (2 * 4 * 16 * 512, 16 * 512, 512)
    assert c.v - c.k == 4 * 16 * 512 * 2  # V half starts one [H, P, D] block later, in bytes
    c8 = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_FP8_E4M3FN, 10, 4, 64, 512, 0.5, 0.25)
    assert c8.v - c8.k == 4 * 64 * 512 and (c8.k_scale, c8.v_scale) == (0.5, 0.25)
    s = pa.pa_kv_cache_separate(0x10000, 0x20000, pa.PA_DTYPE_BF16, 7, 8, 64, 512, 256)
    assert (s.k_stride_page, s.v_stride_page) == (8 * 64 * 512, 8 * 64 * 256)
    assert (s.head_dim_qk, s.head_dim_vo) == (512, 256)


def lens_to_table(lens, P):
    n = [(L + P - 1) // P for L in lens]
    indptr = np.zeros(len(lens) + 1, np.int32)
    indptr[1:] = np.cumsum(n)
    last = np.array([(L - 1) % P + 1 if L > 0 else 0 for L in lens], np.int32)
    return indptr, last


DECODE_CASES = [
    ([37, 64], 16, 0, 1, 1),
    ([37, 64], 16, 0, 2, 1),
    ([1, 15, 16, 17, 0, 300], 16, 0, 8, 2),
    ([1024, 8192, 5000, 4097], 16, 0, 8, 4),
    ([4096, 32768, 9000], 64, 0, 0, 4),
    ([512, 16384, 1000, 1023, 1025], 1, 1024, 0, 8),
    ([512, 16384, 1000], 32, 1024, 0, 8),
    ([100, 5, 0], 3, 7, 3, 1),
    (list(np.random.default_rng(0).integers(1024, 8193, size=32)), 16, 0, 8, 4),
    (list(np.random.default_rng(1).integers(4096, 32769, size=64)), 64, 0, 0, 4),
    # pair-aligned pieces of very different lengths (pairs of 3, 63, 1 and 2 blocks)
    ([40, 1000, 3, 17], 16, 0, 0, 2),
]


def deferred_rule(waves):
    """The planner parks split results in LDS when at least a quarter of the waves finish a
    split segment (slot >= 0) before their last segment."""
    mid = sum(any(seg[4] >= 0 for seg in w[:-1]) for w in waves)
    return int(len(waves) > 0 and 4 * mid >= len(waves))


@pytest.mark.parametrize("lens,P,window,splits,hkv", DECODE_CASES)
def test_decode_plan_matches_reference_partition(lens, P, window, splits, hkv):
    indptr, last = lens_to_table(lens, P)
    cache = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_BF16, int(indptr[-1]) + 1, hkv, P, 512)
    plan, buf = pa.pa_decode_plan(params(hq=hkv * 2, window=window), cache, indptr, last, splits)
    waves = pa.decode_waves(plan, buf)
    merges = pa.decode_merges(plan, buf)
    # Record layout: every segment carries its request's first kv_indices entry; the head
    # segment of wave w sits at index w and names the wave's further segments, which follow
    # the heads wave after wave.
    segs = pa.decode_segments(plan, buf)
    assert (segs[:, 5] == indptr[segs[:, 0]]).all()
    nxt = plan.num_workers
    for w in range(plan.num_workers):
        assert segs[w, 6] == nxt
        nxt += segs[w, 7] & 0xFFFF
    assert nxt == plan.num_items and plan.workers_offset == 32 * plan.num_workers
    assert plan.grouped_partials == 1  # bf16, 2 heads per KV head at 512: results fit LDS
    ref_waves, ref_merges, ref_groups = decode_partition_ref(lens, window, splits, hkv,
                                                             group_last=True)
    assert [[tuple(r) for r in w.tolist()] for w in waves] == ref_waves
    assert [tuple(r) for r in merges.tolist()] == ref_merges
    assert pa.decode_groups(plan, buf) == ref_groups
    assert plan.num_workers == len(ref_waves) and plan.num_merges == len(ref_merges)
    assert plan.num_items == sum(len(w) for w in ref_waves)
    assert plan.num_slots == sum(m[3] for m in ref_merges)
    assert plan.deferred_partials == deferred_rule(ref_waves)
    group, dvo = 2, 512
    assert plan.partial_lse_offset - plan.partial_o_offset >= plan.num_slots * group * dvo * 4
    assert plan.workspace_bytes >= plan.partial_lse_offset + plan.num_slots * group * 4


@pytest.mark.parametrize("lens,P,window,splits,hkv", DECODE_CASES)
def test_reference_partition_covers_visible_keys_exactly(lens, P, window, splits, hkv):
    """Every visible key of every (request, KV head) lies in exactly one segment; inner
    cuts fall on 16-key blocks; waves differ by at most one block; a fixed split's chunk
    boundaries are segment boundaries; slots of a merged pair are consecutive in key
    order; single-segment pairs write directly."""
    waves, merges, _ = decode_partition_ref(lens, window, splits, hkv)
    per_pair = {}
    for w in waves:
        for b, h, t0, t1, slot in w:
            per_pair.setdefault((b, h), []).append((t0, t1, slot))
    merged = {(b, h): (s0, k) for b, h, s0, k in merges}
    for b, L in enumerate(lens):
        L = int(L)
        start = max(0, L - window) if window > 0 else 0
        for h in range(hkv):
            segs = sorted(per_pair.get((b, h), []))
            if L == 0:
                assert segs == [] and merged[(b, h)][1] == 0
                continue
            assert segs[0][0] == start and segs[-1][1] == L
            for (a0, a1, _), (b0, b1, _) in zip(segs, segs[1:]):
                assert a1 == b0 and b0 % 16 == 0
            assert all(t1 > t0 for t0, t1, _ in segs)
            if len(segs) == 1:
                assert segs[0][2] == -1 and (b, h) not in merged
            else:
                s0, k = merged[(b, h)]
                assert k == len(segs) and [s for _, _, s in segs] == list(range(s0, s0 + k))
            if splits > 0:
                # split-K S: the S near-equal chunk boundaries of the pair's blocks are
                # segment boundaries (each chunk is one or more whole segments).
                fb, n = start // 16, -(-L // 16) - start // 16
                c = min(splits, n)
                starts = {t0 for t0, _, _ in segs}
                assert {16 * (fb + n * k // c) for k in range(1, c)} <= starts
                assert len(segs) >= c
    blocks = [sum(-(-t1 // 16) - t0 // 16 for _, _, t0, t1, _ in w) for w in waves]
    assert blocks == sorted(blocks, reverse=True)  # longest first
    # Balanced pieces of at most m blocks (m from the total and the 2048 wave slots); with
    # no fixed split, pieces follow the pair boundaries whenever cutting each pair on its own
    # into pieces of at most m blocks fits the slots: one segment per wave, a pair's pieces
    # within one block of each other.  Otherwise the flattened axis in near-equal parts.
    nblk = [0 if int(L) == 0 else -(-int(L) // 16) - (max(0, int(L) - window) if window > 0 else 0) // 16
            for L in lens]
    units = hkv * sum(nblk)
    if waves:
        m = -(-units // min(2048, -(-units // 8)))
        assert max(blocks) <= m and len(waves) <= 2048
        aligned = splits == 0 and hkv * sum(-(-n // m) for n in nblk) <= 2048
        if aligned:
            assert all(len(w) == 1 for w in waves)
            per_pair = {}
            for w, nb in zip(waves, blocks):
                per_pair.setdefault(tuple(w[0][:2]), []).append(nb)
            assert all(max(v) - min(v) <= 1 for v in per_pair.values())
        else:
            assert max(blocks) - min(blocks) <= 1
    slots = sorted(s for w in waves for *_, s in w if s >= 0)
    assert slots == list(range(len(slots)))  # every slot written once


def test_balanced_partition_of_the_gqa_decode_shape_gives_equal_pieces():
    """The GQA decode shape: at most 2048 waves, every piece holds the largest size that
    2048 pieces would need (ceil(units / 2048) blocks) or one block less, and the fewest
    waves that size allows run, so almost none is short."""
    lens = list(np.random.default_rng(5).integers(1024, 8193, size=32))
    waves, merges, _ = decode_partition_ref(lens, 0, 0, 4)
    total = 4 * sum(-(-int(L) // 16) for L in lens)
    blocks = [sum(-(-t1 // 16) - t0 // 16 for _, _, t0, t1, _ in w) for w in waves]
    m = -(-total // 2048)
    assert sum(blocks) == total
    assert len(waves) <= 2048 and len(waves) == -(-total // m)
    assert max(blocks) == m and min(blocks) >= m - 1
    assert sum(b < m for b in blocks) < len(waves) // 100 + 1
    assert all(1 <= len(w) <= 2 for w in waves)  # pieces of ~36 blocks vs pairs of >= 64


PREFILL_CASES = [
    ([4096] * 4, [5120] * 4, 2, True, 0),
    ([5, 1, 0], [37, 20, 9], 3, True, 0),
    ([33, 7], [40, 7], 6, True, 5),
    ([17], [17], 1, False, 0),
    ([200, 64], [1000, 64], 8, True, 100),
    # short queries over long KV: tiles are split into key chunks
    ([3, 1, 16], [3000, 5000, 2100], 2, True, 0),
    ([16] * 8, [16384] * 8, 2, True, 0),
    ([1, 40], [20000, 700], 4, False, 0),
    ([8, 8], [9000, 9000], 2, True, 3000),
]


def short_tiles_rule(items):
    """The planner's choice of the prefill kernel form for short tiles: 1 when waves left
    without rows (a tile of r rows keeps ceil(r / 16) of its 8 waves busy) hold at least an
    eighth of the wave-stages (32-key stages x 8 waves, summed over the items)."""
    total = idle = 0
    for b, r0, r1, k0, k1, slot in items:
        stages = (k1 + 31) // 32 - k0 // 32 if k1 > k0 else 0
        total += 8 * stages
        idle += (8 - (r1 - r0 + 15) // 16) * stages
    return int(total > 0 and 8 * idle >= total)


@pytest.mark.parametrize("qo,kv,group,causal,window", PREFILL_CASES)
def test_prefill_plan_matches_reference_tiles(qo, kv, group, causal, window):
    P = 16
    indptr, last = lens_to_table(kv, P)
    qo_indptr = np.zeros(len(qo) + 1, np.int32)
    qo_indptr[1:] = np.cumsum(qo)
    hkv = 2
    cache = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_BF16, int(indptr[-1]) + 1, hkv, P, 512)
    plan, buf = pa.pa_prefill_plan(params(hq=hkv * group, window=window, causal=int(causal)),
                                   cache, qo_indptr, indptr, last)
    items = pa.prefill_items(plan, buf)
    merges = pa.prefill_merges(plan, buf)
    ref_items, ref_merges = prefill_plan_ref(qo, kv, group, plan.tile_rows, causal, window, hkv,
                                             kv_bytes_per_key=2 * (512 + 512))
    assert [tuple(r[:5]) + (r[8],) for r in items.tolist()] == [tuple(r) for r in ref_items]
    assert [tuple(r) for r in merges.tolist()] == [tuple(r) for r in ref_merges]
    for r in items:
        b = r[0]
        assert (r[5], r[6], r[7]) == (qo_indptr[b], kv[b], qo[b])
    assert plan.total_q == sum(qo)
    assert plan.short_tiles == short_tiles_rule(ref_items)
    assert plan.num_merges == len(ref_merges)
    assert plan.num_slots == sum(m[5] for m in ref_merges)
    part_rows = plan.num_slots * hkv * plan.tile_rows
    assert plan.partial_lse_offset - plan.partial_o_offset >= part_rows * 512 * 4
    assert plan.workspace_bytes >= plan.partial_lse_offset + part_rows * 8


@pytest.mark.parametrize("seed", range(24))
def test_random_plans_match_the_reference(seed):
    """Random batches (empty and one-key requests, page sizes 1..128, windows, fixed
    splits, group sizes 1..8 or 16): both planners' integers equal the reference rule.
    Run under the host sanitizers too (tests/test_host_sanitized.py)."""
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 40))
    P = int(rng.choice([1, 3, 16, 32, 64, 128]))
    lens = [int(x) for x in rng.integers(0, 3000, size=B)]
    lens[0] = 1
    if B > 1:
        lens[1] = 0
    window = int(rng.choice([0, 0, 1, 17, 1024]))
    splits = int(rng.choice([0, 0, 1, 3, 8, 64]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 3, 6, 8]))
    indptr, last = lens_to_table(lens, P)
    cache = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_BF16, int(indptr[-1]) + 1, hkv, P, 512)
    plan, buf = pa.pa_decode_plan(params(hq=hkv * group, window=window), cache, indptr, last,
                                  splits)
    # bf16 at 512/512: up to 6 heads per KV head leave LDS room for a result per wave
    assert plan.grouped_partials == int(group <= 6)
    ref_waves, ref_merges, ref_groups = decode_partition_ref(lens, window, splits, hkv,
                                                             group_last=group <= 6)
    assert [[tuple(r) for r in w.tolist()] for w in pa.decode_waves(plan, buf)] == ref_waves
    assert [tuple(r) for r in pa.decode_merges(plan, buf).tolist()] == ref_merges
    assert pa.decode_groups(plan, buf) == ref_groups
    assert plan.deferred_partials == deferred_rule(ref_waves)
    qo = [int(rng.integers(0, L + 1)) for L in lens]
    causal = bool(rng.integers(0, 2))
    pgroup = int(rng.choice([1, 2, 6, 16]))
    qo_indptr = np.zeros(B + 1, np.int32)
    qo_indptr[1:] = np.cumsum(qo)
    plan, buf = pa.pa_prefill_plan(params(hq=hkv * pgroup, window=window, causal=int(causal)),
                                   cache, qo_indptr, indptr, last)
    ref_items, ref_pmerges = prefill_plan_ref(qo, lens, pgroup, plan.tile_rows, causal, window,
                                              hkv, kv_bytes_per_key=2 * (512 + 512))
    items = pa.prefill_items(plan, buf)
    assert [tuple(r[:5]) + (r[8],) for r in items.tolist()] == [tuple(r) for r in ref_items]
    assert [tuple(r) for r in pa.prefill_merges(plan, buf).tolist()] == [tuple(r) for r in ref_pmerges]
    assert plan.short_tiles == short_tiles_rule(ref_items)


def test_tiles_run_request_by_request_when_their_keys_exceed_the_last_level_cache():
    """4 x 4096 new tokens (no split-K): over 20000-key requests the tiles read 328 MB of K
    and V, more than the 256 MB last-level cache, so they run request by request (longest
    first within each); over 5120-key requests (84 MB) the longest tiles of all requests run
    first."""
    def order(kv_len):
        indptr, last = lens_to_table([kv_len] * 4, 16)
        qo_indptr = np.arange(5, dtype=np.int32) * 4096
        cache = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_BF16, int(indptr[-1]) + 1, 2, 16, 512)
        plan, buf = pa.pa_prefill_plan(params(hq=4), cache, qo_indptr, indptr, last)
        assert plan.num_merges == 0
        items = pa.prefill_items(plan, buf)
        return items[:, 0].tolist(), (items[:, 4] - items[:, 3]).tolist()
    reqs, lens = order(20000)
    assert reqs == sorted(reqs) and len(set(reqs)) == 4
    for b in range(4):
        run = [n for r, n in zip(reqs, lens) if r == b]
        assert run == sorted(run, reverse=True)
    reqs, lens = order(5120)
    assert lens == sorted(lens, reverse=True) and reqs[:4] == [0, 1, 2, 3]


def test_short_tile_form_is_chosen_for_tiles_of_few_rows():
    """16 new tokens x group 2 fill 2 of a tile's 8 waves: the short-tile form; 4096 new
    tokens fill whole tiles: the plain form."""
    def plan_of(qo, kv):
        indptr, last = lens_to_table(kv, 64)
        qo_indptr = np.zeros(len(qo) + 1, np.int32)
        qo_indptr[1:] = np.cumsum(qo)
        cache = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_BF16, int(indptr[-1]) + 1, 8, 64, 512)
        return pa.pa_prefill_plan(params(hq=16), cache, qo_indptr, indptr, last)[0]
    assert plan_of([16] * 8, [16384] * 8).short_tiles == 1
    assert plan_of([4096] * 4, [5120] * 4).short_tiles == 0
    assert plan_of([4096, 16], [5120, 16384]).short_tiles == 0  # 1 % of the wave-stages idle


@pytest.mark.parametrize("qo,kv,group,causal,window", PREFILL_CASES)
def test_prefill_reference_chunks_cover_each_tile_exactly(qo, kv, group, causal, window):
    """A split tile's chunks are contiguous, cover its key range exactly, start on 32-key
    stages (but the first) and take consecutive slots; whole tiles keep slot -1."""
    hkv = 2
    items, merges = prefill_plan_ref(qo, kv, group, 128, causal, window, hkv)
    by_tile = {}
    for b, r0, r1, kb, ke, slot in items:
        by_tile.setdefault((b, r0, r1), []).append((kb, ke, slot))
    split = {(b, r0, r1): (s0, c) for b, r0, r1, _, s0, c in merges}
    for key, chunks in by_tile.items():
        chunks.sort()
        if key not in split:
            assert len(chunks) == 1 and chunks[0][2] == -1
            continue
        s0, c = split[key]
        assert len(chunks) == c and [s for *_, s in chunks] == list(range(s0, s0 + c))
        for (a0, a1, _), (b0, b1, _) in zip(chunks, chunks[1:]):
            assert a1 == b0 and b0 % 32 == 0 and a1 > a0
    if len(by_tile) * hkv >= 512:
        assert merges == []


# ----------------------------------------------------------------------------- error paths

def decode_plan_status(lens=(37, 64), P=16, hq=8, hkv=1, dim=512, dvo=None, splits=1,
                       kv_dtype=pa.PA_DTYPE_BF16, indptr=None, last=None, scale=(1.0, 1.0)):
    ip, la = lens_to_table(list(lens), P)
    ip = ip if indptr is None else np.asarray(indptr, np.int32)
    la = la if last is None else np.asarray(last, np.int32)
    c = pa.pa_kv_cache()
    c.k, c.v, c.kv_dtype, c.num_pages, c.num_kv_heads, c.page_size = 0, 0, kv_dtype, 100, hkv, P
    c.head_dim_qk, c.head_dim_vo = dim, dim if dvo is None else dvo
    c.k_stride_token = c.v_stride_token = dim
    c.k_stride_head = c.v_stride_head = P * dim
    c.k_stride_page = c.v_stride_page = 2 * hkv * P * dim
    c.k_scale, c.v_scale = scale
    try:
        pa.pa_decode_plan(params(hq=hq), c, ip, la, splits)
        return pa.PA_OK
    except pa.PaError as e:
        assert e.message  # every failure names its cause
        return e.status


@pytest.mark.parametrize("kw,status", [
    (dict(), pa.PA_OK),
    (dict(indptr=[0, 3, 2], last=[5, 16]), pa.PA_ERR_INVALID_ARG),       # decreasing indptr
    (dict(indptr=[1, 3, 7], last=[5, 16]), pa.PA_ERR_INVALID_ARG),       # indptr[0] != 0
    (dict(last=[0, 16]), pa.PA_ERR_INVALID_ARG),                         # last page empty
    (dict(last=[5, 17]), pa.PA_ERR_INVALID_ARG),                         # last page > P
    (dict(hq=6, hkv=4), pa.PA_ERR_INVALID_ARG),                          # Hq % Hkv != 0
    (dict(hq=18, hkv=2), pa.PA_ERR_UNSUPPORTED),                         # group 9 > 8
    (dict(hq=16, hkv=2), pa.PA_OK),                                      # group 8: control
    (dict(dim=128), pa.PA_ERR_UNSUPPORTED),                              # head_dim 128
    (dict(dim=256, dvo=512), pa.PA_ERR_UNSUPPORTED),                     # (256, 512)
    (dict(dim=512, dvo=256), pa.PA_OK),                                  # (512, 256): control
    (dict(kv_dtype=pa.PA_DTYPE_FP32), pa.PA_ERR_UNSUPPORTED),            # fp32 KV
    (dict(kv_dtype=pa.PA_DTYPE_FP8_E4M3FN, scale=(0.5, 2.0)), pa.PA_OK), # fp8: control
    (dict(scale=(0.5, 1.0)), pa.PA_ERR_INVALID_ARG),                     # bf16 with a scale
    (dict(kv_dtype=pa.PA_DTYPE_FP8_E4M3FN, scale=(0.0, 1.0)), pa.PA_ERR_INVALID_ARG),
    (dict(splits=65), pa.PA_ERR_UNSUPPORTED),
    (dict(splits=-1), pa.PA_ERR_UNSUPPORTED),
    (dict(splits=64), pa.PA_OK),
])
def test_decode_plan_rejects_bad_input_with_positive_controls(kw, status):
    assert decode_plan_status(**kw) == status


def test_misaligned_strides_are_rejected_and_aligned_padding_is_accepted():
    c = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_BF16, 10, 2, 16, 512)
    c.v_stride_token = 520  # 1040 bytes: padded rows, still 16-byte aligned
    pa.pa_decode_plan(params(hq=2), c, *lens_to_table([20], 16), 1)
    c.v_stride_token = 516  # 1032 bytes: breaks 16-byte alignment
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode_plan(params(hq=2), c, *lens_to_table([20], 16), 1)
    assert e.value.status == pa.PA_ERR_UNSUPPORTED and "v_stride_token" in e.value.message


def test_prefill_rejects_more_new_tokens_than_keys_and_plans_every_kv_format():
    P = 16
    ip, la = lens_to_table([10], P)
    c = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_BF16, 10, 2, P, 512)
    pa.pa_prefill_plan(params(hq=4), c, [0, 10], ip, la)  # control: q_len == kv_len
    with pytest.raises(pa.PaError) as e:
        pa.pa_prefill_plan(params(hq=4), c, [0, 11], ip, la)
    assert e.value.status == pa.PA_ERR_INVALID_ARG
    # FP8 E4M3FN (cast on load in both phases) and NVFP4 plan like bf16: same items.
    ref, ref_buf = pa.pa_prefill_plan(params(hq=4), c, [0, 10], ip, la)
    c8 = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_FP8_E4M3FN, 10, 2, P, 512, 0.5, 2.0)
    c4 = pa.pa_kv_cache_nvfp4_hnd(0x10000, 0x90000, 10, 2, P, 512, 0.5, 2.0)
    for cq in (c8, c4):
        plan, buf = pa.pa_prefill_plan(params(hq=4), cq, [0, 10], ip, la)
        assert plan.kv_dtype == cq.kv_dtype
        assert np.array_equal(pa.prefill_items(plan, buf), pa.prefill_items(ref, ref_buf))
    # A KV format the library does not implement is still refused.
    cf = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_BF16, 10, 2, P, 512)
    cf.kv_dtype = pa.PA_DTYPE_FP32
    with pytest.raises(pa.PaError) as e:
        pa.pa_prefill_plan(params(hq=4), cf, [0, 10], ip, la)
    assert e.value.status == pa.PA_ERR_UNSUPPORTED


def test_nvfp4_constructors_give_byte_strides_of_data_and_block_scales():
    c = pa.pa_kv_cache_nvfp4_hnd(0x10000, 0x90000, 10, 2, 16, 512, 0.5, 0.25)
    assert c.kv_dtype == pa.PA_DTYPE_NVFP4 and c.head_dim_qk == c.head_dim_vo == 512
    assert (c.k_stride_token, c.k_stride_head, c.k_stride_page) == (256, 16 * 256, 2 * 2 * 16 * 256)
    assert (c.k_sf_stride_token, c.k_sf_stride_head, c.k_sf_stride_page) == (32, 16 * 32,
                                                                              2 * 2 * 16 * 32)
    assert c.v == 0x10000 + 2 * 16 * 256 and c.v_sf == 0x90000 + 2 * 16 * 32
    assert (c.v_stride_page, c.v_sf_stride_page) == (c.k_stride_page, c.k_sf_stride_page)
    s = pa.pa_kv_cache_nvfp4_separate(0x10000, 0x20000, 0x30000, 0x40000, 10, 2, 1, 512, 256)
    assert (s.k_stride_token, s.v_stride_token, s.k_sf_stride_token, s.v_sf_stride_token) == (
        256, 128, 32, 16)
    assert (s.k_stride_page, s.v_sf_stride_page) == (2 * 256, 2 * 16)
    pa.pa_decode_plan(params(hq=8), c, *lens_to_table([37, 64], 16), 0)  # decode plans


def test_nvfp4_misuse_is_refused():
    ip, la = lens_to_table([20], 16)
    with pytest.raises(pa.PaError) as e:  # the plain constructors have no block scales
        pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_NVFP4, 10, 2, 16, 512)
    assert e.value.status == pa.PA_ERR_INVALID_ARG and "nvfp4" in e.value.message
    c = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_FP8_E4M3FN, 10, 2, 16, 512, 1.0, 1.0)
    c.k_sf = 0x90000  # a stray block-scale tensor on an FP8 cache
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode_plan(params(hq=2), c, ip, la, 0)
    assert e.value.status == pa.PA_ERR_INVALID_ARG and "k_sf" in e.value.message
    f = pa.pa_kv_cache_nvfp4_hnd(0x10000, 0x90000, 10, 2, 16, 512)
    f.v_sf_stride_token = 40  # not a multiple of 16 bytes
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode_plan(params(hq=2), f, ip, la, 0)
    assert e.value.status == pa.PA_ERR_UNSUPPORTED and "v_sf_stride_token" in e.value.message
    f = pa.pa_kv_cache_nvfp4_hnd(0x10000, 0x90000, 10, 2, 16, 512)
    pa.pa_prefill_plan(params(hq=4), f, [0, 20], ip, la)  # prefill reads nvfp4 too


def test_plan_buffer_too_small_is_rejected():
    ip, la = lens_to_table([100, 200], 16)
    c = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_BF16, 20, 1, 16, 512)
    p = params(hq=8)
    plan = pa.pa_plan()
    lib = pa.lib()
    ipa, ipp = pa._i32(ip)
    laa, lap = pa._i32(la)
    assert lib.pa_decode_plan(ctypes.byref(p), ctypes.byref(c), ipp, lap, 2, 2, None, 0,
                              ctypes.byref(plan)) == pa.PA_OK
    small = np.zeros(plan.plan_bytes - 1, np.uint8)
    st = lib.pa_decode_plan(ctypes.byref(p), ctypes.byref(c), ipp, lap, 2, 2,
                            small.ctypes.data_as(ctypes.c_void_p), small.nbytes,
                            ctypes.byref(plan))
    assert st == pa.PA_ERR_WORKSPACE_TOO_SMALL


def test_validate_page_table_host():
    pa.pa_validate_page_table_host([0, 2, 3], [4, 1, 0], [5, 16], 5, 16)
    with pytest.raises(pa.PaError):
        pa.pa_validate_page_table_host([0, 2, 3], [4, 5, 0], [5, 16], 5, 16)  # index 5 >= 5
    with pytest.raises(pa.PaError):
        pa.pa_validate_page_table_host([0, 2, 3], [4, -1, 0], [5, 16], 5, 16)


def test_run_calls_refuse_a_plan_made_for_other_sizes():
    """Forced from the host: the check fails before anything reaches HIP."""
    ip, la = lens_to_table([37, 64], 16)
    c = pa.pa_kv_cache_hnd(0x10000, pa.PA_DTYPE_BF16, 10, 1, 16, 512)
    p = params(hq=8)
    plan, buf = pa.pa_decode_plan(p, c, ip, la, 2)
    table = pa.pa_page_table(0x1000, 0x2000, 0x3000, 2)
    p_other = params(hq=8, window=4)
    with pytest.raises(pa.PaError) as e:
        pa.pa_paged_decode(plan, 0x4000, c, table, p_other, 0x5000, None, 0x6000, 1 << 20)
    assert e.value.status == pa.PA_ERR_INVALID_ARG
    with pytest.raises(pa.PaError) as e:
        pa.pa_paged_decode(plan, 0x4000, c, table, p, 0x5000, None, 0x6000, 16)
    assert e.value.status == pa.PA_ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(pa.PaError) as e:
        pa.pa_paged_decode(plan, 0x4001, c, table, p, 0x5000, None, 0x6000, 1 << 20)
    assert e.value.status == pa.PA_ERR_UNSUPPORTED  # misaligned q


def test_nvfp4_prefill_widens_pages_only_when_tiles_re_read_keys():
    """NVFP4 prefill plans reserve bf16 pages for every page-table entry (2 (D_qk + D_vo)
    bytes per entry, KV head and slot, plus one int32 per entry) exactly when the plan does
    not split keys and its tiles read each key at least four times on average; bf16 and
    FP8 plans never do."""
    def plan_for(qo, kv, dtype, hq=16, hkv=8, P=16, dvo=512):
        indptr, last = lens_to_table(kv, P)
        qo_indptr = np.zeros(len(qo) + 1, np.int32)
        qo_indptr[1:] = np.cumsum(qo)
        pages = int(indptr[-1]) + 1
        if dtype == pa.PA_DTYPE_NVFP4:
            cache = pa.pa_kv_cache_nvfp4_hnd(0x10000, 0x20000, pages, hkv, P, 512)
        else:
            cache = pa.pa_kv_cache_hnd(0x10000, dtype, pages, hkv, P, 512)
        plan, _ = pa.pa_prefill_plan(params(hq=hq), cache, qo_indptr, indptr, last)
        return plan, int(indptr[-1])

    # 2 x 2048 new tokens (16/8 heads: 64 tiles of 128 rows per KV head), no split-K, each
    # key read by many tiles: widened.
    plan, entries = plan_for([2048, 2048], [2600, 2200], pa.PA_DTYPE_NVFP4)
    assert plan.num_merges == 0 and plan.staged_pages == entries
    assert plan.staged_offset >= plan.partial_lse_offset and plan.staged_offset % 256 == 0
    need = entries * 8 * 16 * (512 + 512) * 2 + entries * 4
    assert plan.staged_offset + need <= plan.workspace_bytes < plan.staged_offset + need + 256
    # The same shapes over bf16 and FP8 caches: never.
    for dt in (pa.PA_DTYPE_BF16, pa.PA_DTYPE_FP8_E4M3FN):
        assert plan_for([2048, 2048], [2600, 2200], dt)[0].staged_pages == 0
    # A few new tokens over long KV: the plan splits keys, so no widening.
    plan, _ = plan_for([16] * 4, [6000] * 4, pa.PA_DTYPE_NVFP4)
    assert plan.num_merges > 0 and plan.staged_pages == 0 and plan.staged_offset == 0
    # No split, but each key read by fewer than four tiles on average (one 128-row tile per
    # 16 tokens at group 8, keys mostly behind a long prefix read by one tile each).
    plan, _ = plan_for([16] * 512, [4000] * 512, pa.PA_DTYPE_NVFP4, hq=64, hkv=8)
    assert plan.num_merges == 0 and plan.staged_pages == 0
