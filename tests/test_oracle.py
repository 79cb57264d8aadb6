"""Pins of the fp64 oracle against things other than itself.

Each test names what pins the oracle: torch's own dtype conversions, hand-derived
examples (tests/golden), brute-force attention written with scalar Python loops,
closed forms, and exact invariants of attention.  A second group plants plausible
mistakes in copies of the oracle's steps and checks that these pins catch them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (bf16_bits_to_f64, E4M3FN_VALUES, kv_values, request_kv_len,
                    gather_request_kv, visible_mask, softmax_attention, decode_ref,
                    prefill_ref, chunk_partial_ref, merge_ref)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def bf16_bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------- numerics

def test_bf16_decode_matches_torch_for_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_e4m3fn_table_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(E4M3FN_VALUES), nan)
    assert np.array_equal(E4M3FN_VALUES[~nan], ref[~nan])
    assert nan.sum() == 2


def test_e4m3fn_golden_codes():
    g = json.load(open(GOLDEN))["e4m3fn_codes"]
    for c, v in zip(g["codes"], g["values"]):
        assert E4M3FN_VALUES[c] == v
    for c in g["nan_codes"]:
        assert math.isnan(E4M3FN_VALUES[c])
    assert math.copysign(1.0, E4M3FN_VALUES[0x80]) == -1.0 and E4M3FN_VALUES[0x80] == 0.0


def test_kv_values_scale_and_dtype_rules():
    assert np.array_equal(kv_values(np.array([0x38, 0x40], np.uint8), "fp8", 0.5), [0.5, 1.0])
    with pytest.raises(ValueError):
        kv_values(np.zeros(2, np.uint16), "bf16", 2.0)
    with pytest.raises(ValueError):
        kv_values(np.zeros(2, np.uint16), "fp16")


# --------------------------------------------------------------------------- paging

def test_request_lengths_partial_exact_and_empty():
    # L=37 over 3 pages of 16 (last holds 5); L=64 over 4 pages (last holds 16); empty.
    lens = request_kv_len([0, 3, 7, 7], [5, 16, 0], 16)
    assert list(lens) == [37, 64, 0]


@pytest.mark.parametrize("page_size", [1, 3, 16])
def test_gather_inverts_an_independent_scatter(page_size):
    """Scatter a dense logical KV into shuffled pages by the layout rule, gather it back."""
    rng = np.random.default_rng(7)
    lens = [1, 5, 2 * page_size, 17]
    heads, dim = 2, 4
    dense = [rng.integers(0, 65535, size=(L, heads, dim)).astype(np.uint16) for L in lens]
    n_pages = [-(-L // page_size) for L in lens]
    num_pages = sum(n_pages) + 3
    perm = rng.permutation(num_pages)
    pool = np.full((num_pages, heads, page_size, dim), 0xFFFF, dtype=np.uint16)
    indptr, indices, last, p = [0], [], [], 0
    for b, L in enumerate(lens):
        mine = perm[p:p + n_pages[b]]
        p += n_pages[b]
        indices.extend(mine)
        indptr.append(len(indices))
        last.append((L - 1) % page_size + 1)
        for t in range(L):  # token t -> its page's slot t % page_size
            pool[mine[t // page_size], :, t % page_size, :] = dense[b][t]
    for b in range(len(lens)):
        got = gather_request_kv(pool, indptr, indices, last, page_size, b)
        assert got.dtype == np.uint16 and np.array_equal(got, dense[b])


def test_golden_paged_decode_window_and_prefill():
    g = json.load(open(GOLDEN))
    pd = g["paged_decode"]
    kp = bf16_bits(pd["k_pages"])
    vp = bf16_bits(pd["v_pages"])
    q = bf16_bits_to_f64(bf16_bits(pd["q"]))
    args = (kp, vp, pd["kv_indptr"], pd["kv_indices"], pd["kv_last_page_len"],
            pd["page_size"], pd["sm_scale"])
    o, lse = decode_ref(q, *args)
    assert np.array_equal(o, np.asarray(pd["o"]))
    assert abs(lse[0, 0] - math.log(3)) < 1e-15
    o, lse = decode_ref(q, *args, window=g["paged_decode_window2"]["window"])
    assert np.array_equal(o, np.asarray(g["paged_decode_window2"]["o"]))
    assert abs(lse[0, 0] - math.log(2)) < 1e-15
    pf = g["paged_prefill_causal"]
    q2 = bf16_bits_to_f64(bf16_bits(pf["q"]))
    o, lse = prefill_ref(q2, pf["qo_indptr"], *args)
    assert np.array_equal(o, np.asarray(pf["o"]))
    assert np.allclose(lse[:, 0], [math.log(2), math.log(3)], rtol=0, atol=1e-15)


def test_golden_two_keys_and_gqa():
    g = json.load(open(GOLDEN))
    tk = g["two_keys"]
    o, lse = softmax_attention(np.array([tk["q"]]), np.array(tk["k"]), np.array(tk["v"]),
                               np.ones((1, 2), bool), tk["sm_scale"])
    assert np.allclose(o[0], tk["o"], rtol=0, atol=1e-14)
    assert abs(lse[0] - math.log(4)) < 1e-14
    gq = g["gqa_two_heads"]
    # One KV head shared by two query heads, through the paged decode path.
    kp = bf16_bits(np.array(gq["k"])[None, None])  # [1 page, 1 head, 2 slots, 2]
    vp = bf16_bits(np.array(gq["v"])[None, None])
    q = np.array(gq["q"])[None]  # [1, 2 heads, 2]
    o, _ = decode_ref(q, kp, vp, [0, 1], [0], [2], 2, gq["sm_scale"])
    assert np.allclose(o[0], gq["o"], rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- attention core

def brute_force_attention(q, k, v, visible, scale):
    """Scalar-loop softmax attention using only the math module."""
    n, dv = len(q), len(v[0]) if len(v) else 0
    out, lses = [], []
    for i in range(n):
        s = [scale * sum(q[i][d] * k[t][d] for d in range(len(q[i]))) if visible[i][t]
             else None for t in range(len(k))]
        vals = [x for x in s if x is not None]
        if not vals:
            out.append([0.0] * dv)
            lses.append(-math.inf)
            continue
        m = max(vals)
        w = [math.exp(x - m) if x is not None else 0.0 for x in s]
        z = sum(w)
        out.append([sum(w[t] * v[t][d] for t in range(len(k))) / z for d in range(dv)])
        lses.append(m + math.log(z))
    return np.array(out), np.array(lses)


@pytest.mark.parametrize("dim,length,causal,window", [(8, 1, False, 0), (16, 40, True, 0),
                                                       (8, 23, True, 5), (16, 17, False, 4)])
def test_softmax_attention_matches_brute_force(dim, length, causal, window):
    rng = np.random.default_rng(dim * 100 + length)
    q = rng.standard_normal((6, dim))
    k = rng.standard_normal((length, dim))
    v = rng.standard_normal((length, dim + 3))
    pos = rng.integers(0, length, size=6)
    mask = visible_mask(pos, length, causal, window)
    o, lse = softmax_attention(q, k, v, mask, 0.3)
    ob, lb = brute_force_attention(q.tolist(), k.tolist(), v.tolist(), mask.tolist(), 0.3)
    assert np.allclose(o, ob, rtol=0, atol=1e-12)
    assert np.allclose(lse, lb, rtol=0, atol=1e-12)


def test_softmax_attention_hd512_brute_force():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 512))
    k = rng.standard_normal((9, 512))
    v = rng.standard_normal((9, 512))
    mask = np.ones((2, 9), bool)
    o, lse = softmax_attention(q, k, v, mask, 1 / math.sqrt(512))
    ob, lb = brute_force_attention(q.tolist(), k.tolist(), v.tolist(), mask.tolist(),
                                   1 / math.sqrt(512))
    assert np.allclose(o, ob, rtol=0, atol=1e-12) and np.allclose(lse, lb, rtol=0, atol=1e-12)


def test_visible_mask_window_counts_the_query_position():
    m = visible_mask([9], 10, True, 3)
    assert list(np.nonzero(m[0])[0]) == [7, 8, 9]
    m = visible_mask([4], 10, True, 0)
    assert list(np.nonzero(m[0])[0]) == [0, 1, 2, 3, 4]
    m = visible_mask([4], 10, False, 2)
    assert list(np.nonzero(m[0])[0]) == [3, 4, 5, 6, 7, 8, 9]


def test_closed_forms():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 16))
    k = rng.standard_normal((5, 16))
    v = rng.standard_normal((5, 7))
    ones = np.ones((1, 5), bool)
    # A single key returns its value exactly, with lse = the score.
    o, lse = softmax_attention(q, k[:1], v[:1], ones[:, :1], 0.25)
    assert np.array_equal(o[0], v[0]) and lse[0] == 0.25 * (q[0] @ k[0])
    # Constant V returns V.
    vc = np.tile(v[:1], (5, 1))
    o, _ = softmax_attention(q, k, vc, ones, 0.25)
    assert np.allclose(o[0], v[0], rtol=0, atol=1e-14)
    # q = 0 gives the mean of the visible values, lse = ln(count).
    o, lse = softmax_attention(np.zeros((1, 16)), k, v, ones, 0.25)
    assert np.allclose(o[0], v.mean(axis=0), rtol=0, atol=1e-14)
    assert abs(lse[0] - math.log(5)) < 1e-14
    # Two keys: weights (1 - sigma, sigma) with sigma = sigmoid(s1 - s0).
    s = 0.25 * (k[:2] @ q[0])
    sig = 1 / (1 + math.exp(-(s[1] - s[0])))
    o, _ = softmax_attention(q, k[:2], v[:2], ones[:, :2], 0.25)
    assert np.allclose(o[0], (1 - sig) * v[0] + sig * v[1], rtol=0, atol=1e-14)
    # Window 1 returns the last value.
    o, _ = softmax_attention(q, k, v, visible_mask([4], 5, True, 1), 0.25)
    assert np.array_equal(o[0], v[4])
    # Nothing visible: o = 0, lse = -inf.
    o, lse = softmax_attention(q, k, v, np.zeros((1, 5), bool), 0.25)
    assert np.array_equal(o[0], np.zeros(7)) and lse[0] == -np.inf


# --------------------------------------------------------------------------- helpers for paged invariants

def small_decode(seed=5, lens=(37, 64, 1, 16), hq=8, hkv=2, dim=32, page=16, dvo=None,
                 kv_dtype="bf16"):
    from synth import make_decode_case
    c = make_decode_case(lens, hq, hkv, dim, page, head_dim_vo=dvo, kv_dtype=kv_dtype,
                         seed=seed, out_dtype="fp32")
    kp = c.k_pool.contiguous().view(torch.int16 if kv_dtype == "bf16" else torch.uint8).numpy()
    vp = c.v_pool.contiguous().view(torch.int16 if kv_dtype == "bf16" else torch.uint8).numpy()
    if kv_dtype == "bf16":
        kp, vp = kp.view(np.uint16), vp.view(np.uint16)
    q = bf16_bits_to_f64(c.q.view(torch.int16).numpy().view(np.uint16))
    return c, q, kp, vp


def run_decode(c, q, kp, vp, window=0, **kw):
    return decode_ref(q, kp, vp, c.kv_indptr, c.kv_indices, c.kv_last_page_len, c.page_size,
                      c.sm_scale, window=window, kv_dtype=c.kv_dtype, k_scale=c.k_scale,
                      v_scale=c.v_scale, **kw)


def test_page_permutation_invariance_is_bit_exact():
    c, q, kp, vp = small_decode()
    o, lse = run_decode(c, q, kp, vp)
    rng = np.random.default_rng(1)
    perm = rng.permutation(c.num_pages)  # new page id of old page p is perm[p]
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    idx2 = perm[c.kv_indices].astype(np.int32)
    o2, lse2 = decode_ref(q, kp2, vp2, c.kv_indptr, idx2, c.kv_last_page_len, c.page_size,
                          c.sm_scale)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_gqa_equals_mha_with_duplicated_kv_heads():
    c, q, kp, vp = small_decode(hq=6, hkv=2)
    o, lse = run_decode(c, q, kp, vp)
    group = 3
    kp_m = np.repeat(kp, group, axis=1)  # kv head j*3+g is a copy of kv head j
    vp_m = np.repeat(vp, group, axis=1)
    o2, lse2 = decode_ref(q, kp_m, vp_m, c.kv_indptr, c.kv_indices, c.kv_last_page_len,
                          c.page_size, c.sm_scale)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def truncated_table(c, keep_from):
    """Page table of the same requests with their first keep_from[b] tokens dropped,
    rebuilt on fresh pages (contents copied token by token)."""
    kp_src = c.k_pool.contiguous().view(torch.int16).numpy().view(np.uint16)
    vp_src = c.v_pool.contiguous().view(torch.int16).numpy().view(np.uint16)
    P = c.page_size
    k_new, v_new, indptr, indices, last = [], [], [0], [], []
    for b, L in enumerate(c.kv_lens):
        toks = list(range(int(keep_from[b]), int(L)))
        n = -(-len(toks) // P)
        for j in range(n):
            kpage = np.zeros(kp_src.shape[1:], np.uint16)
            vpage = np.zeros(vp_src.shape[1:], np.uint16)
            for s, t in enumerate(toks[j * P:(j + 1) * P]):
                src_page = c.kv_indices[c.kv_indptr[b] + t // P]
                kpage[:, s] = kp_src[src_page, :, t % P]
                vpage[:, s] = vp_src[src_page, :, t % P]
            indices.append(len(k_new))
            k_new.append(kpage)
            v_new.append(vpage)
        indptr.append(len(indices))
        last.append((len(toks) - 1) % P + 1 if toks else 0)
    return (np.stack(k_new), np.stack(v_new), np.array(indptr), np.array(indices),
            np.array(last))


@pytest.mark.parametrize("window", [1, 5, 16, 33])
def test_window_equals_truncated_kv(window):
    c, q, kp, vp = small_decode(lens=(37, 64, 1, 16, 40), page=3)
    o, lse = run_decode(c, q, kp, vp, window=window)
    kn, vn, ip, ix, la = truncated_table(c, np.maximum(0, c.kv_lens - window))
    o2, lse2 = decode_ref(q, kn, vn, ip, ix, la, c.page_size, c.sm_scale)
    assert np.allclose(o, o2, rtol=0, atol=1e-12) and np.allclose(lse, lse2, rtol=0, atol=1e-12)


def test_window_at_least_length_equals_no_window():
    c, q, kp, vp = small_decode()
    o, lse = run_decode(c, q, kp, vp)
    o2, lse2 = run_decode(c, q, kp, vp, window=int(c.kv_lens.max()))
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_split_merge_equals_unsplit(seed):
    c, q, kp, vp = small_decode(seed=seed, lens=(37, 64, 50), page=16)
    o, lse = run_decode(c, q, kp, vp, window=20 if seed == 2 else 0)
    rng = np.random.default_rng(seed)
    for b in range(c.batch):
        L = int(c.kv_lens[b])
        k = kv_values(gather_request_kv(kp, c.kv_indptr, c.kv_indices, c.kv_last_page_len,
                                        c.page_size, b), "bf16")
        v = kv_values(gather_request_kv(vp, c.kv_indptr, c.kv_indices, c.kv_last_page_len,
                                        c.page_size, b), "bf16")
        mask = visible_mask([L - 1], L, True, 20 if seed == 2 else 0)[0]
        # Random cut points, duplicates allowed, so some chunks are empty.
        cuts = np.sort(rng.integers(0, L + 1, size=5))
        bounds = [0] + list(cuts) + [L]
        for h in range(c.num_qo_heads):
            kvh = h // (c.num_qo_heads // c.num_kv_heads)
            parts = [chunk_partial_ref(q[b, h], k[:, kvh], v[:, kvh], mask, lo, hi,
                                       c.sm_scale) for lo, hi in zip(bounds[:-1], bounds[1:])]
            om, lm = merge_ref([p[0] for p in parts], [p[1] for p in parts])
            assert np.allclose(om, o[b, h], rtol=0, atol=1e-12)
            assert abs(lm - lse[b, h]) < 1e-12


def test_merge_of_all_empty_chunks():
    o, lse = merge_ref(np.zeros((3, 4)), np.full(3, -np.inf))
    assert np.array_equal(o, np.zeros(4)) and lse == -np.inf


def test_prefill_rows_equal_decode_on_truncated_kv_and_qlen1_equals_decode():
    from synth import make_prefill_case
    c = make_prefill_case([5, 1], [37, 20], 4, 2, 32, 16, seed=9)
    kp = c.k_pool.contiguous().view(torch.int16).numpy().view(np.uint16)
    vp = c.v_pool.contiguous().view(torch.int16).numpy().view(np.uint16)
    q = bf16_bits_to_f64(c.q.view(torch.int16).numpy().view(np.uint16))
    o, lse = prefill_ref(q, c.qo_indptr, kp, vp, c.kv_indptr, c.kv_indices,
                         c.kv_last_page_len, c.page_size, c.sm_scale)
    for b in range(c.batch):
        q0, q1 = c.qo_indptr[b], c.qo_indptr[b + 1]
        L = int(c.kv_lens[b])
        for i in range(q1 - q0):
            pos = L - (q1 - q0) + i
            # Decode over the same pages with the length cut to pos + 1.
            n_pages = pos // c.page_size + 1
            indptr = [0, n_pages]
            indices = c.kv_indices[c.kv_indptr[b]:c.kv_indptr[b] + n_pages]
            last = [pos % c.page_size + 1]
            od, ld = decode_ref(q[q0 + i][None], kp, vp, indptr, indices, last, c.page_size,
                                c.sm_scale)
            assert np.allclose(o[q0 + i], od[0], rtol=0, atol=1e-12)
            assert np.allclose(lse[q0 + i], ld[0], rtol=0, atol=1e-12)


def test_asymmetric_equals_symmetric_with_zero_padded_v():
    c, q, kp, vp = small_decode(dim=32, dvo=16)
    o, lse = run_decode(c, q, kp, vp)
    vpad = np.concatenate([vp, np.zeros_like(vp)], axis=3)  # [.., 16] -> [.., 32]
    o2, lse2 = decode_ref(q, kp, vpad, c.kv_indptr, c.kv_indices, c.kv_last_page_len,
                          c.page_size, c.sm_scale)
    assert np.allclose(o, o2[..., :16], rtol=0, atol=1e-12)
    assert np.array_equal(o2[..., 16:], np.zeros_like(o2[..., 16:]))
    assert np.allclose(lse, lse2, rtol=0, atol=1e-12)


def test_fp8_cache_is_read_through_the_code_table():
    c, q, kp, vp = small_decode(kv_dtype="fp8")
    o, lse = run_decode(c, q, kp, vp)
    # The same attention on a float64 cache holding the decoded values times the scales.
    kf = E4M3FN_VALUES[kp] * c.k_scale
    vf = E4M3FN_VALUES[vp] * c.v_scale
    kbits = kf  # float64 pools go through softmax_attention directly
    for b in range(c.batch):
        L = int(c.kv_lens[b])
        k = gather_request_kv(kbits, c.kv_indptr, c.kv_indices, c.kv_last_page_len,
                              c.page_size, b)
        v = gather_request_kv(vf, c.kv_indptr, c.kv_indices, c.kv_last_page_len,
                              c.page_size, b)
        for h in range(c.num_qo_heads):
            kvh = h // (c.num_qo_heads // c.num_kv_heads)
            ob, lb = brute_force_attention([q[b, h].tolist()], k[:, kvh].tolist(),
                                           v[:, kvh].tolist(), [[True] * L], c.sm_scale)
            assert np.allclose(o[b, h], ob[0], rtol=0, atol=1e-12)
            assert abs(lse[b, h] - lb[0]) < 1e-12


def test_poison_never_reaches_the_output():
    c, q, kp, vp = small_decode()
    o, _ = run_decode(c, q, kp, vp)
    assert np.abs(o).max() < 10.0  # a poisoned V (|v| = 30000) would show up here


# --------------------------------------------------------------------------- planted mistakes

def test_planted_last_page_off_by_one_is_caught(monkeypatch):
    """Counting the last page as full breaks the hand-derived paged example."""
    import oracle.attention as att
    real = att.request_kv_len

    def wrong(indptr, last, page_size):
        lens = real(indptr, last, page_size)
        return np.where(lens > 0, lens + (page_size - np.asarray(last)), 0)
    monkeypatch.setattr(att, "request_kv_len", wrong)
    g = json.load(open(GOLDEN))["paged_decode"]
    kp, vp = bf16_bits(g["k_pages"]), bf16_bits(g["v_pages"])
    q = bf16_bits_to_f64(bf16_bits(g["q"]))
    with pytest.raises(Exception):
        o, _ = att.decode_ref(q, kp, vp, g["kv_indptr"], g["kv_indices"],
                              g["kv_last_page_len"], g["page_size"], g["sm_scale"])
        assert np.array_equal(o, np.asarray(g["o"]))


def test_planted_window_off_by_one_is_caught():
    m_wrong = np.arange(10)[None, :] >= 9 - 3  # t >= pos - W instead of t > pos - W
    m_right = visible_mask([9], 10, True, 3)
    assert not np.array_equal(m_wrong, m_right)


def test_planted_kv_head_mapping_is_caught():
    """h % Hkv instead of h // G differs from GQA = MHA-with-duplicates."""
    c, q, kp, vp = small_decode(hq=6, hkv=2)
    o, _ = run_decode(c, q, kp, vp)
    kp_wrong = np.concatenate([kp[:, [0]], kp[:, [1]], kp[:, [0]], kp[:, [1]], kp[:, [0]],
                               kp[:, [1]]], axis=1)  # head h reads h % 2
    vp_wrong = np.concatenate([vp[:, [0]], vp[:, [1]], vp[:, [0]], vp[:, [1]], vp[:, [0]],
                               vp[:, [1]]], axis=1)
    o2, _ = decode_ref(q, kp_wrong, vp_wrong, c.kv_indptr, c.kv_indices, c.kv_last_page_len,
                       c.page_size, c.sm_scale)
    assert not np.allclose(o, o2, atol=1e-3)


# --------------------------------------------------------------------------- NVFP4 KV

def test_e2m1_codes_follow_the_format_structure():
    """The 16 E2M1 codes, pinned by the structure of a sign-magnitude float with 2 exponent
    bits and 1 mantissa bit rather than by the closed form: codes 8..15 negate 0..7 (with
    -0), magnitudes rise strictly, the subnormal step is half the smallest normal, and each
    binade doubles the one below (code c + 2 is twice code c for normal codes)."""
    v = oracle.E2M1_VALUES
    assert v.shape == (16,)
    assert np.array_equal(v[8:], -v[:8]) and math.copysign(1.0, v[8]) == -1.0
    assert np.all(np.diff(v[:8]) > 0) and v[0] == 0.0
    assert v[2] == 1.0 and v[1] == v[2] / 2  # smallest normal 2^0; subnormal step 1/2
    for c in range(2, 6):
        assert v[c + 2] == 2 * v[c]
    assert v[7] == 6.0 and v[3] == 1.5  # largest finite magnitude; mantissa bit = +1/2


def test_nvfp4_hand_derived_rows():
    """Hand-derived values: byte 0x21 holds elements (code 1, code 2) = (0.5, 1.0), byte 0xF7
    holds (code 7, code 15) = (6.0, -6.0); block scale code 0x40 is E4M3FN 2.0, 0x38 is 1.0."""
    packed = np.array([[0x21, 0xF7] + [0x00] * 6, [0x00] * 7 + [0x9B]], dtype=np.uint8)
    scales = np.array([[0x40], [0x38]], dtype=np.uint8)
    got = oracle.nvfp4_values(packed, scales, 0.25)
    want = np.zeros((2, 16))
    want[0, :4] = np.array([0.5, 1.0, 6.0, -6.0]) * 2.0 * 0.25
    # 0x9B: low nibble 0xB = 1|011 = -1.5, high nibble 0x9 = 1|001 = -0.5
    want[1, 14:] = np.array([-1.5, -0.5]) * 1.0 * 0.25
    assert np.array_equal(got, want)


def test_nvfp4_block_scale_index_is_element_over_16():
    packed = np.full((1, 32), 0x22, dtype=np.uint8)  # every element 1.0, 64 elements
    scales = np.array([[0x38, 0x40, 0x48, 0x50]], dtype=np.uint8)  # 1, 2, 4, 8
    got = oracle.nvfp4_values(packed, scales)
    assert np.array_equal(got[0], np.repeat([1.0, 2.0, 4.0, 8.0], 16))
    with pytest.raises(ValueError):
        oracle.nvfp4_values(packed, scales[:, :3])


@pytest.mark.parametrize("seed", [0, 1])
def test_nvfp4_round_trip_within_the_quantisation_bound(seed):
    """The input generator's quantiser (its own E2M1 table and packing) followed by the
    oracle's dequantisation lands within the rounding bound: each element's error is at
    most half of the E2M1 spacing at its magnitude (1 at the top, 4..6) times its block's
    scale, plus the clamp at 6 when the block scale rounded down."""
    from synth.workloads import _nvfp4_encode
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn((64, 512), generator=gen)
    g = float(x.abs().max()) / (6 * 448)
    packed, bs = _nvfp4_encode(x, g)
    deq = oracle.nvfp4_values(packed.numpy(), bs.numpy(), g)
    xs = x.double().numpy()
    step = np.repeat(oracle.E4M3FN_VALUES[bs.numpy()], 16, axis=-1) * g
    assert np.all(np.abs(xs - deq) <= 1.0 * step * (1 + 2 ** -3) + 1e-12)
    # Relative RMS error of E2M1 with per-16 scales is about 10 %; a swapped nibble order or
    # a wrong block index gives errors of the order of the values themselves.
    assert np.sqrt(np.mean((xs - deq) ** 2)) < 0.15 * np.sqrt(np.mean(xs ** 2))


def nvfp4_small_decode(seed=7, lens=(37, 64, 1, 16), hq=8, hkv=2, dim=64, page=16, dvo=None):
    from synth import make_decode_case
    c = make_decode_case(lens, hq, hkv, dim, page, head_dim_vo=dvo, kv_dtype="nvfp4",
                         seed=seed, out_dtype="fp32")
    q = bf16_bits_to_f64(c.q.view(torch.int16).numpy().view(np.uint16))
    arrs = [t.contiguous().numpy() for t in (c.k_pool, c.v_pool, c.k_sf, c.v_sf)]
    return (c, q) + tuple(arrs)


def test_nvfp4_decode_matches_brute_force_on_decoded_values():
    c, q, kp, vp, ksf, vsf = nvfp4_small_decode(dim=32, lens=(19, 1, 40))
    o, lse = decode_ref(q, kp, vp, c.kv_indptr, c.kv_indices, c.kv_last_page_len, c.page_size,
                        c.sm_scale, kv_dtype="nvfp4", k_scale=c.k_scale, v_scale=c.v_scale,
                        k_sf=ksf, v_sf=vsf)
    for b in range(c.batch):
        L = int(c.kv_lens[b])
        pages = c.kv_indices[c.kv_indptr[b]:c.kv_indptr[b + 1]]
        for h in range(c.num_qo_heads):
            kvh = h // (c.num_qo_heads // c.num_kv_heads)
            ks, vs = [], []
            for t in range(L):  # token by token, element by element, from the bytes
                pg, sl = int(pages[t // c.page_size]), t % c.page_size
                def elem(pool, sfp, d, scale):
                    byte = int(pool[pg, kvh, sl, d // 2])
                    nib = byte & 15 if d % 2 == 0 else byte >> 4
                    mag = [0, 0.5, 1, 1.5, 2, 3, 4, 6][nib & 7]
                    return (-mag if nib & 8 else mag) * \
                        oracle.E4M3FN_VALUES[sfp[pg, kvh, sl, d // 16]] * scale
                ks.append([elem(kp, ksf, d, c.k_scale) for d in range(32)])
                vs.append([elem(vp, vsf, d, c.v_scale) for d in range(32)])
            ob, lb = brute_force_attention([q[b, h].tolist()], ks, vs, [[True] * L], c.sm_scale)
            assert np.allclose(o[b, h], ob[0], rtol=0, atol=1e-12)
            assert abs(lse[b, h] - lb[0]) < 1e-12


def test_nvfp4_block_scales_follow_the_page_table():
    """Permuting pages of data and block scales together is invisible (bit-exact); permuting
    the data alone is not."""
    c, q, kp, vp, ksf, vsf = nvfp4_small_decode()
    kw = dict(kv_dtype="nvfp4", k_scale=c.k_scale, v_scale=c.v_scale)
    o, lse = decode_ref(q, kp, vp, c.kv_indptr, c.kv_indices, c.kv_last_page_len, c.page_size,
                        c.sm_scale, k_sf=ksf, v_sf=vsf, **kw)
    perm = np.random.default_rng(3).permutation(c.num_pages)
    moved = []
    for a in (kp, vp, ksf, vsf):
        a2 = np.empty_like(a)
        a2[perm] = a
        moved.append(a2)
    idx2 = perm[c.kv_indices].astype(np.int32)
    o2, lse2 = decode_ref(q, moved[0], moved[1], c.kv_indptr, idx2, c.kv_last_page_len,
                          c.page_size, c.sm_scale, k_sf=moved[2], v_sf=moved[3], **kw)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    o3, _ = decode_ref(q, moved[0], moved[1], c.kv_indptr, idx2, c.kv_last_page_len,
                       c.page_size, c.sm_scale, k_sf=ksf, v_sf=vsf, **kw)
    assert not np.allclose(o, o3, atol=1e-3)


def test_nvfp4_poison_never_reaches_the_output():
    c, q, kp, vp, ksf, vsf = nvfp4_small_decode(lens=(37, 5, 64))
    o, _ = decode_ref(q, kp, vp, c.kv_indptr, c.kv_indices, c.kv_last_page_len, c.page_size,
                      c.sm_scale, kv_dtype="nvfp4", k_scale=c.k_scale, v_scale=c.v_scale,
                      k_sf=ksf, v_sf=vsf)
    vmax = np.abs(oracle.nvfp4_values(vp, vsf, c.v_scale))
    poison = 6 * 448 * c.v_scale
    assert np.abs(o).max() < 0.5 * poison and vmax.max() >= poison


def test_planted_nibble_swap_is_caught():
    """Reading element 2i from the high nibble breaks the hand-derived rows."""
    packed = np.array([[0x21] + [0] * 7], dtype=np.uint8)
    swapped = ((packed & 15) << 4) | (packed >> 4)
    right = oracle.nvfp4_values(packed, np.array([[0x38]], np.uint8))
    wrong = oracle.nvfp4_values(swapped, np.array([[0x38]], np.uint8))
    assert right[0, 0] == 0.5 and wrong[0, 0] != 0.5


def test_nvfp4_prefill_rows_equal_decode_on_truncated_kv():
    """Row i of an NVFP4 prefill is the decode of a request cut after its position, read
    through the same pages and block scales (to fp64 rounding of the products)."""
    from synth import make_prefill_case
    c = make_prefill_case([5, 3], [21, 40], 4, 2, 32, 8, kv_dtype="nvfp4", seed=9)
    q = bf16_bits_to_f64(c.q.view(torch.int16).numpy().view(np.uint16))
    arrs = [t.contiguous().numpy() for t in (c.k_pool, c.v_pool, c.k_sf, c.v_sf)]
    kw = dict(kv_dtype="nvfp4", k_scale=c.k_scale, v_scale=c.v_scale, k_sf=arrs[2], v_sf=arrs[3])
    o, lse = prefill_ref(q, c.qo_indptr, arrs[0], arrs[1], c.kv_indptr, c.kv_indices,
                         c.kv_last_page_len, c.page_size, c.sm_scale, **kw)
    for b in range(c.batch):
        q_len, L = int(c.qo_lens[b]), int(c.kv_lens[b])
        for i in range(q_len):
            pos = L - q_len + i
            n_pages = pos // c.page_size + 1
            ip = np.array([0, n_pages], np.int32)
            idx = c.kv_indices[c.kv_indptr[b]:c.kv_indptr[b] + n_pages]
            last = np.array([pos % c.page_size + 1], np.int32)
            row = int(c.qo_indptr[b]) + i
            od, ld = decode_ref(q[row][None], arrs[0], arrs[1], ip, idx, last, c.page_size,
                                c.sm_scale, **kw)
            assert np.allclose(o[row], od[0], rtol=0, atol=1e-12)
            assert np.abs(lse[row] - ld[0]).max() < 1e-12
