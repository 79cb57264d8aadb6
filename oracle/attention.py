"""Paged softmax attention, written out as its plain definition in float64.

Test infrastructure only (see the package docstring).

The definition, with the page citations for each step:

1. Paged KV addressing.  [Triton-hd512], section "Approach": the decode kernel reads the
   combined HND cache ``[num_pages, 2, num_kv_heads, page_size, head_dim]`` through
   ``kv_indptr`` / ``kv_indices`` / ``kv_last_page_len``, with the same slicing as the
   FlashInfer decode plan.  Reading taken: request b owns pages
   ``kv_indices[kv_indptr[b]:kv_indptr[b+1]]`` in logical order; every page is full except
   the last, which holds ``kv_last_page_len[b]`` tokens (1..page_size, so an exact multiple
   has a last page length of page_size).  Logical token t sits in page
   ``kv_indices[kv_indptr[b] + t // page_size]`` at slot ``t % page_size``.  In the combined
   layout index 0 of the "2" axis is K and index 1 is V.
2. Separate K and V pools.  [VO-split], section "Summary" and its test commit: K and V may
   live in separately allocated pools with their own strides and widths (qk=512, vo=256);
   they share the page table.
3. Grouped query heads.  [Triton-hd512], section "Test Coverage": GQA ratios, including
   non-power-of-two ones such as 12/4 and 24/4.  Reading taken: query head h reads KV head
   ``h // (Hq // Hkv)``.
4. Visibility.  Decode is one query token at the last position ``L_b - 1``.  Prefill
   ([Triton-hd512], section "Approach": causal attention when no custom mask is given;
   section "Not covered": the current tokens are the ones after the cached prefix) puts
   the ``q_len`` new tokens at the end of the request, so row i sits at
   ``pos_i = L_b - q_len + i`` and sees keys ``t <= pos_i``.  A sliding window W
   ([Triton-hd512], sections "Approach" and "Test Coverage") keeps the W most recent keys,
   the query's own position included: ``t > pos - W``.
   NVFP4 caches ([VO-split], sections "Summary" and "NVFP4 split-KV correctness (added)")
   carry a block-scale tensor per pool, addressed like the data (same page, head and slot),
   so the oracle gathers both and dequantises (numerics.nvfp4_values).
5. Softmax attention with the natural-log log-sum-exp ([VO-split], release notes: "lse
   values"): ``s_t = scale * q . k_t``; ``o = sum_t exp(s_t - m) v_t / Z``;
   ``lse = m + ln Z``.  An empty visible set gives o = 0 and lse = -inf.
6. Split-K merge ([Triton-hd512], section "Not covered": split-K workspaces; [VO-split],
   section "NVFP4 split-KV correctness (added)": split-KV is flash-decoding): partial
   states over disjoint chunks of the key axis combine by log-sum-exp weights.
"""

import numpy as np

from .numerics import kv_values


def request_kv_len(kv_indptr, kv_last_page_len, page_size):
    """Number of KV tokens of every request (step 1 of the definition)."""
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    last = np.asarray(kv_last_page_len, dtype=np.int64)
    out = np.zeros(len(kv_indptr) - 1, dtype=np.int64)
    for b in range(len(out)):
        n_pages = kv_indptr[b + 1] - kv_indptr[b]
        out[b] = 0 if n_pages == 0 else (n_pages - 1) * page_size + last[b]
    return out


def gather_request_kv(pool, kv_indptr, kv_indices, kv_last_page_len, page_size, b):
    """Stored elements of request b in logical token order: ``[L_b, H, D]``.

    ``pool`` is one of the two halves of the cache, indexed ``[page, head, slot, dim]``.
    The stored element type is kept (bf16 bit patterns or FP8 codes stay raw), so that a
    device-side gather can be compared with this one bit for bit.
    """
    start, end = int(kv_indptr[b]), int(kv_indptr[b + 1])
    n_pages = end - start
    rows = []
    for j in range(n_pages):
        page = int(kv_indices[start + j])
        count = page_size if j < n_pages - 1 else int(kv_last_page_len[b])
        rows.append(pool[page, :, :count, :])  # [H, count, D]
    if not rows:
        return np.zeros((0, pool.shape[1], pool.shape[3]), dtype=pool.dtype)
    return np.concatenate(rows, axis=1).transpose(1, 0, 2)  # [L, H, D]


def visible_mask(pos, kv_len, causal, window):
    """Boolean ``[len(pos), kv_len]``: key t visible to the query at position pos."""
    pos = np.asarray(pos, dtype=np.int64)[:, None]
    t = np.arange(kv_len, dtype=np.int64)[None, :]
    mask = np.ones((pos.shape[0], kv_len), dtype=bool)
    if causal:
        mask &= t <= pos
    if window > 0:
        mask &= t > pos - window
    return mask


def softmax_attention(q, k, v, mask, sm_scale):
    """Masked softmax attention rows in float64.

    q ``[n, Dqk]``, k ``[L, Dqk]``, v ``[L, Dvo]``, mask ``[n, L]`` ->
    (o ``[n, Dvo]``, lse ``[n]``).  Rows with nothing visible give o = 0, lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    o = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    if k.shape[0] == 0 or n == 0:
        return o, lse
    s = sm_scale * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    any_visible = mask.any(axis=1)
    m = np.where(any_visible, s.max(axis=1), 0.0)
    p = np.where(mask, np.exp(s - m[:, None]), 0.0)
    z = p.sum(axis=1)
    nz = z > 0
    o[nz] = (p[nz] @ v) / z[nz, None]
    lse[nz] = m[nz] + np.log(z[nz])
    return o, lse


def _request_kv_f64(k_pool, v_pool, kv_dtype, k_scale, v_scale, kv_indptr, kv_indices,
                    kv_last_page_len, page_size, b, k_sf=None, v_sf=None):
    """Dequantised K and V of request b, ``[L_b, H, D]`` each.  NVFP4 block scales are
    gathered through the same page table as the data they scale."""
    def gather(pool):
        return gather_request_kv(pool, kv_indptr, kv_indices, kv_last_page_len, page_size, b)
    k_bs = None if k_sf is None else gather(k_sf)
    v_bs = None if v_sf is None else gather(v_sf)
    return (kv_values(gather(k_pool), kv_dtype, k_scale, k_bs),
            kv_values(gather(v_pool), kv_dtype, v_scale, v_bs))


def _value_width(pool, kv_dtype):
    """head_dim of a pool: NVFP4 stores two elements per byte."""
    return pool.shape[3] * (2 if kv_dtype == "nvfp4" else 1)


def decode_ref(q, k_pool, v_pool, kv_indptr, kv_indices, kv_last_page_len, page_size,
               sm_scale, window=0, kv_dtype="bf16", k_scale=1.0, v_scale=1.0,
               requests=None, k_sf=None, v_sf=None):
    """Single-token paged decode.

    q: float64 ``[B, Hq, Dqk]`` (one query token per request, at position L_b - 1).
    k_pool / v_pool: stored elements ``[num_pages, Hkv, P, Dqk]`` / ``[..., Dvo]`` (NVFP4:
    packed bytes ``[..., D/2]`` with block scales k_sf / v_sf ``[..., D/16]``).
    Returns (o ``[B, Hq, Dvo]``, lse ``[B, Hq]``), or only the rows of ``requests``.
    """
    q = np.asarray(q, dtype=np.float64)
    batch, hq, _ = q.shape
    hkv = k_pool.shape[1]
    if hq % hkv:
        raise ValueError("num_qo_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    dvo = _value_width(v_pool, kv_dtype)
    lens = request_kv_len(kv_indptr, kv_last_page_len, page_size)
    reqs = list(range(batch)) if requests is None else list(requests)
    o = np.zeros((len(reqs), hq, dvo), dtype=np.float64)
    lse = np.full((len(reqs), hq), -np.inf, dtype=np.float64)
    for r, b in enumerate(reqs):
        k, v = _request_kv_f64(k_pool, v_pool, kv_dtype, k_scale, v_scale, kv_indptr,
                               kv_indices, kv_last_page_len, page_size, b, k_sf, v_sf)
        length = int(lens[b])
        mask = visible_mask([length - 1], length, True, window)
        for h in range(hq):
            kvh = h // group
            o_h, lse_h = softmax_attention(q[b, h][None, :], k[:, kvh, :], v[:, kvh, :],
                                           mask, sm_scale)
            o[r, h], lse[r, h] = o_h[0], lse_h[0]
    return o, lse


def prefill_ref(q, qo_indptr, k_pool, v_pool, kv_indptr, kv_indices, kv_last_page_len,
                page_size, sm_scale, causal=True, window=0, kv_dtype="bf16", k_scale=1.0,
                v_scale=1.0, tokens=None, k_sf=None, v_sf=None):
    """Paged prefill of the new tokens of every request.

    q: float64 ``[Nq, Hq, Dqk]``, ragged by ``qo_indptr``.  The q_len_b new tokens of
    request b are its last q_len_b KV tokens, so row i sits at ``L_b - q_len_b + i``.
    Returns (o ``[Nq, Hq, Dvo]``, lse ``[Nq, Hq]``), or only the rows listed in
    ``tokens`` (global query-token indices), in that order.
    """
    q = np.asarray(q, dtype=np.float64)
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    n_q, hq, _ = q.shape
    hkv = k_pool.shape[1]
    if hq % hkv:
        raise ValueError("num_qo_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    dvo = _value_width(v_pool, kv_dtype)
    lens = request_kv_len(kv_indptr, kv_last_page_len, page_size)
    sel = np.arange(n_q) if tokens is None else np.asarray(tokens, dtype=np.int64)
    o = np.zeros((len(sel), hq, dvo), dtype=np.float64)
    lse = np.full((len(sel), hq), -np.inf, dtype=np.float64)
    batch = len(qo_indptr) - 1
    for b in range(batch):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        rows = np.nonzero((sel >= q0) & (sel < q1))[0]
        if len(rows) == 0:
            continue
        q_len, length = q1 - q0, int(lens[b])
        if q_len > length:
            raise ValueError("a request has more new tokens than KV tokens")
        k, v = _request_kv_f64(k_pool, v_pool, kv_dtype, k_scale, v_scale, kv_indptr,
                               kv_indices, kv_last_page_len, page_size, b, k_sf, v_sf)
        pos = length - q_len + (sel[rows] - q0)
        mask = visible_mask(pos, length, causal, window)
        for h in range(hq):
            kvh = h // group
            o_h, lse_h = softmax_attention(q[sel[rows], h, :], k[:, kvh, :], v[:, kvh, :],
                                           mask, sm_scale)
            o[rows, h], lse[rows, h] = o_h, lse_h
    return o, lse


def chunk_partial_ref(q, k, v, mask_row, t_begin, t_end, sm_scale):
    """Partial state of one query over the keys of ``[t_begin, t_end)`` it can see.

    q ``[Dqk]``, k ``[L, Dqk]``, v ``[L, Dvo]``, mask_row ``[L]`` (its visible set) ->
    (o_c ``[Dvo]`` normalised within the chunk, lse_c).
    """
    length = k.shape[0]
    chunk = np.zeros(length, dtype=bool)
    chunk[t_begin:t_end] = True
    o, lse = softmax_attention(np.asarray(q)[None, :], k, v,
                               (np.asarray(mask_row) & chunk)[None, :], sm_scale)
    return o[0], lse[0]


def merge_ref(o_parts, lse_parts):
    """Log-sum-exp merge of partial states over disjoint key chunks.

    o_parts ``[S, ..., D]`` (each normalised within its chunk), lse_parts ``[S, ...]`` ->
    (o ``[..., D]``, lse ``[...]``).  Chunks with lse = -inf (nothing visible) carry no
    weight; if every chunk is empty the result is o = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    finite = np.isfinite(lse_parts)
    any_finite = finite.any(axis=0)
    m = np.where(any_finite, np.where(finite, lse_parts, -np.inf).max(axis=0), 0.0)
    w = np.where(finite, np.exp(np.where(finite, lse_parts, 0.0) - m), 0.0)
    total = w.sum(axis=0)
    safe = np.where(total > 0, total, 1.0)
    o = (w[..., None] * o_parts).sum(axis=0) / safe[..., None]
    o = np.where(any_finite[..., None], o, 0.0)
    lse = np.where(any_finite, m + np.log(safe), -np.inf)
    return o, lse
