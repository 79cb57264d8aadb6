"""Seeded generators for paged-attention inputs.

Recipe (every case): request lengths and the page permutation come from a numpy PCG64
generator seeded with ``seed``; Q, K and V values come from a torch generator seeded with
``seed + 1`` on the target device (CPU for the small cases, the GPU for the large ones),
drawn as float32 N(0, 1) and rounded to bf16 (round-to-nearest-even).  FP8 K and V are
N(0, 1) divided by a per-tensor scale amax/448 of the drawn data, clamped to +-448 and
rounded to E4M3FN; the scale (rounded to fp32, the type the library takes) is returned
with the case.  NVFP4 K and V are N(0, 1) quantised
the usual two-level way: a per-tensor fp32 scale g = amax / (6 * 448), then per 16
consecutive head_dim elements of one token a block scale amax_block / (6 g) rounded to
E4M3FN, then each element x / (block scale * g) rounded to the nearest E2M1 value and
packed two per byte (element 2i in the low nibble).  The block scales sit in a separate
uint8 tensor shaped like the data with head_dim / 16 per row.

The pool holds the pages the requests need plus slack; pages are handed out in a random
order.  Every element no query can see -- slots past a request's last-page length, pages
no request uses, and keys before a sliding window -- holds a finite poison value (bf16
+-30000, FP8 code 0x7E, NVFP4 byte 0x77 with block scale 0x7E) so that a kernel reading them produces a visibly wrong result.

The cache is the combined HND layout ``[num_pages, 2, num_kv_heads, page_size, head_dim]``
(K at index 0, V at 1) when K and V have the same width, or two pools
``[num_pages, num_kv_heads, page_size, head_dim_{qk,vo}]`` sharing one page table
otherwise.
"""

from dataclasses import dataclass, field
from typing import Optional

import math

import numpy as np
import torch

BF16_POISON_K = 30000.0
BF16_POISON_V = -30000.0
FP8_POISON_CODE = 0x7E
FP8_MAX = 448.0
FP4_POISON_BYTE = 0x77
FP4_MAX = 6.0
# E2M1 magnitudes of codes 0..7 and the midpoints between neighbours (for rounding).
_E2M1_MAGS = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
_E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


@dataclass
class DecodeCase:
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_vo: int
    page_size: int
    kv_dtype: str  # "bf16" | "fp8" | "nvfp4"
    window: int
    num_splits: int
    out_dtype: str  # "fp32" | "bf16"
    sm_scale: float
    kv_lens: np.ndarray
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    kv_last_page_len: np.ndarray
    num_pages: int
    q: torch.Tensor  # bf16 [B, Hq, Dqk]
    k_pool: torch.Tensor  # [NP, Hkv, P, Dqk] view (bf16 or uint8 codes)
    v_pool: torch.Tensor  # [NP, Hkv, P, Dvo] view
    cache: Optional[torch.Tensor] = None  # combined [NP, 2, Hkv, P, D] when Dqk == Dvo
    k_scale: float = 1.0
    v_scale: float = 1.0
    name: str = ""
    meta: dict = field(default_factory=dict)
    k_sf: Optional[torch.Tensor] = None  # NVFP4 block scales [NP, Hkv, P, Dqk/16] view
    v_sf: Optional[torch.Tensor] = None
    sf_cache: Optional[torch.Tensor] = None  # combined [NP, 2, Hkv, P, D/16]


@dataclass
class PrefillCase:
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_vo: int
    page_size: int
    kv_dtype: str
    window: int
    causal: bool
    out_dtype: str
    sm_scale: float
    qo_lens: np.ndarray
    qo_indptr: np.ndarray
    kv_lens: np.ndarray
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    kv_last_page_len: np.ndarray
    num_pages: int
    q: torch.Tensor  # bf16 [Nq, Hq, Dqk]
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    cache: Optional[torch.Tensor] = None
    k_scale: float = 1.0
    v_scale: float = 1.0
    name: str = ""
    meta: dict = field(default_factory=dict)
    k_sf: Optional[torch.Tensor] = None  # NVFP4 block scales [NP, Hkv, P, Dqk/16] view
    v_sf: Optional[torch.Tensor] = None
    sf_cache: Optional[torch.Tensor] = None  # combined [NP, 2, Hkv, P, D/16]


def _page_table(rng, kv_lens, page_size, slack_pages):
    """Shuffled page pool: returns indptr, indices, last_page_len, num_pages."""
    n_pages = [(int(L) + page_size - 1) // page_size for L in kv_lens]
    needed = int(sum(n_pages))
    num_pages = needed + int(slack_pages)
    perm = rng.permutation(num_pages).astype(np.int32)
    indptr = np.zeros(len(kv_lens) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(n_pages)
    indices = perm[:needed].copy()
    last = np.array([(int(L) - 1) % page_size + 1 if L > 0 else 0 for L in kv_lens],
                    dtype=np.int32)
    return indptr, indices, last, num_pages


def _visible_slots(kv_lens, indptr, indices, page_size, num_pages, first_visible):
    """Boolean [num_pages, page_size]: slot holds a key some query can see."""
    valid = np.zeros((num_pages, page_size), dtype=bool)
    for b, length in enumerate(kv_lens):
        length = int(length)
        if length == 0:
            continue
        t = np.arange(int(first_visible[b]), length, dtype=np.int64)
        pages = indices[indptr[b] + t // page_size]
        valid[pages, t % page_size] = True
    return valid


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _bf16_pool(shape, gen, device, chunk_elems=1 << 28):
    """N(0,1) rounded to bf16, generated in slabs along dim 0 to bound temporaries."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    per = max(1, chunk_elems // max(1, math.prod(shape[1:])))
    for s in range(0, shape[0], per):
        e = min(shape[0], s + per)
        out[s:e] = _randn((e - s,) + tuple(shape[1:]), gen, device).to(torch.bfloat16)
    return out


def _fp8_pool(shape, gen, device, chunk_elems=1 << 28):
    """N(0,1) / (amax/448) rounded to E4M3FN; returns (uint8 codes, scale)."""
    codes = torch.empty(shape, dtype=torch.uint8, device=device)
    per = max(1, chunk_elems // max(1, math.prod(shape[1:])))
    slabs = []
    amax = 0.0
    # Draw once, remember the slabs' generator states so the same values are re-drawn
    # for encoding without holding the float32 pool in memory.
    for s in range(0, shape[0], per):
        e = min(shape[0], s + per)
        state = gen.get_state()
        x = _randn((e - s,) + tuple(shape[1:]), gen, device)
        amax = max(amax, float(x.abs().max()))
        slabs.append((s, e, state))
    scale = float(np.float32(amax / FP8_MAX))  # the C ABI takes fp32 scales
    for s, e, state in slabs:
        gen.set_state(state)
        x = _randn((e - s,) + tuple(shape[1:]), gen, device)
        x = torch.clamp(x / scale, -FP8_MAX, FP8_MAX)
        codes[s:e] = x.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def _nvfp4_encode(x, g):
    """x float32 [..., D], tensor scale g -> (packed uint8 [..., D/2], block scales [..., D/16])."""
    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // 16, 16))
    bs = (blocks.abs().amax(dim=-1) / (FP4_MAX * g)).clamp(max=FP8_MAX)
    bs_codes = bs.to(torch.float8_e4m3fn)
    bs_val = bs_codes.to(torch.float32)
    y = blocks / (torch.where(bs_val > 0, bs_val, torch.ones_like(bs_val)) * g)[..., None]
    y = y.clamp(-FP4_MAX, FP4_MAX).reshape(x.shape)
    mids = torch.tensor(_E2M1_MIDS, dtype=torch.float32, device=x.device)
    mag = torch.bucketize(y.abs(), mids).to(torch.uint8)
    codes = mag | ((y < 0) & (mag > 0)).to(torch.uint8) << 3
    packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
    return packed, bs_codes.view(torch.uint8)


def _nvfp4_pool(shape, gen, device, chunk_elems=1 << 26):
    """N(0,1) quantised to NVFP4; returns (packed [..., D/2], block scales [..., D/16], g)."""
    d = shape[-1]
    packed = torch.empty(tuple(shape[:-1]) + (d // 2,), dtype=torch.uint8, device=device)
    scales = torch.empty(tuple(shape[:-1]) + (d // 16,), dtype=torch.uint8, device=device)
    per = max(1, chunk_elems // max(1, math.prod(shape[1:])))
    slabs = []
    amax = 0.0
    for s in range(0, shape[0], per):
        e = min(shape[0], s + per)
        state = gen.get_state()
        x = _randn((e - s,) + tuple(shape[1:]), gen, device)
        amax = max(amax, float(x.abs().max()))
        slabs.append((s, e, state))
    g = float(np.float32(amax / (FP4_MAX * FP8_MAX)))  # the C ABI takes fp32 scales
    for s, e, state in slabs:
        gen.set_state(state)
        x = _randn((e - s,) + tuple(shape[1:]), gen, device)
        packed[s:e], scales[s:e] = _nvfp4_encode(x, g)
    return packed, scales, g


def _poison(pool_k, pool_v, valid, kv_dtype, k_sf=None, v_sf=None):
    dev = pool_k.device
    invalid = torch.from_numpy(~valid).to(dev)[:, None, :, None]  # [NP, 1, P, 1]
    if kv_dtype == "bf16":
        pool_k.masked_fill_(invalid, BF16_POISON_K)
        pool_v.masked_fill_(invalid, BF16_POISON_V)
    elif kv_dtype == "fp8":
        pool_k.masked_fill_(invalid, FP8_POISON_CODE)
        pool_v.masked_fill_(invalid, FP8_POISON_CODE)
    else:
        pool_k.masked_fill_(invalid, FP4_POISON_BYTE)
        pool_v.masked_fill_(invalid, FP4_POISON_BYTE)
        k_sf.masked_fill_(invalid, FP8_POISON_CODE)
        v_sf.masked_fill_(invalid, FP8_POISON_CODE)


def _kv_pools(num_pages, hkv, page_size, dqk, dvo, kv_dtype, gen, device):
    """Returns (cache or None, k_pool, v_pool, k_scale, v_scale, block-scale dict)."""
    if kv_dtype == "nvfp4":
        k, k_sf, k_scale = _nvfp4_pool((num_pages, hkv, page_size, dqk), gen, device)
        v, v_sf, v_scale = _nvfp4_pool((num_pages, hkv, page_size, dvo), gen, device)
        if dqk != dvo:
            return None, k, v, k_scale, v_scale, dict(k_sf=k_sf, v_sf=v_sf)
        cache = torch.stack([k, v], dim=1)
        sf_cache = torch.stack([k_sf, v_sf], dim=1)
        del k, v, k_sf, v_sf
        return (cache, cache[:, 0], cache[:, 1], k_scale, v_scale,
                dict(k_sf=sf_cache[:, 0], v_sf=sf_cache[:, 1], sf_cache=sf_cache))
    return _kv_pools_8_16(num_pages, hkv, page_size, dqk, dvo, kv_dtype, gen, device) + ({},)


def _kv_pools_8_16(num_pages, hkv, page_size, dqk, dvo, kv_dtype, gen, device):
    if dqk == dvo:
        shape = (num_pages, 2, hkv, page_size, dqk)
        if kv_dtype == "bf16":
            cache = _bf16_pool(shape, gen, device)
            return cache, cache[:, 0], cache[:, 1], 1.0, 1.0
        # One scale per tensor: draw K and V halves separately.
        cache = torch.empty(shape, dtype=torch.uint8, device=device)
        k_codes, k_scale = _fp8_pool((num_pages, hkv, page_size, dqk), gen, device)
        v_codes, v_scale = _fp8_pool((num_pages, hkv, page_size, dvo), gen, device)
        cache[:, 0] = k_codes
        cache[:, 1] = v_codes
        del k_codes, v_codes
        return cache, cache[:, 0], cache[:, 1], k_scale, v_scale
    if kv_dtype == "bf16":
        k = _bf16_pool((num_pages, hkv, page_size, dqk), gen, device)
        v = _bf16_pool((num_pages, hkv, page_size, dvo), gen, device)
        return None, k, v, 1.0, 1.0
    k, k_scale = _fp8_pool((num_pages, hkv, page_size, dqk), gen, device)
    v, v_scale = _fp8_pool((num_pages, hkv, page_size, dvo), gen, device)
    return None, k, v, k_scale, v_scale


def make_decode_case(kv_lens, num_qo_heads, num_kv_heads, head_dim_qk, page_size, *,
                     head_dim_vo=None, kv_dtype="bf16", window=0, num_splits=0,
                     out_dtype="bf16", sm_scale=None, seed=0, device="cpu",
                     slack_pages=None, name="", poison_window=True):
    """One decode batch: one query token per request at position L_b - 1."""
    head_dim_vo = head_dim_qk if head_dim_vo is None else head_dim_vo
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(seed))
    needed = int(sum((int(L) + page_size - 1) // page_size for L in kv_lens))
    slack = max(2, needed // 10) if slack_pages is None else slack_pages
    indptr, indices, last, num_pages = _page_table(rng, kv_lens, page_size, slack)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 1)
    batch = len(kv_lens)
    q = _randn((batch, num_qo_heads, head_dim_qk), gen, device).to(torch.bfloat16)
    cache, k_pool, v_pool, k_scale, v_scale, sf = _kv_pools(
        num_pages, num_kv_heads, page_size, head_dim_qk, head_dim_vo, kv_dtype, gen, device)
    if window > 0 and poison_window:
        first = np.maximum(0, kv_lens - window)
    else:
        first = np.zeros_like(kv_lens)
    valid = _visible_slots(kv_lens, indptr, indices, page_size, num_pages, first)
    _poison(k_pool, v_pool, valid, kv_dtype, sf.get("k_sf"), sf.get("v_sf"))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim_qk)
    return DecodeCase(batch, num_qo_heads, num_kv_heads, head_dim_qk, head_dim_vo, page_size,
                      kv_dtype, window, num_splits, out_dtype, sm_scale, kv_lens, indptr,
                      indices, last, num_pages, q, k_pool, v_pool, cache, k_scale, v_scale,
                      name, **sf)


def make_prefill_case(qo_lens, kv_lens, num_qo_heads, num_kv_heads, head_dim_qk, page_size,
                      *, head_dim_vo=None, kv_dtype="bf16", window=0, causal=True,
                      out_dtype="bf16", sm_scale=None, seed=0, device="cpu",
                      slack_pages=None, name=""):
    """Paged prefill: the q_len new tokens of a request are its last KV tokens."""
    head_dim_vo = head_dim_qk if head_dim_vo is None else head_dim_vo
    qo_lens = np.asarray(qo_lens, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    if np.any(qo_lens > kv_lens):
        raise ValueError("q_len must not exceed kv_len")
    rng = np.random.Generator(np.random.PCG64(seed))
    needed = int(sum((int(L) + page_size - 1) // page_size for L in kv_lens))
    slack = max(2, needed // 10) if slack_pages is None else slack_pages
    indptr, indices, last, num_pages = _page_table(rng, kv_lens, page_size, slack)
    qo_indptr = np.zeros(len(qo_lens) + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_lens)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 1)
    n_q = int(qo_indptr[-1])
    q = _randn((n_q, num_qo_heads, head_dim_qk), gen, device).to(torch.bfloat16)
    cache, k_pool, v_pool, k_scale, v_scale, sf = _kv_pools(
        num_pages, num_kv_heads, page_size, head_dim_qk, head_dim_vo, kv_dtype, gen, device)
    if window > 0:
        first = np.maximum(0, kv_lens - qo_lens - window + 1)
    else:
        first = np.zeros_like(kv_lens)
    valid = _visible_slots(kv_lens, indptr, indices, page_size, num_pages, first)
    _poison(k_pool, v_pool, valid, kv_dtype, sf.get("k_sf"), sf.get("v_sf"))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim_qk)
    return PrefillCase(len(qo_lens), num_qo_heads, num_kv_heads, head_dim_qk, head_dim_vo,
                       page_size, kv_dtype, window, causal, out_dtype, sm_scale, qo_lens,
                       qo_indptr, kv_lens, indptr, indices, last, num_pages, q, k_pool,
                       v_pool, cache, k_scale, v_scale, name, **sf)


# The workloads (sizes, head counts, page sizes, length mixes and dtypes) the benchmark
# and the full-size parity tests run.  Seeds are 1000 + workload number.
WORKLOADS = {
    "tiny_decode": dict(kind="decode", kv_lens=[37, 64], num_qo_heads=8, num_kv_heads=1,
                        head_dim_qk=512, page_size=16, out_dtype="fp32", num_splits=1,
                        slack_pages=9, seed=1001),
    # The GQA decode runs the balanced partition (num_splits 0); variant "splitk8" runs the
    # same inputs with every request cut into exactly 8 key chunks.
    "gqa_decode": dict(kind="decode", batch=32, len_range=(1024, 8192), num_qo_heads=24,
                       num_kv_heads=4, head_dim_qk=512, page_size=16, num_splits=0,
                       seed=1002),
    "fp8_decode": dict(kind="decode", batch=64, len_range=(4096, 32768), num_qo_heads=12,
                       num_kv_heads=4, head_dim_qk=512, page_size=64, kv_dtype="fp8",
                       num_splits=0, seed=1003),
    # NVFP4 KV at the FP8 workload's geometry: 4-bit codes plus one E4M3 scale per 16.
    "nvfp4_decode": dict(kind="decode", batch=64, len_range=(4096, 32768), num_qo_heads=12,
                         num_kv_heads=4, head_dim_qk=512, page_size=64, kv_dtype="nvfp4",
                         num_splits=0, seed=1007),
    "window_decode": dict(kind="decode", batch=48, len_range=(512, 16384), num_qo_heads=16,
                          num_kv_heads=8, window=1024, num_splits=0, seed=1004,
                          variants=[(512, 1), (512, 32), (256, 1), (256, 32)]),
    "causal_prefill": dict(kind="prefill", batch=4, qo_len=4096, prefix=1024,
                           num_qo_heads=16, num_kv_heads=8, head_dim_qk=512, page_size=64,
                           variants=[512, 256], seed=1005),
    # The causal prefill geometry over an FP8 E4M3FN cache (cast on load).
    "fp8_prefill": dict(kind="prefill", batch=4, qo_len=4096, prefix=1024,
                        num_qo_heads=16, num_kv_heads=8, head_dim_qk=512, page_size=64,
                        kv_dtype="fp8", variants=[512, 256], seed=1009),
    # The NVFP4 page's shape: asymmetric qk 512 / vo 256 prefill over an NVFP4 cache.
    "nvfp4_prefill": dict(kind="prefill", batch=4, qo_len=4096, prefix=1024,
                          num_qo_heads=16, num_kv_heads=8, head_dim_qk=512, page_size=64,
                          kv_dtype="nvfp4", variants=[256], seed=1008),
    # Short-query extend (a few new tokens over a long cached prefix): the split-K prefill
    # geometry; HBM-bound.
    "extend_prefill": dict(kind="prefill", batch=8, qo_len=16, prefix=16368,
                           num_qo_heads=16, num_kv_heads=8, head_dim_qk=512, page_size=64,
                           variants=[512], seed=1006),
}


def decode_workload(name, device="cpu", variant=None):
    """Builds one decode workload by name (a variant picks (head_dim, page_size))."""
    w = dict(WORKLOADS[name])
    assert w.pop("kind") == "decode"
    seed = w.pop("seed")
    if "len_range" in w:
        lo, hi = w.pop("len_range")
        batch = w.pop("batch")
        rng = np.random.Generator(np.random.PCG64(seed + 500))
        kv_lens = rng.integers(lo, hi + 1, size=batch)
    else:
        kv_lens = w.pop("kv_lens")
    variants = w.pop("variants", None)
    if isinstance(variant, str):
        assert variant.startswith("splitk"), variant
        w["num_splits"] = int(variant[len("splitk"):])
    elif variants is not None:
        dim, page = variants[0] if variant is None else variant
        w["head_dim_qk"], w["page_size"] = dim, page
    return make_decode_case(kv_lens, seed=seed, device=device, name=name, **w)


def prefill_workload(name, device="cpu", head_dim_vo=None):
    w = dict(WORKLOADS[name])
    assert w.pop("kind") == "prefill"
    seed = w.pop("seed")
    batch, qo_len, prefix = w.pop("batch"), w.pop("qo_len"), w.pop("prefix")
    w.pop("variants")
    qo_lens = [qo_len] * batch
    kv_lens = [qo_len + prefix] * batch
    return make_prefill_case(qo_lens, kv_lens, seed=seed, device=device, name=name,
                             head_dim_vo=head_dim_vo, **w)


def extract_requests(case, requests, device="cpu"):
    """Copies the pages of some requests into a compact case (pages renumbered in order).

    Used to run the CPU check on a sample of a large batch; only inputs are moved.
    """
    requests = list(requests)
    page_lists, lens, lasts = [], [], []
    for b in requests:
        s, e = int(case.kv_indptr[b]), int(case.kv_indptr[b + 1])
        page_lists.append(case.kv_indices[s:e])
        lens.append(int(case.kv_lens[b]))
        lasts.append(int(case.kv_last_page_len[b]))
    pages = np.concatenate(page_lists) if page_lists else np.zeros(0, np.int32)
    sel = torch.from_numpy(pages.astype(np.int64)).to(case.k_pool.device)
    k_pool = case.k_pool.index_select(0, sel).to(device)
    v_pool = case.v_pool.index_select(0, sel).to(device)
    indptr = np.zeros(len(requests) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum([len(p) for p in page_lists])
    out = dict(kv_lens=np.asarray(lens, np.int64), kv_indptr=indptr,
               kv_indices=np.arange(len(pages), dtype=np.int32),
               kv_last_page_len=np.asarray(lasts, np.int32), k_pool=k_pool, v_pool=v_pool)
    if case.k_sf is not None:
        out["k_sf"] = case.k_sf.index_select(0, sel).to(device)
        out["v_sf"] = case.v_sf.index_select(0, sel).to(device)
    if isinstance(case, DecodeCase):
        out["q"] = case.q[requests].to(device)
    else:
        rows = [np.arange(case.qo_indptr[b], case.qo_indptr[b + 1]) for b in requests]
        qo_lens = np.asarray([len(r) for r in rows], np.int64)
        qo_indptr = np.zeros(len(requests) + 1, dtype=np.int32)
        qo_indptr[1:] = np.cumsum(qo_lens)
        idx = torch.from_numpy(np.concatenate(rows).astype(np.int64)).to(case.q.device)
        out["q"] = case.q.index_select(0, idx).to(device)
        out["qo_indptr"] = qo_indptr
        out["qo_lens"] = qo_lens
    return out
