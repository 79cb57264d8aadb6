"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerances: for bf16 inputs with fp32 accumulation, max-abs error <= 1e-2 and mean-abs
error <= 1e-3 over every valid output element; lse max-abs <= 1e-3 where finite, and the
same -inf positions.  FP8 and NVFP4 KV are compared with the oracle run on the stored
codes (and block scales), which it dequantises itself.

A bf16 output also carries the rounding of the exact result to bf16, up to half an ulp,
i.e. 2^-8 |ref|; that alone exceeds 1e-2 once |ref| > 2.56 (rows that see few keys).  For
bf16 outputs the per-element bound is therefore 1e-2 + 2^-8 |ref|, and a separate
bit-exact test checks that the bf16 output is the round-to-nearest-even of the fp32
output of the same computation.
"""

import sys

import numpy as np
import torch

import oracle
from synth import extract_requests

MAX_ABS = 1e-2
MEAN_ABS = 1e-3
LSE_ABS = 1e-3


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def bf16_to_np(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def pool_to_np(t, kv_dtype):
    t = t.detach().contiguous().cpu()
    if kv_dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.uint8).numpy()


def out_to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(name, got, ref, got_lse=None, ref_lse=None, out_dtype="fp32"):
    err = np.abs(got - ref)
    max_abs, mean_abs = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    msg = f"{name}: max_abs={max_abs:.3e} mean_abs={mean_abs:.3e}"
    bound = MAX_ABS + (np.abs(ref) * 2.0 ** -8 if out_dtype == "bf16" else 0.0)
    ok = bool(np.all(err <= bound)) and mean_abs <= MEAN_ABS and np.isfinite(got).all()
    if got_lse is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(got_lse), fin), f"{name}: lse -inf pattern differs"
        lerr = float(np.abs(got_lse[fin] - ref_lse[fin]).max(initial=0.0))
        msg += f" lse_max_abs={lerr:.3e}"
        ok = ok and lerr <= LSE_ABS
    say(msg)
    assert ok, msg
    return max_abs, mean_abs


def _scales_np(src):
    """NVFP4 block-scale pools of a case (or of a copied-out sample) as numpy, else None."""
    if src.get("k_sf") is None:
        return {}
    return dict(k_sf=pool_to_np(src["k_sf"], "nvfp4"), v_sf=pool_to_np(src["v_sf"], "nvfp4"))


def oracle_decode(case, requests=None):
    """Oracle on the case's inputs (all requests, or a sample copied out page by page)."""
    if requests is None:
        kp = pool_to_np(case.k_pool, case.kv_dtype)
        vp = pool_to_np(case.v_pool, case.kv_dtype)
        q = oracle.bf16_bits_to_f64(bf16_to_np(case.q))
        return oracle.decode_ref(q, kp, vp, case.kv_indptr, case.kv_indices,
                                 case.kv_last_page_len, case.page_size, case.sm_scale,
                                 window=case.window, kv_dtype=case.kv_dtype,
                                 k_scale=case.k_scale, v_scale=case.v_scale,
                                 **_scales_np(dict(k_sf=case.k_sf, v_sf=case.v_sf)))
    sub = extract_requests(case, requests)
    q = oracle.bf16_bits_to_f64(bf16_to_np(sub["q"]))
    return oracle.decode_ref(q, pool_to_np(sub["k_pool"], case.kv_dtype),
                             pool_to_np(sub["v_pool"], case.kv_dtype), sub["kv_indptr"],
                             sub["kv_indices"], sub["kv_last_page_len"], case.page_size,
                             case.sm_scale, window=case.window, kv_dtype=case.kv_dtype,
                             k_scale=case.k_scale, v_scale=case.v_scale, **_scales_np(sub))


def oracle_prefill(case, tokens=None, requests=None):
    scales = dict(k_scale=case.k_scale, v_scale=case.v_scale)
    if requests is None:
        kp = pool_to_np(case.k_pool, case.kv_dtype)
        vp = pool_to_np(case.v_pool, case.kv_dtype)
        q = oracle.bf16_bits_to_f64(bf16_to_np(case.q))
        return oracle.prefill_ref(q, case.qo_indptr, kp, vp, case.kv_indptr, case.kv_indices,
                                  case.kv_last_page_len, case.page_size, case.sm_scale,
                                  causal=case.causal, window=case.window,
                                  kv_dtype=case.kv_dtype, tokens=tokens, **scales,
                                  **_scales_np(dict(k_sf=case.k_sf, v_sf=case.v_sf)))
    sub = extract_requests(case, requests)
    q = oracle.bf16_bits_to_f64(bf16_to_np(sub["q"]))
    return oracle.prefill_ref(q, sub["qo_indptr"], pool_to_np(sub["k_pool"], case.kv_dtype),
                              pool_to_np(sub["v_pool"], case.kv_dtype), sub["kv_indptr"],
                              sub["kv_indices"], sub["kv_last_page_len"], case.page_size,
                              case.sm_scale, causal=case.causal, window=case.window,
                              kv_dtype=case.kv_dtype, tokens=tokens, **scales,
                              **_scales_np(sub))


def gpu_decode(case, num_splits=None, out_dtype=None, with_lse=True):
    from paged_attention_hd512_amd import PagedDecode
    runner = PagedDecode(case.k_pool, case.v_pool, case.kv_indptr, case.kv_indices,
                         case.kv_last_page_len, case.num_qo_heads, kv_dtype=case.kv_dtype,
                         k_scale=case.k_scale, v_scale=case.v_scale, sm_scale=case.sm_scale,
                         window=case.window,
                         num_splits=case.num_splits if num_splits is None else num_splits,
                         out_dtype=out_dtype or case.out_dtype, k_sf=case.k_sf, v_sf=case.v_sf)
    out, lse = runner.run(case.q, with_lse=with_lse)
    torch.cuda.synchronize()
    return runner, out, lse


def gpu_prefill(case, out_dtype=None):
    from paged_attention_hd512_amd import PagedPrefill
    runner = PagedPrefill(case.k_pool, case.v_pool, case.qo_indptr, case.kv_indptr,
                          case.kv_indices, case.kv_last_page_len, case.num_qo_heads,
                          kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale,
                          sm_scale=case.sm_scale, window=case.window, causal=case.causal,
                          out_dtype=out_dtype or case.out_dtype, k_sf=case.k_sf, v_sf=case.v_sf)
    out, lse = runner.run(case.q)
    torch.cuda.synchronize()
    return runner, out, lse


def bf16_rne_bits(x):
    """Round-to-nearest-even of float32 values to bf16 bit patterns (test-side helper)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def repad(t, extra):
    """The same values in a new allocation whose rows are `extra` elements longer: a
    strided view with its own stride family."""
    parent = torch.zeros(tuple(t.shape[:-1]) + (t.shape[-1] + extra,), dtype=t.dtype,
                         device=t.device)
    parent[..., :t.shape[-1]] = t
    return parent[..., :t.shape[-1]]
