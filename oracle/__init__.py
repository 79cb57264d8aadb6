"""Plain fp64 CPU oracle for paged GQA softmax attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The HIP
library never calls it, and it shares no code with the HIP library: no kernels, no
headers, no helpers, no tables.

What it computes is the plain definition of attention over a paged KV cache, written out
in float64 with numpy, with no tiling, no split and no online softmax.  The pages it
follows are cited by title and section:

* [Triton-hd512]  "[None][feat] Run Gemma4 head_dim 512 attention on Triton"
  (TensorRT-LLM pull request 17772).
* [FA2-SM120]     "[https://nvbugs/6566891][fix] Use FlashInfer FA2 for Gemma4 on SM120 and
  SM121" (TensorRT-LLM pull request 17557).
* [VO-split]      "feat(attention): asymmetric VO-split NVFP4 paged prefill (qk=512/vo=256)
  for Gemma-4 on SM120/121" (FlashInfer pull request 3684).

Every function below is pinned by the CPU tests against something other than itself
(brute-force dense attention, closed forms, invariants, torch's own dtype conversions).
Nothing here is "parity unpinned".
"""

from .numerics import (bf16_bits_to_f64, e4m3fn_value, E4M3FN_VALUES, e2m1_value, E2M1_VALUES,
                       nvfp4_values, kv_values)
from .attention import (
    request_kv_len,
    gather_request_kv,
    visible_mask,
    softmax_attention,
    decode_ref,
    prefill_ref,
    chunk_partial_ref,
    merge_ref,
)
from .partition import decode_partition_ref, prefill_plan_ref

__all__ = [
    "bf16_bits_to_f64",
    "e4m3fn_value",
    "E4M3FN_VALUES",
    "e2m1_value",
    "E2M1_VALUES",
    "nvfp4_values",
    "kv_values",
    "request_kv_len",
    "gather_request_kv",
    "visible_mask",
    "softmax_attention",
    "decode_ref",
    "prefill_ref",
    "chunk_partial_ref",
    "merge_ref",
    "decode_partition_ref",
    "prefill_plan_ref",
]
