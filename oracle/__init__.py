"""Plain, slow CPU oracle for one decode step of a parallel-layer MoE transformer.

This package is TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path (``libmk.so`` and its Python
binding) never imports, links or runs anything in here, and nothing in here imports the product.

Sources. The method is described by three web pages about Cohere's decode megakernel:

* P1 - the aimodeling.com article "cohere-megakernel-north-mini-code-h100", sections
  "Decode is a bandwidth game", "One persistent kernel for the whole decode step",
  "From demo to a full serving system", "Caveats and takeaways".
* P2 - "Cohere Megakernel Beats vLLM by 1.58x on H100 GPUs" (latestnews.news), single body.
* P3 - "Cohere Releases Megakernel Engine for North Mini Code, Achieving Up to 1.41x Speedup
  Over vLLM" (aibriefing.imbch.dev), sections "Key Technologies and Architecture",
  "Scheduling and Performance Benchmarks", "Limitations and Future Plans".

The megakernel is an execution strategy; what it computes is an ordinary decode step, so the
oracle is that plain definition written out (``oracle.decode``). Readings taken where the pages
are silent are listed in ``oracle.decode``'s docstring, each marked "reading". A prompt's prefill
(``oracle.prefill``) is the same layers over all prompt positions at once, causally masked.

Pins (tests marked ``not gpu``): bf16 codec exhaustive + library cross-check; GEMV vs fp64 with
the standard dot-product error bound; RMSNorm closed form and invariants; RoPE vs complex
multiplication, identity at pos 0, norm and relative-position invariants; attention vs an explicit
per-key loop, one-key / identical-key / dominant-key special cases, GQA == repeated-KV MHA; paged ==
contiguous gather; top-k vs brute-force rank counting with constructed ties; router weights vs the
full softmax renormalised; MoE sparse sum vs a dense loop over every expert with a mask; whole step
fp32 vs fp64, batch-row independence, zero branch weights -> identity. Prefill: equal to the
decode step one position at a time, to itself on a split prompt, causal, and a one-position
prefill equal to a decode step; planted mistakes (mask off by one, no mask, RoPE positions, stale
keys, unweighted experts) each fail a pin. FP8 weights: E4M3 decoder vs torch's float8_e4m3fn for all
256 codes and at the format's landmarks; packed-row layout; an FP8 model with power-of-two row scales
equals its bf16 twin bit for bit (decode step and prefill), and misapplied scales break the equality.
MXFP4 weights: E2M1 decoder vs the element table of the OCP MX specification, E8M0 decoder vs torch's
float8_e8m0fnu for all 256 codes, packed-row layout byte by byte, and an MXFP4 model equal to its
bf16 twin bit for bit (swapped nibbles, shifted or dropped block scales break the equality).

Parity unpinned: nothing the pages print can be recomputed here (the pages give no model
dimensions and no worked example), so no whole-step value is pinned to the pages themselves.
"""

from .bf16 import bf16_to_f32, f32_to_bf16, f64_to_bf16  # noqa: F401
from .decode import (  # noqa: F401
    Dims,
    DenseWeights,
    PagedKV,
    StepResult,
    decode_step,
    greedy_decode,
    rmsnorm,
    rope,
    rope_cos_sin,
    decode_attention,
    gather_paged,
    route,
    expert_ffn,
    silu,
)
from . import mxfp4, prefill  # noqa: F401  (oracle.prefill.prefill, oracle.mxfp4.Mxfp4Rows)
