"""CPU oracle for one expert-parallel rank's MoE expert computation on the
expanded dispatch layout.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``expanded_dispatch_layout_amd``) and imports nothing from it.

It is a plain, slow, obviously-correct restatement of what the pages define:

* ``fp8``    OCP E4M3 (fn) codec and the round-up power-of-two (UE8M0) scale
             rule.
* ``quant``  per-group fp8 quantisation (1x128 activation groups, 128x128
             weight blocks) in fp32 and UE8M0 scale formats.
* ``layout`` capacity bound, expand-mode prefix sum, stable slot ranking,
             scatter of rows/scales/weights into aligned expert blocks and
             the row-to-expert labels.
* ``layer``  block-scaled grouped GEMM, SiLU*up with per-group quantisation
             (and the top-k weight fold), the weighted gather, the whole
             layer, the standard (non-EP) path (bf16 rows quantised per
             1x128 group, top-k weights and the routed scaling factor in the
             gather), and a per-token brute force that uses no layout at all.
* ``masked`` the decode path's fixed-height masked slab: the bridges from
             and back to the expanded layout and the layer on the slab.

Sources (cited by title and section in every function):

* SGLang pull request 37261, "feat(deepep_v2): expanded (do_expand=True)
  prefill dispatch for DeepEP-V2" (the method; its Modifications/Core list,
  the SGLANG_DEEPEP_V2_PREFILL_DO_EXPAND section and the review thread).
* vLLM pull request 54109, PaddedStandard activation format (Motivation,
  Design and Testing sections): the padded-input contract.
* SGLang source page ``moe_runner/deep_gemm.py`` (functions named where
  used): the stages around the layout.

Every function is pinned by tests under ``tests/`` that check it against
closed forms, library routines, invariants and brute force.  Parity
unpinned: none of the functions; the exact fp8 codes of the activation
quantisation at rounding ties after a different fp32 accumulation order are
bounded only by the output tolerance (see the layer tests).
"""

from . import fp8, quant, layout, layer, masked  # noqa: F401
