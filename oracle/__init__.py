"""CPU oracle for the fused MoE expert-FFN forward (test infrastructure).

This package is the slow, plainly written fp64 reference that the HIP path is
checked against.  It is test infrastructure, not product code: only the test
suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it.  It shares no code with the HIP library (no kernels, headers,
helpers, tables or constants) and never imports the library's package.

Modules
-------
codecs   e4m3 (OCP E4M3FN), e8m0 and bfloat16 encode/decode, written from the
         format definitions.
align    the planner's output written as its plain definition (a stable
         grouping of route ids by expert, padded to ``block_m``).
moe      the expert FFN step by step in fp64: dequantize, gate/up GEMM,
         SwiGLU, requantize, down GEMM, top-k weighted sum.
router   the gate's routing from router logits: softmax over the experts,
         the top-k largest (ties to the lower id), renormalized weights.

Every function cites the page and passage of the source pages it follows.
The sources are five web pages on fused MoE kernels:
  [hpc-ops RFC]   "[RFC] Fused W8A8 MoE megakernel on H20" (Tencent/hpc-ops #94)
  [prime-flash]   "Prime Flash MoE: Fused MoE Kernels for Blackwell"
  [DeepGEMM #411] "SM90 FP8 x MXFP4 MegaMoE" (DeepGEMM PR #411 mirror)
  [DeepGEMM #88]  "[SM90] Ring-buffered FP8 MegaMoE with a lag-ordered L1/L2
                  schedule" (sgl-project/DeepGEMM PR #88)

Parity status: every function here is pinned by tests under ``tests/`` marked
``not gpu`` (exhaustive codec checks against the format definitions and an
independent torch cast, brute-force alignment, per-token brute-force FFN loops,
a dense-FFN special case, linearity, permutation and empty-expert invariants,
and hand-derived golden fixtures).
"""

from . import codecs, align, moe  # noqa: F401
