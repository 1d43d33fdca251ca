"""CPU oracle for the KronQ per-layer quantization engine (test infrastructure).

Plain, slow, fp64 numpy code that states what the engine computes, step by
step, so the GPU path can be checked against it.  It is test infrastructure:
only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import it.  It shares no code with the HIP library and imports nothing
from it.

Every function cites the passage it follows.  Sources are named by page title
and section:
  [KronQ-README]   "KronQ: LLM Quantization via a Kronecker-Factored Hessian",
                   repository README (GitLite mirror of the KronQ GitHub repo).
  [KronQ-abstract] "KronQ: LLM Quantization via Kronecker-Factored Hessian",
                   arXiv 2607.07964 abstract (fugumt.com mirror).
  [KronQ-news]     "KronQ makes 2-bit models work where the standard method
                   collapses" (groundtruth.day).
  [WaterKron]      "WaterKron and FlipFlop Hessian: Information-Theoretically
                   Grounded Quantization with Kronecker-factored Hessians"
                   (thelatestinai.com), Figure 1 and Table 1.

Readings where the pages are silent are marked READING and listed in the
repository's design notes.  One function carries no independent pin:
  * the BiIP rescale exponent rule (`rescale_vectors`): only the loss
    invariance and the proxy-bound optimality constrain it -- its alpha
    choice is "parity unpinned".
"""
from .kronq import *  # noqa: F401,F403
from .kronq import __all__  # noqa: F401
