"""Float64 CPU oracle for absorbed (latent) MLA decode over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``mla_latent_attention_amd``) and imports nothing from it.

Pages cited in this package (the passages are named by page title and section):

* [Issue] "[Kimi-K3 MLA TP8] MLA performance" (ROCm/aiter issue 4541).
  Sec. 2 "K3 MLA geometry", Sec. 3 "Entry point", Sec. 4.1/4.2 "Arguments",
  Sec. 5.1-5.5 "Notes for optimization".
* [Blog] "Kimi K3 on AMD Instinct MI355X: vLLM Serving Matches NVIDIA HGX B300
  Throughput per GPU on AgentX".  Sec. "1. Cache: keep conversation state
  available for reuse" and Sec. "4. MLA: faster long-context decoding with AMD
  AITER assembly".

Modules:

* ``codecs``  - exact decoders of float8_e4m3fn and bfloat16 codes to float64.
* ``mla``     - the plain definition: per request, gather the referenced latent
                rows, score every query row against all visible rows, softmax,
                weight the first 512 dims; plus the LSE merge of partial answers.
* ``brute``   - an independent scalar brute force (exact integer dot products,
                50-digit mpmath softmax, exact fixed-point weighted sums) used
                only to pin ``mla`` on tiny inputs.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(exhaustive codec checks against torch's casts, brute force, closed forms and
invariants).  The absolute values of o and lse at the benchmark shapes are not
printed anywhere on the pages, so those rest on the pinned definition.
"""

from . import codecs, mla  # noqa: F401

__all__ = ["codecs", "mla"]
