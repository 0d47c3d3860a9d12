"""CPU oracle for Decode Context Parallel (DCP) decode attention.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The product path (``sequence_sharded_paged_amd``) never imports, calls or links
anything here, and this package imports nothing from the product path: the two
share no code.

What it computes, each function citing the passage it follows:

* ``formats``   - exact decoding of the stored KV formats (fp32, bf16, OCP
                  fp8 e4m3fn) into float64.
* ``layout``    - brute-force slot mapper: the four per-token layout formulas of
                  "Decode Context Parallel (DCP)" (vLLM Ascend design doc),
                  section "KV-cache layout", evaluated literally, plus a running
                  per-rank counter; local sequence lengths are the counters'
                  final values.
* ``cache``     - the KV-cache write: new rows stored (fp32 as is, bf16 and fp8
                  e4m3 by nearest-value rounding, fp8 through the per-head
                  scale) at the slots the slot mapping gives, non-owners
                  skipped ("Decode Context Parallel (DCP)", section "KV-cache
                  layout"; "DeepSeek V4.1 context parallelism", section
                  "Cache ownership").
* ``gather``    - the context gather of (chunked) prefill: every cached
                  position's stored row copied from its owner back into
                  request-contiguous order ("Decode Context Parallel (DCP)",
                  section "Prefill and chunked prefill").
* ``attention`` - plain full-softmax decode attention over the *unsharded*
                  sequence in float64, the per-rank partial (O, LSE) over the
                  tokens a rank owns, the log-sum-exp merge with an attention
                  sink applied once, multi-token decode (causal among the last
                  q_len tokens) and a replicated segment counted by one rank
                  ("DeepSeek V4.1 context parallelism", section "Decode
                  computation").

Every function here is pinned by ``-m "not gpu"`` tests against something other
than itself (hand-derived worked example, closed forms, invariants, torch's
float64 scaled-dot-product attention, torch's float8 decoding, brute force,
the E4M3 code table's own values).
No function is "parity unpinned".
"""

from . import formats, layout, attention, cache, gather  # noqa: F401
