"""Seeded synthetic inputs for DCP decode attention.

This module generates inputs only: sequence lengths, block tables, queries,
canonical (unsharded, request-contiguous) keys and values in their stored
format, fp8 scales and attention sinks. It holds none of the method's
arithmetic (no slot mapping, no attention, no merge), so the CPU oracle and
the HIP path can both consume what it produces without sharing code.

The workloads stand in for the agentic long-context trace described in
"Efficient Decode Context Parallelism with vLLM for Long Context Workloads",
section 2.1 (median input ~67k tokens, bimodal: about half at 64k and above
with a tail to ~1M, ~18% under 8k, ~8% over 128k). None of that trace's items
are used; only its length statistics shape the mixtures below.
"""

from .configs import (KV_WRITE_WORKLOADS, SEGMENT_WORKLOADS, VERIFY_WORKLOADS, WORKLOADS,  # noqa: F401
                      KvWriteWorkload, SegmentWorkload, VerifyWorkload, Workload, get_kv_write_workload,
                      get_segment_workload, get_verify_workload, get_workload)
from .generate import (Case, KvWriteCase, Segment, make_case, make_kv_write_case, make_segment,  # noqa: F401
                       make_verify_queries)
