"""CPU oracle for single-token decode attention -- TEST INFRASTRUCTURE ONLY.

Plain float64 numpy definitions of what the decode-attention path computes,
used to check the HIP library. Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package; the library itself
never calls it and shares no code, constants or helpers with it.

Modules:
  attention -- GQA/MQA/MHA decode, absorbed MLA decode, explicit (up-projected)
               MLA decode, split-KV log-sum-exp combine.
  sizes     -- closed-form KV-cache sizes, FLOPs and arithmetic intensity.
"""
from .attention import (  # noqa: F401
    gqa_decode_ref, mla_absorbed_ref, mla_explicit_ref, combine_ref, absorb_query_ref,
)
from . import sizes  # noqa: F401
