"""CPU oracle of the KDA mixer: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library.
"""
from .ref import (OracleCfg, bf16, commit, decode_case, load, prefill_case,
                  round_bf16, run_heads, run_heads_chunked, verify_case)

__all__ = ["OracleCfg", "bf16", "commit", "decode_case", "load",
           "prefill_case", "round_bf16", "run_heads", "run_heads_chunked",
           "verify_case"]
