"""Test infrastructure: a plain fp64 CPU oracle for attention forward and
backward.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  The GPU library never imports, links or calls it.
"""
from .attention import (attention_bwd_ref, attention_bwd_ref_masked, attention_online_merge, attention_ref,
                        attention_ref_masked)

__all__ = ["attention_ref", "attention_ref_masked", "attention_online_merge", "attention_bwd_ref",
           "attention_bwd_ref_masked"]
