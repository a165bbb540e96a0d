"""Test infrastructure: a plain fp64 CPU oracle for attention forward.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  The GPU library never imports, links or calls it.
"""
from .attention import attention_ref, attention_online_merge

__all__ = ["attention_ref", "attention_online_merge"]
