"""CPU reference implementations of exact attention (TEST INFRASTRUCTURE ONLY).

Plain, slow, fp64 code written from the pages' definitions, used to check the
HIP library. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import it; the library and its Python binding never do, and share no
code with it.

Modules:
  attention      - the materialised definition (S, P in fp64), forward and backward
  softmax_forms  - three-pass, online-normalizer and one-pass softmax recurrences
  brute          - pure-Python loops for tiny inputs (pins the NumPy version)
  decode         - decoding: the newest Nq queries over Nk cached keys (bottom-right causal)
"""
from .attention import (allowed, attention, attention_dq_rows, attention_head,
                        attention_rows, softmax_rows)

__all__ = ["allowed", "attention", "attention_dq_rows", "attention_head", "attention_rows",
           "softmax_rows"]
