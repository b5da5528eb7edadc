"""Plain CPU oracle for the quantized-KV decode-attention path.

TEST INFRASTRUCTURE ONLY.  This package is a slow, direct restatement of what the path
computes, used to check the HIP library.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library never does, and the oracle
shares no code, tables or constants with it.  Inputs come from ``workloads/`` (seeded
generators only, no method arithmetic).

Modules:
  formats    binary16 / E4M3FN / E2M1 / bfloat16 encoders and decoders from their definitions
  quantize   group statistics, outlier predicate, INT4 / FP4 / 2-bit-centroid / FP8-row fits,
             packing and dequantization of single rows
  cache      one (sequence, KV head, K-or-V) list: rows in token order + sorted COO outliers
  attention  float64 decode attention with GQA, chunk states and the log-sum-exp merge
  kvbytes    KV-cache byte counts (the pages' size formula and its quantized analogue)

Every function is pinned by the CPU tests under ``tests/test_oracle_*.py``.
"""
