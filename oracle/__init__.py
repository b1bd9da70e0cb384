"""CPU oracle for the speculative-decoding verification step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link or
run anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, tables or helpers with
the HIP library; the two meet only at the seeded inputs.

What it computes, in fp64 unless stated, straight from the definitions:
  * attention of the 1 + D verified positions over a paged KV cache, with a full
    (not online) softmax per query row                    -- attention.py
  * the online-softmax and split-merge formulation of the same result, written
    from the running-max / running-sum update on the pages, used only to pin
    the identity "online softmax equals full softmax"     -- attention.py
  * greedy acceptance: per-row vocab argmax (fp32 compares, lowest index on
    ties), keep drafts up to the first mismatch, commit the KV length -- accept.py
  * storage decoders for bf16 and OCP e4m3                -- formats.py
  * the pages' closed forms (expected tokens per verification, KV-cache size,
    score-table size, decode arithmetic intensity)        -- closed_forms.py

Parity status: every function here is pinned by a test in tests/test_oracle_*.py
against something other than itself (printed values, closed forms, brute force,
library routines, invariants); none is "parity unpinned".
"""
from .formats import bf16_bits_to_f64, e4m3_bits_to_f64
from .attention import (gather_kv, oracle_attn, oracle_attn_online, merge_partial_states,
                        online_softmax_rows)
from .accept import oracle_argmax, oracle_accept
from . import closed_forms
