"""Greedy acceptance, oracle form (test infrastructure).

Sources on the pages:
  * Draft length D and acceptance length AL; the target accepts drafts up to the
    first mismatch and always adds one token of its own, so AL lies in 1 .. 1+D:
    NVIDIA co-design summary (papanda925.com), section "Basic structure of
    speculative decoding" (definitions and the draft/verify/accept flowchart).
  * The worked example in which three drafts are accepted and the fourth is
    replaced by the target's own token: "GPU and LLM" ch. 5 (animemo.app),
    section "Speculative decoding (2): verify in one pass".
  * At temperature zero the target's token at a position is the argmax of its
    logits there; the acceptance rule that keeps the target's output
    distribution reduces to "accept iff draft == argmax" (same section).

Readings where the pages are silent:
  * row j of the logits (input position j, position 0 = the last committed
    token) checks draft j for j < D; row D gives the bonus token;
  * argmax ties go to the lowest vocabulary index; values are compared as fp32
    (so -0 and +0 tie); an all -inf row gives index 0;
  * committed KV length = L_b - (1 + D) + AL: the context, the last committed
    token and the accepted drafts (the bonus token's KV is written next step).
"""
from __future__ import annotations

import numpy as np


def oracle_argmax(logits: np.ndarray) -> np.ndarray:
    """Lowest index of the maximum along the last axis, comparing fp32 values.

    numpy's argmax returns the first occurrence of the maximum and compares with
    ordinary floating-point ordering (-0 == +0), which is the definition above.
    """
    x = np.asarray(logits, dtype=np.float32)
    return np.argmax(x, axis=-1).astype(np.int32)


def oracle_accept(logits, draft, kv_lens_in, D):
    """Returns dict(target [B][R], accept_len [B], out_tokens [B][R], kv_lens_out [B])."""
    logits = np.asarray(logits, dtype=np.float32)
    B, R, V = logits.shape
    assert R == D + 1
    draft = np.asarray(draft, dtype=np.int64).reshape(B, D)
    target = oracle_argmax(logits)                          # [B][R]
    accept_len = np.empty(B, dtype=np.int32)
    out_tokens = np.full((B, R), -1, dtype=np.int32)
    kv_out = np.empty(B, dtype=np.int32)
    for b in range(B):
        n = D
        for j in range(D):
            if draft[b, j] != target[b, j]:
                n = j
                break
        accept_len[b] = n + 1
        out_tokens[b, :n] = draft[b, :n]
        out_tokens[b, n] = target[b, n]
        kv_out[b] = int(kv_lens_in[b]) - R + n + 1
    return dict(target=target, accept_len=accept_len, out_tokens=out_tokens,
                kv_lens_out=kv_out)
