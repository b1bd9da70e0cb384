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


# ---------------------------------------------------------------------------
# Stochastic (lossless) acceptance.
#
# The pages state the property: the acceptance rule keeps the output
# distribution the same as the large model's alone ("GPU and LLM" ch. 5,
# section "Speculative decoding (2): verify in one pass"), and they cite the
# rule's source (Leviathan et al., ICML 2023, in "Speculative decoding (1)").
# The rule restated from that paper: the draft token d_j, drawn from the draft
# distribution q_j, is kept with probability min(1, p_j(d_j) / q_j(d_j)); at
# the first draft not kept, the emitted token is drawn from the residual
# max(0, p_j - q_j), renormalised; when every draft is kept, one more token is
# drawn from p_D.
#
# Readings (the pages give no interface):
#   * p_j = softmax(target_logits[b][j] / tau), q_j = softmax(draft_logits[b][j]
#     / tau), one temperature tau > 0 for both;
#   * "kept with probability min(1, p/q)" is the test u_j * q_j(d_j) < p_j(d_j)
#     with a uniform u_j in [0, 1) passed in (q_j(d_j) = 0: kept iff p_j(d_j) > 0);
#   * drawing from a distribution w uses one uniform u in [0, 1): the first
#     index whose running sum of w exceeds u * sum(w);
#   * a residual that is zero everywhere (p_j == q_j) is replaced by p_j;
#   * row alignment, AL, out_tokens and the KV commit as in greedy acceptance.
# ---------------------------------------------------------------------------
def _softmax64(z, tau):
    x = np.asarray(z, dtype=np.float64) / float(tau)
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def oracle_draw(w, u):
    """First index whose running sum of w exceeds u * sum(w) (w >= 0, sum > 0)."""
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    i = int(np.searchsorted(c, float(u) * c[-1], side="right"))
    if i >= len(c):                      # u * sum rounded onto the total: last nonzero entry
        i = int(np.flatnonzero(np.asarray(w) > 0)[-1])
    return i


def keep_draft(u, p_d, q_d):
    """The draft is kept with probability min(1, p_d / q_d): u * q_d < p_d."""
    return float(u) * q_d < p_d


def residual(p_j, q_j):
    """max(0, p_j - q_j) (unnormalised), or p_j itself where that is zero everywhere."""
    r = np.maximum(p_j - q_j, 0.0)
    return r if r.sum() > 0 else p_j


def oracle_accept_sampled(target_logits, draft_logits, draft, u_accept, u_sample, tau,
                          kv_lens_in, D):
    """Returns dict(accept_len [B], out_tokens [B][R], kv_lens_out [B])."""
    z = np.asarray(target_logits, dtype=np.float32)
    B, R, V = z.shape
    assert R == D + 1
    y = np.asarray(draft_logits, dtype=np.float32).reshape(B, D, V)
    draft = np.asarray(draft, dtype=np.int64).reshape(B, D)
    u_accept = np.asarray(u_accept, dtype=np.float32).reshape(B, D)
    u_sample = np.asarray(u_sample, dtype=np.float32).reshape(B)
    accept_len = np.empty(B, dtype=np.int32)
    out_tokens = np.full((B, R), -1, dtype=np.int32)
    kv_out = np.empty(B, dtype=np.int32)
    for b in range(B):
        p = _softmax64(z[b], tau)
        q = _softmax64(y[b], tau) if D else np.zeros((0, V))
        n, dist = D, p[D]
        for j in range(D):
            d = draft[b, j]
            if keep_draft(u_accept[b, j], p[j, d], q[j, d]):
                continue
            n, dist = j, residual(p[j], q[j])
            break
        accept_len[b] = n + 1
        out_tokens[b, :n] = draft[b, :n]
        out_tokens[b, n] = oracle_draw(dist, u_sample[b])
        kv_out[b] = int(kv_lens_in[b]) - R + n + 1
    return dict(accept_len=accept_len, out_tokens=out_tokens, kv_lens_out=kv_out)
