"""Draft-side signals and the choice of the next draft length (oracle; TEST
INFRASTRUCTURE ONLY -- only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it).

What the pages give:
  * SpecKV summary (arXiv 2605.02888), section "Technical core": two signals
    read from the draft model's output distribution -- confidence (the largest
    next-token probability) and entropy (the spread of the distribution) --
    predict the acceptance rate; a controller picks the speculation length
    gamma that maximises the expected number of tokens per step.
  * "GPU and LLM" ch. 5, section "Speculative decoding (2)": with each draft
    accepted with probability alpha, a verification of k drafts yields
    (1 - alpha^(k+1)) / (1 - alpha) tokens on average.
  * NVIDIA co-design summary, guideline 4: drafting costs rho * D relative to
    one target pass (rho = draft layers / target layers); guideline 3: above
    D = 128/G - 1, pick D with G (1 + D) a multiple of the 128-row tile.

Readings (SpecKV's trained MLP and its gamma x rate objective are not used):
  S1  p = softmax(z / tau) over the row; confidence c = max_v p_v; entropy
      H = -sum_v p_v ln p_v (nats, 0 ln 0 = 0).
  S2  The acceptance estimate is alpha = c (the draft's own probability of its
      most likely token).
  S3  The next draft length maximises tokens per unit time
          f(D) = E(alpha, D) / (1 + rho D),  E(alpha, D) = sum_{i=0..D} alpha^i
      over the candidates D in [0, D_max]; with a group size G > 0 the
      candidates above 128/G - 1 are only those with G (1 + D) a multiple of
      128.  Ties go to the smaller D.
  S4  Evaluation order (fixed so that the kernel can reproduce the decision
      bit for bit from the same confidence): in fp64, a = min(c, 1);
      P_0 = 1 and P_{D+1} = P_D * a; E = D + 1 if a == 1 else (1 - P_{D+1}) / (1 - a);
      cost = 1 + rho * D (product rounded, then the sum); f = E / cost; a
      candidate replaces the best only if its f is strictly larger.
"""
from __future__ import annotations

import numpy as np

TILE_ROWS = 128


def oracle_signals(logits, tau: float = 1.0):
    """(confidence [rows], entropy [rows]) in fp64 for fp32 logits [rows][V]
    (finite or -inf, at least one finite value per row)."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64) / float(tau)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    S = e.sum(axis=-1)
    p = e / S[:, None]
    conf = p.max(axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(p), 0.0)
    return conf, -plogp.sum(axis=-1)


def candidate_lengths(max_draft_len: int, G: int):
    """Reading S3: all of 0..D_max, or with G > 0 those up to 128/G - 1 and the
    longer ones that fill whole 128-row tiles."""
    out = []
    for D in range(max_draft_len + 1):
        if G > 0 and G * (D + 1) > TILE_ROWS and (G * (D + 1)) % TILE_ROWS != 0:
            continue
        out.append(D)
    return out


def choose_draft_len(confidence: float, max_draft_len: int, rho: float, G: int) -> int:
    """Reading S4, step by step in fp64 (numpy scalars: IEEE operations)."""
    a = np.float64(min(float(confidence), 1.0))
    rho = np.float64(np.float32(rho))
    cands = set(candidate_lengths(max_draft_len, G))
    best_D, best_f = -1, np.float64(-1.0)
    P = np.float64(1.0)
    for D in range(max_draft_len + 1):
        P = P * a                                   # a^(D+1)
        if D not in cands:
            continue
        E = np.float64(D + 1) if a == 1.0 else (np.float64(1.0) - P) / (np.float64(1.0) - a)
        cost = np.float64(1.0) + rho * np.float64(D)
        f = E / cost
        if f > best_f:
            best_D, best_f = D, f
    return best_D


def oracle_draft_signals(logits, tau: float, max_draft_len: int, rho: float, G: int):
    """Returns dict(confidence, entropy, next_draft_len) per row."""
    conf, ent = oracle_signals(logits, tau)
    nd = np.array([choose_draft_len(c, max_draft_len, rho, G) for c in conf], dtype=np.int32)
    return dict(confidence=conf, entropy=ent, next_draft_len=nd)
