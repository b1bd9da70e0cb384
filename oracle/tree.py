"""Draft-tree verification (oracle; TEST INFRASTRUCTURE ONLY -- only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it).

The pages' drafter proposes several candidate tokens per position and the
target scores the grouped candidates in one pass (novita.ai blog,
"Revolutionizing LLM inference ...", section "Implementation": candidate
generation and batch verification).  They do not fix a tree layout; the
readings below are taken in both the oracle and the library.

  T1  A sequence's R = 1 + D new positions are the nodes of a draft tree in
      topological order: parent[0] = -1 (node 0 = the last committed token, the
      root), parent[j] < j for j >= 1; node j's K/V sit at new position j.
  T2  Attention: node i sees the context and the nodes on its root path (itself
      and its ancestors) -- oracle.attention._visible_tree; a chain tree
      (parent[j] = j - 1) is the causal rule of chain verification.
  T3  Greedy acceptance: a_i = argmax of logits row i (lowest index on ties, as
      in chain acceptance).  From the root, step to the lowest-indexed child c
      of the current node i with token[c] == a_i while one exists.  The path's
      nodes after the root are the accepted drafts; AL = path length (1 .. 1 +
      depth); out_tokens = the accepted drafts' tokens, then a_last, -1 padded;
      accept_path = the path's node indices, -1 padded.
  T4  The committed length counts the root and the accepted drafts,
      kv_len' = kv_len - R + AL, as in chain acceptance; the accepted nodes'
      K/V rows are accept_path[1..AL-1] of the new positions, which the caller
      moves to positions 1 .. AL - 1 (for a chain they are already there).
"""
from __future__ import annotations

import numpy as np

from .accept import oracle_argmax


def ancestor_masks(parents) -> np.ndarray:
    """[B][R] uint64: bit j of mask[b][i] set iff node j is node i or one of its
    ancestors (reading T2), by walking the parent links."""
    parents = np.asarray(parents, dtype=np.int64)
    B, R = parents.shape
    out = np.zeros((B, R), dtype=np.uint64)
    for b in range(B):
        for i in range(R):
            m, j = 0, i
            while j >= 0:
                m |= 1 << j
                j = int(parents[b, j])
            out[b, i] = np.uint64(m)
    return out


def oracle_accept_tree(logits, tokens, parents, kv_lens_in):
    """Reading T3/T4.  logits [B][R][V] fp32, tokens [B][R] (token of each node;
    tokens[b][0] is not used), parents [B][R].  Returns dict(target, accept_len,
    out_tokens, accept_path, kv_lens_out)."""
    logits = np.asarray(logits, dtype=np.float32)
    B, R, V = logits.shape
    tokens = np.asarray(tokens, dtype=np.int64)
    parents = np.asarray(parents, dtype=np.int64)
    target = oracle_argmax(logits)
    accept_len = np.empty(B, dtype=np.int32)
    out_tokens = np.full((B, R), -1, dtype=np.int32)
    accept_path = np.full((B, R), -1, dtype=np.int32)
    kv_out = np.empty(B, dtype=np.int32)
    for b in range(B):
        path = [0]
        while True:
            cur = path[-1]
            nxt = next((c for c in range(cur + 1, R)
                        if parents[b, c] == cur and tokens[b, c] == target[b, cur]), None)
            if nxt is None:
                break
            path.append(nxt)
        AL = len(path)
        accept_len[b] = AL
        accept_path[b, :AL] = path
        out_tokens[b, :AL - 1] = tokens[b, path[1:]]
        out_tokens[b, AL - 1] = target[b, path[-1]]
        kv_out[b] = int(kv_lens_in[b]) - R + AL
    return dict(target=target, accept_len=accept_len, out_tokens=out_tokens,
                accept_path=accept_path, kv_lens_out=kv_out)
