"""Verification attention, oracle form (test infrastructure; fp64).

What is computed (for each sequence b, KV head kvh, query head h in kvh's group,
verified position i in 0..D):

    P_b      = L_b - (1 + D)             context length before this step
    s_t      = sm_scale * <q[b,i,h,:], K[b,t,kvh,:]>      for t = 0 .. P_b + i
    out[b,i,h,:] = sum_t softmax(s)_t * V[b,t,kvh,:]

Sources on the pages:
  * One target forward over the D drafted positions plus the bonus position,
    shaped like a prefill: "GPU and LLM", chapter 5 (animemo.app), section
    "Speculative decoding (2): verify in one pass"; the NVIDIA co-design summary
    (papanda925.com), section "Basic structure of speculative decoding".
  * Query heads share KV heads in contiguous groups of G (the GQA figure groups
    adjacent query heads four at a time): "GPU and LLM" ch. 5, section "GQA".
  * Fixed 16-token KV blocks located through a per-sequence block table:
    "GPU and LLM" ch. 5, section "PagedAttention (2)".
  * Per-row running max m and running exponent sum l, rescaled by exp(m - m_new)
    when the max grows, and a final division by l that gives exactly the full
    softmax: "GPU and LLM" ch. 5, section "Online softmax: carry the max and the
    sum".  ``oracle_attn`` uses the full softmax (the plain definition);
    ``oracle_attn_online`` follows the update rule tile by tile and merges
    independent key ranges with the same rule applied to whole states.

Readings where the pages are silent (each is listed in the design notes):
  * the cache already holds the 1 + D new positions, so L_b includes them;
  * position i sees keys 0 .. P_b + i (causal among the new positions);
  * query head h uses KV head h // G;
  * sm_scale = 1/sqrt(hd); K and V of an e4m3 cache are code * scale[block][kvh].

The storage layouts read here are the ones the C header documents:
  q        [B][R][H_q][hd] bf16 bits
  k_cache  [num_blocks][H_kv][hd/X][16][X]   (X = 8 for bf16, 16 for e4m3)
  v_cache  [num_blocks][H_kv][hd][16]
  k_scale, v_scale  [num_blocks][H_kv] fp32 (e4m3 only)
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, e4m3_bits_to_f64

BLOCK = 16


def _decode(codes: np.ndarray) -> np.ndarray:
    if codes.dtype == np.uint16:
        return bf16_bits_to_f64(codes)
    if codes.dtype == np.uint8:
        return e4m3_bits_to_f64(codes)
    raise TypeError(f"unsupported cache element type {codes.dtype}")


def gather_kv(k_cache, v_cache, k_scale, v_scale, block_table, b, L, kv_heads=None):
    """Logical K and V of sequence ``b`` for tokens 0..L-1, as fp64 [L][H_kv][hd].

    Token t lives in physical block block_table[b][t // 16], slot t % 16.  With
    ``kv_heads`` only those KV heads are decoded (the others are NaN).
    """
    nb = -(-int(L) // BLOCK)
    blocks = np.asarray(block_table[b, :nb], dtype=np.int64)
    if nb and (blocks < 0).any():
        raise ValueError("block table entry < 0 inside the sequence")
    H_kv = k_cache.shape[1]
    heads = np.arange(H_kv) if kv_heads is None else np.asarray(list(kv_heads), dtype=np.int64)
    kb = k_cache[blocks][:, heads]                    # [nb][h][hd/X][16][X]
    _, nh, nx, bs, X = kb.shape
    k_tok = kb.transpose(0, 3, 1, 2, 4).reshape(nb * BLOCK, nh, nx * X)
    vb = v_cache[blocks][:, heads]                    # [nb][h][hd][16]
    v_tok = vb.transpose(0, 3, 1, 2).reshape(nb * BLOCK, nh, vb.shape[2])
    Kh = _decode(k_tok[:L])
    Vh = _decode(v_tok[:L])
    if k_cache.dtype == np.uint8:
        sel = np.ix_(blocks, heads)
        ks = np.repeat(np.asarray(k_scale, np.float64)[sel], BLOCK, axis=0)[:L]  # [L][h]
        vs = np.repeat(np.asarray(v_scale, np.float64)[sel], BLOCK, axis=0)[:L]
        Kh = Kh * ks[:, :, None]
        Vh = Vh * vs[:, :, None]
    if kv_heads is None:
        return Kh, Vh
    K = np.full((int(L), H_kv, nx * X), np.nan)
    V = np.full((int(L), H_kv, vb.shape[2]), np.nan)
    K[:, heads] = Kh
    V[:, heads] = Vh
    return K, V


def _visible(R: int, L: int) -> np.ndarray:
    """visible[i, t]: position i (0..R-1) may attend key t (0..L-1)."""
    P = L - R
    return np.arange(L)[None, :] <= (P + np.arange(R))[:, None]


def _visible_tree(parents, L: int) -> np.ndarray:
    """visible[i, t] for draft-tree verification: new position j holds tree node
    j (parent[j] < j, parent[0] = -1); node i sees every context key t < L - R
    and the new keys of itself and its ancestors, found by walking parents."""
    R = len(parents)
    P = L - R
    vis = np.zeros((R, L), dtype=bool)
    vis[:, :P] = True
    for i in range(R):
        j = i
        while j >= 0:
            vis[i, P + j] = True
            j = int(parents[j])
    return vis


def oracle_attn(q, k_cache, v_cache, k_scale, v_scale, block_table, kv_lens, *,
                D, H_kv, sm_scale, seqs=None, kv_heads=None, parents=None):
    """Full-softmax attention of the R = D + 1 verified positions.

    With ``parents`` ([B][R] int, a draft tree per sequence) the new positions
    are tree nodes and each sees its ancestors instead of every earlier
    position (``_visible_tree``).  Returns fp64 [B][R][H_q][hd]; rows outside
    ``seqs`` x ``kv_heads`` (when given) are NaN.
    """
    B, R, H_q, hd = q.shape
    assert R == D + 1 and H_q % H_kv == 0
    G = H_q // H_kv
    out = np.full((B, R, H_q, hd), np.nan)
    seqs = range(B) if seqs is None else seqs
    for b in seqs:
        L = int(kv_lens[b])
        if L < R:
            raise ValueError("kv_lens[b] must include the R new positions")
        K, V = gather_kv(k_cache, v_cache, k_scale, v_scale, block_table, b, L,
                         None if kv_heads is None else list(kv_heads))
        Q = bf16_bits_to_f64(q[b])                     # [R][H_q][hd]
        vis = _visible(R, L) if parents is None else _visible_tree(parents[b], L)
        for kvh in (range(H_kv) if kv_heads is None else kv_heads):
            for g in range(G):
                h = kvh * G + g
                s = sm_scale * (Q[:, h, :] @ K[:, kvh, :].T)      # [R][L]
                s = np.where(vis, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                w = np.exp(s - m)
                out[b, :, h, :] = (w @ V[:, kvh, :]) / w.sum(axis=1, keepdims=True)
    return out


def online_softmax_rows(s: np.ndarray, v: np.ndarray, tile: int):
    """Running (O, m, l) over the key axis of ``s`` [n][L] in tiles of ``tile`` keys.

    For every new tile of scores s:
        m_new = max(m, max s);  l = l*exp(m - m_new) + sum exp(s - m_new)
        O = O*exp(m - m_new) + sum exp(s - m_new) * v;  m = m_new
    Masked scores are -inf.  While a row has seen no visible key its state stays
    (O = 0, m = -inf, l = 0).  Returns the unnormalised state (O, m, l).
    """
    n, L = s.shape
    O = np.zeros((n, v.shape[1]))
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    for t0 in range(0, L, tile):
        st = s[:, t0:t0 + tile]
        if st.shape[1] == 0:
            continue
        m_new = np.maximum(m, st.max(axis=1))
        live = np.isfinite(m_new)
        # a row whose max was -inf has O = 0 and l = 0, so its rescale factor is moot
        m_safe = np.where(np.isfinite(m), m, 0.0)
        m_new_safe = np.where(live, m_new, 0.0)
        alpha = np.where(live & np.isfinite(m), np.exp(m_safe - m_new_safe), 1.0)
        p = np.where(live[:, None], np.exp(st - np.where(live, m_new, 0.0)[:, None]), 0.0)
        l = l * alpha + p.sum(axis=1)
        O = O * alpha[:, None] + p @ v[t0:t0 + tile]
        m = m_new
    return O, m, l


def merge_partial_states(states):
    """Merge (O_s, m_s, l_s) of disjoint key ranges with the same rescaling rule:
    m = max_s m_s, l = sum_s l_s exp(m_s - m), O = sum_s O_s exp(m_s - m)."""
    ms = np.stack([st[1] for st in states])            # [S][n]
    m = ms.max(axis=0)
    live = np.isfinite(m)
    ms_safe = np.where(np.isfinite(ms), ms, 0.0)
    w = np.exp(ms_safe - np.where(live, m, 0.0)[None, :])
    w = np.where(np.isfinite(ms) & live[None, :], w, 0.0)
    l = sum(wi * st[2] for wi, st in zip(w, states))
    O = sum(wi[:, None] * st[0] for wi, st in zip(w, states))
    return O, m, l


def oracle_attn_online(q, k_cache, v_cache, k_scale, v_scale, block_table, kv_lens, *,
                       D, H_kv, sm_scale, tile=64, split_tokens=None):
    """Same result as ``oracle_attn`` by the online-softmax route: keys split into
    ranges of ``split_tokens`` (all keys in one range when None), each range
    processed tile by tile, then the range states merged and divided by l."""
    B, R, H_q, hd = q.shape
    G = H_q // H_kv
    out = np.empty((B, R, H_q, hd))
    for b in range(B):
        L = int(kv_lens[b])
        K, V = gather_kv(k_cache, v_cache, k_scale, v_scale, block_table, b, L)
        Q = bf16_bits_to_f64(q[b])
        vis = _visible(R, L)
        step = L if not split_tokens else split_tokens
        for kvh in range(H_kv):
            for g in range(G):
                h = kvh * G + g
                s = sm_scale * (Q[:, h, :] @ K[:, kvh, :].T)
                s = np.where(vis, s, -np.inf)
                states = [online_softmax_rows(s[:, a:a + step], V[a:a + step, kvh, :], tile)
                          for a in range(0, L, step)]
                O, m, l = merge_partial_states(states)
                out[b, :, h, :] = O / l[:, None]
    return out
