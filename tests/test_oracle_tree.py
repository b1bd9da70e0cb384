"""Pins for draft-tree verification in the oracle (oracle/tree.py and the tree
visibility of oracle/attention.py).

  * a chain tree reproduces chain verification exactly: attention equals
    oracle_attn without a tree, acceptance equals oracle_accept (both pinned
    elsewhere to the pages and to library routines);
  * tree attention equals torch's fp64 scaled-dot-product attention with a mask
    built element by element from the parent links, and a pure-Python loop on
    tiny inputs; a star tree's node sees exactly the context, the root and itself;
  * tree acceptance against brute force over every small tree and token
    assignment (V = 2, R <= 5): with distinct sibling tokens the accepted path
    ends at the deepest node whose whole root path agrees with the target;
    with equal sibling tokens the lowest-indexed child is taken;
  * the generator's ancestor masks against the oracle's.
"""
import itertools

import numpy as np
import pytest
import torch

from oracle.accept import oracle_accept, oracle_argmax
from oracle.attention import oracle_attn
from oracle.formats import bf16_bits_to_f64
from oracle.attention import gather_kv
from oracle.tree import ancestor_masks, oracle_accept_tree
from workloads import MINI, make_attn_inputs, make_tree_plan, tree_tokens_from_target


def _attn(inp, parents=None, seqs=None):
    w = inp.w
    return oracle_attn(inp.q, inp.k_cache, inp.v_cache, inp.k_scale, inp.v_scale, inp.block_table,
                       inp.kv_lens, D=w.D, H_kv=w.H_kv, sm_scale=w.sm_scale, parents=parents,
                       seqs=seqs)


@pytest.mark.parametrize("name", ["mini_gqa8_d15", "mini_fp8_hd64"])
def test_chain_tree_is_chain_attention(name):
    inp = make_attn_inputs(MINI[name])
    plan = make_tree_plan(inp.w, shape="chain")
    np.testing.assert_array_equal(_attn(inp, plan.parents), _attn(inp))


def _mask_from_parents(parents_b, L, R):
    """Visibility written out per element: t is visible to node i when t is a
    context key, or t - P is i, or t - P is reached from i by parent links."""
    P = L - R
    vis = np.zeros((R, L), dtype=bool)
    for i in range(R):
        for t in range(L):
            if t < P:
                vis[i, t] = True
                continue
            j, seen = i, False
            while j != -1:
                if j == t - P:
                    seen = True
                j = int(parents_b[j])
            vis[i, t] = seen
    return vis


def test_tree_attention_matches_torch_sdpa():
    w = MINI["mini_gqa8_d15"]
    inp = make_attn_inputs(w)
    plan = make_tree_plan(w, shape="random")
    got = _attn(inp, plan.parents)
    G = w.H_q // w.H_kv
    for b in range(w.B):
        L = int(inp.kv_lens[b])
        K, V = gather_kv(inp.k_cache, inp.v_cache, None, None, inp.block_table, b, L)
        Q = bf16_bits_to_f64(inp.q[b])
        vis = torch.from_numpy(_mask_from_parents(plan.parents[b], L, w.R))
        for h in range(w.H_q):
            kvh = h // G
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(Q[:, h, :])[None], torch.from_numpy(K[:, kvh, :])[None],
                torch.from_numpy(V[:, kvh, :])[None], attn_mask=vis[None], scale=w.sm_scale)[0]
            np.testing.assert_allclose(got[b, :, h, :], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_star_tree_sees_context_root_and_itself_tiny_loops():
    w = MINI["mini_hd64_g4"].replace(B=1, T_range=(5, 5))
    inp = make_attn_inputs(w)
    plan = make_tree_plan(w, shape="star")
    got = _attn(inp, plan.parents)
    L = int(inp.kv_lens[0])
    P = L - w.R
    K, V = gather_kv(inp.k_cache, inp.v_cache, None, None, inp.block_table, 0, L)
    Q = bf16_bits_to_f64(inp.q[0])
    G = w.H_q // w.H_kv
    for i in range(w.R):
        keys = list(range(P)) + [P] + ([P + i] if i > 0 else [])
        for h in range(w.H_q):
            s = [w.sm_scale * sum(Q[i, h, d] * K[t, h // G, d] for d in range(w.hd)) for t in keys]
            m = max(s)
            e = [np.exp(x - m) for x in s]
            want = [sum(e[k] * V[t, h // G, d] for k, t in enumerate(keys)) / sum(e)
                    for d in range(w.hd)]
            np.testing.assert_allclose(got[0, i, h], want, rtol=1e-11, atol=1e-13)


def test_generator_masks_match_oracle_ancestors():
    for shape in ("random", "chain", "star"):
        plan = make_tree_plan(MINI["mini_gqa8_d15"], shape=shape)
        np.testing.assert_array_equal(plan.masks, ancestor_masks(plan.parents))
    plan = make_tree_plan(MINI["mini_gqa8_d15"], shape="chain")
    assert [int(x) for x in plan.masks[0]] == [(1 << (i + 1)) - 1 for i in range(16)]


def test_chain_tree_acceptance_is_chain_acceptance():
    w = MINI["mini_gqa8_d15"]
    rng = np.random.default_rng(0)
    logits = rng.standard_normal((w.B, w.R, 40)).astype(np.float32)
    target = oracle_argmax(logits)
    plan = make_tree_plan(w.replace(V=40), shape="chain", p_match=0.8)
    tok = tree_tokens_from_target(plan, target)
    kv = np.full(w.B, 100, np.int32)
    t = oracle_accept_tree(logits, tok, plan.parents, kv)
    c = oracle_accept(logits, tok[:, 1:], kv, w.D)
    for k in ("target", "accept_len", "out_tokens", "kv_lens_out"):
        np.testing.assert_array_equal(t[k], c[k])
    for b in range(w.B):
        np.testing.assert_array_equal(t["accept_path"][b, : t["accept_len"][b]],
                                      np.arange(t["accept_len"][b]))


def _all_trees(R):
    for ps in itertools.product(*[range(j) for j in range(1, R)]):
        yield np.array((-1,) + ps, dtype=np.int64)


def test_tree_acceptance_brute_force_small():
    V = 2
    for R in range(1, 5):
        for parents in _all_trees(R):
            for targets in itertools.product(range(V), repeat=R):
                logits = np.full((1, R, V), -1.0, np.float32)
                for i, a in enumerate(targets):
                    logits[0, i, a] = 1.0
                for toks in itertools.product(range(V), repeat=R - 1):
                    tok = np.array([[0, *toks]], np.int64)
                    r = oracle_accept_tree(logits, tok, parents[None], np.array([50]))
                    path = list(r["accept_path"][0, : r["accept_len"][0]])
                    # every step follows a parent link and agrees with the target
                    assert path[0] == 0
                    for u, v in zip(path, path[1:]):
                        assert parents[v] == u and tok[0, v] == targets[u]
                    # the last node has no agreeing child; lower agreeing siblings never skipped
                    last = path[-1]
                    assert not any(parents[c] == last and tok[0, c] == targets[last]
                                   for c in range(R))
                    for u, v in zip(path, path[1:]):
                        assert not any(parents[c] == u and tok[0, c] == targets[u]
                                       for c in range(1, v))
                    # distinct sibling tokens: the deepest fully agreeing node ends the path
                    sib_ok = all(len({tok[0, c] for c in range(1, R) if parents[c] == p}) ==
                                 sum(1 for c in range(1, R) if parents[c] == p) for p in range(R))
                    if sib_ok:
                        good = [i for i in range(R) if all(
                            tok[0, n] == targets[parents[n]] for n in _root_path(parents, i)[1:])]
                        deepest = max(good, key=lambda i: len(_root_path(parents, i)))
                        assert last == deepest
                    assert r["kv_lens_out"][0] == 50 - R + len(path)
                    assert list(r["out_tokens"][0, : len(path)]) == \
                        [int(tok[0, v]) for v in path[1:]] + [targets[last]]
                    assert (r["out_tokens"][0, len(path):] == -1).all()


def _root_path(parents, i):
    p = []
    while i != -1:
        p.append(i)
        i = int(parents[i])
    return p[::-1]
