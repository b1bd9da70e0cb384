"""Pins for the acceptance oracle.

  * argmax: exhaustive enumeration of short vectors over a value set with ties,
    signed zeros and -inf, against a pure-Python "lowest index of the maximum";
  * prefix / commit: exhaustive enumeration of target and draft sequences on a
    tiny vocabulary (drafts include an out-of-range id) against first-principles
    counting;
  * the pages' worked example (three accepted, the fourth replaced);
  * invariants: AL in 1..1+D, committed length = context + AL, output layout;
  * statistics: with drafts that match with probability p independently, the
    mean AL converges to (1 - p^(D+1)) / (1 - p), the pages' closed form.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle.accept import oracle_accept, oracle_argmax
from oracle.closed_forms import expected_tokens
from workloads import (EDGE, MINI, TINY, LLAMA3_8B, Workload, drafts_from_target,
                       make_accept_plan)

NEG_INF = float("-inf")


def _lowest_index_of_max(row):
    best = max(row)
    for i, v in enumerate(row):
        if v == best:
            return i


@pytest.mark.parametrize("V", [1, 2, 3, 4])
def test_argmax_exhaustive_small(V):
    values = [NEG_INF, -1.5, -0.0, 0.0, 2.0]
    rows = list(itertools.product(values, repeat=V))
    x = np.array(rows, dtype=np.float32)
    got = oracle_argmax(x)
    want = [_lowest_index_of_max(r) for r in rows]
    assert got.tolist() == want


def test_argmax_signed_zero_and_all_neg_inf():
    x = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0], [NEG_INF] * 3,
                  [-3.0, NEG_INF, -3.0]], np.float32)
    assert oracle_argmax(x).tolist() == [0, 0, 0, 0]


def _brute_accept(target, draft, D):
    n = 0
    while n < D and draft[n] == target[n]:
        n += 1
    return n + 1, list(draft[:n]) + [target[n]] + [-1] * (D - n)


@pytest.mark.parametrize("D", [0, 1, 2, 3])
def test_prefix_exhaustive(D):
    V = 3
    R = D + 1
    targets = list(itertools.product(range(V), repeat=R))
    drafts = list(itertools.product(range(V + 1), repeat=D))   # id V never matches
    B = len(targets) * len(drafts)
    logits = np.full((B, R, V), -1.0, np.float32)
    tg = np.empty((B, R), np.int64)
    dr = np.empty((B, D), np.int64)
    for k, (t, d) in enumerate(itertools.product(targets, drafts)):
        tg[k], dr[k] = t, d
        logits[k, np.arange(R), list(t)] = 1.0
    kv_in = np.full(B, 100 + R, np.int32)
    res = oracle_accept(logits, dr, kv_in, D)
    assert (res["target"] == tg).all()
    for k in range(B):
        al, out = _brute_accept(tg[k], dr[k], D)
        assert res["accept_len"][k] == al
        assert res["out_tokens"][k].tolist() == out
        assert res["kv_lens_out"][k] == 100 + al


def test_worked_example_from_pages(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "worked_verification_example.json")))
    vocab = {w: i for i, w in enumerate(ex["vocab"])}
    D = len(ex["draft"])
    R = D + 1
    logits = np.zeros((1, R, len(vocab)), np.float32)
    for j, tok in enumerate(ex["target_argmax_first4"]):
        logits[0, j, vocab[tok]] = 5.0
    logits[0, D, vocab["kyou"]] = 5.0          # the bonus row is never reached here
    draft = np.array([[vocab[t] for t in ex["draft"]]])
    ctx = len(ex["context"])
    res = oracle_accept(logits, draft, np.array([ctx + R]), D)
    assert res["accept_len"][0] == ex["expected_accept_len"]
    got = [ex["vocab"][i] for i in res["out_tokens"][0] if i >= 0]
    assert got == ex["expected_out_tokens"]
    assert res["kv_lens_out"][0] == ctx + ex["expected_accept_len"]


@pytest.mark.parametrize("w", [TINY, MINI["mini_gqa4_d7"], MINI["mini_gqa8_d15"],
                               EDGE["edge_d63"], EDGE["edge_plain_decode"]],
                         ids=lambda w: w.name)
def test_invariants_on_generated_inputs(w):
    plan = make_accept_plan(w)
    target = oracle_argmax(plan.logits)
    draft = drafts_from_target(plan, target)
    kv_in = np.arange(w.B, dtype=np.int32) + 5 * w.R
    res = oracle_accept(plan.logits, draft, kv_in, w.D)
    AL = res["accept_len"]
    assert ((AL >= 1) & (AL <= w.R)).all()
    assert (res["kv_lens_out"] - (kv_in - w.R) == AL).all()
    for b in range(w.B):
        n = AL[b] - 1
        assert (res["out_tokens"][b, :n] == draft[b, :n]).all()
        assert res["out_tokens"][b, n] == target[b, n]
        assert (res["out_tokens"][b, n + 1:] == -1).all()
        # every rejection happened at a planned mismatch, every acceptance at a planned match
        assert plan.match[b, :n].all()
        if n < w.D:
            assert not plan.match[b, n]


@pytest.mark.parametrize("p,D", [(0.5, 4), (0.7, 4), (0.9, 4), (0.7, 3), (0.6, 7)])
def test_mean_accept_len_converges_to_closed_form(p, D):
    w = Workload(f"mc_{p}_{D}", 5000 + D, B=40000, H_q=1, H_kv=1, hd=8, D=D, T=0, V=16,
                 p_match=p)
    plan = make_accept_plan(w)
    target = oracle_argmax(plan.logits)
    res = oracle_accept(plan.logits, drafts_from_target(plan, target),
                        np.full(w.B, w.R, np.int32), D)
    AL = res["accept_len"].astype(np.float64)
    mu = expected_tokens(p, D)
    se = AL.std() / np.sqrt(w.B)
    assert abs(AL.mean() - mu) < 4 * se, (AL.mean(), mu, se)


def test_mean_accept_len_with_per_sequence_probability():
    # D = 15, p ~ U[0.3, 0.9] per sequence: E[AL] = mean over p of the closed form
    w = Workload("mc_range", 5100, B=40000, H_q=1, H_kv=1, hd=8, D=15, T=0, V=16,
                 p_range=(0.3, 0.9))
    plan = make_accept_plan(w)
    target = oracle_argmax(plan.logits)
    res = oracle_accept(plan.logits, drafts_from_target(plan, target),
                        np.full(w.B, w.R, np.int32), w.D)
    ps = np.linspace(0.3, 0.9, 200001)
    mu = np.trapezoid([expected_tokens(x, 15) for x in ps[::100]], ps[::100]) / 0.6
    AL = res["accept_len"].astype(np.float64)
    assert abs(AL.mean() - mu) < 4 * AL.std() / np.sqrt(w.B)
    assert abs(mu - 3.126) < 5e-4
