"""GPU parity of spec_accept against the oracle: bit-exact target tokens,
acceptance lengths, output tokens and committed KV lengths."""
import numpy as np
import pytest

from oracle.accept import oracle_accept
from tests.gpu_util import note, run_accept
from workloads import (EDGE, FP8_LONG, LLAMA3_8B, LLAMA31_70B, MINI, TINY, Workload,
                       drafts_from_target, make_accept_plan)

pytestmark = pytest.mark.gpu

WITH_VOCAB = [w for w in [TINY, *MINI.values(), *EDGE.values()] if w.V > 0]


def compare(logits, draft, kv_in, inplace=False):
    D = logits.shape[1] - 1
    ref = oracle_accept(logits, draft, kv_in, D)
    got = run_accept(logits, draft, kv_in, inplace=inplace)
    for key in ("target", "accept_len", "out_tokens", "kv_lens_out"):
        assert np.array_equal(got[key], ref[key]), key
    return got


def plan_inputs(w):
    plan = make_accept_plan(w)
    from oracle.accept import oracle_argmax
    draft = drafts_from_target(plan, oracle_argmax(plan.logits))
    kv_in = (np.arange(w.B, dtype=np.int32) * 7 + 3 * w.R).astype(np.int32)
    return plan.logits, draft, kv_in


@pytest.mark.parametrize("w", WITH_VOCAB + [LLAMA3_8B, LLAMA31_70B, FP8_LONG],
                         ids=lambda w: w.name)
def test_accept_bit_exact(w):
    logits, draft, kv_in = plan_inputs(w)
    got = compare(logits, draft, kv_in)
    note(f"  {w.name}: sum AL = {int(got['accept_len'].sum())}")


def test_accept_in_place_commit():
    logits, draft, kv_in = plan_inputs(MINI["mini_gqa8_d15"])
    compare(logits, draft, kv_in, inplace=True)


def _tie_logits(B, R, V, rng):
    x = rng.standard_normal((B, R, V)).astype(np.float32)
    CH = 4096
    for b in range(B):
        for j in range(R):
            kind = (b * R + j) % 6
            row = x[b, j]
            if kind == 0:       # ties straddling a chunk boundary
                idx = [i for i in (CH - 1, CH, 2 * CH - 1) if i < V] or [V - 1]
                row[idx] = 9.0
            elif kind == 1:     # +0 / -0 tie as the maximum
                row[:] = -1.0
                pos = sorted(rng.choice(V, size=min(2, V), replace=False))
                row[pos[0]] = -0.0
                row[pos[-1]] = 0.0
            elif kind == 2:     # all -inf
                row[:] = -np.inf
            elif kind == 3:     # maximum in the very last element
                row[-1] = 50.0
            elif kind == 4:     # many equal maxima spread over the row
                row[rng.choice(V, size=min(17, V), replace=False)] = 7.5
            # kind 5: plain N(0, 1)
    return x


@pytest.mark.parametrize("V", [1, 3, 4, 5, 1023, 4095, 4096, 4097, 8191, 8192, 8193, 16387, 40000, 128256])
def test_argmax_ties_and_edges(V):
    rng = np.random.default_rng(V)
    B, D = 3, 5
    logits = _tie_logits(B, D + 1, V, rng)
    draft = rng.integers(-2, V + 2, size=(B, D)).astype(np.int32)
    kv_in = np.full(B, 100, np.int32)
    compare(logits, draft, kv_in)


def test_drafts_equal_to_target_are_all_accepted():
    w = Workload("all_match", 6001, B=8, H_q=1, H_kv=1, hd=64, D=31, T=0, V=50000, p_match=1.0)
    logits, draft, kv_in = plan_inputs(w)
    got = compare(logits, draft, kv_in)
    assert (got["accept_len"] == w.R).all()


def test_first_draft_wrong_gives_one_token():
    w = Workload("none_match", 6002, B=8, H_q=1, H_kv=1, hd=64, D=7, T=0, V=3000, p_match=0.0)
    logits, draft, kv_in = plan_inputs(w)
    got = compare(logits, draft, kv_in)
    assert (got["accept_len"] == 1).all()


def test_workspace_contents_on_entry_are_ignored():
    """One workspace, filled with junk before every call, serves a chain of
    greedy and tree calls of different shapes, each bit-exact against the
    oracle."""
    import torch

    import speculative_decoding_verification_15_amd as sv
    from oracle.tree import oracle_accept_tree
    from tests.gpu_util import dev
    from workloads import make_tree_plan, tree_tokens_from_target

    rng = np.random.default_rng(77)
    shapes = [(16, 15, 128256), (3, 5, 4097), (16, 15, 128256), (7, 0, 1), (9, 63, 300),
              (16, 15, 5000)]
    big = max(sv.spec_accept_workspace_size(*s) for s in shapes)
    ws = torch.empty(big, dtype=torch.uint8, device="cuda")
    for i, (B, D, V) in enumerate(shapes):
        R = D + 1
        logits = _tie_logits(B, R, V, rng) if i % 2 else \
            rng.standard_normal((B, R, V)).astype(np.float32)
        kv_in = np.full(B, 40 + R, np.int32)
        target = np.argmax(logits, axis=-1)
        draft = np.where(rng.random((B, D)) < 0.7, target[:, :D],
                         rng.integers(0, V, size=(B, D))).astype(np.int32)
        ref = oracle_accept(logits, draft, kv_in, D)
        outs = {k: torch.full(s, -7, dtype=torch.int32, device="cuda") for k, s in
                (("target", (B, R)), ("accept_len", (B,)), ("out_tokens", (B, R)),
                 ("kv_lens_out", (B,)), ("accept_path", (B, R)))}
        ws.random_(0, 256)
        note(f"[gpu] junk workspace call {i}: B={B} D={D} V={V}")
        sv.spec_accept(B, D, V, dev(logits), dev(draft) if D else None, outs["target"],
                       outs["accept_len"], outs["out_tokens"], dev(kv_in), outs["kv_lens_out"],
                       ws, big)
        torch.cuda.synchronize()
        for k in ("target", "accept_len", "out_tokens", "kv_lens_out"):
            assert np.array_equal(outs[k].cpu().numpy(), ref[k]), (i, k)
        if D > 0:                   # a tree call on the same workspace
            w = Workload("ws_tree", 100 + i, B=B, H_q=1, H_kv=1, hd=64, D=D, T=0, V=V)
            tp = make_tree_plan(w, shape="random", width=3, p_match=0.7)
            tok = tree_tokens_from_target(tp, target)
            tref = oracle_accept_tree(logits, tok, tp.parents, kv_in)
            ws.random_(0, 256)
            sv.spec_accept_tree(B, D, V, dev(logits), dev(tok), dev(tp.parents), outs["target"],
                                outs["accept_len"], outs["out_tokens"], outs["accept_path"],
                                dev(kv_in), outs["kv_lens_out"], ws, big)
            torch.cuda.synchronize()
            for k in ("target", "accept_len", "out_tokens", "accept_path", "kv_lens_out"):
                assert np.array_equal(outs[k].cpu().numpy(), tref[k]), (i, "tree", k)
