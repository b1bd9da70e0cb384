"""GPU parity of spec_accept_sampled against the stochastic-acceptance oracle.

Exact: accept_len, out_tokens and the committed KV lengths equal the oracle's
for every sequence whose decisions are not near-ties.  The GPU evaluates p and
q from fp32 exponentials (a few ulp each, independent per logit) with fp64 sums,
so a decision whose margin is inside that rounding may go either way:
  * a keep test u*q < p with |u*q - p| <= 1e-5 * max(p, u*q);
  * a draw whose u * total lies within 2e-8 * total of a running-sum boundary.
Sequences with a near-tie must still be valid: AL in 1..1+D, the drafts before
the emitted token, a token of positive weight, -1 padding, the KV commit.
Also checked on the GPU's own outputs: with V = 6 and 20000 sequences the first
emitted token follows the target distribution (chi-square) and the first draft
is kept at the rate sum_v min(p, q).
"""
import numpy as np
import pytest
import torch
from scipy import stats

import speculative_decoding_verification_15_amd as sv
from oracle.accept import _softmax64, oracle_accept_sampled
from tests.gpu_util import dev, note
from workloads import LLAMA31_70B, Workload, make_sampled_accept_inputs

pytestmark = pytest.mark.gpu


def run_sampled(zt, zd, draft, ua, us, tau, kv_in, inplace=False):
    B, R, V = zt.shape
    D = R - 1
    t_zt = dev(np.ascontiguousarray(zt, np.float32))
    t_zd = dev(np.ascontiguousarray(zd, np.float32)) if D else None
    t_dr = dev(np.ascontiguousarray(draft, np.int32)) if D else None
    t_ua = dev(np.ascontiguousarray(ua, np.float32)) if D else None
    t_us = dev(np.ascontiguousarray(us, np.float32))
    al = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, R), -7, dtype=torch.int32, device="cuda")
    kin = dev(np.asarray(kv_in, np.int32))
    kout = kin if inplace else torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ws_bytes = sv.spec_accept_sampled_workspace_size(B, D, V)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    note(f"[gpu] spec_accept_sampled B={B} D={D} V={V} tau={tau}")
    sv.spec_accept_sampled(B, D, V, tau, t_zt, t_zd, t_dr, t_ua, t_us, al, out, kin, kout, ws,
                           ws_bytes)
    torch.cuda.synchronize()
    return dict(accept_len=al.cpu().numpy(), out_tokens=out.cpu().numpy(),
                kv_lens_out=kout.cpu().numpy())


def _near_tie_and_weights(zt, zd, draft, ua, us, tau, b, n_ref):
    """Whether sequence b's oracle decisions include a near-tie, and the weights
    of the distribution the emitted token is drawn from (for validity checks)."""
    D = zt.shape[1] - 1
    p = _softmax64(zt[b], tau)
    q = _softmax64(zd[b], tau) if D else None
    tie = False
    for j in range(min(n_ref + 1, D)):
        d = int(draft[b, j])
        a, c = float(ua[b, j]) * q[j, d], p[j, d]
        tie |= abs(a - c) <= 1e-5 * max(a, c)
    if n_ref < D:
        w = np.maximum(p[n_ref] - q[n_ref], 0.0)
        w = w if w.sum() > 0 else p[n_ref]
    else:
        w = p[D]
    cs = np.cumsum(w)
    T = float(us[b]) * cs[-1]
    i = int(np.searchsorted(cs, T, side="right"))
    lo = cs[i - 1] if i > 0 else 0.0
    hi = cs[min(i, len(cs) - 1)]
    tie |= min(T - lo, hi - T) <= 2e-8 * cs[-1]
    return tie, w


def compare(zt, zd, draft, ua, us, tau, kv_in, inplace=False):
    B, R, V = zt.shape
    D = R - 1
    ref = oracle_accept_sampled(zt, zd, draft, ua, us, tau, kv_in, D)
    got = run_sampled(zt, zd, draft, ua, us, tau, kv_in, inplace=inplace)
    n_tie = 0
    for b in range(B):
        same = (got["accept_len"][b] == ref["accept_len"][b]
                and (got["out_tokens"][b] == ref["out_tokens"][b]).all()
                and got["kv_lens_out"][b] == ref["kv_lens_out"][b])
        if same:
            continue
        tie, _ = _near_tie_and_weights(zt, zd, draft, ua, us, tau, b, int(ref["accept_len"][b]) - 1)
        assert tie, (b, got["accept_len"][b], ref["accept_len"][b], got["out_tokens"][b],
                     ref["out_tokens"][b])
        n_tie += 1
        # still a valid outcome
        n = int(got["accept_len"][b]) - 1
        assert 0 <= n <= D
        assert (got["out_tokens"][b, :n] == draft[b, :n]).all()
        assert (got["out_tokens"][b, n + 1:] == -1).all()
        _, w = _near_tie_and_weights(zt, zd, draft, ua, us, tau, b, n)
        assert w[got["out_tokens"][b, n]] > 0
        assert got["kv_lens_out"][b] == kv_in[b] - R + n + 1
    note(f"  B={B} D={D} V={V} tau={tau}: sum AL = {int(got['accept_len'].sum())}, "
         f"near-tie differences {n_tie}")
    assert n_tie <= max(1, B // 50)
    return got


def _inputs(B, D, V, tau=1.0, seed=3100, noise=0.5):
    w = Workload(f"smp_{B}_{D}_{V}", seed, B=B, H_q=1, H_kv=1, hd=8, D=D, T=0, V=V)
    x = make_sampled_accept_inputs(w, tau=tau, noise=noise)
    kv_in = (np.arange(B, dtype=np.int32) * 5 + 3 * w.R).astype(np.int32)
    return x, kv_in


@pytest.mark.parametrize("B,D,V,tau", [(64, 3, 1024, 1.0), (64, 3, 1024, 0.7), (16, 7, 5003, 1.0),
                                       (8, 0, 4096, 1.0), (40, 15, 4097, 1.3), (4, 63, 300, 1.0)])
def test_sampled_matches_oracle(B, D, V, tau):
    x, kv_in = _inputs(B, D, V, tau)
    compare(x.target_logits, x.draft_logits, x.draft, x.u_accept, x.u_sample, tau, kv_in)


def test_sampled_full_size_70b_like():
    # B = 32, D = 15, V = 128256 (the 70B-like acceptance shape)
    x = make_sampled_accept_inputs(LLAMA31_70B)
    kv_in = np.full(LLAMA31_70B.B, 4096, np.int32)
    compare(x.target_logits, x.draft_logits, x.draft, x.u_accept, x.u_sample, x.tau, kv_in)


def test_sampled_in_place_commit_and_far_drafts():
    x, kv_in = _inputs(32, 5, 2048, seed=3200, noise=3.0)   # a poor draft model: early rejections
    got = compare(x.target_logits, x.draft_logits, x.draft, x.u_accept, x.u_sample, 1.0, kv_in,
                  inplace=True)
    assert (got["accept_len"] < 6).any()


def test_gpu_emitted_tokens_follow_the_target():
    from tests.test_oracle_accept_sampled import Y, Z
    N, V = 20000, Z.shape[1]
    rng = np.random.default_rng(77)
    q0 = _softmax64(Y[0], 1.0)
    draft = rng.choice(V, size=(N, 1), p=q0)
    zt = np.broadcast_to(Z[:2], (N, 2, V)).copy()
    zd = np.broadcast_to(Y[:1], (N, 1, V)).copy()
    ua = rng.random((N, 1)).astype(np.float32)
    us = rng.random(N).astype(np.float32)
    got = run_sampled(zt, zd, draft, ua, us, 1.0, np.full(N, 2, np.int32))
    p0 = _softmax64(Z[0], 1.0)
    counts = np.bincount(got["out_tokens"][:, 0], minlength=V)
    assert stats.chisquare(counts, p0 * N).pvalue > 1e-4
    alpha = np.minimum(p0, q0).sum()
    kept = (got["accept_len"] == 2).mean()
    assert abs(kept - alpha) < 4 * np.sqrt(alpha * (1 - alpha) / N), (kept, alpha)
