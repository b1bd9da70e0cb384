"""Pins of the stochastic-acceptance oracle (CPU only).

What the pages fix: the rule keeps the output distribution of the large model
alone ("GPU and LLM" ch. 5, section "Speculative decoding (2)"), and with each
draft kept independently with probability alpha the expected tokens per
verification is (1 - alpha^(k+1)) / (1 - alpha) (same section).  The rule's
source (Leviathan et al., cited there) gives alpha = sum_v min(p(v), q(v)).
Checked here:
  * the emitted tokens follow the target distribution (chi-square, at the first
    position and at the second given the first draft kept);
  * the keep rate is sum_v min(p, q), and the mean AL is the closed form;
  * p == q keeps every draft; p(d) = 0 rejects d and draws from p;
  * the inverse-CDF draw against its definition, exhaustively on a grid.
"""
import numpy as np
import pytest
from scipy import stats

from oracle.accept import oracle_accept_sampled, oracle_draw
from oracle.closed_forms import expected_tokens

V = 6


def _softmax(x):
    e = np.exp(np.asarray(x, np.float64) - np.max(x))
    return e / e.sum()


def _trials(z_rows, y_rows, N, seed, tau=1.0):
    """N sequences sharing the per-position target logits z_rows [R][V] and draft
    logits y_rows [D][V]; drafts drawn from q with numpy's own sampler."""
    rng = np.random.default_rng(seed)
    R, D = len(z_rows), len(y_rows)
    q = [_softmax(np.asarray(y, np.float64) / tau) for y in y_rows]
    draft = np.stack([rng.choice(len(z_rows[0]), size=N, p=q[j]) for j in range(D)], axis=1) \
        if D else np.zeros((N, 0), np.int64)
    z = np.broadcast_to(np.asarray(z_rows, np.float32), (N, R, len(z_rows[0])))
    y = np.broadcast_to(np.asarray(y_rows, np.float32).reshape(D, len(z_rows[0])), (N, D, len(z_rows[0])))
    u_acc = rng.random((N, D)).astype(np.float32)
    u_smp = rng.random(N).astype(np.float32)
    res = oracle_accept_sampled(z, y, draft, u_acc, u_smp, tau, np.full(N, R, np.int32), D)
    return res, draft


def _chi2_ok(samples, p, pmin=1e-4):
    counts = np.bincount(samples, minlength=len(p)).astype(np.float64)
    exp = p * counts.sum()
    keep = exp > 0
    assert counts[~keep].sum() == 0, "drew a token of probability zero"
    return stats.chisquare(counts[keep], exp[keep] / exp[keep].sum() * counts.sum()).pvalue > pmin


Z = np.array([[1.0, 0.2, -0.5, 2.0, 0.0, -1.0],
              [0.3, 1.5, 0.1, -0.7, 0.9, 0.0],
              [-0.2, 0.4, 1.1, 0.0, -1.3, 0.6]], np.float32)
Y = np.array([[0.1, 1.2, 0.4, 0.5, -0.3, 0.8],
              [1.4, 0.2, -0.6, 0.3, 0.9, -0.1]], np.float32)


@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_emitted_tokens_follow_the_target(tau):
    N = 30000
    res, draft = _trials(Z, Y, N, seed=11, tau=tau)
    p0, p1 = _softmax(Z[0] / tau), _softmax(Z[1] / tau)
    out = res["out_tokens"]
    assert _chi2_ok(out[:, 0], p0)
    kept0 = res["accept_len"] >= 2               # first draft kept: the second emitted token
    assert _chi2_ok(out[kept0, 1], p1)
    # keep rate of the first draft: sum_v min(p, q)
    alpha0 = np.minimum(p0, _softmax(Y[0] / tau)).sum()
    se = np.sqrt(alpha0 * (1 - alpha0) / N)
    assert abs(kept0.mean() - alpha0) < 4 * se, (kept0.mean(), alpha0)


@pytest.mark.parametrize("D", [1, 4])
def test_mean_accept_len_is_the_closed_form(D):
    # the same p and q at every position: each draft kept with alpha = sum min(p, q)
    N = 20000
    res, _ = _trials([Z[0]] * (D + 1), [Y[0]] * D, N, seed=12 + D)
    alpha = np.minimum(_softmax(Z[0]), _softmax(Y[0])).sum()
    AL = res["accept_len"].astype(np.float64)
    mu = expected_tokens(alpha, D)
    assert abs(AL.mean() - mu) < 4 * AL.std() / np.sqrt(N), (AL.mean(), mu)


def test_equal_distributions_keep_every_draft():
    N, D = 8000, 2
    res, draft = _trials(Z, Z[:D], N, seed=13)
    assert (res["accept_len"] == D + 1).all()
    assert (res["out_tokens"][:, :D] == draft).all()
    assert _chi2_ok(res["out_tokens"][:, D], _softmax(Z[D]))


def test_zero_target_probability_rejects_and_draws_from_target():
    z = Z[:2].copy()
    z[0, 3] = -np.inf                              # p0(3) = 0
    y = np.full((1, V), -40.0, np.float32)
    y[0, 3] = 40.0                                 # q0 all but one-hot on token 3
    N = 20000
    res, draft = _trials(z, y, N, seed=14)
    assert (draft[:, 0] == 3).all()
    assert (res["accept_len"] == 1).all()
    assert _chi2_ok(res["out_tokens"][:, 0], _softmax(z[0]))


def _draw_by_definition(w, u):
    T = u * sum(w)
    run = 0.0
    for i, x in enumerate(w):
        run += x
        if run > T:
            return i
    return max(i for i, x in enumerate(w) if x > 0)


@pytest.mark.parametrize("w", [[0.0, 0.2, 0.0, 0.5, 0.3], [1.0], [0.0, 0.0, 2.0], [0.25] * 4,
                               [0.0, 1e-30, 0.0, 1.0, 0.0]])
def test_draw_matches_its_definition(w):
    for u in np.concatenate([np.linspace(0, 1, 2001, endpoint=False),
                             np.cumsum(w)[:-1] / max(sum(w), 1e-300)]):
        u = min(float(u), np.nextafter(1.0, 0.0))
        assert oracle_draw(np.array(w), u) == _draw_by_definition(w, u), (w, u)
    # boundaries: a running sum equal to u * total is not "exceeded"
    assert oracle_draw(np.array([0.0, 0.2, 0.0, 0.5, 0.3]), 0.2) == 3
    assert oracle_draw(np.array([0.0, 0.2, 0.0, 0.5, 0.3]), 0.0) == 1


def test_no_drafts_draws_the_bonus_from_the_target():
    N = 20000
    res, _ = _trials(Z[:1], np.zeros((0, V), np.float32), N, seed=15)
    assert (res["accept_len"] == 1).all()
    assert _chi2_ok(res["out_tokens"][:, 0], _softmax(Z[0]))
