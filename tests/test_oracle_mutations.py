"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin fails.

Each case swaps one piece of the oracle for a wrong variant -- an off-by-one
mask, a wrong KV-head index, a transposed V block, a dropped rescale, a wrong
exponent bias, the last instead of the first maximum, an AL off by one -- and
runs the pin that should catch it.  The real oracle is restored afterwards.
"""
import numpy as np
import pytest

import oracle.accept as acc
import oracle.attention as att
import oracle.formats as fmt
from tests import test_oracle_accept as T_acc
from tests import test_oracle_attention as T_att
from tests import test_oracle_formats as T_fmt
from workloads import MINI


def _expect_pin_failure(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_mask_off_by_one_is_caught(monkeypatch):
    # position i no longer sees itself
    monkeypatch.setattr(att, "_visible",
                        lambda R, L: np.arange(L)[None, :] < (L - R + np.arange(R))[:, None])
    _expect_pin_failure(T_att.test_oracle_matches_torch_sdpa, MINI["mini_gqa4_d7"])


def test_wrong_kv_head_is_caught(monkeypatch):
    real = att.gather_kv

    def swapped(*a):
        K, V = real(*a)
        return K[:, ::-1], V[:, ::-1]
    monkeypatch.setattr(att, "gather_kv", swapped)
    _expect_pin_failure(T_att.test_oracle_matches_torch_sdpa, MINI["mini_gqa4_d7"])


def test_transposed_v_block_is_caught(monkeypatch):
    def wrong_gather(k_cache, v_cache, k_scale, v_scale, block_table, b, L, kv_heads=None):
        nb = -(-int(L) // 16)
        blocks = np.asarray(block_table[b, :nb], dtype=np.int64)
        kb = k_cache[blocks]
        n, H, nx, bs, X = kb.shape
        K = att._decode(kb.transpose(0, 3, 1, 2, 4).reshape(nb * 16, H, nx * X)[:L])
        # reads V as if it were token-major [16][hd] inside each block
        vb = v_cache[blocks].reshape(nb, H, 16, -1)
        V = att._decode(vb.transpose(0, 2, 1, 3).reshape(nb * 16, H, -1)[:L])
        return K, V
    monkeypatch.setattr(att, "gather_kv", wrong_gather)
    _expect_pin_failure(T_att.test_oracle_matches_torch_sdpa, MINI["mini_gqa4_d7"])


def test_dropped_rescale_is_caught(monkeypatch):
    def no_rescale(s, v, tile):
        n, L = s.shape
        O = np.zeros((n, v.shape[1])); m = np.full(n, -np.inf); l = np.zeros(n)
        for t0 in range(0, L, tile):
            st = s[:, t0:t0 + tile]
            m_new = np.maximum(m, st.max(axis=1))
            p = np.exp(st - m_new[:, None])
            l = l + p.sum(axis=1)          # missing l * exp(m - m_new)
            O = O + p @ v[t0:t0 + tile]    # missing O * exp(m - m_new)
            m = m_new
        return O, m, l
    monkeypatch.setattr(att, "online_softmax_rows", no_rescale)
    _expect_pin_failure(T_att.test_online_softmax_equals_full_softmax, "mini_gqa4_d7",
                        (64,), (None,))


def test_wrong_e4m3_bias_is_caught(monkeypatch):
    def bias8(bits):
        b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
        s, e, m = (b >> 7) & 1, (b >> 3) & 0xF, b & 7
        sign = np.where(s == 1, -1.0, 1.0)
        v = np.where(e == 0, sign * np.ldexp(m / 8.0, -7), sign * np.ldexp(1 + m / 8.0, e - 8))
        return np.where((e == 15) & (m == 7), np.nan, v)
    monkeypatch.setattr(T_fmt, "e4m3_bits_to_f64", bias8)
    _expect_pin_failure(T_fmt.test_e4m3_all_codes_match_torch)


def test_last_maximum_is_caught(monkeypatch):
    def last_max(x):
        x = np.asarray(x, np.float32)
        return (x.shape[-1] - 1 - np.argmax(x[..., ::-1], axis=-1)).astype(np.int32)
    monkeypatch.setattr(T_acc, "oracle_argmax", last_max)
    _expect_pin_failure(T_acc.test_argmax_exhaustive_small, 3)


def test_accept_len_off_by_one_is_caught(monkeypatch):
    real = acc.oracle_accept

    def short(*a):
        r = real(*a)
        r["accept_len"] = np.maximum(r["accept_len"] - 1, 0)
        return r
    monkeypatch.setattr(T_acc, "oracle_accept", short)
    _expect_pin_failure(T_acc.test_prefix_exhaustive, 2)


def test_bf16_half_shift_is_caught(monkeypatch):
    def wrong(bits):
        u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return u.view(np.float32).astype(np.float64)
    monkeypatch.setattr(T_fmt, "bf16_bits_to_f64", wrong)
    _expect_pin_failure(T_fmt.test_bf16_all_patterns_match_torch)


from tests import test_oracle_accept_sampled as T_smp  # noqa: E402


def test_inverted_keep_ratio_is_caught(monkeypatch):
    # keep with probability min(1, q/p) instead of min(1, p/q)
    monkeypatch.setattr(acc, "keep_draft", lambda u, p_d, q_d: float(u) * p_d < q_d)
    _expect_pin_failure(T_smp.test_emitted_tokens_follow_the_target, 1.0)


def test_residual_without_subtraction_is_caught(monkeypatch):
    monkeypatch.setattr(acc, "residual", lambda p_j, q_j: p_j)
    _expect_pin_failure(T_smp.test_emitted_tokens_follow_the_target, 1.0)


def test_draw_off_by_one_is_caught(monkeypatch):
    def left(w, u):
        c = np.cumsum(np.asarray(w, np.float64))
        return min(int(np.searchsorted(c, float(u) * c[-1], side="left")), len(c) - 1)
    monkeypatch.setattr(T_smp, "oracle_draw", left)
    _expect_pin_failure(T_smp.test_draw_matches_its_definition, [0.0, 0.2, 0.0, 0.5, 0.3])


import oracle.append as app  # noqa: E402
from tests import test_oracle_append as T_app  # noqa: E402


def test_block_scale_without_448_is_caught(monkeypatch):
    # scale = amax (codes would top out at 1.0 instead of 448)
    monkeypatch.setattr(app, "_block_scale", lambda amax: np.float32(amax) if amax else np.float32(1))
    _expect_pin_failure(T_app.test_block_aligned_appends_match_generator_placement, True)


def test_encode_ties_away_from_zero_is_caught(monkeypatch):
    real = app.e4m3_encode_f32

    def away(y):
        y = np.asarray(y, np.float32)
        # nudge exact halfway cases upwards before the correct encoder
        return real(np.nextafter(y, np.sign(y) * np.float32(np.inf)).astype(np.float32))
    monkeypatch.setattr(app, "e4m3_encode_f32", away)
    _expect_pin_failure(T_app.test_block_aligned_appends_match_generator_placement, True)


def test_held_codes_not_reencoded_is_caught(monkeypatch):
    # on a scale change the held codes keep their old bytes (their values change)
    real = app.oracle_kv_append

    def no_reencode(k_new, v_new, k_cache, v_cache, k_scale, v_scale, table, lens, fp8):
        out = real(k_new, v_new, k_cache, v_cache, k_scale, v_scale, table, lens, fp8)
        kc = out[0]
        for b, c in enumerate(np.asarray(lens)):
            blk, a = table[b][int(c) // 16], int(c) % 16
            kc[blk, :, :, :a, :] = np.asarray(k_cache)[blk, :, :, :a, :]
        return out
    monkeypatch.setattr(T_app, "oracle_kv_append", no_reencode)
    _expect_pin_failure(T_app.test_fp8_held_codes_kept_when_values_fit_and_reencoded_when_they_outgrow)


def test_append_at_wrong_position_is_caught(monkeypatch):
    real = app.oracle_kv_append
    monkeypatch.setattr(T_app, "oracle_kv_append",
                        lambda kn, vn, kc, vc, ks, vs, t, lens, fp8:
                        real(kn, vn, kc, vc, ks, vs, t, np.asarray(lens) + 1, fp8))
    _expect_pin_failure(T_app.test_bf16_rows_land_where_the_attention_gather_reads_them)


import oracle.draft_signals as dsg  # noqa: E402
from tests import test_oracle_draft_signals as T_dsg  # noqa: E402


def test_entropy_in_bits_is_caught(monkeypatch):
    real = dsg.oracle_signals
    monkeypatch.setattr(T_dsg, "oracle_signals",
                        lambda z, tau=1.0: (real(z, tau)[0], real(z, tau)[1] / np.log(2)))
    _expect_pin_failure(T_dsg.test_signals_match_scipy, 1.0)


def test_ties_to_longer_draft_are_caught(monkeypatch):
    real = dsg.choose_draft_len

    def longer(c, Dmax, rho, G):
        d = real(c, Dmax, rho, G)
        return max(dsg.candidate_lengths(Dmax, G)) if c == 0.0 and rho == 0.0 else d
    monkeypatch.setattr(T_dsg, "choose_draft_len", longer)
    _expect_pin_failure(T_dsg.test_choice_special_cases)


def test_tile_rule_off_by_one_is_caught(monkeypatch):
    def loose(Dmax, G):
        return [D for D in range(Dmax + 1)
                if not (G > 0 and G * D > 128 and (G * (D + 1)) % 128 != 0)]
    monkeypatch.setattr(T_dsg, "candidate_lengths", loose)
    _expect_pin_failure(T_dsg.test_tile_rule_candidates)


def test_objective_without_draft_cost_is_caught(monkeypatch):
    real = dsg.choose_draft_len
    monkeypatch.setattr(T_dsg, "choose_draft_len", lambda c, Dmax, rho, G: real(c, Dmax, 0.0, G))
    _expect_pin_failure(T_dsg.test_choice_matches_brute_force_grid)


import oracle.tree as otree  # noqa: E402
from tests import test_oracle_tree as T_tree  # noqa: E402


def test_tree_parent_only_visibility_is_caught(monkeypatch):
    # node i sees itself and its parent, not the whole root path
    def shallow(parents, L):
        R = len(parents)
        vis = np.zeros((R, L), dtype=bool)
        vis[:, : L - R] = True
        for i in range(R):
            vis[i, L - R + i] = True
            if parents[i] >= 0:
                vis[i, L - R + int(parents[i])] = True
        return vis
    monkeypatch.setattr(att, "_visible_tree", shallow)
    _expect_pin_failure(T_tree.test_tree_attention_matches_torch_sdpa)


def test_tree_walk_takes_highest_child_is_caught(monkeypatch):
    def highest(logits, tokens, parents, kv):
        logits = np.asarray(logits, np.float32)
        B, R, V = logits.shape
        tgt = acc.oracle_argmax(logits)
        out = otree.oracle_accept_tree(logits, tokens, parents, kv)
        for b in range(B):
            path = [0]
            while True:
                cs = [c for c in range(R - 1, path[-1], -1)
                      if parents[b][c] == path[-1] and tokens[b][c] == tgt[b, path[-1]]]
                if not cs:
                    break
                path.append(cs[0])
            out["accept_path"][b, :] = -1
            out["accept_path"][b, : len(path)] = path
        return out
    monkeypatch.setattr(T_tree, "oracle_accept_tree", highest)
    _expect_pin_failure(T_tree.test_tree_acceptance_brute_force_small)
