"""Pins for the attention oracle.

Each check compares the oracle with something other than itself:
  * torch's fp64 scaled_dot_product_attention on K/V gathered here by explicit
    per-element index arithmetic (a second reading of the cache layout) and
    decoded by torch's own bf16 / float8 types;
  * pure-Python loops over the definition on tiny inputs;
  * the online-softmax identity (running max and sum, split ranges merged)
    against the full softmax, to 1e-12;
  * special cases with known answers (one visible key, q = 0, one dominant
    score, causal self-attention with an empty context);
  * invariance to the physical block placement, and poisoned (NaN) slots past
    each sequence's length never reaching an output.
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import oracle_attn, oracle_attn_online
from workloads import EDGE, MINI, TINY, KV_FP8, Workload, make_attn_inputs


def _decode_torch(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes))
    if codes.dtype == np.uint16:
        return t.view(torch.int16).view(torch.bfloat16).to(torch.float64)
    return t.view(torch.float8_e4m3fn).to(torch.float64)


def logical_kv(inp, b):
    """K, V of sequence b as [L][H_kv][hd] fp64, read element by element through
    the block table with the documented index formulas."""
    L = int(inp.kv_lens[b])
    X = inp.k_cache.shape[-1]
    H_kv, hd = inp.w.H_kv, inp.w.hd
    t = np.arange(L)[:, None, None]
    kvh = np.arange(H_kv)[None, :, None]
    d = np.arange(hd)[None, None, :]
    blk = inp.block_table[b][t // 16]
    slot = t % 16
    kc = inp.k_cache[blk, kvh, d // X, slot, d % X]
    vc = inp.v_cache[blk, kvh, d, slot]
    K, V = _decode_torch(kc), _decode_torch(vc)
    if inp.k_cache.dtype == np.uint8:
        K = K * torch.from_numpy(inp.k_scale[blk[:, :, 0], np.arange(H_kv)[None, :]].astype(np.float64))[:, :, None]
        V = V * torch.from_numpy(inp.v_scale[blk[:, :, 0], np.arange(H_kv)[None, :]].astype(np.float64))[:, :, None]
    return K, V


def sdpa_reference(inp):
    w = inp.w
    out = np.empty((w.B, w.R, w.H_q, w.hd))
    for b in range(w.B):
        K, V = logical_kv(inp, b)
        L = K.shape[0]
        Q = _decode_torch(inp.q[b]).permute(1, 0, 2)[None]           # [1][H_q][R][hd]
        Kr = K.permute(1, 0, 2).repeat_interleave(w.G, dim=0)[None]   # [1][H_q][L][hd]
        Vr = V.permute(1, 0, 2).repeat_interleave(w.G, dim=0)[None]
        P = L - w.R
        mask = torch.arange(L)[None, :] <= (P + torch.arange(w.R))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(Q, Kr, Vr, attn_mask=mask,
                                                             scale=w.sm_scale)
        out[b] = o[0].permute(1, 0, 2).numpy()
    return out


def run_oracle(inp, **kw):
    w = inp.w
    return oracle_attn(inp.q, inp.k_cache, inp.v_cache, inp.k_scale, inp.v_scale,
                       inp.block_table, inp.kv_lens, D=w.D, H_kv=w.H_kv,
                       sm_scale=w.sm_scale, **kw)


SMALL = [TINY] + list(MINI.values()) + list(EDGE.values())


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_oracle_matches_torch_sdpa(w):
    inp = make_attn_inputs(w)
    ours = run_oracle(inp)
    ref = sdpa_reference(inp)
    assert np.isfinite(ours).all()
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


def _python_brute_force(inp):
    w = inp.w
    out = np.empty((w.B, w.R, w.H_q, w.hd))
    for b in range(w.B):
        K, V = logical_kv(inp, b)
        K, V = K.tolist(), V.tolist()
        Q = _decode_torch(inp.q[b]).tolist()
        L = len(K)
        for i in range(w.R):
            last = L - w.R + i
            for h in range(w.H_q):
                kvh = h // w.G
                s = [w.sm_scale * math.fsum(Q[i][h][d] * K[t][kvh][d] for d in range(w.hd))
                     for t in range(last + 1)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = math.fsum(e)
                for d in range(w.hd):
                    out[b, i, h, d] = math.fsum(e[t] * V[t][kvh][d] for t in range(last + 1)) / z
    return out


@pytest.mark.parametrize("w", [
    Workload("bf_tiny_bf16", 4001, B=2, H_q=4, H_kv=2, hd=8, D=2, T_range=(0, 37)),
    Workload("bf_tiny_fp8", 4002, B=2, H_q=2, H_kv=1, hd=16, D=3, T_range=(1, 30),
             kv_dtype=KV_FP8),
], ids=lambda w: w.name)
def test_oracle_matches_python_loops(w):
    inp = make_attn_inputs(w)
    np.testing.assert_allclose(run_oracle(inp), _python_brute_force(inp), rtol=0, atol=1e-12)


@pytest.mark.parametrize("name,tiles,splits", [
    ("mini_gqa4_d7", (5, 64), (None, 16, 100, 1000)),
    ("mini_fp8_d15", (64, 128), (None, 16, 64, 512)),
    ("mini_hd64_g4", (1, 64), (None, 16)),
])
def test_online_softmax_equals_full_softmax(name, tiles, splits):
    inp = make_attn_inputs(MINI[name])
    w = inp.w
    full = run_oracle(inp)
    for tile in tiles:
        for split in splits:
            online = oracle_attn_online(inp.q, inp.k_cache, inp.v_cache, inp.k_scale,
                                        inp.v_scale, inp.block_table, inp.kv_lens, D=w.D,
                                        H_kv=w.H_kv, sm_scale=w.sm_scale, tile=tile,
                                        split_tokens=split)
            rel = np.abs(online - full).max() / np.abs(full).max()
            assert rel <= 1e-12, (tile, split, rel)


def test_one_visible_key_returns_that_value_exactly():
    inp = make_attn_inputs(EDGE["edge_one_key"])
    out = run_oracle(inp)
    K, V = logical_kv(inp, 0)
    for h in range(inp.w.H_q):
        np.testing.assert_array_equal(out[0, 0, h], V[0, h // inp.w.G].numpy())


def test_zero_query_gives_mean_of_visible_values():
    inp = make_attn_inputs(MINI["mini_gqa4_d7"])
    inp.q[:] = 0
    out = run_oracle(inp)
    w = inp.w
    for b in range(w.B):
        _, V = logical_kv(inp, b)
        V = V.numpy()
        L = V.shape[0]
        for i in range(w.R):
            mean = V[: L - w.R + i + 1].mean(axis=0)          # [H_kv][hd]
            for h in range(w.H_q):
                np.testing.assert_allclose(out[b, i, h], mean[h // w.G], rtol=0, atol=1e-13)


def test_dominant_score_selects_its_value():
    w = Workload("dominant", 4003, B=1, H_q=2, H_kv=1, hd=64, D=1, T=40)
    inp = make_attn_inputs(w)
    L = int(inp.kv_lens[0])
    star = 17
    # K = 0 except key `star`, which is 8 * e_3; q = 64 * e_3 -> score 512/8 = 64 vs 0
    blk = inp.block_table[0]
    for t in range(L):
        for d in range(w.hd):
            inp.k_cache[blk[t // 16], 0, d // 8, t % 16, d % 8] = 0
    inp.k_cache[blk[star // 16], 0, 3 // 8, star % 16, 3 % 8] = 0x4100   # 8.0
    inp.q[:] = 0
    inp.q[:, :, :, 3] = 0x4280                                             # 64.0
    out = run_oracle(inp)
    _, V = logical_kv(inp, 0)
    # every other key gets weight exp(-64) relative to the dominant one
    for i in range(w.R):
        for h in range(w.H_q):
            np.testing.assert_allclose(out[0, i, h], V[star, 0].numpy(), rtol=0, atol=1e-24 * L + 1e-26)


def test_block_placement_does_not_change_outputs():
    w = MINI["mini_gqa8_d15"]
    a = run_oracle(make_attn_inputs(w))
    b = run_oracle(make_attn_inputs(w.replace(identity_table=True)))
    np.testing.assert_array_equal(a, b)


def test_empty_context_is_causal_self_attention():
    inp = make_attn_inputs(EDGE["edge_empty_context"])
    w = inp.w
    out = run_oracle(inp)
    for b in range(w.B):
        K, V = logical_kv(inp, b)
        assert K.shape[0] == w.R
        Q = _decode_torch(inp.q[b]).permute(1, 0, 2)[None]
        Kr = K.permute(1, 0, 2).repeat_interleave(w.G, dim=0)[None]
        Vr = V.permute(1, 0, 2).repeat_interleave(w.G, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kr, Vr, is_causal=True,
                                                               scale=w.sm_scale)
        np.testing.assert_allclose(out[b], ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_poisoned_slots_and_subset_rows():
    w = MINI["mini_fp8_d15"]
    inp = make_attn_inputs(w)
    # slots past L_b and the spare blocks hold NaN codes
    assert (inp.k_cache == 0x7F).any()
    full = run_oracle(inp)
    assert np.isfinite(full).all()
    part = run_oracle(inp, seqs=[1], kv_heads=[1])
    np.testing.assert_array_equal(part[1, :, w.G:2 * w.G], full[1, :, w.G:2 * w.G])
    assert np.isnan(part[0]).all() and np.isnan(part[1, :, :w.G]).all()
