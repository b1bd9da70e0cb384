"""Pins for the KV-append oracle (oracle/append.py).

What fixes the expected values, other than the oracle itself:
  - torch's float8_e4m3fn conversion (a library routine) for the encoder, over
    every bf16 value and a million fp32 bit patterns;
  - the input generator's cache construction (reshape/transpose placement and
    torch's e4m3 conversion) for blocks that start and fill inside one append;
  - the attention oracle's gather (its own index formulas) for where bf16 rows land;
  - the e4m3 rounding bound, the amax/448 rule (the largest held value of every
    block encodes to 448) and the byte-for-byte untouched rest of the cache.
"""
import numpy as np
import pytest
import torch

from oracle.accept import oracle_accept
from oracle.append import e4m3_encode_f32, oracle_kv_append
from oracle.attention import gather_kv
from oracle.formats import bf16_bits_to_f64, e4m3_bits_to_f64
from workloads import KV_FP8, MINI, make_append_inputs
from workloads.generate import FP8_POISON, BF16_POISON, f32_to_bf16_bits

BLOCK = 16


def _torch_e4m3(y):
    t = torch.from_numpy(np.clip(np.asarray(y, np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_every_bf16_value_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16_bits_to_f64(bits).astype(np.float32)
    x = x[np.isfinite(x)]
    np.testing.assert_array_equal(e4m3_encode_f32(x), _torch_e4m3(x))


def test_encode_random_f32_patterns_match_torch():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # exponents spread over the whole e4m3 range and past it
    u = (u & np.uint32(0x807FFFFF)) | ((rng.integers(100, 140, size=u.size).astype(np.uint32)) << 23)
    x = u.view(np.float32)
    np.testing.assert_array_equal(e4m3_encode_f32(x), _torch_e4m3(x))


def test_encode_round_trip_and_hand_values():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    y = e4m3_bits_to_f64(codes).astype(np.float32)
    np.testing.assert_array_equal(e4m3_encode_f32(y), codes)
    cases = {448.0: 0x7E, 1000.0: 0x7E, -1e9: 0xFE, 1.0: 0x38, 1.0625: 0x38, 1.1875: 0x3A,
             1.125 + 2 ** -10: 0x39, 2.0 ** -10: 0x00, 3 * 2.0 ** -11: 0x01, -0.0: 0x80,
             -2.0 ** -12: 0x80, 464.0: 0x7E, 2.0 ** -9 * 1.5: 0x02}
    for v, c in cases.items():
        assert int(e4m3_encode_f32(np.float32(v))) == c, (v, hex(c))


def _empty_cache(B, H_kv, hd, fp8, max_tokens, seed=0):
    """A paged cache of poison with a permuted table covering max_tokens per sequence."""
    nb = -(-max_tokens // BLOCK)
    perm = np.random.default_rng(seed).permutation(B * nb + 2).astype(np.int32)
    table = perm[: B * nb].reshape(B, nb)
    X = 16 if fp8 else 8
    dt, poison = (np.uint8, FP8_POISON) if fp8 else (np.uint16, BF16_POISON)
    kc = np.full((B * nb + 2, H_kv, hd // X, BLOCK, X), poison, dtype=dt)
    vc = np.full((B * nb + 2, H_kv, hd, BLOCK), poison, dtype=dt)
    ks = np.full((B * nb + 2, H_kv), np.nan, np.float32) if fp8 else None
    vs = np.full((B * nb + 2, H_kv), np.nan, np.float32) if fp8 else None
    return kc, vc, ks, vs, table


def _rows(rng, shape, gain=1.0):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(gain))


@pytest.mark.parametrize("fp8", [False, True])
def test_block_aligned_appends_match_generator_placement(fp8):
    """Whole-block appends from an empty cache give the bytes of a one-shot
    quantization: per (block, KV head) scale amax/448, torch's e4m3 conversion,
    placed by the generator's reshape/transpose."""
    B, H, hd, nblk = 2, 2, 64, 3
    rng = np.random.default_rng(11)
    k = _rows(rng, (B, nblk * BLOCK, H, hd))
    v = _rows(rng, (B, nblk * BLOCK, H, hd))
    kc, vc, ks, vs, table = _empty_cache(B, H, hd, fp8, nblk * BLOCK)
    lens = np.zeros(B, np.int32)
    for j in range(nblk):
        sl = slice(j * BLOCK, (j + 1) * BLOCK)
        kc, vc, ks, vs, lens = oracle_kv_append(k[:, sl], v[:, sl], kc, vc, ks, vs, table, lens, fp8)
    assert (lens == nblk * BLOCK).all()
    X = 16 if fp8 else 8
    for b in range(B):
        for name, rows, cache, scale in (("k", k, kc, ks), ("v", v, vc, vs)):
            x = bf16_bits_to_f64(rows[b]).astype(np.float32).reshape(nblk, BLOCK, H, hd)
            if fp8:
                amax = np.abs(x).max(axis=(1, 3))
                s = (amax / np.float32(448.0)).astype(np.float32)
                np.testing.assert_array_equal(scale[table[b]], s)
                codes = _torch_e4m3(x / s[:, None, :, None])
            else:
                codes = rows[b].reshape(nblk, BLOCK, H, hd)
            if name == "k":
                want = codes.reshape(nblk, BLOCK, H, hd // X, X).transpose(0, 2, 3, 1, 4)
            else:
                want = codes.transpose(0, 2, 3, 1)
            np.testing.assert_array_equal(cache[table[b]], want)


def test_bf16_rows_land_where_the_attention_gather_reads_them():
    w = MINI["mini_gqa4_d7"]
    ap = make_append_inputs(w)
    base = ap.base
    kc, vc, _, _, lens = oracle_kv_append(ap.k_new, ap.v_new, base.k_cache, base.v_cache, None,
                                          None, base.block_table, ap.committed, fp8=False)
    np.testing.assert_array_equal(lens, ap.committed + w.R)
    for b in range(w.B):
        c, L = int(ap.committed[b]), int(lens[b])
        K, V = gather_kv(kc, vc, None, None, base.block_table, b, L)
        K0, V0 = gather_kv(base.k_cache, base.v_cache, None, None, base.block_table, b, L)
        np.testing.assert_array_equal(K[:c], K0[:c])
        np.testing.assert_array_equal(V[:c], V0[:c])
        np.testing.assert_array_equal(K[c:], bf16_bits_to_f64(ap.k_new[b]))
        np.testing.assert_array_equal(V[c:], bf16_bits_to_f64(ap.v_new[b]))


def _written_mask(shape_blocks, table, committed, R, fp8, H_kv, hd):
    """Boolean masks over the K and V caches of the slots an append may write
    (held slots of touched blocks too, for e4m3 re-encoding)."""
    X = 16 if fp8 else 8
    mk = np.zeros((shape_blocks, H_kv, hd // X, BLOCK, X), bool)
    mv = np.zeros((shape_blocks, H_kv, hd, BLOCK), bool)
    for b, c in enumerate(committed):
        for j in range(int(c) // BLOCK, (int(c) + R - 1) // BLOCK + 1):
            lo = 0 if fp8 else max(int(c) - j * BLOCK, 0)
            hi = min(int(c) + R - j * BLOCK, BLOCK)
            mk[table[b][j], :, :, lo:hi, :] = True
            mv[table[b][j], :, :, lo:hi] = True
    return mk, mv


@pytest.mark.parametrize("name", ["mini_gqa4_d7", "mini_fp8_d15", "mini_fp8_hd64"])
def test_untouched_bytes_and_scales_keep_their_values(name):
    w = MINI[name]
    fp8 = w.kv_dtype == KV_FP8
    ap = make_append_inputs(w, gains=(0.5, 1.0, 4.0))
    base = ap.base
    kc, vc, ks, vs, _ = oracle_kv_append(ap.k_new, ap.v_new, base.k_cache, base.v_cache,
                                         base.k_scale, base.v_scale, base.block_table,
                                         ap.committed, fp8)
    mk, mv = _written_mask(base.num_blocks, base.block_table, ap.committed, w.R, fp8, w.H_kv, w.hd)
    np.testing.assert_array_equal(kc[~mk], base.k_cache[~mk])
    np.testing.assert_array_equal(vc[~mv], base.v_cache[~mv])
    if fp8:
        touched = np.zeros(base.num_blocks, bool)
        for b, c in enumerate(ap.committed):
            touched[base.block_table[b][int(c) // BLOCK: (int(c) + w.R - 1) // BLOCK + 1]] = True
        np.testing.assert_array_equal(ks[~touched], base.k_scale[~touched])   # NaN == NaN here
        np.testing.assert_array_equal(vs[~touched], base.v_scale[~touched])


def _half_step(y):
    """Half the e4m3 grid spacing around |y| (y already divided by the scale)."""
    a = np.minimum(np.abs(y.astype(np.float64)), 448.0)
    e = np.maximum(np.floor(np.log2(np.maximum(a, 2.0 ** -9))), -6)
    return 2.0 ** (e - 3) / 2


def _decoded_block(cache, scale, blk, h, slots, fp8_X=16):
    if cache.ndim == 5:
        c = cache[blk, h].transpose(1, 0, 2).reshape(BLOCK, -1)[slots]
    else:
        c = cache[blk, h].T[slots]
    return e4m3_bits_to_f64(c) * np.float64(scale[blk, h]), c


def test_fp8_held_codes_kept_when_values_fit_and_reencoded_when_they_outgrow():
    B, H, hd = 3, 2, 64
    rng = np.random.default_rng(5)
    kc, vc, ks, vs, table = _empty_cache(B, H, hd, True, 64)
    lens = np.zeros(B, np.int32)
    first_k, first_v = _rows(rng, (B, 5, H, hd)), _rows(rng, (B, 5, H, hd))
    kc, vc, ks, vs, lens = oracle_kv_append(first_k, first_v, kc, vc, ks, vs, table, lens, True)
    kc1, ks1 = kc.copy(), ks.copy()
    # smaller values: codes of slots 0..4 and the scale stay
    small_k, small_v = _rows(rng, (B, 4, H, hd), 0.25), _rows(rng, (B, 4, H, hd), 0.25)
    kc2, vc2, ks2, vs2, lens2 = oracle_kv_append(small_k, small_v, kc, vc, ks, vs, table, lens, True)
    for b in range(B):
        blk = table[b][0]
        np.testing.assert_array_equal(kc2[blk][:, :, :5, :], kc1[blk][:, :, :5, :])
        np.testing.assert_array_equal(ks2[blk], ks1[blk])
    # larger values: scale = amax_new / 448, held values re-encoded within two roundings
    big_k, big_v = _rows(rng, (B, 4, H, hd), 8.0), _rows(rng, (B, 4, H, hd), 8.0)
    kc3, vc3, ks3, vs3, _ = oracle_kv_append(big_k, big_v, kc, vc, ks, vs, table, lens, True)
    for b in range(B):
        blk = table[b][0]
        for h in range(H):
            amax = np.float32(np.abs(bf16_bits_to_f64(big_k[b, :, h])).max())
            assert ks3[blk, h] == np.float32(amax / np.float32(448.0))
            x0 = bf16_bits_to_f64(first_k[b, :, h])
            dec, codes = _decoded_block(kc3, ks3, blk, h, slice(0, 5))
            bound = (_half_step(x0 / ks1[blk, h]) * ks1[blk, h]
                     + _half_step(x0 / ks3[blk, h]) * ks3[blk, h]) * (1 + 1e-6)
            assert (np.abs(dec - x0) <= bound).all()
            _, filled = _decoded_block(kc3, ks3, blk, h, slice(0, 9))
            assert (filled & 0x7F).max() == 0x7E


def test_fp8_append_chain_keeps_amax_rule_and_rounding_bound():
    """Random append sizes from an empty cache: every filled (block, KV head) holds
    448 as its largest code magnitude (its largest value encodes to 448, the
    amax/448 rule), and the last-appended values decode within one rounding."""
    B, H, hd = 3, 2, 64
    rng = np.random.default_rng(9)
    kc, vc, ks, vs, table = _empty_cache(B, H, hd, True, 200)
    lens = np.zeros(B, np.int32)
    for step in range(12):
        R = int(rng.integers(1, 17))
        if int(lens.max()) + R > 200:
            break
        gain = float(rng.choice([0.1, 1.0, 3.0, 30.0]))
        k, v = _rows(rng, (B, R, H, hd), gain), _rows(rng, (B, R, H, hd), gain)
        c0 = lens.copy()
        kc, vc, ks, vs, lens = oracle_kv_append(k, v, kc, vc, ks, vs, table, lens, True)
        for b in range(B):
            for h in range(H):
                for cache, scale, rows in ((kc, ks, k), (vc, vs, v)):
                    for t in range(R):
                        pos = int(c0[b]) + t
                        blk, slot = table[b][pos // BLOCK], pos % BLOCK
                        dec, _ = _decoded_block(cache, scale, blk, h, slice(slot, slot + 1))
                        x = bf16_bits_to_f64(rows[b, t, h])
                        y = (x.astype(np.float32) / scale[blk, h]).astype(np.float64)
                        assert (np.abs(dec[0] / scale[blk, h] - y) <= _half_step(y)).all()
        for b in range(B):
            for j in range(-(-int(lens[b]) // BLOCK)):
                n = min(BLOCK, int(lens[b]) - j * BLOCK)
                for h in range(H):
                    for cache, scale in ((kc, ks), (vc, vs)):
                        _, codes = _decoded_block(cache, scale, table[b][j], h, slice(0, n))
                        assert (codes & 0x7F).max() == 0x7E


def test_fp8_chunked_equals_one_shot_when_first_chunk_holds_the_max():
    B, H, hd = 2, 2, 128
    rng = np.random.default_rng(3)
    k = rng.standard_normal((B, 16, H, hd), dtype=np.float32)
    k[:, 0] *= 10.0                                   # the max sits in the first chunk
    v = rng.standard_normal((B, 16, H, hd), dtype=np.float32)
    v[:, 2] *= 10.0
    k, v = f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    st = _empty_cache(B, H, hd, True, 32)
    table = st[4]
    one = oracle_kv_append(k, v, *st[:4], table, np.zeros(B, np.int32), True)
    part = oracle_kv_append(k[:, :6], v[:, :6], *st[:4], table, np.zeros(B, np.int32), True)
    part = oracle_kv_append(k[:, 6:], v[:, 6:], *part[:4], table, part[4], True)
    for a, b in zip(one, part):
        np.testing.assert_array_equal(a, b)


def test_rollback_by_length_then_append_overwrites_rejected_rows():
    """Append R rows, accept AL of them (the greedy oracle commits the length),
    append the next R rows: the visible cache is the held tokens + the AL
    accepted rows + the new rows (bf16, exactly)."""
    B, H, hd, D = 3, 2, 64, 7
    R = D + 1
    rng = np.random.default_rng(4)
    kc, vc, _, _, table = _empty_cache(B, H, hd, False, 128)
    committed = np.array([37, 16, 5], np.int32)        # held slots hold poison
    k1, v1 = _rows(rng, (B, R, H, hd)), _rows(rng, (B, R, H, hd))
    kc1, vc1, _, _, lens = oracle_kv_append(k1, v1, kc, vc, None, None, table, committed, False)
    logits = rng.standard_normal((B, R, 50)).astype(np.float32)
    target = logits.argmax(-1)
    draft = target[:, :D].copy()
    draft[0, 2] = (draft[0, 2] + 1) % 50               # sequence 0 rejects draft 2
    draft[1, 0] = (draft[1, 0] + 1) % 50               # sequence 1 rejects draft 0
    acc = oracle_accept(logits, draft.astype(np.int32), lens, D)
    kept = acc["kv_lens_out"]
    np.testing.assert_array_equal(kept - committed, acc["accept_len"])
    np.testing.assert_array_equal(acc["accept_len"], [3, 1, R])
    k2, v2 = _rows(rng, (B, R, H, hd)), _rows(rng, (B, R, H, hd))
    kc2, vc2, _, _, lens2 = oracle_kv_append(k2, v2, kc1, vc1, None, None, table, kept, False)
    np.testing.assert_array_equal(lens2, kept + R)
    for b in range(B):
        c, al = int(committed[b]), int(acc["accept_len"][b])
        K, V = gather_kv(kc2, vc2, None, None, table, b, int(lens2[b]))
        np.testing.assert_array_equal(K[c: c + al], bf16_bits_to_f64(k1[b, :al]))
        np.testing.assert_array_equal(V[c: c + al], bf16_bits_to_f64(v1[b, :al]))
        np.testing.assert_array_equal(K[c + al:], bf16_bits_to_f64(k2[b]))
        np.testing.assert_array_equal(V[c + al:], bf16_bits_to_f64(v2[b]))


def _tree_step(fp8, seed=21):
    """An append of a random tree's 16 node rows after ragged contexts, then the
    greedy tree acceptance of the oracle: returns everything the commit needs."""
    from oracle.accept import oracle_argmax
    from oracle.tree import oracle_accept_tree
    from workloads import make_tree_plan, tree_tokens_from_target
    w = MINI["mini_gqa8_d15"].replace(B=3, V=30)
    B, R, H, hd = w.B, w.R, 2, 64
    rng = np.random.default_rng(seed)
    kc, vc, ks, vs, table = _empty_cache(B, H, hd, fp8, 160, seed=seed)
    # held context: one whole block each, then lengths 16, 5, 13 (valid codes)
    ctx = [_rows(rng, (B, 16, H, hd)) for _ in range(2)]
    kc, vc, ks, vs, _ = oracle_kv_append(*ctx, kc, vc, ks, vs, table, np.zeros(B, np.int32), fp8)
    T = np.array([16, 5, 13], np.int32)
    k_new, v_new = _rows(rng, (B, R, H, hd), 2.0), _rows(rng, (B, R, H, hd), 2.0)
    kc, vc, ks, vs, L = oracle_kv_append(k_new, v_new, kc, vc, ks, vs, table, T, fp8)
    logits = rng.standard_normal((B, R, w.V)).astype(np.float32)
    tp = make_tree_plan(w, shape="random", width=3, p_match=0.9)
    tok = tree_tokens_from_target(tp, oracle_argmax(logits))
    acc = oracle_accept_tree(logits, tok, tp.parents, L)
    return dict(k_new=k_new, v_new=v_new, kc=kc, vc=vc, ks=ks, vs=vs, table=table, T=T, acc=acc)


def test_tree_commit_moves_accepted_rows_behind_the_root_bf16():
    st = _tree_step(False)
    acc = st["acc"]
    assert acc["accept_len"].max() > 2
    kc, vc, _, _, lens = oracle_kv_append(st["k_new"], st["v_new"], st["kc"], st["vc"], None,
                                          None, st["table"], acc["kv_lens_out"], False,
                                          accept_path=acc["accept_path"])
    np.testing.assert_array_equal(lens, acc["kv_lens_out"])
    for b in range(3):
        AL, T = int(acc["accept_len"][b]), int(st["T"][b])
        assert lens[b] == T + AL
        path = acc["accept_path"][b, :AL]
        K, V = gather_kv(kc, vc, None, None, st["table"], b, int(lens[b]))
        np.testing.assert_array_equal(K[T:], bf16_bits_to_f64(st["k_new"][b, path]))
        np.testing.assert_array_equal(V[T:], bf16_bits_to_f64(st["v_new"][b, path]))
        K0, _ = gather_kv(st["kc"], st["vc"], None, None, st["table"], b, T)
        np.testing.assert_array_equal(K[:T], K0)


def test_tree_commit_of_a_chain_leaves_a_bf16_cache_unchanged():
    st = _tree_step(False)
    AL = np.array([16, 3, 1], np.int32)
    path = np.full((3, 16), -1, np.int32)
    for b in range(3):
        path[b, :AL[b]] = np.arange(AL[b])
    kv = st["T"] + AL
    kc, vc, _, _, lens = oracle_kv_append(st["k_new"], st["v_new"], st["kc"], st["vc"], None,
                                          None, st["table"], kv, False, accept_path=path)
    np.testing.assert_array_equal(kc, st["kc"])
    np.testing.assert_array_equal(vc, st["vc"])
    np.testing.assert_array_equal(lens, kv)


def test_tree_commit_e4m3_rounding_and_amax_rule():
    st = _tree_step(True)
    acc = st["acc"]
    kc, vc, ks, vs, lens = oracle_kv_append(st["k_new"], st["v_new"], st["kc"], st["vc"],
                                            st["ks"], st["vs"], st["table"], acc["kv_lens_out"],
                                            True, accept_path=acc["accept_path"])
    for b in range(3):
        AL, T = int(acc["accept_len"][b]), int(st["T"][b])
        for k, node in enumerate(acc["accept_path"][b, 1:AL], start=1):
            pos = T + k
            blk, slot = st["table"][b][pos // BLOCK], pos % BLOCK
            for cache, scale, rows in ((kc, ks, st["k_new"]), (vc, vs, st["v_new"])):
                for h in range(2):
                    dec, _ = _decoded_block(cache, scale, blk, h, slice(slot, slot + 1))
                    x = bf16_bits_to_f64(rows[b, node, h])
                    y = (x.astype(np.float32) / scale[blk, h]).astype(np.float64)
                    assert (np.abs(dec[0] / scale[blk, h] - y) <= _half_step(y)).all()
        # a block whose scale the commit recomputed holds 448 as its largest code;
        # one that kept its scale may not (a rejected row may have set it)
        for j in range((T + 1) // BLOCK, (T + AL - 1) // BLOCK + 1) if AL > 1 else []:
            n = min(BLOCK, int(lens[b]) - j * BLOCK)
            blk = st["table"][b][j]
            for h in range(2):
                for cache, scale, before in ((kc, ks, st["ks"]), (vc, vs, st["vs"])):
                    if scale[blk, h] == before[blk, h]:
                        continue
                    _, codes = _decoded_block(cache, scale, blk, h, slice(0, n))
                    assert (codes & 0x7F).max() == 0x7E
