"""KV append with e4m3 quantize-on-write (oracle; TEST INFRASTRUCTURE ONLY).

Nothing in the product path may import or call this module: only the tests, the
smoke check and the benchmark's CPU-baseline leg do.

The step before verification attention: the K and V rows of the R = 1 + D new
positions of every sequence are written into its paged cache at token
positions kv_lens[b] .. kv_lens[b] + R - 1, and the length grows by R.
  - 16-token blocks behind a block table, a block taken as it is needed:
    "GPU and LLM" ch. 5 (animemo.app), section "PagedAttention (2)".
  - KV data stored as FP8 for long inputs, with scaling factors, and the
    KV cache updated dynamically: novita.ai blog "Revolutionizing LLM
    inference ...", sections "Proprietary FP8 quantization scheme",
    "KVCache quantization" and "Inference process optimization".
  - Rejected drafts are undone by the length alone: the acceptance step
    commits kv_len' = kv_len - (1 + D) + AL, and the next append writes over
    the slots past it.

Readings taken where the pages are silent (the same in the library):
  A1  e4m3 scale per (physical block, KV head) = amax / 448 of the block's
      filled values (1 when amax is 0); K and V separately.
  A2  A block that already holds tokens keeps its scale and its codes when the
      appended values fit under the block's current largest value,
      fp32(max|decode(code)| * scale); otherwise the scale becomes
      amax_new / 448 and the held codes are re-encoded from their fp32 values
      fp32(decode(code) * old_scale).  A block that starts in this append
      takes amax / 448 of its new values.
  A3  Encoding: fp32 quotient x / scale (IEEE division), then the nearest e4m3
      value, ties to the even code, magnitudes above 448 saturated to 448; the
      sign bit is the sign of the quotient (so -0 and negative values that
      round to zero give 0x80).
  A4  Slots other than the written ones, and the scales of blocks not written,
      keep their bytes.

Layouts (as the C header states them):
  k_cache bf16 [num_blocks][H_kv][hd/8][16][8], e4m3 [num_blocks][H_kv][hd/16][16][16]
  v_cache      [num_blocks][H_kv][hd][16]
  k_scale, v_scale [num_blocks][H_kv] fp32
  k_new, v_new [B][R][H_kv][hd] bf16 bits
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, e4m3_bits_to_f64

BLOCK = 16
E4M3_MAX = 448.0


def _e4m3_grid():
    """The 127 non-negative finite e4m3 values, ascending, and their codes."""
    codes = np.arange(0, 127, dtype=np.uint8)      # 0x00 .. 0x7E (0x7F is NaN)
    vals = e4m3_bits_to_f64(codes)
    assert np.all(np.diff(vals) > 0)
    return vals, codes


def e4m3_encode_f32(y) -> np.ndarray:
    """fp32 values -> e4m3 codes by reading A3: nearest grid value, ties to the even
    code (the code's lowest bit is the mantissa's), saturation at 448, sign bit
    copied from y.  Written as a search over the decoded grid, so it depends only
    on the decoder's definition of each code."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64)).ravel()
    vals, codes = _e4m3_grid()
    a = np.minimum(a, E4M3_MAX)
    hi = np.searchsorted(vals, a, side="left")         # first grid value >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = vals[hi] - a                                # exact in fp64 (see below)
    d_lo = a - vals[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    mag = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    sign = np.signbit(y.ravel()).astype(np.uint8) << np.uint8(7)
    return (mag | sign).reshape(y.shape)
# The differences above are exact: a is an fp32 value (24 significant bits) and
# its neighbours on the grid lie within a factor 2 of it or are 0, so a - g fits
# in well under 53 bits.


def _block_scale(amax: np.float32) -> np.float32:
    """Reading A1: amax / 448 in fp32, 1 for an all-zero block."""
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(E4M3_MAX))


def oracle_kv_append(k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table, kv_lens,
                     fp8: bool, accept_path=None):
    """Append the R new K/V rows of every sequence; returns new arrays
    (k_cache, v_cache, k_scale, v_scale, kv_lens_out).  Inputs are not modified.

    k_new, v_new  [B][R][H_kv][hd] uint16 bf16 bits
    kv_lens       [B] committed lengths before the append (c_b)

    With ``accept_path`` ([B][R], a tree acceptance's walked nodes, root first,
    -1 padded): the tree commit.  kv_lens are then the committed lengths after
    the acceptance; the rows of the accepted nodes after the root, in path
    order, are appended by the same rule at kv_lens[b] - (AL - 1), right behind
    the root, and the lengths are returned unchanged (reading T4).
    """
    k_new = np.asarray(k_new, dtype=np.uint16)
    v_new = np.asarray(v_new, dtype=np.uint16)
    B, R, H_kv, hd = k_new.shape
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    ks = None if k_scale is None else np.array(k_scale, dtype=np.float32, copy=True)
    vs = None if v_scale is None else np.array(v_scale, dtype=np.float32, copy=True)
    X = 16 if fp8 else 8                                # elements per 16-byte K vector
    lens = np.asarray(kv_lens, dtype=np.int64)

    d = np.arange(hd)

    def k_at(blk, h, slots):
        """Index of K elements (slot, dim) of (blk, h): [n][hd]."""
        t = np.asarray(slots)[:, None]
        return (blk, h, (d // X)[None, :], t, (d % X)[None, :])

    def v_at(blk, h, slots):
        t = np.asarray(slots)[:, None]
        return (blk, h, d[None, :], t)

    def append_seq(b, krows, vrows, c):
        """Rows krows/vrows [n][H_kv][hd] (bf16 bits) of sequence b at positions c .. c+n-1."""
        n = krows.shape[0]
        if n == 0:
            return
        if not fp8:
            for i in range(n):
                pos = c + i
                blk = int(block_table[b][pos // BLOCK])
                slot = pos % BLOCK
                for h in range(H_kv):
                    kc[k_at(blk, h, [slot])] = krows[i, h, :][None, :]
                    vc[v_at(blk, h, [slot])] = vrows[i, h, :][None, :]
            return
        # e4m3: per touched block and KV head, for K and V independently
        first_blk, last_blk = c // BLOCK, (c + n - 1) // BLOCK
        for j in range(first_blk, last_blk + 1):
            blk = int(block_table[b][j])
            start = j * BLOCK
            a = max(c - start, 0)                       # held slots 0 .. a-1
            lo, hi = max(c, start), min(c + n, start + BLOCK)
            for h in range(H_kv):
                for rows, cache, scale, at in ((krows, kc, ks, k_at), (vrows, vc, vs, v_at)):
                    x = bf16_bits_to_f64(rows[lo - c: hi - c, h, :]).astype(np.float32)
                    amax_new = np.float32(np.abs(x).max()) if x.size else np.float32(0)
                    if a == 0:
                        s = _block_scale(amax_new)
                        regrow = False
                    else:
                        s_old = np.float32(scale[blk, h])
                        held = cache[at(blk, h, range(a))]            # [a][hd] codes
                        held_max = np.float32(np.abs(e4m3_bits_to_f64(held)).max())
                        a_held = np.float32(held_max * s_old)
                        if amax_new <= a_held:
                            s, regrow = s_old, False
                        else:
                            s, regrow = _block_scale(amax_new), True
                        if regrow:
                            xo = (e4m3_bits_to_f64(held).astype(np.float32) * s_old).astype(np.float32)
                            cache[at(blk, h, range(a))] = e4m3_encode_f32((xo / s).astype(np.float32))
                    cache[at(blk, h, range(lo - start, hi - start))] = \
                        e4m3_encode_f32((x / s).astype(np.float32))
                    scale[blk, h] = s

    if accept_path is None:
        for b in range(B):
            append_seq(b, k_new[b], v_new[b], int(lens[b]))
        return kc, vc, ks, vs, (lens + R).astype(np.int32)
    # tree commit: the accepted nodes after the root, right behind it
    path = np.asarray(accept_path, dtype=np.int64)
    for b in range(B):
        nodes = []
        for x in path[b, 1:]:
            if x < 0:
                break
            nodes.append(int(x))
        append_seq(b, k_new[b, nodes], v_new[b, nodes], int(lens[b]) - len(nodes))
    return kc, vc, ks, vs, lens.astype(np.int32)
