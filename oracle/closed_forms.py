"""Closed forms the pages give for the verification step (oracle; test infrastructure).

  * Expected tokens per verification with k drafts each accepted independently
    with probability alpha: (1 - alpha^(k+1)) / (1 - alpha), capped at k + 1
    when alpha -> 1.  "GPU and LLM" ch. 5 (animemo.app), section "Speculative
    decoding (2): verify in one pass" (prints 1.9 / 2.8 / 4.1 at k = 4 for
    alpha = 0.5 / 0.7 / 0.9).
  * KV-cache size = 2 x layers x KV heads x head dim x context x bytes.
    "GPU and LLM" ch. 5, section "The KV-cache formula: which term to shrink",
    with the MHA / GQA / MQA figures in that section and the next two.
  * Score-table size T x T (the table FlashAttention never writes to HBM).
    "GPU and LLM" ch. 5, section "FlashAttention: do not write the T x T table".
  * Decode-attention arithmetic intensity about 2G flops per KV element,
    2G(1 + D) with speculative decoding, and the draft length 128/G - 1 that
    fills a 128-row tile.  NVIDIA co-design summary (papanda925.com), guidelines
    2 and 3.
"""
from __future__ import annotations


def expected_tokens(alpha: float, k: int) -> float:
    """E[tokens per verification] = sum_{j=0..k} alpha^j."""
    if alpha == 1.0:
        return float(k + 1)
    return (1.0 - alpha ** (k + 1)) / (1.0 - alpha)


def kv_elements_per_layer_token(H_kv: int, d: int) -> int:
    """K and V values stored per layer per token: 2 * H_kv * d."""
    return 2 * H_kv * d


def kv_cache_bytes(layers: int, H_kv: int, d: int, T: int, bytes_per_value: float) -> float:
    return 2 * layers * H_kv * d * T * bytes_per_value


def score_table_entries(T: int) -> int:
    return T * T


def attention_flops_per_key(M: int, hd: int) -> int:
    """Flops spent on one key of one KV head by M query rows: a length-hd dot
    product for each score (2*hd) and an hd-wide multiply-add into the output
    for each probability (2*hd)."""
    return 2 * M * hd + 2 * M * hd


def decode_intensity_flops_per_kv_element(G: int, D: int, hd: int = 128) -> float:
    """Flops per stored K/V element when M = G*(1+D) query rows read one key
    (2*hd elements: its K row and its V row)."""
    M = G * (1 + D)
    return attention_flops_per_key(M, hd) / (2 * hd)


def tile_filling_draft_len(G: int, tile_rows: int = 128) -> int:
    """Largest D with G*(1+D) <= tile_rows: tile_rows/G - 1 when G divides it."""
    return tile_rows // G - 1
