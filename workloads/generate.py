"""Seeded synthetic inputs for the verification step.

This module only makes inputs: random draws, their encoding into the storage
formats the kernels read (bf16 by round-to-nearest-even, OCP e4m3 through
PyTorch's float8 conversion), and their placement into the paged KV cache.  It
holds none of the verification arithmetic (no attention, softmax, argmax or
acceptance); both the oracle and the GPU path consume the same host bytes it
produces.

Random streams: ``SeedSequence(seed).spawn(8)`` in the fixed order
lens, perm, q, k, v, logits, match, other-id.

Storage layouts written here (the C header documents the same layouts):
  q            [B][R][H_q][hd]                      bf16 bits (uint16)
  k_cache      [num_blocks][H_kv][hd/X][16][X]      X = 16 bytes / element size
  v_cache      [num_blocks][H_kv][hd][16]
  k_scale      [num_blocks][H_kv] fp32              (e4m3 caches only)
  v_scale      [num_blocks][H_kv] fp32
  block_table  [B][max_blocks_per_seq] int32, -1 where unused
  kv_lens      [B] int32, L_b = T_b + R
Slots past L_b in a sequence's last block, and blocks no sequence uses, hold
poison (NaN encodings) that must never reach an output.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from .configs import BLOCK_SIZE, KV_BF16, KV_FP8, Workload

BF16_POISON = np.uint16(0x7FC1)   # a quiet NaN
FP8_POISON = np.uint8(0x7F)       # e4m3 NaN
FP8_MAX = 448.0

STREAMS = ("lens", "perm", "q", "k", "v", "logits", "match", "other")


def seed_streams(seed: int) -> dict:
    ss = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: np.random.default_rng(s) for name, s in zip(STREAMS, ss)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Encode fp32 values as OCP e4m3 (round to nearest even, saturated to +-448)."""
    import torch

    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32), -FP8_MAX, FP8_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@dataclasses.dataclass
class AttnInputs:
    w: Workload
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    k_scale: Optional[np.ndarray]
    v_scale: Optional[np.ndarray]
    block_table: np.ndarray
    kv_lens: np.ndarray
    num_blocks: int
    max_kv_len: int

    @property
    def context_lens(self) -> np.ndarray:
        return self.kv_lens - self.w.R


@dataclasses.dataclass
class AcceptPlan:
    """Acceptance inputs: target logits plus the recipe for the draft tokens.

    Drafts depend on the target tokens, which the caller computes; see
    ``drafts_from_target``.
    """
    w: Workload
    logits: np.ndarray          # [B][R][V] fp32
    p_seq: np.ndarray           # [B] per-sequence match probability
    match: np.ndarray           # [B][D] bool
    other: np.ndarray           # [B][D] uniform draws in [0, V-2]


def context_lengths(w: Workload, rng) -> np.ndarray:
    if w.T is not None:
        return np.full(w.B, w.T, dtype=np.int64)
    lo, hi = w.T_range
    return rng.integers(lo, hi + 1, size=w.B, dtype=np.int64)


def kv_elem_bytes(w: Workload) -> int:
    return 1 if w.kv_dtype == KV_FP8 else 2


def make_attn_inputs(w: Workload, T_override: Optional[np.ndarray] = None) -> AttnInputs:
    """Draw Q, the KV cache, the block table and the lengths for workload ``w``."""
    rs = seed_streams(w.seed)
    T = context_lengths(w, rs["lens"])
    if T_override is not None:
        T = np.asarray(T_override, dtype=np.int64)
    L = T + w.R
    nblk = -(-L // BLOCK_SIZE)
    used = int(nblk.sum())
    num_blocks = used + w.spare_blocks
    perm = (np.arange(num_blocks) if w.identity_table
            else rs["perm"].permutation(num_blocks)).astype(np.int32)
    max_blocks = max(w.max_blocks_per_seq, int(nblk.max()))
    table = np.full((w.B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(w.B):
        table[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += int(nblk[b])

    q = f32_to_bf16_bits(rs["q"].standard_normal((w.B, w.R, w.H_q, w.hd), dtype=np.float32))

    fp8 = w.kv_dtype == KV_FP8
    X = 16 // kv_elem_bytes(w)
    cdt = np.uint8 if fp8 else np.uint16
    poison = FP8_POISON if fp8 else BF16_POISON
    k_cache = np.full((num_blocks, w.H_kv, w.hd // X, BLOCK_SIZE, X), poison, dtype=cdt)
    v_cache = np.full((num_blocks, w.H_kv, w.hd, BLOCK_SIZE), poison, dtype=cdt)
    k_scale = np.full((num_blocks, w.H_kv), np.nan, dtype=np.float32) if fp8 else None
    v_scale = np.full((num_blocks, w.H_kv), np.nan, dtype=np.float32) if fp8 else None

    for b in range(w.B):
        Lb, nb = int(L[b]), int(nblk[b])
        phys = table[b, :nb]
        for name, cache, scale in (("k", k_cache, k_scale), ("v", v_cache, v_scale)):
            x = rs[name].standard_normal((Lb, w.H_kv, w.hd), dtype=np.float32)
            xp = np.zeros((nb * BLOCK_SIZE, w.H_kv, w.hd), dtype=np.float32)
            xp[:Lb] = x
            xp = xp.reshape(nb, BLOCK_SIZE, w.H_kv, w.hd)
            if fp8:
                amax = np.abs(xp).max(axis=(1, 3))                      # [nb][H_kv]
                s = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0))
                s = s.astype(np.float32)
                scale[phys] = s
                codes = f32_to_e4m3_bits(xp / s[:, None, :, None])
            else:
                codes = f32_to_bf16_bits(xp)
            # slots past L_b keep their poison
            valid = np.zeros((nb * BLOCK_SIZE,), dtype=bool)
            valid[:Lb] = True
            valid = valid.reshape(nb, BLOCK_SIZE)
            codes = np.where(valid[:, :, None, None], codes, poison)
            if name == "k":
                # [nb][16][H_kv][hd] -> [nb][H_kv][hd/X][16][X]
                c = codes.reshape(nb, BLOCK_SIZE, w.H_kv, w.hd // X, X).transpose(0, 2, 3, 1, 4)
            else:
                # [nb][16][H_kv][hd] -> [nb][H_kv][hd][16]
                c = codes.transpose(0, 2, 3, 1)
            cache[phys] = c

    return AttnInputs(w=w, q=q, k_cache=k_cache, v_cache=v_cache, k_scale=k_scale,
                      v_scale=v_scale, block_table=table, kv_lens=L.astype(np.int32),
                      num_blocks=num_blocks, max_kv_len=max(w.max_kv_len, int(L.max())))


def make_accept_plan(w: Workload, n_logit_sets: int = 1):
    """Target logits (N(0,1) fp32) and the draft recipe for workload ``w``.

    With ``n_logit_sets > 1`` the logits stream keeps drawing further sets of the
    same shape (used to rotate buffers when timing); the first set is identical
    either way.
    """
    rs = seed_streams(w.seed)
    sets = [rs["logits"].standard_normal((w.B, w.R, w.V), dtype=np.float32)
            for _ in range(n_logit_sets)]
    if w.p_range is not None:
        p = rs["match"].uniform(w.p_range[0], w.p_range[1], size=w.B)
    else:
        p = np.full(w.B, w.p_match, dtype=np.float64)
    match = rs["match"].random((w.B, w.D)) < p[:, None]
    other = rs["other"].integers(0, max(w.V - 1, 1), size=(w.B, w.D), dtype=np.int64)
    plan = AcceptPlan(w=w, logits=sets[0], p_seq=p, match=match, other=other)
    return (plan, sets) if n_logit_sets > 1 else plan


def drafts_from_target(plan: AcceptPlan, target: np.ndarray) -> np.ndarray:
    """Draft j of sequence b equals the target token of row j with the planned
    probability, otherwise a uniformly drawn different id (r + (r >= target))."""
    t = np.asarray(target, dtype=np.int64)[:, : plan.w.D]
    r = plan.other
    d = np.where(plan.match, t, r + (r >= t))
    return d.astype(np.int32)


@dataclasses.dataclass
class SampledAcceptInputs:
    w: Workload
    target_logits: np.ndarray   # [B][R][V] fp32
    draft_logits: np.ndarray    # [B][D][V] fp32
    draft: np.ndarray           # [B][D] int32, drawn from softmax(draft_logits / tau)
    u_accept: np.ndarray        # [B][D] fp32 in [0, 1)
    u_sample: np.ndarray        # [B] fp32 in [0, 1)
    tau: float


def _uniform01_f32(rng, shape):
    u = rng.random(shape).astype(np.float32)
    return np.minimum(u, np.float32(np.nextafter(np.float32(1), np.float32(0))))


def make_sampled_accept_inputs(w: Workload, tau: float = 1.0, noise: float = 0.5) -> SampledAcceptInputs:
    """Inputs of stochastic acceptance: target logits N(0,1); a draft model whose
    logits are the target's plus N(0, noise^2); drafts drawn from the draft
    model's distribution at temperature tau by the Gumbel-max trick (the index of
    the largest y / tau + g with g standard Gumbel, which is a draw from
    softmax(y / tau) without computing it); uniforms in [0, 1) for the tests and
    the emitted token.  Streams: SeedSequence([seed, 2]).spawn(5)."""
    ss = np.random.SeedSequence([w.seed, 2]).spawn(5)
    rz, ry, rg, ru, rs = (np.random.default_rng(s) for s in ss)
    z = rz.standard_normal((w.B, w.R, w.V), dtype=np.float32)
    y = (z[:, : w.D] + np.float32(noise) * ry.standard_normal((w.B, w.D, w.V), dtype=np.float32))
    y = np.ascontiguousarray(y, dtype=np.float32)
    draft = np.empty((w.B, w.D), dtype=np.int32)
    for b in range(w.B):               # per sequence, to bound the temporary
        g = rg.gumbel(size=(w.D, w.V))
        draft[b] = np.argmax(y[b].astype(np.float64) / tau + g, axis=-1)
    return SampledAcceptInputs(w=w, target_logits=z, draft_logits=y, draft=draft,
                               u_accept=_uniform01_f32(ru, (w.B, w.D)),
                               u_sample=_uniform01_f32(rs, (w.B,)), tau=float(tau))



@dataclasses.dataclass
class AppendInputs:
    """A paged cache holding each sequence's committed tokens, and the K/V rows of
    its R new positions to append."""
    base: AttnInputs            # cache, scales and block table (room for c_b + R tokens)
    committed: np.ndarray       # [B] int32: c_b, tokens held before the append
    k_new: np.ndarray           # [B][R][H_kv][hd] bf16 bits
    v_new: np.ndarray


def make_append_inputs(w: Workload, gains=(1.0,), base: Optional[AttnInputs] = None) -> AppendInputs:
    """The cache of ``make_attn_inputs(w)`` with its committed length set to the
    context T_b (the R positions after it are overwritten by the append), and new
    K/V rows N(0,1) * g, g drawn per (sequence, KV head) from ``gains`` (gains
    above 1 make appended values outgrow a block's e4m3 scale).
    Streams: SeedSequence([seed, 3]).spawn(3) in the order k, v, gain.  ``base``:
    the already drawn ``make_attn_inputs(w)``, to avoid drawing it again."""
    base = make_attn_inputs(w) if base is None else base
    ss = np.random.SeedSequence([w.seed, 3]).spawn(3)
    rk, rv, rg = (np.random.default_rng(s) for s in ss)
    g = np.asarray(gains, dtype=np.float32)[rg.integers(0, len(gains), size=(w.B, 1, w.H_kv, 1))]
    k = rk.standard_normal((w.B, w.R, w.H_kv, w.hd), dtype=np.float32) * g
    v = rv.standard_normal((w.B, w.R, w.H_kv, w.hd), dtype=np.float32) * g
    return AppendInputs(base=base, committed=(base.kv_lens - w.R).astype(np.int32),
                        k_new=f32_to_bf16_bits(k), v_new=f32_to_bf16_bits(v))


def make_draft_logits(rows: int, V: int, seed: int, sharp=(0.3, 8.0)) -> np.ndarray:
    """Draft-model logits [rows][V] fp32: N(0,1) times a per-row sharpness drawn
    log-uniformly from ``sharp`` (so the rows' confidences span flat to peaked
    distributions).  Streams: SeedSequence([seed, 4]).spawn(2) (logits, sharpness)."""
    ss = np.random.SeedSequence([seed, 4]).spawn(2)
    rz, rs = (np.random.default_rng(s) for s in ss)
    z = rz.standard_normal((rows, V), dtype=np.float32)
    s = np.exp(rs.uniform(np.log(sharp[0]), np.log(sharp[1]), size=(rows, 1))).astype(np.float32)
    return np.ascontiguousarray(z * s, dtype=np.float32)


@dataclasses.dataclass
class TreePlan:
    """A draft tree per sequence over the R new positions (node 0 = the root, the
    last committed token; parents[b][j] < j), its ancestor masks in the layout
    the tree attention reads, and the recipe for the node tokens."""
    w: Workload
    parents: np.ndarray         # [B][R] int32, parents[:, 0] = -1
    masks: np.ndarray           # [B][R] uint64: bit j of masks[b][i] = j is i or an ancestor
    match: np.ndarray           # [B][R] bool: node j carries its parent's target token
    other: np.ndarray           # [B][R] uniform draws in [0, V-2]


def make_tree_plan(w: Workload, shape: str = "random", width: int = 3,
                   p_match: float = 0.6) -> TreePlan:
    """Trees of R = 1 + D nodes: "random" (each node's parent drawn uniformly from
    the ``width`` nodes before it), "chain" (parent j - 1), "star" (parent 0).
    Streams: SeedSequence([seed, 5]).spawn(3) in the order parent, match, other."""
    ss = np.random.SeedSequence([w.seed, 5]).spawn(3)
    rp, rm, ro = (np.random.default_rng(s) for s in ss)
    B, R = w.B, w.R
    parents = np.full((B, R), -1, dtype=np.int32)
    for j in range(1, R):
        if shape == "chain":
            parents[:, j] = j - 1
        elif shape == "star":
            parents[:, j] = 0
        else:
            parents[:, j] = rp.integers(max(0, j - width), j, size=B)
    masks = np.zeros((B, R), dtype=np.uint64)
    for b in range(B):
        for i in range(R):
            m = np.uint64(1) << np.uint64(i)
            if i > 0:
                m |= masks[b, parents[b, i]]
            masks[b, i] = m
    match = rm.random((B, R)) < p_match
    other = ro.integers(0, max(w.V - 1, 1), size=(B, R), dtype=np.int64)
    return TreePlan(w=w, parents=parents, masks=masks, match=match, other=other)


def tree_tokens_from_target(plan: TreePlan, target: np.ndarray) -> np.ndarray:
    """Node j's token is its parent's target token with the planned probability,
    otherwise another uniformly drawn id; entry 0 (the root) is 0."""
    t = np.asarray(target, dtype=np.int64)
    B, R = plan.parents.shape
    tok = np.zeros((B, R), dtype=np.int32)
    for j in range(1, R):
        pt = t[np.arange(B), plan.parents[:, j]]
        r = plan.other[:, j]
        tok[:, j] = np.where(plan.match[:, j], pt, r + (r >= pt))
    return tok


def split_path_lengths(B, seed, long_every=64):
    """Contexts for the many-sequence split path: mostly short (32 to 200
    tokens), every ``long_every``-th sequence long (1000 to 2000 tokens), so
    that 256-token splits cut the long ones into up to eight pieces."""
    rng = np.random.default_rng(seed)
    T = rng.integers(32, 201, B)
    T[::long_every] = rng.integers(1000, 2001, len(T[::long_every]))
    return T
