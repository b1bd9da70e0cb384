"""spec_accept_noalloc (no workspace argument: the row keys and counters live in
the library's fixed device array) against spec_accept with a workspace, through
the C ABI, bit for bit: two calls in a row, the second with a smaller input,
then the first shape again, and a graph replay."""
import numpy as np
import pytest
import torch

import speculative_decoding_verification_15_amd as sv
from oracle.accept import oracle_accept
from tests.gpu_util import dev, note

pytestmark = pytest.mark.gpu


def _inputs(B, D, V, seed, ties=False):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((B, D + 1, V)).astype(np.float32)
    if ties:                                    # equal maxima across chunks, +0/-0, -inf rows
        logits[0, :, [min(5, V - 1), min(4096, V - 1)]] = 9.0
        if B > 1:
            logits[1, 0, :] = -np.inf
        if B > 2 and V > 2:
            logits[2, :, :] = -1.0
            logits[2, :, 1] = -0.0
            logits[2, :, V - 1] = 0.0
    target = np.argmax(logits, axis=-1)
    draft = np.where(rng.random((B, D)) < 0.7, target[:, :D],
                     rng.integers(0, V, size=(B, D))).astype(np.int32)
    kv_in = (np.arange(B, dtype=np.int32) * 3 + 50).astype(np.int32)
    return logits, draft, kv_in


def _outs(B, R):
    return {k: torch.full(s, -7, dtype=torch.int32, device="cuda") for k, s in
            (("target", (B, R)), ("accept_len", (B,)), ("out_tokens", (B, R)),
             ("kv_lens_out", (B,)))}


def _both(B, D, V, seed, ties=False):
    logits, draft, kv_in = _inputs(B, D, V, seed, ties)
    lg, dr, kin = dev(logits), (dev(draft) if D else None), dev(kv_in)
    R = D + 1
    a, b = _outs(B, R), _outs(B, R)
    ws_bytes = sv.spec_accept_workspace_size(B, D, V)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    note(f"[gpu] spec_accept vs spec_accept_noalloc B={B} D={D} V={V}")
    sv.spec_accept(B, D, V, lg, dr, a["target"], a["accept_len"], a["out_tokens"], kin,
                   a["kv_lens_out"], ws, ws_bytes)
    sv.spec_accept_noalloc(B, D, V, lg, dr, b["target"], b["accept_len"], b["out_tokens"], kin,
                           b["kv_lens_out"])
    torch.cuda.synchronize()
    ref = oracle_accept(logits, draft, kv_in, D)
    for k in a:
        got_a, got_b = a[k].cpu().numpy(), b[k].cpu().numpy()
        assert np.array_equal(got_b, got_a), k
        assert np.array_equal(got_b, ref[k]), k


def test_no_alloc_matches_spec_accept_twice_then_smaller():
    _both(32, 15, 128256, 1)          # the 70B-like acceptance shape
    _both(3, 5, 4097, 2, ties=True)   # a smaller input on the same array
    _both(32, 15, 128256, 3)          # and the large one again
    _both(5, 0, 1, 4)                 # D = 0, V = 1


def test_no_alloc_inside_a_graph():
    B, D, V = 8, 7, 20000
    logits, draft, kv_in = _inputs(B, D, V, 9, ties=True)
    lg, dr, kin = dev(logits), dev(draft), dev(kv_in)
    o = _outs(B, D + 1)
    ref = oracle_accept(logits, draft, kv_in, D)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):            # the set-up (first call) happens outside capture
        sv.spec_accept_noalloc(B, D, V, lg, dr, o["target"], o["accept_len"], o["out_tokens"],
                               kin, o["kv_lens_out"], stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sv.spec_accept_noalloc(B, D, V, lg, dr, o["target"], o["accept_len"], o["out_tokens"],
                               kin, o["kv_lens_out"])
    for rep in range(4):
        for t in o.values():
            t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in o:
            assert np.array_equal(o[k].cpu().numpy(), ref[k]), (rep, k)
        _both(3, 2, 300, 20 + rep)        # eager work on the same array between replays
