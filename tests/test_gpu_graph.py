"""The verification step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library allocates nothing and records no memset, so a serving loop can
capture spec_kv_append -> spec_verify_attn -> spec_accept once and replay it.
Each replay, with eager work and synchronisations between replays, must give
the eager step's outputs bit for bit (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import speculative_decoding_verification_15_amd as sv
from oracle.accept import oracle_argmax
from tests.gpu_util import DeviceAttn, attn_params, dev, note
from workloads import MINI, drafts_from_target, make_accept_plan, make_append_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["mini_gqa8_d15", "mini_fp8_d15"])
def test_step_in_a_graph_replays_like_eager(name):
    w = MINI[name]
    fp8 = w.kv_dtype == "fp8_e4m3"
    ap = make_append_inputs(w)
    b = ap.base
    plan = make_accept_plan(w)
    draft = drafts_from_target(plan, oracle_argmax(plan.logits))
    d = DeviceAttn(b)
    k0, v0 = d.k.clone(), d.v.clone()
    ks0 = d.ks.clone() if fp8 else None
    vs0 = d.vs.clone() if fp8 else None
    lens0 = dev(ap.committed)
    lens = lens0.clone()
    kn, vn = dev(ap.k_new), dev(ap.v_new)
    lg, dr = dev(plan.logits), dev(draft)
    B, R, V, D = w.B, w.R, w.V, w.D
    app = sv.make_append_params(batch=B, num_new=R, num_kv_heads=w.H_kv, head_dim=w.hd,
                                max_blocks_per_seq=b.block_table.shape[1], num_blocks=b.num_blocks,
                                kv_dtype=sv.SV_KV_FP8_E4M3 if fp8 else sv.SV_KV_BF16)
    p = attn_params(b)
    ws_bytes = sv.spec_verify_attn_workspace_size(p)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty(d.q.shape, dtype=torch.int16, device="cuda")
    tgt = torch.empty((B, R), dtype=torch.int32, device="cuda")
    al = torch.empty((B,), dtype=torch.int32, device="cuda")
    otok = torch.empty((B, R), dtype=torch.int32, device="cuda")
    aws_bytes = sv.spec_accept_workspace_size(B, D, V)
    aws = torch.empty(aws_bytes, dtype=torch.uint8, device="cuda")

    def reset():                      # eager: the cache and lengths before the step
        d.k.copy_(k0)
        d.v.copy_(v0)
        if fp8:
            d.ks.copy_(ks0)
            d.vs.copy_(vs0)
        lens.copy_(lens0)

    def step(stream):
        sv.spec_kv_append(app, kn, vn, d.k, d.v, d.ks, d.vs, d.bt, lens, lens, stream=stream)
        sv.spec_verify_attn(p, d.q, d.k, d.v, d.ks, d.vs, d.bt, lens, out, ws, ws_bytes,
                            stream=stream)
        sv.spec_accept(B, D, V, lg, dr, tgt, al, otok, lens, lens, aws, aws_bytes, stream=stream)

    def snapshot():
        torch.cuda.synchronize()
        return [t.cpu().numpy().copy() for t in (out, tgt, al, otok, lens, d.k, d.v)]

    note(f"[gpu] graph step {name}: eager")
    reset()
    step(None)
    want = snapshot()

    note(f"[gpu] graph step {name}: capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(4):
        reset()                        # eager work between replays
        out.fill_(-1)
        al.fill_(-1)
        torch.cuda.synchronize()
        note(f"[gpu] graph step {name}: replay {rep}")
        g.replay()
        got = snapshot()
        for i, (x, y) in enumerate(zip(got, want)):
            assert np.array_equal(x, y), (rep, i)
