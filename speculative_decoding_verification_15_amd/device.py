"""Device-side plumbing for callers of the binding (the benchmark and the GPU
tests): host arrays to GPU tensors, the attention parameters of a generated
workload, and one workload's attention inputs resident in HBM.  Memory only:
every step of the verification path runs in the library's kernels."""
from __future__ import annotations

import numpy as np
import torch

from ._lib import SV_KV_BF16, SV_KV_FP8_E4M3, make_attn_params, spec_verify_attn, \
    spec_verify_attn_workspace_size

BF16_NAN = np.int16(0x7FC0)
KV_FP8 = "fp8_e4m3"


def dev(a):
    """A contiguous GPU copy of a host array (bf16 bit patterns as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def attn_params(inp, split_tokens=0):
    """sv_attn_params of a generated workload's attention inputs."""
    w = inp.w
    return make_attn_params(
        batch=w.B, draft_len=w.D, num_q_heads=w.H_q, num_kv_heads=w.H_kv, head_dim=w.hd,
        max_blocks_per_seq=inp.block_table.shape[1], num_blocks=inp.num_blocks,
        max_kv_len=inp.max_kv_len,
        kv_dtype=SV_KV_FP8_E4M3 if w.kv_dtype == KV_FP8 else SV_KV_BF16,
        sm_scale=w.sm_scale, split_tokens=split_tokens)


class DeviceAttn:
    """Inputs of one attention call resident on the GPU."""

    def __init__(self, inp):
        self.inp = inp
        self.q = dev(inp.q)
        self.k = dev(inp.k_cache)
        self.v = dev(inp.v_cache)
        self.ks = dev(inp.k_scale) if inp.k_scale is not None else None
        self.vs = dev(inp.v_scale) if inp.v_scale is not None else None
        self.bt = dev(inp.block_table)
        self.kl = dev(inp.kv_lens)

    def run(self, split_tokens=0, stream=None, out=None):
        p = attn_params(self.inp, split_tokens)
        ws_bytes = spec_verify_attn_workspace_size(p)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
        if out is None:
            out = torch.full(self.q.shape, int(BF16_NAN), dtype=torch.int16, device="cuda")
        spec_verify_attn(p, self.q, self.k, self.v, self.ks, self.vs, self.bt, self.kl, out,
                         ws, ws_bytes, stream=stream)
        torch.cuda.synchronize()
        return out

    @staticmethod
    def to_f64(out):
        return out.view(torch.bfloat16).to(torch.float64).cpu().numpy()
