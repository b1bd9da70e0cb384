"""Helpers for the GPU tests: upload seeded inputs, call the library through the
binding (C ABI), bring results back as numpy."""
import sys

import numpy as np
import torch

import speculative_decoding_verification_15_amd as sv

from speculative_decoding_verification_15_amd.device import BF16_NAN, DeviceAttn, attn_params, dev  # noqa: F401


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_attention(inp, split_tokens=0):
    note(f"[gpu] spec_verify_attn {inp.w.name} split_tokens={split_tokens}")
    d = DeviceAttn(inp)
    return DeviceAttn.to_f64(d.run(split_tokens))


def run_accept(logits, draft, kv_in, inplace=False, stream=None):
    B, R, V = logits.shape
    D = R - 1
    lg = dev(logits.astype(np.float32))
    dr = dev(draft.astype(np.int32)) if D > 0 else None
    target = torch.full((B, R), -7, dtype=torch.int32, device="cuda")
    al = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, R), -7, dtype=torch.int32, device="cuda")
    kin = dev(np.asarray(kv_in, np.int32))
    kout = kin if inplace else torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ws_bytes = sv.spec_accept_workspace_size(B, D, V)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    note(f"[gpu] spec_accept B={B} D={D} V={V}")
    sv.spec_accept(B, D, V, lg, dr, target, al, out, kin, kout, ws, ws_bytes, stream=stream)
    torch.cuda.synchronize()
    return dict(target=target.cpu().numpy(), accept_len=al.cpu().numpy(),
                out_tokens=out.cpu().numpy(), kv_lens_out=kout.cpu().numpy())


def attn_errors(gpu, ref):
    """max-abs, mean-abs and relative L2 error over the finite reference entries."""
    sel = np.isfinite(ref)
    d = np.abs(gpu[sel] - ref[sel])
    rel = np.sqrt((d ** 2).sum() / max((ref[sel] ** 2).sum(), 1e-300))
    return float(d.max()), float(d.mean()), float(rel)


MAX_ABS_TOL = 1e-2
MEAN_ABS_TOL = 1e-3
