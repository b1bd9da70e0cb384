"""Benchmark of the verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--split-tokens S] [--no-cpu-baseline]
    python bench.py --tile-sweep       (spec_verify_attn alone on the 14
                                        tile-boundary shapes)

One step = one full pass of the hot path over one batch: spec_verify_attn
(paged GQA attention of the 1 + D verified positions, split-K merge) followed
by spec_accept (vocab argmax, first-mismatch prefix, KV-length commit), both
through the C ABI on the same stream, with all inputs already in HBM.

Printed: one JSON line with the metric (verified tokens/s = sum of acceptance
lengths per step / step time), the attention kernel's achieved HBM bandwidth
against the MI355X peak (the roofline object), the MFMA rate, and the oracle's
throughput on a bounded sample on the host cores (the cpu_baseline object).
The default workload is the 70B-like layer: B=32, H_q=64, H_kv=8, hd=128,
D=15 (G*(1+D) = 128), ragged context T ~ U[2048, 32768], bf16 paged KV,
acceptance over fp32 logits [32, 16, 128256].
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
LEG_WARMUP = 100         # untimed calls before each side measurement
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP8_MFMA_PEAK_TFLOPS = 5000.0
METRIC = "verified tokens/sec + KV HBM GB/s (% peak) at Llama-70B-like GQA, D=15"
KERNEL_SOURCES = ("speculative_decoding_verification_15_amd/csrc/sv_attn.hip",
                  "speculative_decoding_verification_15_amd/csrc/sv_device.h",
                  "speculative_decoding_verification_15_amd/csrc/sv_attn_plan.h",
                  "speculative_decoding_verification_15_amd/csrc/sv_plan.cpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_sv_attn.md")


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence.

    Its record skips the system-scope cache write-back a default event makes:
    the default event torch creates adds ~3 us of stream time per record between
    two kernels here, ~1.5 us with this flag.  The runtime is the libamdhip64
    torch has already loaded (the library's own soname), so the stream handles
    are the ones torch and the library use.  Same calls as torch.cuda.Event.
    """
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                    ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        self._h = ctypes.c_void_p()
        self._check(self._hip.hipEventCreateWithFlags(ctypes.byref(self._h),
                                                      self.DISABLE_SYSTEM_FENCE), "create")

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"hipEvent{what} failed with hipError {rc}")

    def record(self, stream):
        import ctypes
        self._check(self._hip.hipEventRecord(self._h, ctypes.c_void_p(stream.cuda_stream)),
                    "Record")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        import ctypes
        ms = ctypes.c_float()
        self._check(self._hip.hipEventElapsedTime(ctypes.byref(ms), self._h, end._h),
                    "ElapsedTime")
        return ms.value

    def __del__(self):
        if self._hip is not None and self._h:
            self._hip.hipEventDestroy(self._h)


def kernel_source_hash() -> str:
    """Hash of the attention kernels' code (comments and blank space dropped,
    so that a comment edit does not orphan the counter summaries keyed to it)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        src = open(os.path.join(ROOT, p)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def attn_algorithmic_bytes(inp) -> int:
    """Bytes the attention must move at least once: every K and V element of the
    L_b keys of each sequence, the fp8 scales of the blocks read, the block-table
    entries, Q and the output."""
    w = inp.w
    L = inp.kv_lens.astype(np.int64)
    elem = 1 if w.kv_dtype == "fp8_e4m3" else 2
    kv = int(L.sum()) * w.H_kv * w.hd * 2 * elem
    nblk = int(((L + 15) // 16).sum())
    scales = nblk * w.H_kv * 2 * 4 if elem == 1 else 0
    table = nblk * 4
    qo = 2 * w.B * w.R * w.H_q * w.hd * 2
    return kv + scales + table + qo


def attn_algorithmic_kv_bytes(inp) -> int:
    w = inp.w
    elem = 1 if w.kv_dtype == "fp8_e4m3" else 2
    return int(inp.kv_lens.astype(np.int64).sum()) * w.H_kv * w.hd * 2 * elem


def attn_algorithmic_flops(inp) -> int:
    """4 * M * hd flops per (visible key, KV head): QK^T and PV, unpadded M = G*(1+D),
    counting every key of the sequence for every row (the causal tail is ignored)."""
    w = inp.w
    return int(inp.kv_lens.astype(np.int64).sum()) * w.H_kv * 4 * w.M * w.hd


def attn_exps(inp) -> int:
    """Exponentials the softmax needs per launch: one per (query row, visible
    key) pair, M = G*(1+D) rows per (key, KV head) (the causal tail ignored)."""
    w = inp.w
    return int(inp.kv_lens.astype(np.int64).sum()) * w.H_kv * w.M


def attn_kernel_names(w) -> str:
    """The kernels one spec_verify_attn launch runs for this workload (batches
    up to 2048 take the stream-K path)."""
    if w.B > 2048:
        return "spec_verify_attn (split-K partial kernel + sv_attn_combine)"
    main = "sv_attn_streamk_f8" if w.kv_dtype == "fp8_e4m3" else "sv_attn_streamk"
    return f"spec_verify_attn ({main} + sv_attn_streamk_merge)"


def read_traffic(src_hash):
    """HBM traffic per attention launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    m = re.search(r"src_sha=(\w+).*?workload=(\S+).*?bytes_per_launch=(\d+)", txt, re.S)
    if not m or m.group(1) != src_hash:
        return None
    return {"workload": m.group(2), "bytes": int(m.group(3))}


def time_append(w, da, stream, sv, calls=20):
    """spec_kv_append of the step's R new rows per sequence at the committed length
    T_b (the slots the attention reads last), timed with HIP events after the
    step's own timing.  Not part of the step: the cache of the workload already
    holds those rows."""
    import torch
    from speculative_decoding_verification_15_amd.device import dev
    from workloads import make_append_inputs
    ap = make_append_inputs(w, base=da.inp)
    kn, vn = dev(ap.k_new), dev(ap.v_new)
    kin = dev(ap.committed)
    kout = torch.empty_like(kin)
    fp8 = w.kv_dtype == "fp8_e4m3"
    prm = sv.make_append_params(batch=w.B, num_new=w.R, num_kv_heads=w.H_kv, head_dim=w.hd,
                                max_blocks_per_seq=da.inp.block_table.shape[1],
                                num_blocks=da.inp.num_blocks,
                                kv_dtype=sv.SV_KV_FP8_E4M3 if fp8 else sv.SV_KV_BF16)
    sh = stream.cuda_stream
    for _ in range(LEG_WARMUP):        # the GPU idled during input generation: clocks ramp up
        sv.spec_kv_append(prm, kn, vn, da.k, da.v, da.ks, da.vs, da.bt, kin, kout, stream=sh)
    ev = [TimingEvent() for _ in range(2)]
    ev[0].record(stream)
    for _ in range(calls):
        sv.spec_kv_append(prm, kn, vn, da.k, da.v, da.ks, da.vs, da.bt, kin, kout, stream=sh)
    ev[1].record(stream)
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / calls
    rows = w.B * w.R * w.H_kv * 2
    moved = rows * w.hd * (2 + (1 if fp8 else 2))     # bf16 rows in, cache rows out
    return {"kernel": "sv_kv_append", "avg_launch_us": round(us, 2),
            "bytes_new_rows_in_and_out": moved, "GBps": round(moved / (us * 1e-6) / 1e9, 1)}


def time_accept_sampled(w, da, stream, sv, calls=20):
    """spec_accept_sampled (lossless stochastic acceptance) on the workload's shape:
    target logits [B][1+D][V], draft logits [B][D][V], timed with HIP events after
    the step's own timing.  The greedy spec_accept is the step's acceptance; this
    is its sampled-decoding counterpart."""
    import torch
    from speculative_decoding_verification_15_amd.device import dev
    from workloads import make_sampled_accept_inputs
    si = make_sampled_accept_inputs(w)
    B, D, V = w.B, w.D, w.V
    zt, zd = dev(si.target_logits), dev(si.draft_logits)
    dr, ua, us = dev(si.draft), dev(si.u_accept), dev(si.u_sample)
    al = torch.empty((B,), dtype=torch.int32, device="cuda")
    out = torch.empty((B, w.R), dtype=torch.int32, device="cuda")
    kout = torch.empty((B,), dtype=torch.int32, device="cuda")
    ws_bytes = sv.spec_accept_sampled_workspace_size(B, D, V)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    sh = stream.cuda_stream

    def call():
        sv.spec_accept_sampled(B, D, V, si.tau, zt, zd, dr, ua, us, al, out, da.kl, kout, ws,
                               ws_bytes, stream=sh)
    for _ in range(LEG_WARMUP):        # the GPU idled during input generation: clocks ramp up
        call()
    ev = [TimingEvent() for _ in range(2)]
    ev[0].record(stream)
    for _ in range(calls):
        call()
    ev[1].record(stream)
    torch.cuda.synchronize()
    us_call = ev[0].elapsed_time(ev[1]) * 1e3 / calls
    # every target and draft logit once, plus the one row each sequence draws from
    moved = (B * (2 * D + 1) * V + B * V) * 4
    return {"kernels": "sv_sample_stats + sv_sample_keep + sv_sample_chunk_sums + sv_sample_draw", "avg_launch_us": round(us_call, 2),
            "algorithmic_bytes": moved, "GBps": round(moved / (us_call * 1e-6) / 1e9, 1),
            "sum_accept_len": int(al.cpu().sum())}


def time_draft_signals(w, stream, sv, calls=20):
    """spec_draft_signals over one draft-model row per sequence ([B][V] fp32), the
    signals and the next draft length (max_draft_len = D, rho = 0.05, G of the
    workload), timed with HIP events after the step's own timing."""
    import torch
    from speculative_decoding_verification_15_amd.device import dev
    from workloads import make_draft_logits
    z = dev(make_draft_logits(w.B, w.V, seed=w.seed))
    conf = torch.empty((w.B,), dtype=torch.float32, device="cuda")
    ent = torch.empty_like(conf)
    nd = torch.empty((w.B,), dtype=torch.int32, device="cuda")
    ws_bytes = sv.spec_draft_signals_workspace_size(w.B, w.V)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    sh = stream.cuda_stream

    def call():
        sv.spec_draft_signals(w.B, w.V, 1.0, z, conf, ent, nd, w.D, 0.05, w.G, ws, ws_bytes,
                              stream=sh)
    for _ in range(LEG_WARMUP):        # the GPU idled during input generation: clocks ramp up
        call()
    ev = [TimingEvent() for _ in range(2)]
    ev[0].record(stream)
    for _ in range(calls):
        call()
    ev[1].record(stream)
    torch.cuda.synchronize()
    us_call = ev[0].elapsed_time(ev[1]) * 1e3 / calls
    moved = w.B * w.V * 4
    return {"kernels": "sv_draft_stats + sv_draft_decide", "avg_launch_us": round(us_call, 2),
            "algorithmic_bytes": moved, "GBps": round(moved / (us_call * 1e-6) / 1e9, 1),
            "next_draft_len_hist": np.bincount(nd.cpu().numpy(), minlength=w.D + 1).tolist()}


def time_tree(w, da, p, ws, ws_bytes, out, stream, sv, calls=20):
    """Tree verification on the workload's shape: spec_verify_attn_tree with a
    random draft tree of 1 + D nodes per sequence (each node's parent among the 3
    nodes before it), then spec_accept_tree on the first logit set, timed with
    HIP events after the step's own timing."""
    import torch
    from speculative_decoding_verification_15_amd.device import dev
    from workloads import make_accept_plan, make_tree_plan, tree_tokens_from_target
    tp = make_tree_plan(w, shape="random", width=3, p_match=0.7)
    tm = torch.from_numpy(np.ascontiguousarray(tp.masks).view(np.int64)).cuda()
    plan = make_accept_plan(w)
    tok = dev(tree_tokens_from_target(tp, np.argmax(plan.logits, axis=-1)))
    par = dev(tp.parents)
    lg = dev(plan.logits)
    B, D, V, R = w.B, w.D, w.V, w.R
    tgt = torch.empty((B, R), dtype=torch.int32, device="cuda")
    al = torch.empty((B,), dtype=torch.int32, device="cuda")
    otok = torch.empty((B, R), dtype=torch.int32, device="cuda")
    path = torch.empty((B, R), dtype=torch.int32, device="cuda")
    kout = torch.empty((B,), dtype=torch.int32, device="cuda")
    acc_ws_bytes = sv.spec_accept_workspace_size(B, D, V)
    acc_ws = torch.empty(acc_ws_bytes, dtype=torch.uint8, device="cuda")
    sh = stream.cuda_stream

    def attn():
        sv.spec_verify_attn_tree(p, da.q, da.k, da.v, da.ks, da.vs, da.bt, da.kl, tm, out, ws,
                                 ws_bytes, stream=sh)

    def acc():
        sv.spec_accept_tree(B, D, V, lg, tok, par, tgt, al, otok, path, da.kl, kout, acc_ws,
                            acc_ws_bytes, stream=sh)
    res = {}
    for name, fn in (("attn", attn), ("accept", acc)):
        for _ in range(LEG_WARMUP):    # the GPU idled during input generation: clocks ramp up
            fn()
        ev = [TimingEvent() for _ in range(2)]
        ev[0].record(stream)
        for _ in range(calls):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        res[name] = ev[0].elapsed_time(ev[1]) * 1e3 / calls
    return {"kernels": "sv_attn_streamk (tree variant) + merge; sv_argmax_partial + "
                       "sv_accept_tree_finalize",
            "attn_avg_launch_us": round(res["attn"], 2),
            "accept_avg_launch_us": round(res["accept"], 2),
            "sum_accept_len": int(al.cpu().sum())}


def measure_ceilings(stream, sv):
    """The machine's own ceilings, measured after the step's timing: a streaming
    read of 1 GiB (four times the Infinity Cache), a dense bf16 MFMA loop and
    the vector exp2 rate, each the best of a few launches (HIP events)."""
    import torch
    sh = stream.cuda_stream

    def best_us(fn, reps=5):
        ev = [TimingEvent() for _ in range(2 * reps)]
        fn()                                        # first launch: code load
        for r in range(reps):
            ev[2 * r].record(stream)
            fn()
            ev[2 * r + 1].record(stream)
        torch.cuda.synchronize()
        return min(ev[2 * r].elapsed_time(ev[2 * r + 1]) for r in range(reps)) * 1e3

    out = {}
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")   # values are never used
    sink = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    read = {}
    for wgs in (nbytes // 16384, 16384, 4096):    # one, four or sixteen 16 KB chunks each
        us = best_us(lambda: sv.sv_ceiling_read(src, nbytes, wgs, sink, stream=sh))
        read[wgs] = nbytes / (us * 1e-6) / 1e9
    wgs = max(read, key=read.get)
    out["read_stream_GBps"] = round(read[wgs], 1)
    out["read_stream_workgroups"] = wgs
    del src
    m_wgs, m_it = 1024, 2048
    us = best_us(lambda: sv.sv_ceiling_mfma_bf16(m_wgs, m_it, sink, stream=sh))
    out["mfma_bf16_TFLOPs"] = round(m_wgs * 4 * m_it * 4 * 32768 / (us * 1e-6) / 1e12, 1)
    e_wgs, e_it = 2048, 512
    us = best_us(lambda: sv.sv_ceiling_exp2(e_wgs, e_it, sink, stream=sh))
    out["exp2_per_s"] = float(f"{e_wgs * 256 * e_it * 8 / (us * 1e-6):.4g}")
    out["method"] = ("sv_ceiling_read (16-byte non-temporal loads, 16 KB per workgroup at a "
                     "time, best of 65536/16384/4096 workgroups), sv_ceiling_mfma_bf16 (4 independent 32x32x16 bf16 MFMA chains "
                     "per wave), sv_ceiling_exp2 (8 independent v_exp_f32 chains per thread); "
                     "best of 5 launches each, after the timed steps")
    return out


def cpu_baseline(w, inp, plan, draft, budget_s=15.0):
    """Times the oracle (as it is) on whole sequences until ~budget_s of CPU work."""
    from oracle.accept import oracle_accept
    from oracle.attention import oracle_attn
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas = None
    threads = min(affinity, blas) if blas else affinity
    done, tokens, t_total = [], 0, 0.0
    for b in range(w.B):
        t0 = time.perf_counter()
        oracle_attn(inp.q, inp.k_cache, inp.v_cache, inp.k_scale, inp.v_scale, inp.block_table,
                    inp.kv_lens, D=w.D, H_kv=w.H_kv, sm_scale=w.sm_scale, seqs=[b])
        res = oracle_accept(plan.logits[b:b + 1], draft[b:b + 1], inp.kv_lens[b:b + 1], w.D)
        t_total += time.perf_counter() - t0
        tokens += int(res["accept_len"][0])
        done.append(b)
        if t_total >= budget_s:
            break
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": threads,
            "affinity_cores": affinity, "blas_threads": blas, "kind": "oracle",
            "sample": f"{len(done)} of {w.B} sequences (all {w.H_kv} KV heads): fp64 attention "
                      f"+ acceptance, {t_total:.1f} s of host time, sum AL = {tokens}",
            "seconds": round(t_total, 2)}


def tile_sweep_leg(sv, DeviceAttn, attn_params, make_attn_inputs):
    """spec_verify_attn alone on the tile-boundary shapes (B=8, T=16384, bf16;
    H_kv = 8 or 1, D in SWEEP_D): untimed calls for at least 100 calls and 80 ms
    (the GPU idles while each shape's inputs are generated, and its clock dips
    for several ms after it becomes busy again), then the best of three runs of
    10 calls timed with HIP events on the launch stream."""
    import torch
    from workloads import SWEEP_D, tile_sweep
    stream = torch.cuda.current_stream()
    for mqa in (False, True):
        for D in SWEEP_D:
            w = tile_sweep(D, mqa)
            inp = make_attn_inputs(w)
            d = DeviceAttn(inp)
            p = attn_params(inp)
            plan_ws = sv.spec_verify_attn_workspace_size(p)
            ws = torch.empty(max(plan_ws, 256), dtype=torch.uint8, device="cuda")
            out = torch.empty(d.q.shape, dtype=torch.int16, device="cuda")

            def call():
                sv.spec_verify_attn(p, d.q, d.k, d.v, d.ks, d.vs, d.bt, d.kl, out, ws, plan_ws,
                                    stream=stream.cuda_stream)
            e0, e1 = TimingEvent(), TimingEvent()
            e0.record(stream)
            for _ in range(10):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            first_ms = e0.elapsed_time(e1) / 10
            n_warm = max(LEG_WARMUP - 10, int(80.0 / first_ms))
            for _ in range(n_warm):
                call()
            best = float("inf")
            for _ in range(3):
                e0, e1 = TimingEvent(), TimingEvent()
                e0.record(stream)
                for _ in range(10):
                    call()
                e1.record(stream)
                torch.cuda.synchronize()
                best = min(best, e0.elapsed_time(e1) * 1e3 / 10)
            kv = attn_algorithmic_kv_bytes(inp)
            fl = attn_algorithmic_flops(inp)
            m_pad = -(-w.M // 128) * 128              # rows rounded to 128-row tiles
            print(json.dumps({"tile_sweep": w.name, "M": w.M, "M_pad": m_pad, "us": round(best, 1),
                              "calls": 10 + n_warm + 30,
                              "TFLOPs_padded": round(fl * m_pad / w.M / (best * 1e-6) / 1e12, 1),
                              "kv_GBps": round(kv / (best * 1e-6) / 1e9, 1),
                              "TFLOPs": round(fl / (best * 1e-6) / 1e12, 1),
                              "frac_bf16_peak": round(fl / (best * 1e-6) / 1e12 /
                                                      BF16_MFMA_PEAK_TFLOPS, 4)}), flush=True)
            del d, ws, out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="llama31_70b_gqa8_d15")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device-to-device copy (reference for HBM counters)")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="only time spec_verify_attn on the 14 tile-boundary shapes (one JSON "
                         "line each)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n,
                          "launches": 3}), flush=True)
        return

    import speculative_decoding_verification_15_amd as sv
    from speculative_decoding_verification_15_amd.device import DeviceAttn, attn_params, dev
    from workloads import all_workloads, drafts_from_target, make_accept_plan, make_attn_inputs

    if args.tile_sweep:
        tile_sweep_leg(sv, DeviceAttn, attn_params, make_attn_inputs)
        return

    w = all_workloads()[args.workload]
    assert w.V > 0, "the benchmark step needs an acceptance vocabulary"
    t_gen = time.perf_counter()
    inp = make_attn_inputs(w)
    logits_bytes = w.B * w.R * w.V * 4
    n_sets = int(min(8, max(2, -(-512 * 2 ** 20 // logits_bytes))))
    plan, logit_sets = make_accept_plan(w, n_logit_sets=n_sets)
    # Draft synthesis needs the target token of every row (input preparation).
    # Every rotated logit set gets its own drafts from the same match plan, so
    # each step sees the configured match probability.
    drafts = [drafts_from_target(plan, np.argmax(x, axis=-1)) for x in logit_sets]
    draft = drafts[0]
    t_gen = time.perf_counter() - t_gen

    torch.cuda.set_device(0)
    da = DeviceAttn(inp)
    p = attn_params(inp, args.split_tokens)
    ws_bytes = sv.spec_verify_attn_workspace_size(p)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty(da.q.shape, dtype=torch.int16, device="cuda")
    lg = [dev(x) for x in logit_sets]
    dr = [dev(d) for d in drafts] if w.D > 0 else [None] * n_sets
    B, R, V, D = w.B, w.R, w.V, w.D
    tgt = torch.empty((B, R), dtype=torch.int32, device="cuda")
    al = torch.empty((B,), dtype=torch.int32, device="cuda")
    otok = torch.empty((B, R), dtype=torch.int32, device="cuda")
    kv_out = torch.empty((B,), dtype=torch.int32, device="cuda")
    acc_ws_bytes = sv.spec_accept_workspace_size(B, D, V)
    acc_ws = torch.empty(acc_ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    # Two event records per timed step, around the attention call (each adds
    # stream time, ~1.5 us with TimingEvent), so the acceptance call is timed
    # from the second one to the next step's first (the last step: to the stop
    # event) rather than between two records of its own.
    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        sv.spec_verify_attn(p, da.q, da.k, da.v, da.ks, da.vs, da.bt, da.kl, out, ws, ws_bytes,
                            stream=sh)
        if ev is not None:
            ev[1].record(stream)
        sv.spec_accept(B, D, V, lg[i % n_sets], dr[i % n_sets], tgt, al, otok, da.kl, kv_out,
                       acc_ws, acc_ws_bytes, stream=sh)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[TimingEvent() for _ in range(2)] for _ in range(args.steps)]
    start, stop = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(i, evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    t_attn = np.array([e[0].elapsed_time(e[1]) for e in evs])
    t_acc = np.array([evs[i][1].elapsed_time(evs[i + 1][0] if i + 1 < args.steps else stop)
                      for i in range(args.steps)])

    # acceptance lengths of every logit set in use (the step cycles through them)
    al_per_set = []
    for j in range(n_sets):
        sv.spec_accept(B, D, V, lg[j], dr[j], tgt, al, otok, da.kl, kv_out, acc_ws, acc_ws_bytes,
                       stream=sh)
        torch.cuda.synchronize()
        al_per_set.append(int(al.cpu().sum()))
    # the sets share one match plan, so each gives the same acceptance lengths
    assert len(set(al_per_set)) == 1, al_per_set
    tokens_timed = sum(al_per_set[i % n_sets] for i in range(args.steps))

    append = time_append(w, da, stream, sv)
    sampled = time_accept_sampled(w, da, stream, sv)
    signals = time_draft_signals(w, stream, sv)
    tree = time_tree(w, da, p, ws, ws_bytes, out, stream, sv) if w.B <= 2048 else None
    ceilings = measure_ceilings(stream, sv)

    ms_per_step = total_ms / args.steps
    value = tokens_timed / (total_ms / 1e3)
    attn_us = float(np.mean(t_attn) * 1e3)
    acc_us = float(np.mean(t_acc) * 1e3)
    attn_steps = t_attn * 1e3
    last = attn_steps[-min(5, len(attn_steps)):]
    alg_bytes = attn_algorithmic_bytes(inp)
    kv_bytes = attn_algorithmic_kv_bytes(inp)
    achieved = alg_bytes / (attn_us * 1e-6) / 1e9
    kv_gbps = kv_bytes / (attn_us * 1e-6) / 1e9
    flops = attn_algorithmic_flops(inp)
    tflops = flops / (attn_us * 1e-6) / 1e12
    src_hash = kernel_source_hash()
    tr = read_traffic(src_hash)
    traffic = tr["bytes"] if tr and tr["workload"] == w.name else None

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V/logits, permuted paged block table, "
                "drafts matching the target argmax with per-sequence probability)",
        "config": {
            "workload": w.name, "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv, "head_dim": w.hd,
            "D": w.D, "M_rows_per_kv_head": w.M,
            "context": (f"U[{w.T_range[0]},{w.T_range[1]}]" if w.T_range else w.T),
            "sum_kv_len": int(inp.kv_lens.sum()), "kv_dtype": w.kv_dtype, "vocab": w.V,
            "split_tokens": int(p.split_tokens) or "auto",
            "logit_buffers_rotated": n_sets, "parallelism": "single GPU"},
        "roofline": {
            "kernel": attn_kernel_names(w),
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": alg_bytes, "avg_launch_us": round(attn_us, 2),
            "measured_peak": ceilings["read_stream_GBps"],
            "frac_of_measured": round(achieved / ceilings["read_stream_GBps"], 4),
            "median_launch_us": round(float(np.median(attn_steps)), 2),
            "frac_at_median": round(alg_bytes / (np.median(attn_steps) * 1e-6) / 1e9
                                    / HBM_PEAK_GBPS, 4)},
        "attn_us_per_step": {"median": round(float(np.median(attn_steps)), 2),
                             "min": round(float(attn_steps.min()), 2),
                             "max": round(float(attn_steps.max()), 2),
                             "mean_last5": round(float(last.mean()), 2),
                             "all": [round(float(x), 1) for x in attn_steps]},
        "step_ms_median": round(float(np.median(t_attn + t_acc)), 4),
        "kv_hbm_GBps": round(kv_gbps, 1),
        "scored_rows_per_s": round(B * R / (attn_us * 1e-6), 1),
        "kv_hbm_frac_peak": round(kv_gbps / HBM_PEAK_GBPS, 4),
        "mfma": ({"type": "bf16", "achieved_tflops": round(tflops, 1),
                  "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                  "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                  "measured_peak_tflops": ceilings["mfma_bf16_TFLOPs"],
                  "frac_of_measured": round(tflops / ceilings["mfma_bf16_TFLOPs"], 4),
                  "algorithmic_flops_per_launch": flops}
                 if w.kv_dtype != "fp8_e4m3" else
                 {"type": "fp8 (Q and P as hi + lo e4m3 terms: 2x the algorithmic flops "
                          "executed)", "achieved_tflops": round(tflops, 1),
                  "executed_tflops": round(2 * tflops, 1), "peak_tflops": FP8_MFMA_PEAK_TFLOPS,
                  "frac": round(2 * tflops / FP8_MFMA_PEAK_TFLOPS, 4),
                  "algorithmic_flops_per_launch": flops}),
        "softmax_exp2": {"per_launch": attn_exps(inp),
                         "floor_us_at_measured_rate": round(attn_exps(inp) /
                                                            ceilings["exp2_per_s"] * 1e6, 1)},
        "accept": {"timed": "from the event after the attention call to the next step's first "
                            "event (includes that event record)",
                   "avg_launch_us": round(acc_us, 2),
                   "median_launch_us": round(float(np.median(t_acc) * 1e3), 2),
                   "GBps": round(B * R * V * 4 / (acc_us * 1e-6) / 1e9, 1),
                   "frac": round(B * R * V * 4 / (acc_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                   "frac_of_measured": round(B * R * V * 4 / (acc_us * 1e-6) / 1e9
                                             / ceilings["read_stream_GBps"], 4)},
        "ceilings": ceilings,
        "append": append,
        "accept_sampled": sampled,
        "draft_signals": signals,
        "tree": tree,
        "sum_accept_len_per_step": round(tokens_timed / args.steps, 2),
        "kernel_src_sha": src_hash,
        "input_gen_s": round(t_gen, 1),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, inp, plan, draft, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
