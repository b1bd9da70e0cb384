"""ctypes binding of libspecverify.so.

Argument marshalling only: tensors become device pointers, shapes become the
C structs and integers the header declares, and a non-OK status becomes an
SvError.  Every step of the verification path runs in the library's HIP
kernels; nothing here computes.  Importing this module without a built library
raises ImportError (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SV_OK, SV_ERR_INVALID, SV_ERR_WORKSPACE, SV_ERR_UNSUPPORTED, SV_ERR_LAUNCH = range(5)
SV_KV_BF16, SV_KV_FP8_E4M3 = 0, 1

# Every symbol include/spec_verify.h declares.
EXPORTS = ("spec_verify_attn_workspace_size", "spec_verify_attn", "spec_accept_workspace_size",
           "spec_accept", "spec_accept_sampled_workspace_size", "spec_accept_sampled",
           "spec_kv_append", "spec_draft_signals_workspace_size", "spec_draft_signals",
           "spec_verify_attn_tree", "spec_accept_tree", "spec_kv_commit_tree",
           "sv_status_string", "sv_last_error", "sv_abi_version",
           "sv_ceiling_read", "sv_ceiling_mfma_bf16", "sv_ceiling_exp2", "spec_accept_noalloc")


class SvAttnParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("draft_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("split_tokens", ctypes.c_int32),
    ]


class SvAppendParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_new", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
    ]


class SvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)} -- {message}")
        self.status = status


def _load():
    # PyTorch ships its own HIP runtime (same soname as ROCm's).  Loading torch
    # first makes the library bind to that runtime, so the process has exactly
    # one HIP runtime and torch's device memory and streams are valid here.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python -m speculative_decoding_verification_15_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, I32, U = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int
    lib.spec_verify_attn_workspace_size.argtypes = [ctypes.POINTER(SvAttnParams), ctypes.POINTER(S)]
    lib.spec_verify_attn_workspace_size.restype = U
    lib.spec_verify_attn.argtypes = [ctypes.POINTER(SvAttnParams)] + [P] * 9 + [S, P]
    lib.spec_verify_attn.restype = U
    lib.spec_accept_workspace_size.argtypes = [I32, I32, I32, ctypes.POINTER(S)]
    lib.spec_accept_workspace_size.restype = U
    lib.spec_accept.argtypes = [I32, I32, I32] + [P] * 8 + [S, P]
    lib.spec_accept.restype = U
    lib.spec_accept_noalloc.argtypes = [I32, I32, I32] + [P] * 8
    lib.spec_accept_noalloc.restype = U
    lib.spec_accept_sampled_workspace_size.argtypes = [I32, I32, I32, ctypes.POINTER(S)]
    lib.spec_accept_sampled_workspace_size.restype = U
    lib.spec_accept_sampled.argtypes = [I32, I32, I32, ctypes.c_float] + [P] * 10 + [S, P]
    lib.spec_accept_sampled.restype = U
    lib.spec_kv_append.argtypes = [ctypes.POINTER(SvAppendParams)] + [P] * 10
    lib.spec_kv_append.restype = U
    lib.spec_draft_signals_workspace_size.argtypes = [I32, I32, ctypes.POINTER(S)]
    lib.spec_draft_signals_workspace_size.restype = U
    lib.spec_draft_signals.argtypes = [I32, I32, ctypes.c_float, P, P, P, P, I32, ctypes.c_float,
                                       I32, P, S, P]
    lib.spec_draft_signals.restype = U
    lib.spec_verify_attn_tree.argtypes = [ctypes.POINTER(SvAttnParams)] + [P] * 10 + [S, P]
    lib.spec_verify_attn_tree.restype = U
    lib.spec_accept_tree.argtypes = [I32, I32, I32] + [P] * 10 + [S, P]
    lib.spec_accept_tree.restype = U
    lib.spec_kv_commit_tree.argtypes = [ctypes.POINTER(SvAppendParams)] + [P] * 10
    lib.spec_kv_commit_tree.restype = U
    lib.sv_status_string.argtypes = [U]
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.sv_last_error.argtypes = []
    lib.sv_last_error.restype = ctypes.c_char_p
    lib.sv_abi_version.argtypes = []
    lib.sv_abi_version.restype = I32
    lib.sv_ceiling_read.argtypes = [P, S, I32, P, P]
    lib.sv_ceiling_read.restype = U
    lib.sv_ceiling_mfma_bf16.argtypes = [I32, I32, P, P]
    lib.sv_ceiling_mfma_bf16.restype = U
    lib.sv_ceiling_exp2.argtypes = [I32, I32, P, P]
    lib.sv_ceiling_exp2.restype = U
    return lib


_lib = _load()


def library():
    return _lib


def status_string(status: int) -> str:
    return _lib.sv_status_string(status).decode()


def last_error() -> str:
    return _lib.sv_last_error().decode()


def abi_version() -> int:
    return int(_lib.sv_abi_version())


def _check(status: int):
    if status != SV_OK:
        raise SvError(status, last_error())


_I32, _F32, _BF16, _U8, _U64 = ("int32",), ("float32",), ("bfloat16", "int16", "uint16"), \
    ("uint8", "int8", "float8_e4m3fn"), ("int64", "uint64")


def _ptr(t, nbytes=None, name="tensor", dtypes=None):
    """Device address of a tensor (None -> NULL; integers pass through as raw
    addresses).  A tensor must live on the GPU, be contiguous, have one of the
    dtypes the header names for the argument and hold at least `nbytes`
    bytes; otherwise SvError(SV_ERR_INVALID) is raised before any call, since a
    CPU tensor, a strided view or a short buffer would reach a kernel as a bad
    address."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not getattr(t, "is_cuda", False):
        raise SvError(SV_ERR_INVALID, f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise SvError(SV_ERR_INVALID, f"{name} must be contiguous")
    if dtypes is not None and str(t.dtype).replace("torch.", "") not in dtypes:
        raise SvError(SV_ERR_INVALID, f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    have = t.numel() * t.element_size()
    if nbytes is not None and have < nbytes:
        raise SvError(SV_ERR_INVALID, f"{name} holds {have} bytes; the shape needs {nbytes}")
    return t.data_ptr()


def _nbytes(t):
    return 0 if t is None or isinstance(t, int) else t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_attn_params(*, batch, draft_len, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                     num_blocks, max_kv_len, kv_dtype=SV_KV_BF16, sm_scale=None, split_tokens=0,
                     block_size=16) -> SvAttnParams:
    if sm_scale is None:
        sm_scale = head_dim ** -0.5
    return SvAttnParams(batch, draft_len, num_q_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks, max_kv_len, kv_dtype, sm_scale, split_tokens)


def spec_verify_attn_workspace_size(params: SvAttnParams) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.spec_verify_attn_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return int(n.value)


def _attn_ptrs(p: SvAttnParams, q, k_cache, v_cache, k_scale, v_scale, block_table, kv_lens, out,
               workspace, workspace_bytes):
    """Checked addresses of spec_verify_attn's buffers, sized from the params."""
    fp8 = p.kv_dtype == SV_KV_FP8_E4M3
    R = p.draft_len + 1
    qo = max(p.batch, 0) * R * max(p.num_q_heads, 0) * max(p.head_dim, 0) * 2
    cache = max(p.num_blocks, 0) * max(p.num_kv_heads, 0) * 16 * max(p.head_dim, 0) * (1 if fp8 else 2)
    scales = max(p.num_blocks, 0) * max(p.num_kv_heads, 0) * 4
    cdt = _U8 if fp8 else _BF16
    return (_ptr(q, qo, "q", _BF16), _ptr(k_cache, cache, "k_cache", cdt),
            _ptr(v_cache, cache, "v_cache", cdt), _ptr(k_scale, scales, "k_scale", _F32),
            _ptr(v_scale, scales, "v_scale", _F32),
            _ptr(block_table, max(p.batch, 0) * max(p.max_blocks_per_seq, 0) * 4, "block_table", _I32),
            _ptr(kv_lens, max(p.batch, 0) * 4, "kv_lens", _I32), _ptr(out, qo, "out", _BF16),
            _ptr(workspace, workspace_bytes, "workspace"))


def _ws_bytes(workspace, workspace_bytes):
    return _nbytes(workspace) if workspace_bytes is None else workspace_bytes


def spec_verify_attn(params: SvAttnParams, q, k_cache, v_cache, k_scale, v_scale, block_table,
                     kv_lens, out, workspace=None, workspace_bytes=None, stream=None) -> None:
    workspace_bytes = _ws_bytes(workspace, workspace_bytes)
    pq, pk, pv, pks, pvs, pbt, pkl, pout, pws = _attn_ptrs(
        params, q, k_cache, v_cache, k_scale, v_scale, block_table, kv_lens, out, workspace,
        workspace_bytes)
    _check(_lib.spec_verify_attn(ctypes.byref(params), pq, pk, pv, pks, pvs, pbt, pkl, pout, pws,
                                 workspace_bytes, _stream(stream)))


def spec_accept_workspace_size(batch: int, draft_len: int, vocab: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.spec_accept_workspace_size(batch, draft_len, vocab, ctypes.byref(n)))
    return int(n.value)


def _rows(batch, draft_len):
    return max(batch, 0) * (max(draft_len, 0) + 1)


def spec_accept(batch, draft_len, vocab, logits, draft, target_tokens, accept_len, out_tokens,
                kv_lens_in, kv_lens_out, workspace, workspace_bytes=None, stream=None) -> None:
    workspace_bytes = _ws_bytes(workspace, workspace_bytes)
    B, rows = max(batch, 0), _rows(batch, draft_len)
    _check(_lib.spec_accept(batch, draft_len, vocab,
                            _ptr(logits, rows * max(vocab, 0) * 4, "logits", _F32),
                            _ptr(draft, B * max(draft_len, 0) * 4, "draft", _I32),
                            _ptr(target_tokens, rows * 4, "target_tokens", _I32),
                            _ptr(accept_len, B * 4, "accept_len", _I32),
                            _ptr(out_tokens, rows * 4, "out_tokens", _I32),
                            _ptr(kv_lens_in, B * 4, "kv_lens_in", _I32),
                            _ptr(kv_lens_out, B * 4, "kv_lens_out", _I32),
                            _ptr(workspace, workspace_bytes, "workspace"), workspace_bytes,
                            _stream(stream)))


def spec_accept_noalloc(batch, draft_len, vocab, logits, draft, target_tokens, accept_len,
                        out_tokens, kv_lens_in, kv_lens_out, stream=None) -> None:
    B, rows = max(batch, 0), _rows(batch, draft_len)
    _check(_lib.spec_accept_noalloc(batch, draft_len, vocab,
                                    _ptr(logits, rows * max(vocab, 0) * 4, "logits", _F32),
                                    _ptr(draft, B * max(draft_len, 0) * 4, "draft", _I32),
                                    _ptr(target_tokens, rows * 4, "target_tokens", _I32),
                                    _ptr(accept_len, B * 4, "accept_len", _I32),
                                    _ptr(out_tokens, rows * 4, "out_tokens", _I32),
                                    _ptr(kv_lens_in, B * 4, "kv_lens_in", _I32),
                                    _ptr(kv_lens_out, B * 4, "kv_lens_out", _I32), _stream(stream)))


def spec_accept_sampled_workspace_size(batch: int, draft_len: int, vocab: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.spec_accept_sampled_workspace_size(batch, draft_len, vocab, ctypes.byref(n)))
    return int(n.value)


def spec_accept_sampled(batch, draft_len, vocab, temperature, target_logits, draft_logits, draft,
                        u_accept, u_sample, accept_len, out_tokens, kv_lens_in, kv_lens_out,
                        workspace, workspace_bytes=None, stream=None) -> None:
    workspace_bytes = _ws_bytes(workspace, workspace_bytes)
    B, rows, D, V = max(batch, 0), _rows(batch, draft_len), max(draft_len, 0), max(vocab, 0)
    _check(_lib.spec_accept_sampled(batch, draft_len, vocab, float(temperature),
                                    _ptr(target_logits, rows * V * 4, "target_logits", _F32),
                                    _ptr(draft_logits, B * D * V * 4, "draft_logits", _F32),
                                    _ptr(draft, B * D * 4, "draft", _I32),
                                    _ptr(u_accept, B * D * 4, "u_accept", _F32),
                                    _ptr(u_sample, B * 4, "u_sample", _F32),
                                    _ptr(accept_len, B * 4, "accept_len", _I32),
                                    _ptr(out_tokens, rows * 4, "out_tokens", _I32),
                                    _ptr(kv_lens_in, B * 4, "kv_lens_in", _I32),
                                    _ptr(kv_lens_out, B * 4, "kv_lens_out", _I32),
                                    _ptr(workspace, workspace_bytes, "workspace"), workspace_bytes,
                                    _stream(stream)))



def make_append_params(*, batch, num_new, num_kv_heads, head_dim, max_blocks_per_seq, num_blocks,
                       kv_dtype=SV_KV_BF16, block_size=16) -> SvAppendParams:
    return SvAppendParams(batch, num_new, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                          num_blocks, kv_dtype)


def _append_ptrs(p: SvAppendParams, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table):
    """Checked addresses of the buffers spec_kv_append and spec_kv_commit_tree share."""
    fp8 = p.kv_dtype == SV_KV_FP8_E4M3
    rows = max(p.batch, 0) * max(p.num_new, 0) * max(p.num_kv_heads, 0) * max(p.head_dim, 0) * 2
    cache = max(p.num_blocks, 0) * max(p.num_kv_heads, 0) * 16 * max(p.head_dim, 0) * (1 if fp8 else 2)
    scales = max(p.num_blocks, 0) * max(p.num_kv_heads, 0) * 4
    cdt = _U8 if fp8 else _BF16
    return (_ptr(k_new, rows, "k_new", _BF16), _ptr(v_new, rows, "v_new", _BF16),
            _ptr(k_cache, cache, "k_cache", cdt), _ptr(v_cache, cache, "v_cache", cdt),
            _ptr(k_scale, scales, "k_scale", _F32), _ptr(v_scale, scales, "v_scale", _F32),
            _ptr(block_table, max(p.batch, 0) * max(p.max_blocks_per_seq, 0) * 4, "block_table",
                 _I32))


def spec_kv_append(params: SvAppendParams, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                   block_table, kv_lens_in, kv_lens_out, stream=None) -> None:
    B = max(params.batch, 0)
    _check(_lib.spec_kv_append(ctypes.byref(params),
                               *_append_ptrs(params, k_new, v_new, k_cache, v_cache, k_scale,
                                             v_scale, block_table),
                               _ptr(kv_lens_in, B * 4, "kv_lens_in", _I32),
                               _ptr(kv_lens_out, B * 4, "kv_lens_out", _I32), _stream(stream)))


def spec_draft_signals_workspace_size(rows: int, vocab: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.spec_draft_signals_workspace_size(rows, vocab, ctypes.byref(n)))
    return int(n.value)


def spec_draft_signals(rows, vocab, temperature, draft_logits, confidence, entropy, next_draft_len,
                       max_draft_len, rho, group_size, workspace, workspace_bytes=None,
                       stream=None) -> None:
    workspace_bytes = _ws_bytes(workspace, workspace_bytes)
    n = max(rows, 0)
    _check(_lib.spec_draft_signals(rows, vocab, float(temperature),
                                   _ptr(draft_logits, n * max(vocab, 0) * 4, "draft_logits", _F32),
                                   _ptr(confidence, n * 4, "confidence", _F32),
                                   _ptr(entropy, n * 4, "entropy", _F32),
                                   _ptr(next_draft_len, n * 4, "next_draft_len", _I32),
                                   int(max_draft_len), float(rho), int(group_size),
                                   _ptr(workspace, workspace_bytes, "workspace"), workspace_bytes,
                                   _stream(stream)))


def spec_verify_attn_tree(params: SvAttnParams, q, k_cache, v_cache, k_scale, v_scale,
                          block_table, kv_lens, tree_mask, out, workspace=None,
                          workspace_bytes=None, stream=None) -> None:
    workspace_bytes = _ws_bytes(workspace, workspace_bytes)
    pq, pk, pv, pks, pvs, pbt, pkl, pout, pws = _attn_ptrs(
        params, q, k_cache, v_cache, k_scale, v_scale, block_table, kv_lens, out, workspace,
        workspace_bytes)
    ptm = _ptr(tree_mask, _rows(params.batch, params.draft_len) * 8, "tree_mask", _U64)
    _check(_lib.spec_verify_attn_tree(ctypes.byref(params), pq, pk, pv, pks, pvs, pbt, pkl, ptm,
                                      pout, pws, workspace_bytes, _stream(stream)))


def spec_accept_tree(batch, draft_len, vocab, logits, tokens, parents, target_tokens, accept_len,
                     out_tokens, accept_path, kv_lens_in, kv_lens_out, workspace,
                     workspace_bytes=None, stream=None) -> None:
    workspace_bytes = _ws_bytes(workspace, workspace_bytes)
    B, rows = max(batch, 0), _rows(batch, draft_len)
    _check(_lib.spec_accept_tree(batch, draft_len, vocab,
                                 _ptr(logits, rows * max(vocab, 0) * 4, "logits", _F32),
                                 _ptr(tokens, rows * 4, "tokens", _I32),
                                 _ptr(parents, rows * 4, "parents", _I32),
                                 _ptr(target_tokens, rows * 4, "target_tokens", _I32),
                                 _ptr(accept_len, B * 4, "accept_len", _I32),
                                 _ptr(out_tokens, rows * 4, "out_tokens", _I32),
                                 _ptr(accept_path, rows * 4, "accept_path", _I32),
                                 _ptr(kv_lens_in, B * 4, "kv_lens_in", _I32),
                                 _ptr(kv_lens_out, B * 4, "kv_lens_out", _I32),
                                 _ptr(workspace, workspace_bytes, "workspace"), workspace_bytes,
                                 _stream(stream)))


def spec_kv_commit_tree(params: SvAppendParams, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                        block_table, accept_path, kv_lens, stream=None) -> None:
    B = max(params.batch, 0)
    _check(_lib.spec_kv_commit_tree(ctypes.byref(params),
                                    *_append_ptrs(params, k_new, v_new, k_cache, v_cache, k_scale,
                                                  v_scale, block_table),
                                    _ptr(accept_path, B * max(params.num_new, 0) * 4,
                                         "accept_path", _I32),
                                    _ptr(kv_lens, B * 4, "kv_lens", _I32), _stream(stream)))


def sv_ceiling_read(src, nbytes, workgroups, sink, stream=None) -> None:
    _check(_lib.sv_ceiling_read(_ptr(src, nbytes, "src"), nbytes, int(workgroups),
                                _ptr(sink, int(workgroups) * 4, "sink", _F32), _stream(stream)))


def sv_ceiling_mfma_bf16(workgroups, iters, sink, stream=None) -> None:
    _check(_lib.sv_ceiling_mfma_bf16(int(workgroups), int(iters),
                                     _ptr(sink, int(workgroups) * 16, "sink", _F32), _stream(stream)))


def sv_ceiling_exp2(workgroups, iters, sink, stream=None) -> None:
    _check(_lib.sv_ceiling_exp2(int(workgroups), int(iters),
                                _ptr(sink, int(workgroups) * 1024, "sink", _F32), _stream(stream)))
