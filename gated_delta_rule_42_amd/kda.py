"""Thin ctypes binding of libkda.so (include/kda.h): the same entry points,
taking torch tensors.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libkda.so.  PyTorch supplies device memory and the stream.  If the
library is missing, importing this module raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# KDA_LIBRARY names another build of the same sources to load instead (the
# host-sanitized one, for the sanitizer test).
LIBRARY = os.environ.get("KDA_LIBRARY") or os.path.join(_PKG, "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARG = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_WORKSPACE_TOO_SMALL = 3
KDA_ERR_LAUNCH = 4
KDA_ERR_DEVICE = 5
KDA_ERR_SCRATCH_LIMIT = 6

KDA_F32 = 0
KDA_BF16 = 1
KDA_F16 = 2
KDA_FLAG_QK_L2NORM = 1
KDA_FLAG_DIAG_GIVE_UP = 0x80000000
KDA_CONV_SILU = 1
KDA_NORM_SIGMOID = 1
KDA_NORM_RESIDUAL_F32 = 2

_DTYPES = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16, torch.float16: KDA_F16}


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {message} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIBRARY):
        raise ImportError(f"{LIBRARY} is missing; build it with "
                          "`python -m gated_delta_rule_42_amd.build`")
    lib = ctypes.CDLL(LIBRARY)
    vp, i32, i64, u32, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t)
    lib.kda_abi_version.restype = ctypes.c_int
    lib.kda_abi_version.argtypes = []
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [i32]
    lib.kda_chunk_prefill_workspace_size.restype = sz
    lib.kda_chunk_prefill_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32]
    lib.kda_chunk_prefill.restype = i32
    lib.kda_chunk_prefill.argtypes = [
        vp, vp, vp, i32, i64, i64, i64, vp, vp,
        vp, i32, i64, i32, i32, i32,
        vp, i32, i64, vp, vp,
        vp, i64, i32,
        f32, i32, u32, vp, i64, vp, sz, vp]
    lib.kda_chunk_prefill_noalloc.restype = i32
    lib.kda_chunk_prefill_noalloc.argtypes = [
        vp, vp, vp, i32, i64, i64, i64, vp, vp,
        vp, i32, i64, i32, i32, i32,
        vp, i32, i64, vp, vp,
        vp, i64, i32,
        f32, i32, u32, vp, i64, vp]
    lib.kda_chunk_prefill_at.restype = i32
    lib.kda_chunk_prefill_at.argtypes = [
        vp, vp, vp, i32, i64, i64, i64, vp, vp,
        vp, vp, i32, i64, i32, i32, i32,
        vp, i32, i64, vp, vp,
        vp, i64, i32,
        f32, i32, u32, vp, i64, vp, sz, vp]
    lib.kda_conv_chunk_prefill.restype = i32
    lib.kda_conv_chunk_prefill.argtypes = [
        vp, i64, i32, vp, vp, i32, u32, vp, vp, vp,
        vp, i32, i64, i32, i32, i32,
        vp, i32, i64, vp, vp,
        vp, i64, i32,
        f32, i32, u32, vp, i64, vp, sz, vp]
    lib.kda_chunk_prefill_norm_workspace_size.restype = sz
    lib.kda_chunk_prefill_norm_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32]
    lib.kda_chunk_prefill_norm.restype = i32
    lib.kda_chunk_prefill_norm.argtypes = [
        vp, vp, vp, i32, i64, i64, i64, vp, vp,
        vp, i32, i64, i32, i32, i32,
        vp, i32, i64, vp, vp,
        vp, i64, i32,
        f32, i32, u32, vp, i64,
        vp, i64, vp, f32, vp, i64,
        vp, sz, vp]
    lib.kda_conv_chunk_prefill_norm.restype = i32
    lib.kda_conv_chunk_prefill_norm.argtypes = [
        vp, i64, i32, vp, vp, i32, u32, vp, vp, vp,
        vp, i32, i64, i32, i32, i32,
        vp, i32, i64, vp, vp,
        vp, i64, i32,
        f32, i32, u32, vp, i64,
        vp, i64, vp, f32, vp, i64,
        vp, sz, vp]
    lib.kda_recurrent_decode.restype = i32
    lib.kda_recurrent_decode.argtypes = [
        vp, vp, vp, i32, i64, i64, i64, vp, vp, i32, i32, i32, i32,
        vp, i32, i64, vp, f32, u32, vp, i64, vp]
    lib.kda_gated_rmsnorm.restype = i32
    lib.kda_gated_rmsnorm.argtypes = [vp, i64, vp, i64, vp, vp, i64, i32, i64, i32, i32, f32, vp]
    lib.kda_gated_rmsnorm_ex.restype = i32
    lib.kda_gated_rmsnorm_ex.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp, vp, i64, vp, i64,
                                         i32, i64, i32, i32, f32, u32, vp]
    lib.kda_causal_conv1d.restype = i32
    lib.kda_causal_conv1d.argtypes = [
        vp, i64, vp, vp, vp, i64, vp, vp, vp, i32, i64, i32, i32, i32, u32, vp, i64, vp]
    lib.kda_spec_decode.restype = i32
    lib.kda_spec_decode.argtypes = [
        vp, vp, vp, i32, i64, i64, i64, vp, vp, i32, i32, i32, i32, i32,
        vp, i32, i64, vp, vp, f32, u32, vp, i64, vp]
    lib.kda_spec_commit.restype = i32
    lib.kda_spec_commit.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, i32, i64, vp, vp]
    lib.kda_chunk_prefill_check.restype = i32
    lib.kda_chunk_prefill_check.argtypes = [vp, sz, ctypes.POINTER(ctypes.c_uint32), vp]
    return lib


_lib = _load()


def _check(fn: str, status: int) -> None:
    if status != KDA_OK:
        raise KdaError(fn, status, _lib.kda_status_string(status).decode())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _token_stride(t: torch.Tensor, name: str) -> int:
    """[tokens, heads, dim] with heads packed inside a token: stride (s, dim, 1)."""
    if t.dim() == 3 and t.numel() == 0:
        return t.shape[1] * t.shape[2]
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name} must be [tokens, heads, dim] with contiguous heads")
    return t.stride(0)


def _shape(t, name: str, shape, dtype=None) -> None:
    """t (if given) has exactly `shape` (None matches any extent) and, if
    given, `dtype`.  The C ABI takes every size from q (or x), so a tensor of
    another shape would be read or written out of bounds: refuse it here."""
    if t is None:
        return
    if t.dim() != len(shape) or any(w is not None and int(n) != int(w) for n, w in zip(t.shape, shape)):
        want = ", ".join("*" if w is None else str(int(w)) for w in shape)
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected ({want})")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} is {t.dtype}, expected {dtype}")


def _on_device(*named) -> None:
    """Every tensor given lives on the same GPU (host memory would reach the
    kernels as a bad device address)."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor, not on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def _contig(t: torch.Tensor, name: str, dtype: torch.dtype) -> None:
    if t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous {dtype}")


def abi_version() -> int:
    return int(_lib.kda_abi_version())


def status_string(status: int) -> str:
    return _lib.kda_status_string(status).decode()


def chunk_prefill_workspace_size(num_seqs: int, total_tokens: int, num_heads: int, dk: int,
                                 dv: int, chunk_size: int = 64, norm: bool = False) -> int:
    """kda_chunk_prefill_workspace_size, or with `norm` the size the calls
    with the fused gated norm need (kda_chunk_prefill_norm_workspace_size)."""
    fn = _lib.kda_chunk_prefill_norm_workspace_size if norm else _lib.kda_chunk_prefill_workspace_size
    return int(fn(num_seqs, total_tokens, num_heads, dk, dv, chunk_size))


def _norm_args(norm_gate, norm_weight, norm_out, T, H, dv, dtype):
    """Checks the fused norm's tensors' shapes and dtypes (their device is
    checked with the call's other tensors); None when the norm is not asked
    for."""
    if norm_gate is None and norm_out is None:
        if norm_weight is not None:
            raise ValueError("norm_weight needs norm_gate and norm_out")
        return None
    if norm_gate is None or norm_out is None:
        raise ValueError("the fused norm needs both norm_gate and norm_out")
    _shape(norm_gate, "norm_gate", (T, H, dv), dtype)
    _shape(norm_out, "norm_out", (T, H, dv), dtype)
    _shape(norm_weight, "norm_weight", (dv,))
    return norm_gate, norm_out, norm_weight


def _norm_ptrs(nrm, dtype):
    """(gate pointer, gate token stride, weight pointer) of checked norm
    tensors, None for none."""
    if nrm is None:
        return None
    norm_gate, _, norm_weight = nrm
    if norm_weight is not None:
        _contig(norm_weight, "norm_weight", dtype)
    return (_ptr(norm_gate), _token_stride(norm_gate, "norm_gate"), _ptr(norm_weight))


def chunk_prefill(q, k, v, g, beta, cu_seqlens, state_pool, state_indices, out, *,
                  workspace=None, has_initial_state=None, checkpoints=None,
                  ckpt_interval: int = 0, scale: float = 1.0, chunk_size: int = 64,
                  flags: int = 0, norm_gate=None, norm_weight=None, norm_eps: float = 1e-6,
                  norm_out=None, stream=None) -> None:
    """kda_chunk_prefill.  q,k [T,H,dk]; v,out [T,H,dv] (token-strided views
    allowed); g [T,H,dk] fp32; beta [T,H] fp32; cu_seqlens [N+1] int32;
    state_pool [slots,H,dk,dv] fp32/bf16 (updated in place); state_indices [N]
    int32; has_initial_state [N] uint8 or None; checkpoints [cap,H,dk,dv] or
    None.  `workspace` is a uint8 tensor of at least
    chunk_prefill_workspace_size(...) bytes; None allocates one.  With
    norm_gate and norm_out ([T,H,dv], q's dtype) and optionally norm_weight
    [dv], kda_chunk_prefill_norm: the gated RMSNorm of out is written to
    norm_out by the same call (workspace: chunk_prefill_workspace_size(...,
    norm=True))."""
    _prefill_call(None, q, k, v, g, beta, cu_seqlens, state_pool, state_indices, out,
                  workspace, has_initial_state, checkpoints, ckpt_interval, scale, chunk_size,
                  flags, stream, norm=(norm_gate, norm_weight, norm_eps, norm_out))


def chunk_prefill_noalloc(q, k, v, g, beta, cu_seqlens, state_pool, state_indices, out, *,
                          has_initial_state=None, checkpoints=None, ckpt_interval: int = 0,
                          scale: float = 1.0, chunk_size: int = 64, flags: int = 0,
                          stream=None) -> None:
    """kda_chunk_prefill_noalloc: chunk_prefill on the library's fixed 128 MiB
    scratch area instead of a workspace (nothing is allocated, here or in the
    library).  Calls that overlap on one GPU race; a call needing more scratch
    raises (KDA_ERR_SCRATCH_LIMIT)."""
    _prefill_call(None, q, k, v, g, beta, cu_seqlens, state_pool, state_indices, out,
                  None, has_initial_state, checkpoints, ckpt_interval, scale, chunk_size,
                  flags, stream, noalloc=True)


def chunk_prefill_at(q, k, v, g, beta, cu_seqlens, seq_start_pos, state_pool, state_indices,
                     out, *, workspace=None, has_initial_state=None, checkpoints=None,
                     ckpt_interval: int = 0, scale: float = 1.0, chunk_size: int = 64,
                     flags: int = 0, stream=None) -> None:
    """kda_chunk_prefill_at: chunk_prefill for sequences starting at absolute
    positions seq_start_pos [N] int64 (device; chunk boundaries and
    checkpoints follow absolute positions)."""
    _contig(seq_start_pos, "seq_start_pos", torch.int64)
    _prefill_call(seq_start_pos, q, k, v, g, beta, cu_seqlens, state_pool, state_indices, out,
                  workspace, has_initial_state, checkpoints, ckpt_interval, scale, chunk_size,
                  flags, stream)


def _prefill_call(seq_start_pos, q, k, v, g, beta, cu_seqlens, state_pool, state_indices, out,
                  workspace, has_initial_state, checkpoints, ckpt_interval, scale, chunk_size,
                  flags, stream, noalloc: bool = False, norm=(None, None, 1e-6, None)) -> None:
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q and v must be [tokens, heads, dim]")
    T, H, dk = q.shape
    dv = v.shape[2]
    N = state_indices.numel()
    _shape(k, "k", (T, H, dk), q.dtype)
    _shape(v, "v", (T, H, dv), q.dtype)
    _shape(out, "out", (T, H, dv), q.dtype)
    _shape(g, "g", (T, H, dk))
    _shape(beta, "beta", (T, H))
    _shape(cu_seqlens, "cu_seqlens", (N + 1,))
    _shape(state_indices, "state_indices", (N,))
    _shape(has_initial_state, "has_initial_state", (N,))
    _shape(seq_start_pos, "seq_start_pos", (N,))
    _shape(state_pool, "state_pool", (None, H, dk, dv))
    _shape(checkpoints, "checkpoints", (None, H, dk, dv), state_pool.dtype)
    _shape(workspace, "workspace", (None,), torch.uint8)
    norm_gate, norm_weight, norm_eps, norm_out = norm
    nrm = _norm_args(norm_gate, norm_weight, norm_out, T, H, dv, q.dtype)
    _on_device(("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("cu_seqlens", cu_seqlens),
               ("state_pool", state_pool), ("state_indices", state_indices), ("out", out),
               ("workspace", workspace), ("has_initial_state", has_initial_state),
               ("checkpoints", checkpoints), ("seq_start_pos", seq_start_pos),
               ("norm_gate", norm_gate), ("norm_out", norm_out), ("norm_weight", norm_weight))
    _contig(g, "g", torch.float32)
    _contig(beta, "beta", torch.float32)
    _contig(cu_seqlens, "cu_seqlens", torch.int32)
    _contig(state_indices, "state_indices", torch.int32)
    if has_initial_state is not None:
        _contig(has_initial_state, "has_initial_state", torch.uint8)
    if not state_pool.is_contiguous():
        raise ValueError("state_pool must be contiguous")
    nrm = _norm_ptrs(nrm, q.dtype)
    if workspace is None and not noalloc:
        need = chunk_prefill_workspace_size(N, T, H, dk, dv, chunk_size, norm=nrm is not None)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    cap = 0
    if checkpoints is not None:
        if not checkpoints.is_contiguous() or checkpoints.dtype != state_pool.dtype:
            raise ValueError("checkpoints must be contiguous with the state dtype")
        cap = checkpoints.shape[0]
    head = (_ptr(q), _ptr(k), _ptr(v), _dtype(q),
            _token_stride(q, "q"), _token_stride(k, "k"), _token_stride(v, "v"),
            _ptr(g), _ptr(beta), _ptr(cu_seqlens))
    tail = (T, H, dk, dv,
            _ptr(state_pool), _dtype(state_pool), state_pool.shape[0] if state_pool.dim() else 0,
            _ptr(state_indices), _ptr(has_initial_state),
            _ptr(checkpoints), cap, int(ckpt_interval),
            float(scale), int(chunk_size), int(flags),
            _ptr(out), _token_stride(out, "out"))
    if noalloc:
        _check("kda_chunk_prefill_noalloc", _lib.kda_chunk_prefill_noalloc(*head, N, *tail, _stream(stream)))
        return
    ws_tail = (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if nrm is not None:
        _check("kda_chunk_prefill_norm",
               _lib.kda_chunk_prefill_norm(*head, N, *tail, *nrm, float(norm_eps), _ptr(norm_out),
                                           _token_stride(norm_out, "norm_out"), *ws_tail))
        return
    tail += ws_tail
    if seq_start_pos is None:
        _check("kda_chunk_prefill", _lib.kda_chunk_prefill(*head, N, *tail))
    else:
        _check("kda_chunk_prefill_at",
               _lib.kda_chunk_prefill_at(*head, _ptr(seq_start_pos), N, *tail))


def conv_chunk_prefill(x, conv_weight, conv_state_pool, g, beta, cu_seqlens, state_pool,
                       state_indices, out, *, conv_bias=None, silu: bool = True, workspace=None,
                       has_initial_state=None, checkpoints=None, ckpt_interval: int = 0,
                       scale: float = 1.0, chunk_size: int = 64, flags: int = 0,
                       norm_gate=None, norm_weight=None, norm_eps: float = 1e-6, norm_out=None,
                       stream=None) -> None:
    """kda_conv_chunk_prefill.  x [T, 3*H*d] packed q|k|v before the conv
    (token stride allowed, channels contiguous); conv_weight [3Hd, W];
    conv_state_pool [slots, W-1, 3Hd] (updated in place); out [T,H,d]; the
    rest as chunk_prefill, the fused norm included
    (kda_conv_chunk_prefill_norm)."""
    if x.dim() != 2 or out.dim() != 3 or conv_weight.dim() != 2:
        raise ValueError("x must be [tokens, channels], out [tokens, heads, dim], conv_weight [channels, width]")
    T, C = x.shape
    H, dv = out.shape[1], out.shape[2]
    dk = dv
    if C != 3 * H * dk:
        raise ValueError("x must hold 3*H*d channels")
    N = state_indices.numel()
    _shape(out, "out", (T, H, dv), x.dtype)
    _shape(conv_weight, "conv_weight", (C, None))
    _shape(conv_bias, "conv_bias", (C,))
    _shape(conv_state_pool, "conv_state_pool", (None, conv_weight.shape[1] - 1, C))
    _shape(g, "g", (T, H, dk))
    _shape(beta, "beta", (T, H))
    _shape(cu_seqlens, "cu_seqlens", (N + 1,))
    _shape(state_indices, "state_indices", (N,))
    _shape(has_initial_state, "has_initial_state", (N,))
    _shape(state_pool, "state_pool", (None, H, dk, dv))
    _shape(checkpoints, "checkpoints", (None, H, dk, dv), state_pool.dtype)
    _shape(workspace, "workspace", (None,), torch.uint8)
    nrm = _norm_args(norm_gate, norm_weight, norm_out, T, H, dv, x.dtype)
    _on_device(("x", x), ("conv_weight", conv_weight), ("conv_bias", conv_bias),
               ("conv_state_pool", conv_state_pool), ("g", g), ("beta", beta),
               ("cu_seqlens", cu_seqlens), ("state_pool", state_pool),
               ("state_indices", state_indices), ("out", out), ("workspace", workspace),
               ("has_initial_state", has_initial_state), ("checkpoints", checkpoints),
               ("norm_gate", norm_gate), ("norm_out", norm_out), ("norm_weight", norm_weight))
    if x.stride(1) != 1:
        raise ValueError("x needs contiguous channels")
    W = conv_weight.shape[1]
    _contig(conv_weight, "conv_weight", x.dtype)
    if conv_bias is not None:
        _contig(conv_bias, "conv_bias", x.dtype)
    if not conv_state_pool.is_contiguous() or conv_state_pool.dtype != x.dtype:
        raise ValueError("conv_state_pool must be contiguous with x's dtype")
    _contig(g, "g", torch.float32)
    _contig(beta, "beta", torch.float32)
    _contig(cu_seqlens, "cu_seqlens", torch.int32)
    _contig(state_indices, "state_indices", torch.int32)
    if has_initial_state is not None:
        _contig(has_initial_state, "has_initial_state", torch.uint8)
    if not state_pool.is_contiguous():
        raise ValueError("state_pool must be contiguous")
    nrm = _norm_ptrs(nrm, x.dtype)
    need = chunk_prefill_workspace_size(N, T, H, dk, dv, chunk_size, norm=nrm is not None)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    cap = 0
    if checkpoints is not None:
        if not checkpoints.is_contiguous() or checkpoints.dtype != state_pool.dtype:
            raise ValueError("checkpoints must be contiguous with the state dtype")
        cap = checkpoints.shape[0]
    args = (
        _ptr(x), x.stride(0), _dtype(x), _ptr(conv_weight), _ptr(conv_bias), W,
        KDA_CONV_SILU if silu else 0, _ptr(conv_state_pool),
        _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T, H, dk, dv,
        _ptr(state_pool), _dtype(state_pool), state_pool.shape[0] if state_pool.dim() else 0,
        _ptr(state_indices), _ptr(has_initial_state),
        _ptr(checkpoints), cap, int(ckpt_interval),
        float(scale), int(chunk_size), int(flags),
        _ptr(out), _token_stride(out, "out"))
    ws_tail = (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if nrm is not None:
        _check("kda_conv_chunk_prefill_norm",
               _lib.kda_conv_chunk_prefill_norm(*args, *nrm, float(norm_eps), _ptr(norm_out),
                                                _token_stride(norm_out, "norm_out"), *ws_tail))
        return
    _check("kda_conv_chunk_prefill", _lib.kda_conv_chunk_prefill(*args, *ws_tail))


def recurrent_decode(q, k, v, g, beta, state_pool, state_indices, out, *, scale: float = 1.0,
                     flags: int = 0, stream=None) -> None:
    """kda_recurrent_decode.  q,k [B,H,dk]; v,out [B,H,dv] (row-strided views
    allowed); g [B,H,dk] fp32; beta [B,H] fp32; state_pool updated in place."""
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q and v must be [rows, heads, dim]")
    B, H, dk = q.shape
    dv = v.shape[2]
    _shape(k, "k", (B, H, dk), q.dtype)
    _shape(v, "v", (B, H, dv), q.dtype)
    _shape(out, "out", (B, H, dv), q.dtype)
    _shape(g, "g", (B, H, dk))
    _shape(beta, "beta", (B, H))
    _shape(state_indices, "state_indices", (B,))
    _shape(state_pool, "state_pool", (None, H, dk, dv))
    _on_device(("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state_pool", state_pool),
               ("state_indices", state_indices), ("out", out))
    _contig(g, "g", torch.float32)
    _contig(beta, "beta", torch.float32)
    _contig(state_indices, "state_indices", torch.int32)
    if not state_pool.is_contiguous():
        raise ValueError("state_pool must be contiguous")
    status = _lib.kda_recurrent_decode(
        _ptr(q), _ptr(k), _ptr(v), _dtype(q),
        _token_stride(q, "q"), _token_stride(k, "k"), _token_stride(v, "v"),
        _ptr(g), _ptr(beta), B, H, dk, dv,
        _ptr(state_pool), _dtype(state_pool), state_pool.shape[0],
        _ptr(state_indices), float(scale), int(flags), _ptr(out), _token_stride(out, "out"),
        _stream(stream))
    _check("kda_recurrent_decode", status)


def spec_decode(q, k, v, g, beta, state_pool, state_indices, token_states, out, *,
                scale: float = 1.0, flags: int = 0, stream=None) -> None:
    """kda_spec_decode.  q,k [B*ntok,H,dk]; v,out [B*ntok,H,dv]; g [B*ntok,H,dk]
    fp32; beta [B*ntok,H] fp32; state_pool read only; token_states
    [B,ntok,H,dk,dv] with the pool's dtype (written)."""
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q and v must be [rows, heads, dim]")
    R, H, dk = q.shape
    dv = v.shape[2]
    B = state_indices.numel()
    _shape(state_indices, "state_indices", (B,))
    if B == 0:
        return
    if R % B:
        raise ValueError("token rows must be batch * ntok")
    ntok = R // B
    _shape(k, "k", (R, H, dk), q.dtype)
    _shape(v, "v", (R, H, dv), q.dtype)
    _shape(out, "out", (R, H, dv), q.dtype)
    _shape(g, "g", (R, H, dk))
    _shape(beta, "beta", (R, H))
    _shape(state_pool, "state_pool", (None, H, dk, dv))
    _on_device(("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state_pool", state_pool),
               ("state_indices", state_indices), ("token_states", token_states), ("out", out))
    _contig(g, "g", torch.float32)
    _contig(beta, "beta", torch.float32)
    _contig(state_indices, "state_indices", torch.int32)
    if not state_pool.is_contiguous():
        raise ValueError("state_pool must be contiguous")
    if (not token_states.is_contiguous() or token_states.dtype != state_pool.dtype
            or tuple(token_states.shape) != (B, ntok, H, dk, dv)):
        raise ValueError("token_states must be contiguous [B, ntok, H, dk, dv] in the pool dtype")
    status = _lib.kda_spec_decode(
        _ptr(q), _ptr(k), _ptr(v), _dtype(q),
        _token_stride(q, "q"), _token_stride(k, "k"), _token_stride(v, "v"),
        _ptr(g), _ptr(beta), B, ntok, H, dk, dv,
        _ptr(state_pool), _dtype(state_pool), state_pool.shape[0],
        _ptr(state_indices), _ptr(token_states), float(scale), int(flags),
        _ptr(out), _token_stride(out, "out"), _stream(stream))
    _check("kda_spec_decode", status)


def spec_commit(token_states, num_accepted, state_pool, state_indices, *, stream=None) -> None:
    """kda_spec_commit: pool[slot_b] = token_states[b, num_accepted[b] - 1]."""
    if token_states.dim() != 5:
        raise ValueError("token_states must be [B, ntok, H, dk, dv]")
    B, ntok, H, dk, dv = token_states.shape
    _shape(num_accepted, "num_accepted", (B,))
    _shape(state_indices, "state_indices", (B,))
    _shape(state_pool, "state_pool", (None, H, dk, dv))
    _on_device(("token_states", token_states), ("num_accepted", num_accepted),
               ("state_pool", state_pool), ("state_indices", state_indices))
    _contig(num_accepted, "num_accepted", torch.int32)
    _contig(state_indices, "state_indices", torch.int32)
    if not state_pool.is_contiguous() or state_pool.dtype != token_states.dtype:
        raise ValueError("state_pool must be contiguous with the token states' dtype")
    status = _lib.kda_spec_commit(
        _ptr(token_states), B, ntok, H, dk, dv, _ptr(num_accepted), _ptr(state_pool),
        _dtype(state_pool), state_pool.shape[0], _ptr(state_indices), _stream(stream))
    _check("kda_spec_commit", status)


def gated_rmsnorm(x, gate, y, *, weight=None, eps: float = 1e-6, stream=None) -> None:
    """kda_gated_rmsnorm on [T,H,dim] (token-strided views allowed)."""
    if x.dim() != 3:
        raise ValueError("x must be [tokens, heads, dim]")
    T, H, dim = x.shape
    _shape(gate, "gate", (T, H, dim), x.dtype)
    _shape(y, "y", (T, H, dim), x.dtype)
    _shape(weight, "weight", (dim,))
    _on_device(("x", x), ("gate", gate), ("y", y), ("weight", weight))
    if weight is not None:
        _contig(weight, "weight", x.dtype)
    status = _lib.kda_gated_rmsnorm(
        _ptr(x), _token_stride(x, "x"), _ptr(gate), _token_stride(gate, "gate"),
        _ptr(weight), _ptr(y), _token_stride(y, "y"), _dtype(x), T, H, dim, float(eps),
        _stream(stream))
    _check("kda_gated_rmsnorm", status)


def gated_rmsnorm_ex(x, gate, y, *, residual=None, residual_out=None, weight=None, bias=None,
                     activation: str = "silu", eps: float = 1e-6, stream=None) -> None:
    """kda_gated_rmsnorm_ex on [T,H,dim] (token-strided views allowed).
    residual / residual_out: x's dtype, or both fp32 (KDA_NORM_RESIDUAL_F32);
    activation "silu" or "sigmoid"."""
    if x.dim() != 3:
        raise ValueError("x must be [tokens, heads, dim]")
    T, H, dim = x.shape
    _shape(gate, "gate", (T, H, dim), x.dtype)
    _shape(y, "y", (T, H, dim), x.dtype)
    _shape(residual, "residual", (T, H, dim))
    _shape(residual_out, "residual_out", (T, H, dim))
    _shape(weight, "weight", (dim,))
    _shape(bias, "bias", (dim,))
    _on_device(("x", x), ("gate", gate), ("y", y), ("residual", residual),
               ("residual_out", residual_out), ("weight", weight), ("bias", bias))
    if activation not in ("silu", "sigmoid"):
        raise ValueError("activation must be 'silu' or 'sigmoid'")
    for t, name in ((weight, "weight"), (bias, "bias")):
        if t is not None:
            _contig(t, name, x.dtype)
    rdt = {t.dtype for t in (residual, residual_out) if t is not None}
    if len(rdt) > 1 or (rdt and rdt != {x.dtype} and rdt != {torch.float32}):
        raise ValueError("residual and residual_out must share x's dtype or be fp32")
    flags = KDA_NORM_SIGMOID if activation == "sigmoid" else 0
    if rdt == {torch.float32}:
        flags |= KDA_NORM_RESIDUAL_F32
    status = _lib.kda_gated_rmsnorm_ex(
        _ptr(x), _token_stride(x, "x"), _ptr(gate), _token_stride(gate, "gate"),
        _ptr(residual), 0 if residual is None else _token_stride(residual, "residual"),
        _ptr(weight), _ptr(bias), _ptr(y), _token_stride(y, "y"),
        _ptr(residual_out), 0 if residual_out is None else _token_stride(residual_out, "residual_out"),
        _dtype(x), T, H, dim, float(eps), flags, _stream(stream))
    _check("kda_gated_rmsnorm_ex", status)


def causal_conv1d(x, weight, cu_seqlens, conv_state_pool, state_indices, y, *, bias=None,
                  has_initial_state=None, silu: bool = True, stream=None) -> None:
    """kda_causal_conv1d.  x,y [T,C] (token stride allowed, channels
    contiguous); weight [C,W]; conv_state_pool [slots,W-1,C] updated in place."""
    if x.dim() != 2 or weight.dim() != 2:
        raise ValueError("x must be [tokens, channels] and weight [channels, width]")
    T, C = x.shape
    W = weight.shape[1]
    N = state_indices.numel()
    _shape(y, "y", (T, C), x.dtype)
    _shape(weight, "weight", (C, W))
    _shape(bias, "bias", (C,))
    _shape(conv_state_pool, "conv_state_pool", (None, W - 1, C))
    _shape(cu_seqlens, "cu_seqlens", (N + 1,))
    _shape(state_indices, "state_indices", (N,))
    _shape(has_initial_state, "has_initial_state", (N,))
    _on_device(("x", x), ("weight", weight), ("bias", bias), ("cu_seqlens", cu_seqlens),
               ("conv_state_pool", conv_state_pool), ("state_indices", state_indices),
               ("has_initial_state", has_initial_state), ("y", y))
    if x.stride(1) != 1 or y.stride(1) != 1:
        raise ValueError("x and y need contiguous channels")
    _contig(weight, "weight", x.dtype)
    _contig(cu_seqlens, "cu_seqlens", torch.int32)
    _contig(state_indices, "state_indices", torch.int32)
    if has_initial_state is not None:
        _contig(has_initial_state, "has_initial_state", torch.uint8)
    if not conv_state_pool.is_contiguous() or conv_state_pool.dtype != x.dtype:
        raise ValueError("conv_state_pool must be contiguous with x's dtype")
    status = _lib.kda_causal_conv1d(
        _ptr(x), x.stride(0), _ptr(weight), _ptr(bias), _ptr(conv_state_pool),
        conv_state_pool.shape[0], _ptr(cu_seqlens), _ptr(state_indices),
        _ptr(has_initial_state), state_indices.numel(), T, C, W, _dtype(x),
        KDA_CONV_SILU if silu else 0, _ptr(y), y.stride(0), _stream(stream))
    _check("kda_causal_conv1d", status)


def chunk_prefill_check(workspace, *, stream=None) -> int:
    """kda_chunk_prefill_check: waits for the stream and returns the status
    word the last prefill call on `workspace` left (0 = the call completed
    normally).  Synchronises; a diagnostic, not for the hot path."""
    word = ctypes.c_uint32(0)
    status = _lib.kda_chunk_prefill_check(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                          ctypes.byref(word), _stream(stream))
    if status not in (KDA_OK, KDA_ERR_DEVICE):
        _check("kda_chunk_prefill_check", status)
    return int(word.value)
