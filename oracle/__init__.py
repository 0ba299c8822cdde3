"""fp64 CPU oracle for Kimi Delta Attention -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  The product library never calls it, and
it shares no code with the HIP path.  Every array it takes is converted to
float64 exactly (bf16 and fp32 values are exactly representable in fp64), and
every result is fp64.

Functions (all return new arrays; inputs are never modified):
  prefill(...)      token-by-token recurrence over a varlen batch      (kda_oracle.c)
  decode(...)       one recurrent step per row                         (kda_oracle.c)
  spec_decode(...)  ntok draft tokens per row, state after each token  (kda_oracle.c)
  spec_commit(...)  accept a prefix: copy its last state into the pool (kda_oracle.c)
  conv1d(...)       causal depthwise conv1d with rolling conv state    (kda_oracle.c)
  gated_rmsnorm(...) RMSNorm then SiLU gate                           (kda_oracle.c)
  gated_rmsnorm_ex(...) with residual (prenorm sum), bias, sigmoid gate (kda_oracle.c)
  chunk_form.*      the chunked algebra in fp64, a second algorithm used to pin
                    the token loop (see chunk_form.py)

Parity status: the pages print no worked numeric example, so every function
here is pinned by closed forms, invariants, library routines and hand-worked
values (tests/test_oracle_pins.py); none is marked "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):            # a torch tensor: exact widening to fp64
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, dtype=np.int64)


def _ptr(a: np.ndarray | None, kind):
    if a is None:
        return ctypes.cast(None, kind)
    return a.ctypes.data_as(kind)


class Oracle:
    """A loaded oracle library.  `path` may name a rebuilt copy (the mutation
    tests load deliberately broken copies to show the pins catch them)."""

    def __init__(self, path: str):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.kda_oracle_num_threads.restype = ctypes.c_int
        lib.kda_oracle_prefill.restype = ctypes.c_int
        lib.kda_oracle_prefill.argtypes = [
            _f64p, _f64p, _f64p, _f64p, _f64p,
            _i64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _f64p, ctypes.c_int64, _i64p, _u8p,
            _f64p, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_double, ctypes.c_int, ctypes.c_double, _f64p]
        lib.kda_oracle_prefill_at.restype = ctypes.c_int
        lib.kda_oracle_prefill_at.argtypes = [
            _f64p, _f64p, _f64p, _f64p, _f64p,
            _i64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _f64p, ctypes.c_int64, _i64p, _u8p, _i64p,
            _f64p, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_double, ctypes.c_int, ctypes.c_double, _f64p]
        lib.kda_oracle_decode.restype = ctypes.c_int
        lib.kda_oracle_decode.argtypes = [
            _f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _f64p, ctypes.c_int64, _i64p,
            ctypes.c_double, ctypes.c_int, ctypes.c_double, _f64p]
        lib.kda_oracle_spec_decode.restype = ctypes.c_int
        lib.kda_oracle_spec_decode.argtypes = [
            _f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _f64p, ctypes.c_int64, _i64p, _f64p,
            ctypes.c_double, ctypes.c_int, ctypes.c_double, _f64p]
        lib.kda_oracle_spec_commit.restype = ctypes.c_int
        lib.kda_oracle_spec_commit.argtypes = [
            _f64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            _i64p, _f64p, ctypes.c_int64, _i64p]
        lib.kda_oracle_conv1d.restype = ctypes.c_int
        lib.kda_oracle_conv1d.argtypes = [
            _f64p, _f64p, _f64p, _f64p, ctypes.c_int64,
            _i64p, _i64p, _u8p, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int, _f64p]
        lib.kda_oracle_gated_rmsnorm.restype = ctypes.c_int
        lib.kda_oracle_gated_rmsnorm.argtypes = [
            _f64p, _f64p, _f64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, _f64p]
        lib.kda_oracle_gated_rmsnorm_ex.restype = ctypes.c_int
        lib.kda_oracle_gated_rmsnorm_ex.argtypes = [
            _f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            ctypes.c_int, _f64p, _f64p]
        self.lib = lib

    def num_threads(self) -> int:
        return int(self.lib.kda_oracle_num_threads())

    def prefill(self, q, k, v, g, beta, cu_seqlens, pool, slots, has_init=None,
                ckpt_interval: int = 0, ckpt_capacity: int | None = None,
                scale: float = 1.0, l2norm_qk: bool = False, l2_eps: float = 1e-6,
                start_pos=None):
        """Varlen prefill.  q,k,g [T,H,dk]; v [T,H,dv]; beta [T,H];
        cu_seqlens [N+1]; pool [slots,H,dk,dv]; slots [N] (<0 = padding);
        start_pos [N] or None: absolute position of each sequence's first
        token (checkpoints fall at absolute multiples of the interval).
        Returns (o [T,H,dv], new pool, checkpoints [cap,H,dk,dv] or None)."""
        q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
        cu, sl = _i64(cu_seqlens), _i64(slots)
        pool = _f64(pool).copy()
        T, H, dk = q.shape
        dv = v.shape[2]
        n = sl.shape[0]
        assert k.shape == (T, H, dk) and g.shape == (T, H, dk) and v.shape[:2] == (T, H)
        assert beta.shape == (T, H) and cu.shape == (n + 1,) and pool.shape[1:] == (H, dk, dv)
        assert cu[0] == 0 and cu[-1] <= T
        hi = None if has_init is None else np.ascontiguousarray(
            np.asarray(has_init.cpu() if hasattr(has_init, "cpu") else has_init), dtype=np.uint8)
        sp = None if start_pos is None else _i64(start_pos)
        ck = None
        if ckpt_interval > 0:
            lens = np.diff(cu)
            p0 = np.zeros(n, np.int64) if sp is None else sp
            if ckpt_capacity is None:
                ckpt_capacity = int(((p0 + lens) // ckpt_interval - p0 // ckpt_interval).sum())
            ck = np.full((ckpt_capacity, H, dk, dv), np.nan)
        o = np.full((T, H, dv), np.nan)   # rows of no sequence stay NaN
        rc = self.lib.kda_oracle_prefill_at(
            _ptr(q, _f64p), _ptr(k, _f64p), _ptr(v, _f64p), _ptr(g, _f64p), _ptr(beta, _f64p),
            _ptr(cu, _i64p), n, H, dk, dv,
            _ptr(pool, _f64p), pool.shape[0], _ptr(sl, _i64p), _ptr(hi, _u8p), _ptr(sp, _i64p),
            _ptr(ck, _f64p), 0 if ck is None else ck.shape[0], int(ckpt_interval),
            float(scale), int(bool(l2norm_qk)), float(l2_eps), _ptr(o, _f64p))
        if rc != 0:
            raise ValueError(f"kda_oracle_prefill_at failed with status {rc}")
        return o, pool, ck

    def decode(self, q, k, v, g, beta, pool, slots, scale: float = 1.0,
               l2norm_qk: bool = False, l2_eps: float = 1e-6):
        """One step per row.  q,k,g [B,H,dk]; v [B,H,dv]; beta [B,H];
        pool [slots,H,dk,dv]; slots [B] (<0 = padding).  Returns (o, new pool)."""
        q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
        sl = _i64(slots)
        pool = _f64(pool).copy()
        B, H, dk = q.shape
        dv = v.shape[2]
        assert sl.shape == (B,) and pool.shape[1:] == (H, dk, dv)
        o = np.full((B, H, dv), np.nan)
        rc = self.lib.kda_oracle_decode(
            _ptr(q, _f64p), _ptr(k, _f64p), _ptr(v, _f64p), _ptr(g, _f64p), _ptr(beta, _f64p),
            B, H, dk, dv, _ptr(pool, _f64p), pool.shape[0], _ptr(sl, _i64p),
            float(scale), int(bool(l2norm_qk)), float(l2_eps), _ptr(o, _f64p))
        if rc != 0:
            raise ValueError(f"kda_oracle_decode failed with status {rc}")
        return o, pool

    def spec_decode(self, q, k, v, g, beta, pool, slots, ntok: int, scale: float = 1.0,
                    l2norm_qk: bool = False, l2_eps: float = 1e-6):
        """ntok draft tokens per row.  q,k,g [B*ntok,H,dk]; v [B*ntok,H,dv];
        beta [B*ntok,H]; pool [slots,H,dk,dv] (not modified); slots [B].
        Returns (o [B*ntok,H,dv], token_states [B,ntok,H,dk,dv]); token states
        of padding rows are NaN (untouched)."""
        q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
        sl = _i64(slots)
        pool = _f64(pool)
        R, H, dk = q.shape
        dv = v.shape[2]
        B = sl.shape[0]
        assert R == B * ntok and pool.shape[1:] == (H, dk, dv)
        o = np.full((R, H, dv), np.nan)
        ts = np.full((B, ntok, H, dk, dv), np.nan)
        rc = self.lib.kda_oracle_spec_decode(
            _ptr(q, _f64p), _ptr(k, _f64p), _ptr(v, _f64p), _ptr(g, _f64p), _ptr(beta, _f64p),
            B, ntok, H, dk, dv, _ptr(pool, _f64p), pool.shape[0], _ptr(sl, _i64p),
            _ptr(ts, _f64p), float(scale), int(bool(l2norm_qk)), float(l2_eps), _ptr(o, _f64p))
        if rc != 0:
            raise ValueError(f"kda_oracle_spec_decode failed with status {rc}")
        return o, ts

    def spec_commit(self, token_states, accepted, pool, slots):
        """pool[slots[b]] = token_states[b, accepted[b]-1] where accepted[b] > 0.
        Returns the new pool."""
        ts = _f64(token_states)
        acc, sl = _i64(accepted), _i64(slots)
        pool = _f64(pool).copy()
        B, ntok, H, dk, dv = ts.shape
        assert acc.shape == (B,) and sl.shape == (B,) and pool.shape[1:] == (H, dk, dv)
        rc = self.lib.kda_oracle_spec_commit(
            _ptr(ts, _f64p), B, ntok, H, dk, dv, _ptr(acc, _i64p), _ptr(pool, _f64p),
            pool.shape[0], _ptr(sl, _i64p))
        if rc != 0:
            raise ValueError(f"kda_oracle_spec_commit failed with status {rc}")
        return pool

    def conv1d(self, x, w, cu_seqlens, conv_pool, slots, has_init=None, bias=None,
               silu: bool = True):
        """x [T,C]; w [C,W]; conv_pool [slots,W-1,C]. Returns (y, new conv pool)."""
        x, w = _f64(x), _f64(w)
        cu, sl = _i64(cu_seqlens), _i64(slots)
        cp = _f64(conv_pool).copy()
        b = None if bias is None else _f64(bias)
        T, C = x.shape
        W = w.shape[1]
        n = sl.shape[0]
        assert w.shape == (C, W) and cp.shape[1:] == (W - 1, C) and cu.shape == (n + 1,)
        hi = None if has_init is None else np.ascontiguousarray(
            np.asarray(has_init.cpu() if hasattr(has_init, "cpu") else has_init), dtype=np.uint8)
        y = np.full((T, C), np.nan)
        rc = self.lib.kda_oracle_conv1d(
            _ptr(x, _f64p), _ptr(w, _f64p), _ptr(b, _f64p), _ptr(cp, _f64p), cp.shape[0],
            _ptr(cu, _i64p), _ptr(sl, _i64p), _ptr(hi, _u8p), n, C, W, int(bool(silu)),
            _ptr(y, _f64p))
        if rc != 0:
            raise ValueError(f"kda_oracle_conv1d failed with status {rc}")
        return y, cp

    def gated_rmsnorm(self, x, gate, w=None, eps: float = 1e-6):
        """x, gate [..., dim]; w [dim] or None.  Returns y with x's shape."""
        x, gate = _f64(x), _f64(gate)
        shape = x.shape
        dim = shape[-1]
        x2, g2 = x.reshape(-1, dim), gate.reshape(-1, dim)
        ww = None if w is None else _f64(w)
        y = np.full_like(x2, np.nan)
        rc = self.lib.kda_oracle_gated_rmsnorm(
            _ptr(x2, _f64p), _ptr(g2, _f64p), _ptr(ww, _f64p), x2.shape[0], dim, float(eps),
            _ptr(y, _f64p))
        if rc != 0:
            raise ValueError(f"kda_oracle_gated_rmsnorm failed with status {rc}")
        return y.reshape(shape)

    def gated_rmsnorm_ex(self, x, gate, w=None, b=None, eps: float = 1e-6, *, residual=None,
                         sigmoid: bool = False):
        """x, gate, residual [..., dim]; w, b [dim] or None.  Returns (y, h) with
        h = x + residual (x when residual is None), both with x's shape."""
        x, gate = _f64(x), _f64(gate)
        shape = x.shape
        dim = shape[-1]
        x2, g2 = x.reshape(-1, dim), gate.reshape(-1, dim)
        r2 = None if residual is None else _f64(residual).reshape(-1, dim)
        ww = None if w is None else _f64(w)
        bb = None if b is None else _f64(b)
        y = np.full_like(x2, np.nan)
        h = np.full_like(x2, np.nan)
        rc = self.lib.kda_oracle_gated_rmsnorm_ex(
            _ptr(x2, _f64p), _ptr(g2, _f64p), _ptr(r2, _f64p), _ptr(ww, _f64p), _ptr(bb, _f64p),
            x2.shape[0], dim, float(eps), int(bool(sigmoid)), _ptr(y, _f64p), _ptr(h, _f64p))
        if rc != 0:
            raise ValueError(f"kda_oracle_gated_rmsnorm_ex failed with status {rc}")
        return y.reshape(shape), h.reshape(shape)


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    """The oracle built from oracle/kda_oracle.c (built on first use).  The
    environment variable KDA_ORACLE_LIB names another build of the same
    source to load instead (the sanitized one, for the sanitizer test)."""
    global _DEFAULT
    if _DEFAULT is None:
        path = os.environ.get("KDA_ORACLE_LIB")
        if not path:
            path = _build.LIBRARY
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SOURCE):
                _build.build()
        _DEFAULT = Oracle(path)
    return _DEFAULT


def prefill(*args, **kwargs):
    return default().prefill(*args, **kwargs)


def decode(*args, **kwargs):
    return default().decode(*args, **kwargs)


def spec_decode(*args, **kwargs):
    return default().spec_decode(*args, **kwargs)


def spec_commit(*args, **kwargs):
    return default().spec_commit(*args, **kwargs)


def conv1d(*args, **kwargs):
    return default().conv1d(*args, **kwargs)


def gated_rmsnorm(*args, **kwargs):
    return default().gated_rmsnorm(*args, **kwargs)


def gated_rmsnorm_ex(*args, **kwargs):
    return default().gated_rmsnorm_ex(*args, **kwargs)


def num_threads() -> int:
    return default().num_threads()
