"""Seeded synthetic inputs for the KDA workloads.

This module draws inputs only: it imports neither the HIP library nor the
oracle and holds none of the method's arithmetic.  Tests, the smoke check and
the benchmark all take their inputs from here, so the GPU path and the oracle
always see the same values.

Recipe (every workload):
  * numpy.random.default_rng(seed); structure first (lengths, slots), then
    values in the fixed order q, k, v, beta logits, g logits, state, extras;
  * q, k ~ N(0, 1), L2-normalised per (token, head) in fp64 (plain division by
    the norm), then cast round-to-nearest-even to the activation dtype;
    v ~ N(0, 1);
  * beta = sigmoid(N(0, 1)) and g = -softplus(N(0, 1)), drawn in fp64, stored
    fp32 (g is the per-key-channel log-decay, so alpha = exp(g) is in (0, 1));
  * pool states ~ N(0, std) with std 0.02 where a non-zero state is asked for.
The oracle consumes the cast values exactly (widened to fp64).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

BF16 = torch.bfloat16
F32 = torch.float32


def _to(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def _neg_softplus(z: np.ndarray) -> np.ndarray:
    return -(np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z))))


@dataclass
class PrefillCase:
    """One call of the chunk prefill.  All tensors live on the CPU."""
    name: str
    q: torch.Tensor            # [T, H, dk] act dtype
    k: torch.Tensor            # [T, H, dk] act dtype
    v: torch.Tensor            # [T, H, dv] act dtype
    g: torch.Tensor            # [T, H, dk] fp32 log-decay
    beta: torch.Tensor         # [T, H] fp32
    cu_seqlens: torch.Tensor   # [N + 1] int32
    pool: torch.Tensor         # [n_slots, H, dk, dv] state dtype
    slots: torch.Tensor        # [N] int32, < 0 = padding
    has_init: torch.Tensor | None  # [N] uint8 or None (= all have a state)
    chunk_size: int = 64
    ckpt_interval: int = 0
    scale: float = 1.0
    l2norm_qk: bool = False

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_seqs(self) -> int:
        return int(self.slots.shape[0])

    @property
    def lengths(self) -> list[int]:
        cu = self.cu_seqlens.tolist()
        return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]

    def ckpt_rows(self) -> int:
        if self.ckpt_interval <= 0:
            return 0
        return sum(L // self.ckpt_interval for L in self.lengths)


@dataclass
class DecodeCase:
    name: str
    q: torch.Tensor            # [B, H, dk]
    k: torch.Tensor
    v: torch.Tensor            # [B, H, dv]
    g: torch.Tensor            # [B, H, dk] fp32
    beta: torch.Tensor         # [B, H] fp32
    pool: torch.Tensor         # [n_slots, H, dk, dv]
    slots: torch.Tensor        # [B] int32, < 0 = padding row
    scale: float = 1.0
    l2norm_qk: bool = False


def _draw_tokens(rng, T, H, dk, dv, act_dtype, qk_unit=True, g_scale=1.0):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if qk_unit:
        q, k = _unit_rows(q), _unit_rows(k)
    v = rng.standard_normal((T, H, dv))
    beta = _sigmoid(rng.standard_normal((T, H)))
    g = g_scale * _neg_softplus(rng.standard_normal((T, H, dk)))
    return (_to(q, act_dtype), _to(k, act_dtype), _to(v, act_dtype),
            _to(g, F32), _to(beta, F32))


def _draw_pool(rng, n_slots, H, dk, dv, state_dtype, std):
    if std == 0.0:
        return torch.zeros((n_slots, H, dk, dv), dtype=state_dtype)
    x = rng.standard_normal((n_slots, H, dk, dv), dtype=np.float32)
    x *= np.float32(std)
    return torch.from_numpy(x).to(state_dtype)


def random_prefill(seed: int, lengths, H: int, dk: int, dv: int, *,
                   act_dtype=BF16, state_dtype=F32, n_slots: int | None = None,
                   slots=None, has_init=None, chunk_size: int = 64,
                   ckpt_interval: int = 0, scale: float = 1.0, state_std: float = 0.02,
                   qk_unit: bool = True, l2norm_qk: bool = False, g_scale: float = 1.0,
                   name: str = "random_prefill") -> PrefillCase:
    """A varlen prefill with explicit structure.  `slots` defaults to distinct
    random slots; `has_init` None means every sequence carries a state."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in lengths]
    N = len(lengths)
    if n_slots is None:
        n_slots = max(N, 1) * 2
    if slots is None:
        slots = rng.choice(n_slots, N, replace=False) if N else np.zeros(0, np.int64)
    slots = np.asarray(slots, dtype=np.int32)
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q, k, v, g, beta = _draw_tokens(rng, T, H, dk, dv, act_dtype, qk_unit, g_scale)
    pool = _draw_pool(rng, n_slots, H, dk, dv, state_dtype, state_std)
    hi = None if has_init is None else torch.tensor(np.asarray(has_init, dtype=np.uint8))
    return PrefillCase(name, q, k, v, g, beta, torch.from_numpy(cu), pool,
                       torch.from_numpy(slots), hi, chunk_size, ckpt_interval, scale,
                       l2norm_qk)


def tiny_prefill(seed: int = 1) -> PrefillCase:
    """1 sequence, T=64, H=2, d=16, C=16, fp32 everywhere, zero initial state."""
    return random_prefill(seed, [64], 2, 16, 16, act_dtype=F32, state_dtype=F32,
                          n_slots=1, slots=[0], has_init=[0], chunk_size=16,
                          state_std=0.0, name="tiny_prefill_T64_H2_d16_C16_fp32")


def single_seq_prefill(seed: int = 2) -> PrefillCase:
    """T=4096, H=16, d=128, C=64, bf16 q/k/v, fp32 64-slot pool, slot 7."""
    rng = np.random.default_rng(seed)
    T, H, d = 4096, 16, 128
    q, k, v, g, beta = _draw_tokens(rng, T, H, d, d, BF16)
    pool = _draw_pool(rng, 64, H, d, d, F32, 0.02)
    return PrefillCase("prefill_T4096_H16_d128_C64_bf16_f32state", q, k, v, g, beta,
                       torch.tensor([0, T], dtype=torch.int32), pool,
                       torch.tensor([7], dtype=torch.int32), None, 64, 0, 1.0)


def varlen_lengths(rng, n=8, lo=256, hi=4096, cap=16384) -> list[int]:
    while True:
        lens = rng.integers(lo, hi + 1, n)
        if int(lens.sum()) <= cap:
            return [int(x) for x in lens]


def varlen_prefill(seed: int = 3, state_dtype=BF16) -> PrefillCase:
    """8 sequences, lengths U[256,4096] with total <= 16384, H=16, d=128,
    bf16 q/k/v, 256-slot bf16 pool (or fp32: the same draws, rounded to the
    pool dtype) with distinct random slots, checkpoints every 1024 tokens."""
    rng = np.random.default_rng(seed)
    lens = varlen_lengths(rng)
    slots = rng.choice(256, len(lens), replace=False).astype(np.int32)
    H, d = 16, 128
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    q, k, v, g, beta = _draw_tokens(rng, int(cu[-1]), H, d, d, BF16)
    pool = _draw_pool(rng, 256, H, d, d, state_dtype, 0.02)
    tag = "bf16state" if state_dtype == BF16 else "f32state"
    return PrefillCase(f"varlen_prefill_8seq_H16_d128_{tag}_ckpt1024", q, k, v, g, beta,
                       torch.from_numpy(cu), pool, torch.from_numpy(slots), None,
                       64, 1024, 1.0)


def random_decode(seed: int, B: int, H: int, dk: int, dv: int, *, act_dtype=BF16,
                  state_dtype=F32, n_slots: int | None = None, slots=None,
                  scale: float = 1.0, state_std: float = 0.02, qk_unit: bool = True,
                  l2norm_qk: bool = False, name: str = "random_decode") -> DecodeCase:
    rng = np.random.default_rng(seed)
    if n_slots is None:
        n_slots = 2 * B
    if slots is None:
        slots = rng.permutation(n_slots)[:B]
    slots = np.asarray(slots, dtype=np.int32)
    q, k, v, g, beta = _draw_tokens(rng, B, H, dk, dv, act_dtype, qk_unit)
    pool = _draw_pool(rng, n_slots, H, dk, dv, state_dtype, state_std)
    return DecodeCase(name, q, k, v, g, beta, pool, torch.from_numpy(slots), scale, l2norm_qk)


@dataclass
class SpecCase:
    """Speculative decode: ntok draft tokens for each of B rows."""
    name: str
    q: torch.Tensor            # [B*ntok, H, dk]
    k: torch.Tensor
    v: torch.Tensor            # [B*ntok, H, dv]
    g: torch.Tensor            # [B*ntok, H, dk] fp32
    beta: torch.Tensor         # [B*ntok, H] fp32
    pool: torch.Tensor         # [n_slots, H, dk, dv]
    slots: torch.Tensor        # [B] int32, < 0 = padding row
    accepted: torch.Tensor     # [B] int32 in [0, ntok]: a verifier's decision
    ntok: int
    scale: float = 1.0
    l2norm_qk: bool = False


def random_spec(seed: int, B: int, ntok: int, H: int, dk: int, dv: int, *, act_dtype=BF16,
                state_dtype=F32, n_slots: int | None = None, slots=None, scale: float = 1.0,
                state_std: float = 0.02, qk_unit: bool = True, l2norm_qk: bool = False,
                name: str = "random_spec") -> SpecCase:
    """B rows of ntok draft tokens (rows b*ntok + t), slots a random
    permutation prefix, accepted prefix lengths uniform in [0, ntok]."""
    rng = np.random.default_rng(seed)
    if n_slots is None:
        n_slots = 2 * B
    if slots is None:
        slots = rng.permutation(n_slots)[:B]
    slots = np.asarray(slots, dtype=np.int32)
    q, k, v, g, beta = _draw_tokens(rng, B * ntok, H, dk, dv, act_dtype, qk_unit)
    pool = _draw_pool(rng, n_slots, H, dk, dv, state_dtype, state_std)
    accepted = rng.integers(0, ntok + 1, B).astype(np.int32)
    return SpecCase(name, q, k, v, g, beta, pool, torch.from_numpy(slots),
                    torch.from_numpy(accepted), ntok, scale, l2norm_qk)


def spec_batch(seed: int = 6) -> SpecCase:
    """512 rows x 4 draft tokens, H=16, d=128, bf16 q/k/v, fp32 pool of 1024
    slots indexed by a random permutation (the decode batch, speculating 4
    tokens)."""
    return random_spec(seed, 512, 4, 16, 128, 128, n_slots=1024,
                       name="spec_B512_ntok4_H16_d128_bf16_f32pool1024")


def decode_batch(seed: int = 4) -> DecodeCase:
    """512 sequences x 1 token, H=16, d=128, bf16 q/k/v, fp32 pool of 1024
    slots indexed by a random permutation."""
    rng = np.random.default_rng(seed)
    slots = rng.permutation(1024)[:512].astype(np.int32)
    B, H, d = 512, 16, 128
    q, k, v, g, beta = _draw_tokens(rng, B, H, d, d, BF16)
    pool = _draw_pool(rng, 1024, H, d, d, F32, 0.02)
    return DecodeCase("decode_B512_H16_d128_bf16_f32pool1024", q, k, v, g, beta, pool,
                      torch.from_numpy(slots), 1.0)


@dataclass
class LongContextCall:
    """One 4096-token call of the long-context pipeline."""
    x: torch.Tensor        # [T, 3*H*d] bf16 pre-conv packed q|k|v
    g: torch.Tensor        # [T, H, d] fp32
    beta: torch.Tensor     # [T, H] fp32
    gate: torch.Tensor     # [T, H, d] bf16 output gate


@dataclass
class LongContextCase:
    name: str
    T_total: int
    T_call: int
    H: int
    d: int
    conv_width: int
    conv_weight: torch.Tensor   # [3*H*d, W] bf16
    norm_weight: torch.Tensor   # [d] bf16
    eps: float
    state_slot: int
    n_slots: int
    ckpt_interval: int
    seed: int
    scale: float = 1.0
    chunk_size: int = 64
    calls_cache: dict = field(default_factory=dict)

    @property
    def n_calls(self) -> int:
        return self.T_total // self.T_call

    @property
    def channels(self) -> int:
        return 3 * self.H * self.d

    def call(self, i: int) -> LongContextCall:
        """Inputs of call i, drawn from their own stream so that calls can be
        generated one at a time in any order."""
        rng = np.random.default_rng([self.seed, i + 1])
        T, H, d = self.T_call, self.H, self.d
        x = rng.standard_normal((T, self.channels), dtype=np.float32)
        beta = _sigmoid(rng.standard_normal((T, H)))
        g = _neg_softplus(rng.standard_normal((T, H, d)))
        gate = rng.standard_normal((T, H, d), dtype=np.float32)
        return LongContextCall(_to(x, BF16), _to(g, F32), _to(beta, F32), _to(gate, BF16))


def long_context(seed: int = 5, T_total: int = 65536, T_call: int = 4096,
                 H: int = 16, d: int = 128) -> LongContextCase:
    """One sequence of T_total tokens as successive T_call-token calls: causal
    depthwise conv1d (width 4, SiLU) over packed q|k|v, KDA with in-kernel q/k
    L2 normalisation and a bf16 state carried through one pool slot, then the
    per-head gated RMSNorm (eps 1e-6); checkpoints every T_call tokens."""
    rng = np.random.default_rng(seed)
    W = 4
    w = rng.uniform(-0.5, 0.5, (3 * H * d, W))
    nw = 1.0 + 0.1 * rng.standard_normal(d)
    return LongContextCase(f"long_context_T{T_total}_as_{T_total // T_call}x{T_call}_H{H}_d{d}",
                           T_total, T_call, H, d, W, _to(w, BF16), _to(nw, BF16), 1e-6,
                           state_slot=2, n_slots=4, ckpt_interval=T_call, seed=seed)
