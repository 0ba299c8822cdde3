"""kda_chunk_prefill_noalloc -- the prefill on the library's fixed scratch area,
for callers that cannot allocate -- against kda_chunk_prefill, its
workspace twin, through the C ABI on the same inputs.  Both run the same
kernels in the same order, so outputs, final states and checkpoints must be
identical bit for bit (inside the prefill tolerance a fortiori).  Two calls in
a row, the second smaller, so the second starts from the first's leftovers in
the shared area."""
import pytest
import torch

from gated_delta_rule_42_amd import workloads as wl
from tests.gpu_support import DEV, say

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


def _run(case, noalloc: bool):
    from gated_delta_rule_42_amd import kda
    q, k, v = case.q.to(DEV), case.k.to(DEV), case.v.to(DEV)
    g, beta = case.g.to(DEV), case.beta.to(DEV)
    cu, slots = case.cu_seqlens.to(DEV), case.slots.to(DEV)
    hi = None if case.has_init is None else case.has_init.to(DEV)
    pool = case.pool.to(DEV).clone()
    out = torch.full(v.shape, float("nan"), dtype=v.dtype, device=DEV)
    ck = None
    if case.ckpt_interval > 0:
        ck = torch.full((max(case.ckpt_rows(), 1),) + tuple(pool.shape[1:]), float("nan"),
                        dtype=pool.dtype, device=DEV)
    kw = dict(has_initial_state=hi, checkpoints=ck, ckpt_interval=case.ckpt_interval,
              scale=case.scale, chunk_size=case.chunk_size)
    if noalloc:
        kda.chunk_prefill_noalloc(q, k, v, g, beta, cu, pool, slots, out, **kw)
    else:
        kda.chunk_prefill(q, k, v, g, beta, cu, pool, slots, out, **kw)
    torch.cuda.synchronize()
    return out.cpu(), pool.cpu(), None if ck is None else ck.cpu()


def _same(a, b, what):
    assert a.dtype == b.dtype and a.shape == b.shape, what
    assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b), f"{what} differs"


CASES = [
    # A varlen batch with a padding row, checkpoints and a bf16 pool, then a
    # smaller fp32-state call: the second reuses the area the first left.
    ("varlen_bf16_ckpt", lambda: wl.random_prefill(
        31, [700, 1, 257, 1100, 23], 16, 128, 128, act_dtype=BF16, state_dtype=BF16,
        n_slots=12, slots=[3, 0, 7, 11, -1], has_init=[1, 1, 0, 1, 1], chunk_size=64,
        ckpt_interval=256, state_std=0.02, name="noalloc_varlen")),
    ("single_fp32_small", lambda: wl.random_prefill(
        32, [300], 4, 64, 64, act_dtype=BF16, state_dtype=F32, n_slots=2, slots=[1],
        chunk_size=32, state_std=0.02, name="noalloc_small")),
]


def test_noalloc_matches_workspace_prefill_twice():
    for name, make in CASES:
        case = make()
        say(f"noalloc: {name} T={case.total_tokens} H={case.q.shape[1]} d={case.q.shape[2]}")
        ref = _run(case, noalloc=False)
        got = _run(case, noalloc=True)
        _same(got[0], ref[0], f"{name} out")
        _same(got[1], ref[1], f"{name} pool")
        if ref[2] is not None:
            _same(got[2], ref[2], f"{name} checkpoints")
        assert not torch.isnan(got[0].float()).any(), f"{name}: NaN output"


def test_noalloc_rejects_calls_beyond_the_area():
    from gated_delta_rule_42_amd import kda
    # 20,000 tokens at 16 heads of d = 128 need ~640 MB of scratch: refused on
    # the host before anything is enqueued; the outputs stay untouched.
    case = wl.random_prefill(33, [20000], 16, 128, 128, act_dtype=BF16, state_dtype=F32,
                             n_slots=1, slots=[0], chunk_size=64, name="noalloc_too_big")
    assert kda.chunk_prefill_workspace_size(1, 20000, 16, 128, 128, 64) > (128 << 20)
    q = case.q.to(DEV)
    out = torch.zeros(case.v.shape, dtype=case.v.dtype, device=DEV)
    pool = case.pool.to(DEV)
    with pytest.raises(RuntimeError, match="SCRATCH_LIMIT|fixed scratch"):
        kda.chunk_prefill_noalloc(q, case.k.to(DEV), case.v.to(DEV), case.g.to(DEV),
                                  case.beta.to(DEV), case.cu_seqlens.to(DEV), pool,
                                  case.slots.to(DEV), out)
    torch.cuda.synchronize()
    assert not out.any()
