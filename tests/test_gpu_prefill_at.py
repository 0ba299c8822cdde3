"""Chunk prefill at absolute start positions (kda_chunk_prefill_at) on the GPU
against the fp64 oracle: chunk boundaries and checkpoints follow absolute
positions, so a sequence resumed from a cached prefix gets the checkpoints a
single call over the whole sequence would have written."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_42_amd import workloads as wl
from tests.gpu_support import DEV, TOL, bits, f64, gpu_prefill, inv_sqrt, max_err, say

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


def ckpt_rows(case: wl.PrefillCase, start) -> list[int]:
    """Checkpoint rows per sequence: multiples of the interval in (p0, p0 + L]."""
    iv = case.ckpt_interval
    if iv <= 0:
        return [0] * case.num_seqs
    return [(p0 + L) // iv - p0 // iv if L > 0 else 0 for p0, L in zip(start, case.lengths)]


def gpu_prefill_at(case: wl.PrefillCase, start, *, pool=None):
    """kda_chunk_prefill_at; returns (o, pool, checkpoints) on the CPU."""
    from gated_delta_rule_42_amd import kda
    q, k, v = case.q.to(DEV), case.k.to(DEV), case.v.to(DEV)
    p = (case.pool if pool is None else pool).to(DEV).clone()
    out = torch.full(v.shape, float("nan"), dtype=v.dtype, device=DEV)
    ck = None
    if case.ckpt_interval > 0:
        rows = max(sum(ckpt_rows(case, start)), 1)
        ck = torch.full((rows,) + tuple(p.shape[1:]), float("nan"), dtype=p.dtype, device=DEV)
    kda.chunk_prefill_at(
        q, k, v, case.g.to(DEV), case.beta.to(DEV), case.cu_seqlens.to(DEV),
        torch.tensor(start, dtype=torch.int64, device=DEV), p, case.slots.to(DEV), out,
        has_initial_state=None if case.has_init is None else case.has_init.to(DEV),
        checkpoints=ck, ckpt_interval=case.ckpt_interval, scale=case.scale,
        chunk_size=case.chunk_size, flags=kda.KDA_FLAG_QK_L2NORM if case.l2norm_qk else 0)
    torch.cuda.synchronize()
    return out.cpu(), p.cpu(), None if ck is None else ck.cpu()


def oracle_prefill_at(case: wl.PrefillCase, start, heads=None, pool=None):
    sel = slice(None) if heads is None else list(heads)
    p = case.pool if pool is None else pool
    return oracle.prefill(
        f64(case.q)[:, sel], f64(case.k)[:, sel], f64(case.v)[:, sel], f64(case.g)[:, sel],
        f64(case.beta)[:, sel], case.cu_seqlens.numpy(), f64(p)[:, sel], case.slots.numpy(),
        has_init=None if case.has_init is None else case.has_init.numpy(),
        ckpt_interval=case.ckpt_interval, scale=case.scale, l2norm_qk=case.l2norm_qk,
        start_pos=start)


def check_at(case, start, got, label, heads=None):
    o_g, p_g, ck_g = got
    o_r, p_r, ck_r = oracle_prefill_at(case, start, heads)
    sel = slice(None) if heads is None else list(heads)
    tol = TOL[case.pool.dtype]
    cu = case.cu_seqlens.tolist()
    slots = case.slots.tolist()
    real = np.concatenate([np.arange(cu[i], cu[i + 1]) for i, s in enumerate(slots) if s >= 0]
                          + [np.zeros(0, np.int64)])
    errs = {"o": max_err(f64(o_g)[real][:, sel], o_r[real])}
    used = sorted({s for s, L in zip(slots, case.lengths) if s >= 0 and L > 0})
    if used:
        errs["state"] = max_err(f64(p_g)[used][:, sel], p_r[used])
    rows, written, base = ckpt_rows(case, start), [], 0
    for s, n in zip(slots, rows):
        if s >= 0:
            written.extend(range(base, base + n))
        base += n
    if written:
        errs["ckpt"] = max_err(f64(ck_g)[written][:, sel], ck_r[written])
    say(f"  {label}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f" (tol {tol:g}),"
        f" checkpoint rows {base}")
    for key, e in errs.items():
        assert e <= tol, f"{label}: {key} {e:.3e} > {tol}"
    untouched = [s for s in range(case.pool.shape[0]) if s not in used]
    assert torch.equal(bits(p_g[untouched]), bits(case.pool[untouched])), f"{label}: other slots"


LENS = [100, 64, 1, 0, 200, 33, 129, 23]
START = [5, 0, 63, 7, 130, 64, 1, 40]
SLOTS = [1, 3, 5, 7, 9, 11, 13, -1]           # the last sequence is padding


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("state", [F32, BF16])
def test_prefill_at_parity(C, state):
    case = wl.random_prefill(800 + C, LENS, 3, 64, 64, state_dtype=state, n_slots=15,
                             slots=SLOTS, has_init=[1, 1, 0, 1, 1, 1, 1, 1], chunk_size=C,
                             ckpt_interval=2 * C, scale=inv_sqrt(64), state_std=0.3)
    check_at(case, START, gpu_prefill_at(case, START), f"prefill_at C={C} state={state}")


@pytest.mark.parametrize("d", [16, 128])
def test_prefill_at_head_dims(d):
    case = wl.random_prefill(810 + d, LENS, 2, d, d, n_slots=15, slots=SLOTS, chunk_size=64,
                             ckpt_interval=64, scale=inv_sqrt(d), state_std=0.3,
                             l2norm_qk=True, qk_unit=False)
    check_at(case, START, gpu_prefill_at(case, START), f"prefill_at d={d} l2norm")


def test_prefill_at_zero_positions_equal_prefill():
    """All positions 0: bit for bit the results of kda_chunk_prefill."""
    case = wl.random_prefill(820, LENS, 3, 128, 128, n_slots=15, slots=SLOTS, chunk_size=64,
                             ckpt_interval=64, state_std=0.3)
    a = gpu_prefill_at(case, [0] * len(LENS))
    b = gpu_prefill(case)
    for name, u, v in zip(("out", "pool", "checkpoints"), a, b):
        assert torch.equal(bits(u), bits(v)), name


def test_prefill_at_resumed_sequence_matches_one_call():
    """One 700-token sequence as calls of 157 and 543 tokens (the second
    starting at position 157, its state carried in the pool): outputs,
    final state and the second call's checkpoints match the oracle's single
    call over all 700 tokens (checkpoints every 128 absolute tokens)."""
    L, cut, iv = 700, 157, 128
    case = wl.random_prefill(830, [L], 4, 128, 128, n_slots=3, slots=[2], chunk_size=64,
                             ckpt_interval=iv, scale=inv_sqrt(128), state_std=0.3)
    o_r, p_r, ck_r = oracle_prefill_at(case, [0])
    parts, pool, cks = [], case.pool, []
    for a, e in ((0, cut), (cut, L)):
        sub = wl.PrefillCase("part", case.q[a:e], case.k[a:e], case.v[a:e], case.g[a:e],
                             case.beta[a:e], torch.tensor([0, e - a], dtype=torch.int32), pool,
                             case.slots, None, 64, iv, case.scale)
        o, pool, ck = gpu_prefill_at(sub, [a])
        parts.append(o)
        cks.append(ck[:ckpt_rows(sub, [a])[0]])
    e_o = max_err(f64(torch.cat(parts)), o_r)
    e_p = max_err(f64(pool)[2], p_r[2])
    e_c = max_err(f64(torch.cat(cks)), ck_r)
    say(f"  resumed at {cut}: o {e_o:.2e}, state {e_p:.2e}, checkpoints {e_c:.2e} "
        f"({sum(c.shape[0] for c in cks)} rows)")
    assert [c.shape[0] for c in cks] == [1, 4]
    assert max(e_o, e_p, e_c) <= TOL[F32]


def test_prefill_at_full_size():
    """4096 tokens, H=16, d=128, resuming at position 1000 with a bf16 state
    and checkpoints every 1024 absolute tokens (at 1024, 2048, 3072, 4096);
    every head against the oracle."""
    case = wl.random_prefill(840, [4096], 16, 128, 128, state_dtype=BF16, n_slots=8, slots=[7],
                             chunk_size=64, ckpt_interval=1024, scale=inv_sqrt(128),
                             state_std=0.02)
    got = gpu_prefill_at(case, [1000])
    assert ckpt_rows(case, [1000]) == [4]
    check_at(case, [1000], got, "prefill_at full size, start 1000")
