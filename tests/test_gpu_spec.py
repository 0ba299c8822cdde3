"""Speculative multi-token decode and commit on the GPU against the fp64 oracle
(through the C ABI)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_42_amd import workloads as wl
from tests.gpu_support import DEV, TOL, bits, f64, inv_sqrt, max_err, say

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


def gpu_spec(case: wl.SpecCase):
    """Runs kda_spec_decode; returns (o, token_states, pool after) on the CPU."""
    from gated_delta_rule_42_amd import kda
    q, k, v = case.q.to(DEV), case.k.to(DEV), case.v.to(DEV)
    g, beta, slots = case.g.to(DEV), case.beta.to(DEV), case.slots.to(DEV)
    pool = case.pool.to(DEV).clone()
    B, ntok = case.slots.numel(), case.ntok
    H, dk, dv = case.q.shape[1], case.q.shape[2], case.v.shape[2]
    out = torch.full(v.shape, float("nan"), dtype=v.dtype, device=DEV)
    ts = torch.full((B, ntok, H, dk, dv), float("nan"), dtype=pool.dtype, device=DEV)
    kda.spec_decode(q, k, v, g, beta, pool, slots, ts, out, scale=case.scale,
                    flags=kda.KDA_FLAG_QK_L2NORM if case.l2norm_qk else 0)
    torch.cuda.synchronize()
    return out.cpu(), ts.cpu(), pool.cpu()


def check_spec(case: wl.SpecCase, label: str):
    import oracle
    o_g, ts_g, pool_g = gpu_spec(case)
    o_r, ts_r = oracle.spec_decode(case.q, case.k, case.v, case.g, case.beta, case.pool,
                                   case.slots, case.ntok, scale=case.scale,
                                   l2norm_qk=case.l2norm_qk)
    tol = TOL[case.pool.dtype]
    real = [b for b, s in enumerate(case.slots.tolist()) if s >= 0]
    pad = [b for b, s in enumerate(case.slots.tolist()) if s < 0]
    rows = np.concatenate([np.arange(b * case.ntok, (b + 1) * case.ntok) for b in real])
    e_o = max_err(f64(o_g)[rows], o_r[rows])
    e_s = max_err(f64(ts_g)[real], ts_r[real])
    say(f"  {label}: o {e_o:.2e}, token states {e_s:.2e} (tol {tol:g})")
    assert e_o <= tol and e_s <= tol, label
    assert torch.equal(bits(pool_g), bits(case.pool)), f"{label}: the pool was written"
    for b in pad:
        assert torch.count_nonzero(o_g[b * case.ntok:(b + 1) * case.ntok]) == 0
        assert torch.isnan(ts_g[b].float()).all(), f"{label}: padding row token states written"


@pytest.mark.parametrize("ntok", [1, 3, 4])
@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("state", [F32, BF16])
def test_spec_parity(ntok, d, state):
    B = 6
    slots = list(np.random.default_rng(ntok * d).permutation(13)[:B])
    slots[2] = -1                                   # one padding row
    case = wl.random_spec(500 + ntok + d, B, ntok, 3, d, d, state_dtype=state, n_slots=13,
                          slots=slots, scale=inv_sqrt(d), state_std=0.3)
    check_spec(case, f"spec ntok={ntok} d={d} state={state}")


def test_spec_l2norm_and_fp32_activations():
    case = wl.random_spec(61, 4, 3, 2, 64, 64, act_dtype=F32, qk_unit=False, l2norm_qk=True,
                          state_std=0.3)
    check_spec(case, "spec l2norm fp32 act")


def test_spec_one_token_equals_decode():
    """ntok = 1 runs the decode arithmetic: token state 0 equals the state
    decode writes into the pool, bit for bit, and the outputs agree bitwise."""
    from gated_delta_rule_42_amd import kda
    case = wl.random_spec(62, 8, 1, 4, 128, 128, state_std=0.3)
    o_s, ts, _ = gpu_spec(case)
    pool = case.pool.to(DEV).clone()
    out = torch.empty_like(case.v, device=DEV)
    kda.recurrent_decode(case.q.to(DEV), case.k.to(DEV), case.v.to(DEV), case.g.to(DEV),
                         case.beta.to(DEV), pool, case.slots.to(DEV), out)
    torch.cuda.synchronize()
    slots = case.slots.tolist()
    for b, s in enumerate(slots):
        assert torch.equal(bits(ts[b, 0]), bits(pool[s].cpu())), f"row {b}"
    assert torch.equal(bits(o_s), bits(out.cpu()))


@pytest.mark.parametrize("state", [F32, BF16])
def test_spec_commit(state):
    """Commit copies token_states[b, n_b - 1] into the row's slot bit for bit;
    n_b = 0, padding rows and other slots keep their state."""
    from gated_delta_rule_42_amd import kda
    import oracle
    B, ntok = 7, 3
    slots = [5, 0, -1, 9, 2, 11, 7]
    case = wl.random_spec(63, B, ntok, 2, 64, 64, state_dtype=state, n_slots=12, slots=slots,
                          state_std=0.3)
    acc = torch.tensor([2, 0, 3, 3, 1, 0, 3], dtype=torch.int32)
    _, ts, _ = gpu_spec(case)
    pool = case.pool.to(DEV).clone()
    kda.spec_commit(ts.to(DEV), acc.to(DEV), pool, case.slots.to(DEV))
    torch.cuda.synchronize()
    pool = pool.cpu()
    for b, (s, n) in enumerate(zip(slots, acc.tolist())):
        if s < 0:
            continue
        want = ts[b, n - 1] if n > 0 else case.pool[s]
        assert torch.equal(bits(pool[s]), bits(want)), f"row {b}"
    touched = {s for s in slots if s >= 0}
    for s in range(12):
        if s not in touched:
            assert torch.equal(bits(pool[s]), bits(case.pool[s])), f"slot {s}"
    # The committed states match the oracle's commit of its own token states.
    _, ts_r = oracle.spec_decode(case.q, case.k, case.v, case.g, case.beta, case.pool,
                                 case.slots, ntok)
    ts_r = np.nan_to_num(ts_r)
    p_r = oracle.spec_commit(ts_r, acc, case.pool, case.slots)
    e = max_err(f64(pool), p_r)
    say(f"  commit state={state}: pool {e:.2e}")
    assert e <= TOL[state]


def test_spec_full_size():
    """512 rows x 4 draft tokens, H=16, d=128, fp32 pool of 1024 slots; every
    row and head against the oracle."""
    import oracle
    case = wl.spec_batch()
    o_g, ts_g, pool_g = gpu_spec(case)
    assert torch.equal(bits(pool_g), bits(case.pool))
    sel = list(range(case.slots.numel()))
    rows = np.concatenate([np.arange(b * 4, (b + 1) * 4) for b in sel])
    o_r, ts_r = oracle.spec_decode(case.q[rows], case.k[rows], case.v[rows], case.g[rows],
                                   case.beta[rows], case.pool, case.slots[sel], 4)
    e_o = max_err(f64(o_g)[rows], o_r)
    e_s = max_err(f64(ts_g)[sel], ts_r)
    say(f"  {case.name} ({len(sel)} rows): o {e_o:.2e}, token states {e_s:.2e}")
    assert e_o <= TOL[F32] and e_s <= TOL[F32]
