"""Gated RMSNorm and causal conv1d on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_support import bits, f64, max_err, say

pytestmark = pytest.mark.gpu

F32, BF16, F16 = torch.float32, torch.bfloat16, torch.float16


def _excess(got, ref, dtype) -> float:
    """Largest error beyond what rounding the output to `dtype` explains:
    |got - ref| - 2^-8 |ref| for bf16 (RNE is within 2^-9 relative), 2^-10 |ref|
    for fp16 (within 2^-11), the plain error for fp32.  fp32 arithmetic leaves
    ~1e-6."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    slack = {BF16: 2.0 ** -8, F16: 2.0 ** -10}.get(dtype, 0.0) * np.abs(ref)
    return float(np.max(np.abs(got - ref) - slack)) if got.size else 0.0


TOL_ABS = 1e-4


@pytest.mark.parametrize("dtype", [BF16, F32])
@pytest.mark.parametrize("dim", [128, 64, 96, 512])
@pytest.mark.parametrize("weighted", [True, False])
def test_gated_rmsnorm(dtype, dim, weighted):
    from gated_delta_rule_42_amd import kda
    g = torch.Generator().manual_seed(dim)
    T, H = 37, 5
    x = torch.randn(T, H, dim, generator=g).to(dtype)
    gate = torch.randn(T, H, dim, generator=g).to(dtype)
    w = (1 + 0.1 * torch.randn(dim, generator=g)).to(dtype) if weighted else None
    xd, gd = x.cuda(), gate.cuda()
    y = torch.empty_like(xd)
    kda.gated_rmsnorm(xd, gd, y, weight=None if w is None else w.cuda(), eps=1e-6)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(f64(x), f64(gate), None if w is None else f64(w), 1e-6)
    e = _excess(f64(y), ref, dtype)
    say(f"  rmsnorm {dtype} dim={dim} weighted={weighted}: max abs {max_err(f64(y), ref):.2e}, "
        f"beyond output rounding {e:.2e}")
    assert e <= TOL_ABS
    assert torch.equal(bits(xd.cpu()), bits(x)), "input must be preserved"


def test_gated_rmsnorm_packed_gate():
    """The gate read in place from a wider packed tensor."""
    from gated_delta_rule_42_amd import kda
    g = torch.Generator().manual_seed(9)
    T, H, d = 20, 4, 128
    x = torch.randn(T, H, d, generator=g).to(BF16).cuda()
    packed = torch.randn(T, 3 * H * d, generator=g).to(BF16).cuda()
    gate = packed[:, H * d:2 * H * d].view(T, H, d)
    y = torch.empty_like(x)
    kda.gated_rmsnorm(x, gate, y)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(f64(x), f64(gate.contiguous()), None, 1e-6)
    assert _excess(f64(y), ref, BF16) <= TOL_ABS


@pytest.mark.parametrize("dtype", [F16, BF16, F32])
@pytest.mark.parametrize("activation", ["silu", "sigmoid"])
@pytest.mark.parametrize("residual", [None, "same", "fp32"])
def test_gated_rmsnorm_variants(dtype, activation, residual):
    """kda_gated_rmsnorm_ex: fp16/bf16/fp32, SiLU or sigmoid gate, weight and
    bias, a packed (strided) gate, residual in x's dtype or fp32 with the
    prenorm sum written out; inputs preserved."""
    from gated_delta_rule_42_amd import kda
    if residual == "fp32" and dtype == F32:
        pytest.skip("fp32 data already has an fp32 residual")
    g = torch.Generator().manual_seed(17)
    T, H, dim = 29, 3, 128
    x = torch.randn(T, H, dim, generator=g).to(dtype)
    packed = torch.randn(T, 3 * H * dim, generator=g).to(dtype)
    gate_h = packed[:, H * dim:2 * H * dim].reshape(T, H, dim)
    w = (1 + 0.1 * torch.randn(dim, generator=g)).to(dtype)
    b = (0.2 * torch.randn(dim, generator=g)).to(dtype)
    rdt = None if residual is None else (F32 if residual == "fp32" else dtype)
    r = None if rdt is None else torch.randn(T, H, dim, generator=g).to(rdt)
    xd, pd = x.cuda(), packed.cuda()
    gd = pd[:, H * dim:2 * H * dim].view(T, H, dim)
    rd = None if r is None else r.cuda()
    y = torch.full_like(xd, float("nan"))
    ro = torch.full((T, H, dim), float("nan"), dtype=rdt or dtype, device="cuda")
    kda.gated_rmsnorm_ex(xd, gd, y, residual=rd, residual_out=ro, weight=w.cuda(), bias=b.cuda(),
                         activation=activation, eps=1e-6)
    torch.cuda.synchronize()
    y_r, h_r = oracle.gated_rmsnorm_ex(f64(x), f64(gate_h), f64(w), f64(b), 1e-6,
                                       residual=None if r is None else f64(r),
                                       sigmoid=activation == "sigmoid")
    e = _excess(f64(y), y_r, dtype)
    say(f"  norm {dtype} {activation} residual={residual}: max abs {max_err(f64(y), y_r):.2e}, "
        f"beyond output rounding {e:.2e}")
    assert e <= TOL_ABS
    # The prenorm output is the fp32 sum rounded to its type.
    want = x.float() + (0 if r is None else r.float())
    assert torch.equal(bits(ro.cpu()), bits(want.to(rdt or dtype))), "residual_out"
    assert max_err(f64(ro), h_r) <= (0.0 if (rdt or dtype) == F32 and r is None else 2e-2)
    assert torch.equal(bits(xd.cpu()), bits(x)) and torch.equal(bits(pd.cpu()), bits(packed))
    if rd is not None:
        assert torch.equal(bits(rd.cpu()), bits(r))


@pytest.mark.parametrize("dim", [64, 96, 512, 1024, 8])
def test_gated_rmsnorm_variants_dims_no_affine(dim):
    """No weight, no bias, no residual_out, other row widths: equals the
    plain kda_gated_rmsnorm bit for bit for the SiLU gate."""
    from gated_delta_rule_42_amd import kda
    g = torch.Generator().manual_seed(dim + 1)
    T, H = 13, 2
    x = torch.randn(T, H, dim, generator=g).to(F16).cuda()
    gate = torch.randn(T, H, dim, generator=g).to(F16).cuda()
    y1, y2 = torch.empty_like(x), torch.empty_like(x)
    kda.gated_rmsnorm_ex(x, gate, y1)
    kda.gated_rmsnorm(x, gate, y2)
    y3 = torch.empty_like(x)
    kda.gated_rmsnorm_ex(x, gate, y3, activation="sigmoid")
    torch.cuda.synchronize()
    assert torch.equal(bits(y1.cpu()), bits(y2.cpu()))
    ref, _ = oracle.gated_rmsnorm_ex(f64(x), f64(gate), None, None, 1e-6, sigmoid=True)
    assert _excess(f64(y3), ref, F16) <= TOL_ABS


def _conv_case(seed, lens, C, W, dtype, slots, has_init, bias):
    g = torch.Generator().manual_seed(seed)
    T = sum(lens)
    x = torch.randn(T, C, generator=g).to(dtype)
    w = (torch.rand(C, W, generator=g) - 0.5).to(dtype)
    b = torch.randn(C, generator=g).to(dtype) if bias else None
    n_slots = max(slots) + 2
    pool = torch.randn(n_slots, W - 1, C, generator=g).to(dtype)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    return x, w, b, pool, cu, torch.tensor(slots, dtype=torch.int32), \
        None if has_init is None else torch.tensor(has_init, dtype=torch.uint8)


@pytest.mark.parametrize("W", [2, 3, 4, 8])
@pytest.mark.parametrize("dtype", [BF16, F32])
def test_causal_conv1d(W, dtype):
    from gated_delta_rule_42_amd import kda
    lens = [0, 1, 2, 17, 40, 5, 33]
    slots = [0, 1, 2, 3, 4, -1, 6]
    has_init = [1, 1, 0, 1, 0, 1, 1]
    x, w, b, pool, cu, sl, hi = _conv_case(W, lens, 136, W, dtype, slots, has_init, bias=True)
    for silu in (True, False):
        pd = pool.cuda().clone()
        y = torch.full_like(x, float("nan")).cuda()
        kda.causal_conv1d(x.cuda(), w.cuda(), cu.cuda(), pd, sl.cuda(), y, bias=b.cuda(),
                          has_initial_state=hi.cuda(), silu=silu)
        torch.cuda.synchronize()
        y_r, p_r = oracle.conv1d(f64(x), f64(w), cu.numpy(), f64(pool), sl.numpy(),
                                 has_init=hi.numpy(), bias=f64(b), silu=silu)
        cun = cu.numpy()
        real = np.concatenate([np.arange(cun[i], cun[i + 1]) for i in range(len(lens)) if slots[i] >= 0])
        pad = np.arange(cun[5], cun[6])
        e = _excess(f64(y.cpu())[real], y_r[real], dtype)
        assert torch.count_nonzero(y.cpu()[pad]) == 0
        # The new state is a copy of inputs: it must match exactly.
        touched = [s for s, L in zip(slots, lens) if s >= 0 and L > 0]
        assert torch.equal(bits(pd.cpu()[touched]), bits(torch.from_numpy(p_r[touched]).to(dtype)))
        others = [s for s in range(pool.shape[0]) if s not in touched]
        assert torch.equal(bits(pd.cpu()[others]), bits(pool[others]))
        say(f"  conv W={W} {dtype} silu={silu}: beyond output rounding {e:.2e}")
        assert e <= TOL_ABS


def test_causal_conv1d_split_calls():
    """Calls of 1, 2, 37 and 60 tokens in a row through the conv state equal
    one call over the 100 tokens."""
    from gated_delta_rule_42_amd import kda
    x, w, _, pool, _, _, _ = _conv_case(3, [100], 6144, 4, BF16, [1], None, bias=False)
    xd = x.cuda()
    full_pool = pool.cuda().clone()
    y_full = torch.empty_like(xd)
    kda.causal_conv1d(xd, w.cuda(), torch.tensor([0, 100], dtype=torch.int32).cuda(), full_pool,
                      torch.tensor([1], dtype=torch.int32).cuda(), y_full)
    part_pool = pool.cuda().clone()
    ys, a = [], 0
    for n in (1, 2, 37, 60):
        y = torch.empty(n, 6144, dtype=BF16, device="cuda")
        kda.causal_conv1d(xd[a:a + n], w.cuda(), torch.tensor([0, n], dtype=torch.int32).cuda(),
                          part_pool, torch.tensor([1], dtype=torch.int32).cuda(), y)
        ys.append(y)
        a += n
    torch.cuda.synchronize()
    assert torch.equal(bits(torch.cat(ys).cpu()), bits(y_full.cpu()))
    assert torch.equal(bits(part_pool.cpu()), bits(full_pool.cpu()))
