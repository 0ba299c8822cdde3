"""The gated RMSNorm fused into the prefill (kda_chunk_prefill_norm and
kda_conv_chunk_prefill_norm): norm_out bit for bit equal to the plain call
followed by kda_gated_rmsnorm on its output, the call's own results (o,
states, checkpoints, conv states) bit for bit those of the plain call, and at
full size the norm against the fp64 oracle's norm of the stored output on
every head."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_42_amd import workloads as wl
from tests.gpu_support import DEV, assert_device_ok, bits, f64, inv_sqrt, say
from tests.test_gpu_conv_prefill import BF16, F32, _ckpt_buffer, _strided_to_dev, make_case

pytestmark = pytest.mark.gpu


def _gate(T, H, d, dtype, seed, pad=24):
    """A gate read with a token stride wider than H d (a packed projection)."""
    gen = torch.Generator().manual_seed(seed)
    full = torch.randn(T, H * d + pad, generator=gen).to(dtype).to(DEV)
    return full[:, :H * d].view(T, H, d)


def _weight(d, dtype, seed):
    if seed is None:
        return None
    return (1.0 + 0.2 * torch.randn(d, generator=torch.Generator().manual_seed(seed))).to(dtype).to(DEV)


def _same(a, b, what, label):
    if a is None and b is None:
        return
    assert torch.equal(bits(a), bits(b)), f"{label}: {what} differs"


# ---------------------------------------------------------------- plain front end

def _run_plain(case: wl.PrefillCase, *, norm: bool, wseed, eps=1e-6):
    from gated_delta_rule_42_amd import kda
    T, H, d = case.total_tokens, case.g.shape[1], case.g.shape[2]
    q, k, v = case.q.to(DEV), case.k.to(DEV), case.v.to(DEV)
    pool = case.pool.to(DEV).clone()
    ck = _ckpt_buffer(case, pool)
    out = torch.full((T, H, d), float("nan"), dtype=case.v.dtype, device=DEV)
    z = torch.full((T, H, d), float("nan"), dtype=case.v.dtype, device=DEV)
    gate = _gate(T, H, d, case.v.dtype, 7)
    w = _weight(d, case.v.dtype, wseed)
    ws = torch.empty(max(1, kda.chunk_prefill_workspace_size(case.num_seqs, T, H, d, d,
                                                             case.chunk_size, norm=norm)),
                     dtype=torch.uint8, device=DEV)
    kw = dict(workspace=ws, has_initial_state=None if case.has_init is None else case.has_init.to(DEV),
              checkpoints=ck, ckpt_interval=case.ckpt_interval, scale=case.scale,
              chunk_size=case.chunk_size, flags=kda.KDA_FLAG_QK_L2NORM if case.l2norm_qk else 0)
    args = (q, k, v, case.g.to(DEV), case.beta.to(DEV), case.cu_seqlens.to(DEV), pool,
            case.slots.to(DEV), out)
    if norm:
        kda.chunk_prefill(*args, norm_gate=gate, norm_weight=w, norm_eps=eps, norm_out=z, **kw)
    else:
        kda.chunk_prefill(*args, **kw)
        kda.gated_rmsnorm(out, gate, z, weight=w, eps=eps)
    torch.cuda.synchronize()
    assert_device_ok(ws)
    return out.cpu(), pool.cpu(), None if ck is None else ck.cpu(), z.cpu()


PLAIN = [
    # (label, random_prefill args, weight seed)
    ("d=128 C=64 varlen, padding, empty, long", dict(seed=21, lengths=[700, 0, 64, 7, 130], H=4, dk=128, dv=128,
                                                      slots=[3, 1, -1, 0, 5], n_slots=6), 9),
    ("d=64 C=32 bf16 state, ckpt, no init", dict(seed=22, lengths=[300, 33], H=3, dk=64, dv=64,
                                                 state_dtype=BF16, chunk_size=32, ckpt_interval=64,
                                                 has_init=[0, 1]), None),
    ("d=32 C=16 fp32 act", dict(seed=23, lengths=[200, 17], H=2, dk=32, dv=32, act_dtype=F32,
                                chunk_size=16), 9),
    ("d=16 C=16", dict(seed=24, lengths=[150, 1, 23], H=5, dk=16, dv=16, chunk_size=16), None),
    ("d=128 C=16 L2-normalised q,k", dict(seed=25, lengths=[120, 90], H=2, dk=128, dv=128,
                                           chunk_size=16, l2norm_qk=True, qk_unit=False), 9),
    ("d=64 C=64 fp32 act and state", dict(seed=26, lengths=[513], H=2, dk=64, dv=64,
                                          act_dtype=F32, state_dtype=F32), 9),
]


@pytest.mark.parametrize("label,args,wseed", PLAIN, ids=[c[0] for c in PLAIN])
def test_fused_norm_equals_prefill_then_norm(label, args, wseed):
    d = args["dk"]
    case = wl.random_prefill(**args, scale=inv_sqrt(d), state_std=0.3)
    a = _run_plain(case, norm=True, wseed=wseed)
    b = _run_plain(case, norm=False, wseed=wseed)
    for name, u, v in zip(("out", "pool", "checkpoints", "norm out"), a, b):
        _same(u, v, name, label)
    assert not torch.isnan(a[3].float()).any(), f"{label}: NaN left in the norm output"
    say(f"  {label}: fused norm == prefill then norm, bit for bit")


def test_fused_norm_varlen_full_size():
    """The 8-sequence varlen batch (up to 16384 tokens, 16 heads, d = 128,
    checkpoints every 1024): 2048 chain workgroups, more than the chip holds
    at once, so the output workgroups of later pairs start only as earlier
    ones finish.  Everything bit for bit the plain call + the standalone norm."""
    case = wl.varlen_prefill()
    a = _run_plain(case, norm=True, wseed=9)
    b = _run_plain(case, norm=False, wseed=9)
    for name, u, v in zip(("out", "pool", "checkpoints", "norm out"), a, b):
        _same(u, v, name, case.name)
    assert not torch.isnan(a[3].float()).any()
    say(f"  {case.name}: fused norm == prefill then norm, bit for bit")


# ---------------------------------------------------------------- conv front end

def _run_conv(fc, *, norm: bool, wseed, eps=1e-6):
    from gated_delta_rule_42_amd import kda
    base = fc.base
    T, H, d = fc.T, fc.H, fc.d
    x = fc.x.to(DEV) if fc.x.is_contiguous() else _strided_to_dev(fc.x)
    cpool = fc.cpool.to(DEV).clone()
    pool = base.pool.to(DEV).clone()
    ck = _ckpt_buffer(base, pool)
    out = torch.full((T, H, d), float("nan"), dtype=fc.x.dtype, device=DEV)
    z = torch.full((T, H, d), float("nan"), dtype=fc.x.dtype, device=DEV)
    gate = _gate(T, H, d, fc.x.dtype, 8)
    w = _weight(d, fc.x.dtype, wseed)
    ws = torch.empty(max(1, kda.chunk_prefill_workspace_size(base.num_seqs, T, H, d, d,
                                                             base.chunk_size, norm=norm)),
                     dtype=torch.uint8, device=DEV)
    kw = dict(conv_bias=None if fc.b is None else fc.b.to(DEV), silu=fc.silu,
              has_initial_state=None if base.has_init is None else base.has_init.to(DEV),
              checkpoints=ck, ckpt_interval=base.ckpt_interval, scale=base.scale,
              chunk_size=base.chunk_size, flags=kda.KDA_FLAG_QK_L2NORM, workspace=ws)
    args = (x, fc.w.to(DEV), cpool, base.g.to(DEV), base.beta.to(DEV), base.cu_seqlens.to(DEV),
            pool, base.slots.to(DEV), out)
    if norm:
        kda.conv_chunk_prefill(*args, norm_gate=gate, norm_weight=w, norm_eps=eps, norm_out=z, **kw)
    else:
        kda.conv_chunk_prefill(*args, **kw)
        kda.gated_rmsnorm(out, gate, z, weight=w, eps=eps)
    torch.cuda.synchronize()
    assert_device_ok(ws)
    return (out.cpu(), pool.cpu(), None if ck is None else ck.cpu(), cpool.cpu(), z.cpu(),
            gate.cpu(), None if w is None else w.cpu())


CONV = [
    ("d=128 C=64 varlen, padding, empty", dict(seed=1, lens=[450, 0, 64, 7, 200], H=4, d=128, W=4,
                                               slots=[3, 1, -1, 0, 5], n_slots=6), 9),
    ("d=64 C=32 bf16 state, ckpt", dict(seed=2, lens=[290, 33], H=3, d=64, W=3, state=BF16,
                                        chunk=32, ckpt_interval=32), None),
    ("d=32 C=16 fp32 act", dict(seed=3, lens=[150, 17], H=2, d=32, W=2, act=F32, chunk=16), 9),
    ("d=128 C=16 strided x, no bias", dict(seed=5, lens=[177], H=2, d=128, W=4, chunk=16,
                                           bias=False, x_pad=40), 9),
]


@pytest.mark.parametrize("label,args,wseed", CONV, ids=[c[0] for c in CONV])
def test_conv_fused_norm_equals_prefill_then_norm(label, args, wseed):
    fc = make_case(**args)
    a = _run_conv(fc, norm=True, wseed=wseed)
    b = _run_conv(fc, norm=False, wseed=wseed)
    for name, u, v in zip(("out", "pool", "checkpoints", "conv pool", "norm out"), a[:5], b[:5]):
        _same(u, v, name, label)
    assert not torch.isnan(a[4].float()).any(), f"{label}: NaN left in the norm output"
    say(f"  {label}: fused norm == conv prefill then norm, bit for bit")


def test_fused_norm_full_size_all_heads():
    """One 4096-token call, H=16, d=128 (the long-context call's shape: bf16
    state, a checkpoint at 4096): bit for bit the unfused pair, and the norm
    against the fp64 oracle's gated_rmsnorm_ex of the stored output on every
    head, within bf16 output rounding."""
    fc = make_case(seed=6, lens=[4096], H=16, d=128, W=4, state=BF16, slots=[1], n_slots=2,
                   ckpt_interval=4096)
    a = _run_conv(fc, norm=True, wseed=11)
    b = _run_conv(fc, norm=False, wseed=11)
    for name, u, v in zip(("out", "pool", "checkpoints", "conv pool", "norm out"), a[:5], b[:5]):
        _same(u, v, name, "full size")
    o, z, gate, w = f64(a[0]), f64(a[4]), f64(a[5]), f64(a[6])
    z_r, _ = oracle.gated_rmsnorm_ex(o, gate, w, None, 1e-6)
    beyond = float(np.max(np.abs(z - z_r) - 2.0 ** -8 * np.abs(z_r)))
    say(f"  full size, 16 heads: fused norm == unfused; against the oracle's norm of o: "
        f"beyond bf16 output rounding {beyond:.2e}")
    assert beyond <= 1e-4


def test_fused_norm_failure_report():
    """KDA_FLAG_DIAG_GIVE_UP makes every bounded wait of the output
    workgroups give up at once: the call completes, the status word reports
    the timeout and the norm rows are NaN; the next normal call on the same
    workspace is again bit for bit the unfused pair."""
    from gated_delta_rule_42_amd import kda
    case = wl.random_prefill(92, [200, 37], 4, 64, 64, n_slots=4, chunk_size=32, state_std=0.3)
    T, H, d = case.total_tokens, 4, 64
    ws = torch.empty(kda.chunk_prefill_workspace_size(case.num_seqs, T, H, d, d, 32, norm=True),
                     dtype=torch.uint8, device=DEV)
    dev = lambda t: t.to(DEV)
    out = torch.zeros(case.v.shape, dtype=case.v.dtype, device=DEV)
    z = torch.zeros(case.v.shape, dtype=case.v.dtype, device=DEV)
    gate = _gate(T, H, d, case.v.dtype, 7)
    kda.chunk_prefill(dev(case.q), dev(case.k), dev(case.v), dev(case.g), dev(case.beta),
                      dev(case.cu_seqlens), dev(case.pool).clone(), dev(case.slots), out,
                      workspace=ws, chunk_size=32, flags=kda.KDA_FLAG_DIAG_GIVE_UP,
                      norm_gate=gate, norm_out=z)
    torch.cuda.synchronize()
    word = kda.chunk_prefill_check(ws)
    say(f"  status after the forced give-up: {word:#x}")
    assert word == 1, f"status {word:#x}, expected the timeout bit alone"
    assert torch.isnan(z.float()).all(), "norm rows written after a given-up wait must be NaN"
    from gated_delta_rule_42_amd import kda as K
    pool = dev(case.pool).clone()
    out2 = torch.full(case.v.shape, float("nan"), dtype=case.v.dtype, device=DEV)
    z2 = torch.full(case.v.shape, float("nan"), dtype=case.v.dtype, device=DEV)
    K.chunk_prefill(dev(case.q), dev(case.k), dev(case.v), dev(case.g), dev(case.beta),
                    dev(case.cu_seqlens), pool, dev(case.slots), out2, workspace=ws,
                    chunk_size=32, norm_gate=gate, norm_out=z2)
    torch.cuda.synchronize()
    assert_device_ok(ws)
    z3 = torch.full(case.v.shape, float("nan"), dtype=case.v.dtype, device=DEV)
    K.gated_rmsnorm(out2, gate, z3)
    torch.cuda.synchronize()
    assert torch.equal(bits(z2.cpu()), bits(z3.cpu())), "normal call after the give-up differs"


def test_many_short_sequences():
    """64 short sequences (1-300 tokens, two of them padding) x 16 heads, d =
    128: 1,024 (sequence, head) pairs, 16,384 chain workgroups, many times
    what the chip holds at once.  The plain prefill against the oracle on
    every head, and the fused norm bit for bit the plain call + the
    standalone norm: the grid's dispatch order keeps every wait finite at
    this scale, the norm waves' waits for their peers included (both calls'
    chains run two workgroups per CU here)."""
    from tests.gpu_support import check_prefill, gpu_prefill
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(1, 301, size=64)]
    slots = rng.choice(96, 64, replace=False).astype(np.int32)
    slots[[5, 40]] = -1
    case = wl.random_prefill(31, lengths, 16, 128, 128, n_slots=96, slots=slots,
                             state_dtype=BF16, ckpt_interval=128, scale=inv_sqrt(128),
                             state_std=0.3, name="many_short_64seq_H16_d128")
    check_prefill(case, gpu_prefill(case), label=case.name)
    a = _run_plain(case, norm=True, wseed=9)
    b = _run_plain(case, norm=False, wseed=9)
    for name, u, v in zip(("out", "pool", "checkpoints", "norm out"), a, b):
        _same(u, v, name, case.name)
    say(f"  {case.name}: oracle parity, fused norm == prefill then norm, bit for bit")
