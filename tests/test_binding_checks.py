"""The Python binding refuses tensors whose shape, dtype or device does not
match what the C ABI derives from q (or x) -- before any ctypes call, so
these tests run on the CPU and never reach a kernel.  A mismatched tensor
would otherwise be read or written out of bounds on the device."""
import pytest
import torch

BF, F32, I32, U8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8
T, H, D, N = 40, 2, 16, 3


@pytest.fixture(scope="module")
def kda():
    from gated_delta_rule_42_amd import build as kbuild
    import os
    if not os.path.exists(kbuild.LIBRARY):
        kbuild.build()
    from gated_delta_rule_42_amd import kda as k
    return k


def prefill_args(**over):
    a = dict(q=torch.zeros(T, H, D, dtype=BF), k=torch.zeros(T, H, D, dtype=BF),
             v=torch.zeros(T, H, D, dtype=BF), g=torch.zeros(T, H, D, dtype=F32),
             beta=torch.zeros(T, H, dtype=F32), cu_seqlens=torch.tensor([0, 10, 20, 40], dtype=I32),
             state_pool=torch.zeros(5, H, D, D, dtype=F32), state_indices=torch.tensor([0, 1, 2], dtype=I32),
             out=torch.zeros(T, H, D, dtype=BF))
    a.update(over)
    return a


def call_prefill(kda, a, **kw):
    kda.chunk_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu_seqlens"], a["state_pool"],
                      a["state_indices"], a["out"], **kw)


@pytest.mark.parametrize("over,match", [
    (dict(k=torch.zeros(T, H, D, dtype=F32)), "k is"),                  # dtype differs from q
    (dict(v=torch.zeros(T - 1, H, D, dtype=BF)), "v has shape"),
    (dict(out=torch.zeros(T, H + 1, D, dtype=BF)), "out has shape"),
    (dict(g=torch.zeros(T, H, D + 1, dtype=F32)), "g has shape"),
    (dict(beta=torch.zeros(T, 1, dtype=F32)), "beta has shape"),
    (dict(cu_seqlens=torch.tensor([0, 40], dtype=I32)), "cu_seqlens has shape"),
    (dict(state_pool=torch.zeros(5, H - 1, D, D, dtype=F32)), "state_pool has shape"),   # fewer heads
    (dict(state_pool=torch.zeros(5, H, D, 2 * D, dtype=F32)), "state_pool has shape"),
])
def test_prefill_shape_and_dtype_checks(kda, over, match):
    with pytest.raises(ValueError, match=match):
        call_prefill(kda, prefill_args(**over))


def test_prefill_optional_tensors_checked(kda):
    a = prefill_args()
    with pytest.raises(ValueError, match="has_initial_state has shape"):
        call_prefill(kda, a, has_initial_state=torch.ones(N + 1, dtype=U8))
    with pytest.raises(ValueError, match="checkpoints has shape"):
        call_prefill(kda, a, checkpoints=torch.zeros(2, H, D, D + 1, dtype=F32), ckpt_interval=16)
    with pytest.raises(ValueError, match="checkpoints is"):
        call_prefill(kda, a, checkpoints=torch.zeros(2, H, D, D, dtype=BF), ckpt_interval=16)
    with pytest.raises(ValueError, match="workspace is"):
        call_prefill(kda, a, workspace=torch.zeros(100, dtype=F32))
    with pytest.raises(ValueError, match="seq_start_pos has shape"):
        kda.chunk_prefill_at(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu_seqlens"],
                             torch.zeros(N + 1, dtype=torch.int64), a["state_pool"],
                             a["state_indices"], a["out"])


def test_prefill_refuses_host_tensors(kda):
    # Every shape right, but the tensors are in host memory.
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        call_prefill(kda, prefill_args())
    a = prefill_args()
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        kda.chunk_prefill_noalloc(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu_seqlens"],
                                  a["state_pool"], a["state_indices"], a["out"])


def test_decode_checks(kda):
    B = 4
    q = torch.zeros(B, H, D, dtype=BF)
    ok = dict(k=q.clone(), v=q.clone(), g=torch.zeros(B, H, D, dtype=F32),
              beta=torch.zeros(B, H, dtype=F32), pool=torch.zeros(8, H, D, D, dtype=F32),
              idx=torch.zeros(B, dtype=I32), out=q.clone())

    def call(**over):
        a = dict(ok, **over)
        kda.recurrent_decode(q, a["k"], a["v"], a["g"], a["beta"], a["pool"], a["idx"], a["out"])
    with pytest.raises(ValueError, match="state_indices has shape"):
        call(idx=torch.zeros(B + 1, dtype=I32))
    with pytest.raises(ValueError, match="state_pool has shape"):
        call(pool=torch.zeros(8, H + 1, D, D, dtype=F32))
    with pytest.raises(ValueError, match="out is"):
        call(out=torch.zeros(B, H, D, dtype=F32))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        call()


def test_spec_checks(kda):
    B, ntok = 2, 3
    R = B * ntok
    q = torch.zeros(R, H, D, dtype=BF)
    pool = torch.zeros(4, H, D, D, dtype=F32)
    idx = torch.zeros(B, dtype=I32)
    ts = torch.zeros(B, ntok, H, D, D, dtype=F32)
    with pytest.raises(ValueError, match="beta has shape"):
        kda.spec_decode(q, q, q, torch.zeros(R, H, D, dtype=F32), torch.zeros(R, H + 1, dtype=F32),
                        pool, idx, ts, q.clone())
    with pytest.raises(ValueError, match="num_accepted has shape"):
        kda.spec_commit(ts, torch.ones(B + 1, dtype=I32), pool, idx)
    with pytest.raises(ValueError, match="state_pool has shape"):
        kda.spec_commit(ts, torch.ones(B, dtype=I32), torch.zeros(4, H, D, 2 * D, dtype=F32), idx)


def test_norm_and_conv_checks(kda):
    x = torch.zeros(T, H, D, dtype=BF)
    with pytest.raises(ValueError, match="gate has shape"):
        kda.gated_rmsnorm(x, torch.zeros(T, H, D + 1, dtype=BF), x.clone())
    with pytest.raises(ValueError, match="weight has shape"):
        kda.gated_rmsnorm(x, x.clone(), x.clone(), weight=torch.ones(D + 1, dtype=BF))
    with pytest.raises(ValueError, match="residual_out has shape"):
        kda.gated_rmsnorm_ex(x, x.clone(), x.clone(), residual=x.clone(),
                             residual_out=torch.zeros(T, H, 2 * D, dtype=BF))
    C, W = 3 * H * D, 4
    xc = torch.zeros(T, C, dtype=BF)
    cu = torch.tensor([0, T], dtype=I32)
    idx = torch.zeros(1, dtype=I32)
    with pytest.raises(ValueError, match="conv_state_pool has shape"):
        kda.causal_conv1d(xc, torch.zeros(C, W, dtype=BF), cu, torch.zeros(2, W, C, dtype=BF),
                          idx, xc.clone())
    with pytest.raises(ValueError, match="y has shape"):
        kda.causal_conv1d(xc, torch.zeros(C, W, dtype=BF), cu, torch.zeros(2, W - 1, C, dtype=BF),
                          idx, torch.zeros(T, C + 8, dtype=BF))
    with pytest.raises(ValueError, match="conv_state_pool has shape"):
        kda.conv_chunk_prefill(xc, torch.zeros(C, W, dtype=BF), torch.zeros(2, W - 2, C, dtype=BF),
                               torch.zeros(T, H, D, dtype=F32), torch.zeros(T, H, dtype=F32), cu,
                               torch.zeros(2, H, D, D, dtype=F32), idx, torch.zeros(T, H, D, dtype=BF))


def test_fused_norm_checks(kda):
    """The norm arguments of chunk_prefill / conv_chunk_prefill: both tensors
    or neither, [T, H, dv] in q's dtype, a [dv] weight."""
    a = prefill_args()
    gate, z = torch.zeros(T, H, D, dtype=BF), torch.zeros(T, H, D, dtype=BF)
    with pytest.raises(ValueError, match="needs both norm_gate and norm_out"):
        call_prefill(kda, a, norm_gate=gate)
    with pytest.raises(ValueError, match="needs both norm_gate and norm_out"):
        call_prefill(kda, a, norm_out=z)
    with pytest.raises(ValueError, match="norm_weight needs norm_gate and norm_out"):
        call_prefill(kda, a, norm_weight=torch.ones(D, dtype=BF))
    with pytest.raises(ValueError, match="norm_gate has shape"):
        call_prefill(kda, a, norm_gate=torch.zeros(T, H, D + 8, dtype=BF), norm_out=z)
    with pytest.raises(ValueError, match="norm_out has shape"):
        call_prefill(kda, a, norm_gate=gate, norm_out=torch.zeros(T - 1, H, D, dtype=BF))
    with pytest.raises(ValueError, match="norm_gate is"):
        call_prefill(kda, a, norm_gate=torch.zeros(T, H, D, dtype=F32), norm_out=z)
    with pytest.raises(ValueError, match="norm_weight has shape"):
        call_prefill(kda, a, norm_gate=gate, norm_out=z, norm_weight=torch.ones(D + 1, dtype=BF))
    # Every shape right, in host memory: refused before the C call.
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        call_prefill(kda, a, norm_gate=gate, norm_out=z, norm_weight=torch.ones(D, dtype=BF))
