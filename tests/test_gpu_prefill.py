"""Chunk prefill on the GPU against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_42_amd import workloads as wl
from tests.gpu_support import (TOL, bits, check_prefill, f64, gpu_decode, gpu_prefill, inv_sqrt,
                               max_err, say)

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16
# Lengths spanning: empty, one token, a partial chunk, whole chunks, ragged tails.
LENS = [0, 1, 17, 64, 100, 130]


def _varlen(seed, d, C, state, act=BF16, interval=None, scale=1.0, lens=LENS, H=3,
            padding=True, has_init=True, **kw):
    lens = list(lens) + ([23] if padding else [])
    n = len(lens)
    slots = list(range(1, 2 * n, 2))[:n]
    if padding:
        slots[-1] = -1
    hi = [1] * n if has_init else None
    if has_init and n > 2:
        hi[2] = 0
    return wl.random_prefill(seed, lens, H, d, d, act_dtype=act, state_dtype=state,
                             n_slots=2 * n + 1, slots=slots, has_init=hi, chunk_size=C,
                             ckpt_interval=(2 * C if interval is None else interval),
                             scale=scale, state_std=0.3, **kw)


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("state", [F32, BF16])
def test_prefill_parity_small(d, C, state):
    case = _varlen(1000 + d + C, d, C, state, scale=inv_sqrt(d))
    check_prefill(case, gpu_prefill(case), label=f"d={d} C={C} state={state}")


@pytest.mark.parametrize("C", [16, 64])
def test_prefill_fp32_activations(C):
    case = _varlen(77 + C, 64, C, F32, act=F32)
    check_prefill(case, gpu_prefill(case), label=f"fp32 act C={C}")


def test_prefill_l2norm_flag():
    case = _varlen(5, 128, 64, F32, qk_unit=False, l2norm_qk=True)
    check_prefill(case, gpu_prefill(case), label="l2norm flag")


@pytest.mark.parametrize("C,d", [(64, 128), (32, 64)])
def test_prefill_strong_decay(C, d):
    """Decay three times stronger than the workloads': chunk totals of the
    log-decay pass -80 at C=64 (around it at C=32), so the Gram products take
    per-sub-chunk reference points for some or all chunks."""
    case = _varlen(90 + C, d, C, F32, g_scale=3.0, scale=inv_sqrt(d))
    check_prefill(case, gpu_prefill(case), label=f"strong decay C={C} d={d}")


def test_prefill_tiny_config():
    """1 sequence, T=64, H=2, d=16, C=16, fp32 everywhere, zero initial state."""
    case = wl.tiny_prefill()
    check_prefill(case, gpu_prefill(case), label=case.name)


def test_prefill_single_sequence_full_size():
    """T=4096, H=16, d=128, C=64, bf16 q/k/v, fp32 state from slot 7 of 64."""
    case = wl.single_seq_prefill()
    check_prefill(case, gpu_prefill(case), label=case.name)


def test_prefill_varlen_full_size():
    """8 sequences (<=16384 tokens), bf16 256-slot pool, checkpoints every 1024;
    every head against the oracle."""
    case = wl.varlen_prefill()
    check_prefill(case, gpu_prefill(case), label=case.name)


def test_prefill_varlen_full_size_fp32_state():
    """The same batch with an fp32 pool and fp32 checkpoints (tolerance 1e-2)."""
    case = wl.varlen_prefill(state_dtype=F32)
    check_prefill(case, gpu_prefill(case), label=case.name)


def test_prefill_edge_cases():
    # every sequence empty
    case = wl.random_prefill(3, [0, 0, 0], 2, 64, 64, n_slots=4, chunk_size=32)
    o, p, _ = gpu_prefill(case)
    assert torch.equal(bits(p), bits(case.pool))
    # single-token sequences with and without a state, one exactly one chunk long
    case = wl.random_prefill(4, [1, 1, 64, 65], 2, 128, 128, n_slots=6, slots=[5, 0, 2, 3],
                             has_init=[1, 0, 1, 0], chunk_size=64, state_std=0.3)
    check_prefill(case, gpu_prefill(case), label="one-token and one-chunk sequences")
    # only padding
    case = wl.random_prefill(6, [5, 9], 2, 32, 32, n_slots=3, slots=[-1, -1], chunk_size=16)
    o, p, _ = gpu_prefill(case)
    assert torch.count_nonzero(o) == 0 and torch.equal(bits(p), bits(case.pool))


def _self_diff(a, b):
    """Two GPU runs of the same recurrence that round differently: the bf16
    outputs' difference beyond one bf16 step of the value (two outputs a step
    apart are equally good roundings), and the fp32 states' max-abs
    difference."""
    oa, ob = f64(a[0]), f64(b[0])
    e_o = float(np.max(np.abs(oa - ob) - 2.0 ** -7 * np.maximum(np.abs(oa), np.abs(ob)), initial=0.0))
    return e_o, max_err(f64(a[1]), f64(b[1]))


# Bounds for GPU-against-GPU comparisons: a fraction of the oracle tolerance,
# with room over the measured spreads (printed by each test).
SELF_O, SELF_S = 5e-3, 5e-3


def test_prefill_chunk_size_invariance():
    """The chunked method reaches the same result at every chunk size."""
    case = _varlen(21, 128, 64, F32, interval=0, padding=False)
    outs = [gpu_prefill(case, chunk=C) for C in (16, 32, 64)]
    for o, p, _ in outs[1:]:
        e_o, e_s = _self_diff((o, p), outs[0])
        say(f"  chunk-size spread: o beyond one bf16 step {e_o:.2e}, state {e_s:.2e}")
        assert e_o <= SELF_O and e_s <= SELF_S


def test_prefill_split_calls_carry_state():
    """One call over 300 tokens equals three calls of 100 through the pool."""
    case = wl.random_prefill(31, [300], 4, 128, 128, n_slots=3, slots=[1], chunk_size=64,
                             state_std=0.3)
    o_full, p_full, _ = gpu_prefill(case)
    pool = case.pool
    parts = []
    for a in range(0, 300, 100):
        part = wl.PrefillCase("part", case.q[a:a + 100], case.k[a:a + 100], case.v[a:a + 100],
                              case.g[a:a + 100], case.beta[a:a + 100],
                              torch.tensor([0, 100], dtype=torch.int32), pool, case.slots, None,
                              64, 0, 1.0)
        o, pool, _ = gpu_prefill(part)
        parts.append(o)
    e_o, e_s = _self_diff((torch.cat(parts), pool), (o_full, p_full))
    say(f"  split vs one call: o beyond one bf16 step {e_o:.2e}, state {e_s:.2e}")
    assert e_o <= SELF_O and e_s <= SELF_S


def test_prefill_routing_is_bit_exact():
    """Permuting slot assignments and rerunning change no bit of the outputs,
    states or checkpoints."""
    case = _varlen(41, 128, 64, BF16, padding=True)
    a = gpu_prefill(case)
    b = gpu_prefill(case)
    for x, y in zip(a, b):
        assert torch.equal(bits(x), bits(y))
    n_slots = case.pool.shape[0]
    perm = torch.randperm(n_slots, generator=torch.Generator().manual_seed(5)).to(torch.int32)
    pool2 = case.pool.clone()
    pool2[perm.long()] = case.pool
    slots2 = torch.where(case.slots >= 0, perm[case.slots.clamp(min=0).long()], case.slots)
    moved = wl.PrefillCase(case.name, case.q, case.k, case.v, case.g, case.beta,
                           case.cu_seqlens, pool2, slots2.to(torch.int32), case.has_init,
                           case.chunk_size, case.ckpt_interval, case.scale)
    c = gpu_prefill(moved)
    assert torch.equal(bits(a[0]), bits(c[0]))
    assert torch.equal(bits(a[1]), bits(c[1][perm.long()]))
    assert torch.equal(bits(a[2]), bits(c[2]))


def test_prefill_workspace_reuse():
    """A workspace sized for the largest call serves later, smaller calls."""
    from gated_delta_rule_42_amd import kda
    big = _varlen(51, 128, 64, F32)
    small = _varlen(52, 128, 64, F32, lens=[40, 3])
    ws = torch.empty(kda.chunk_prefill_workspace_size(big.num_seqs, big.total_tokens, 3, 128, 128, 64),
                     dtype=torch.uint8, device="cuda")
    check_prefill(big, gpu_prefill(big, workspace=ws), label="workspace first call")
    check_prefill(small, gpu_prefill(small, workspace=ws), label="workspace reused")


@pytest.mark.parametrize("act", [BF16, F32])
def test_packed_chain_equals_per_sequence_calls(act):
    """12 sequences of 200-1,500 tokens x 16 heads, d = 128: a chain grid of
    3,072 workgroups for short sequences, which runs two workgroups per CU.
    Against the oracle on every head, and bit for bit against 12 calls of one
    sequence each (256 chain workgroups, one per CU): the packed build
    computes the same operations.  bf16 and fp32 activations."""
    from gated_delta_rule_42_amd import kda
    from tests.gpu_support import DEV, assert_device_ok
    rng = np.random.default_rng(61)
    lengths = [int(x) for x in rng.integers(200, 1501, size=12)]
    slots = rng.choice(40, 12, replace=False).astype(np.int32)
    has_init = [1] * 12
    has_init[3] = 0
    case = wl.random_prefill(61, lengths, 16, 128, 128, n_slots=40, slots=slots, has_init=has_init,
                             act_dtype=act, state_dtype=F32, scale=inv_sqrt(128), state_std=0.3,
                             name=f"packed_12seq_H16_d128_{'bf16' if act == BF16 else 'fp32'}_act")
    assert case.total_tokens <= 24 * 64 * case.num_seqs      # the packed grid's length bound
    batch = gpu_prefill(case)
    check_prefill(case, batch, label=case.name)
    q, k, v = case.q.to(DEV), case.k.to(DEV), case.v.to(DEV)
    g, beta = case.g.to(DEV), case.beta.to(DEV)
    pool = case.pool.to(DEV).clone()
    out = torch.full(v.shape, float("nan"), dtype=v.dtype, device=DEV)
    cu = case.cu_seqlens.numpy()
    for s in range(case.num_seqs):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        one = torch.tensor([0, t1 - t0], dtype=torch.int32, device=DEV)
        ws = torch.empty(kda.chunk_prefill_workspace_size(1, t1 - t0, 16, 128, 128, 64),
                         dtype=torch.uint8, device=DEV)
        kda.chunk_prefill(q[t0:t1], k[t0:t1], v[t0:t1], g[t0:t1], beta[t0:t1], one, pool,
                          case.slots[s:s + 1].to(DEV), out[t0:t1], workspace=ws,
                          has_initial_state=case.has_init[s:s + 1].to(DEV), scale=case.scale,
                          chunk_size=64)
        torch.cuda.synchronize()
        assert_device_ok(ws)
    assert torch.equal(batch[0].view(torch.uint8), out.cpu().view(torch.uint8)), "packed batch output differs"
    assert torch.equal(bits(batch[1]), bits(pool.cpu())), "packed batch states differ"
    say(f"  {case.name}: oracle parity; equal bit for bit to one call per sequence")


def test_decode_equals_one_token_prefill():
    case = wl.random_decode(61, 40, 4, 128, 128, n_slots=80)
    o_d, p_d = gpu_decode(case)
    pre = wl.PrefillCase("as prefill", case.q, case.k, case.v, case.g, case.beta,
                         torch.arange(41, dtype=torch.int32), case.pool, case.slots, None, 16, 0,
                         case.scale)
    o_p, p_p, _ = gpu_prefill(pre)
    e_o, e_s = _self_diff((o_d, p_d), (o_p, p_p))
    say(f"  decode vs one-token prefill: o beyond one bf16 step {e_o:.2e}, state {e_s:.2e}")
    assert e_o <= SELF_O and e_s <= SELF_S


def test_prefill_strided_inputs():
    """q, k, v read in place from a packed [T, 3*H*d] projection; output into a
    wider buffer."""
    from gated_delta_rule_42_amd import kda
    case = wl.random_prefill(71, [70, 33], 4, 64, 64, n_slots=4, chunk_size=32)
    T, H, d = case.total_tokens, 4, 64
    packed = torch.cat([case.q.reshape(T, -1), case.k.reshape(T, -1), case.v.reshape(T, -1)], 1).cuda()
    q = packed[:, :H * d].view(T, H, d)
    k = packed[:, H * d:2 * H * d].view(T, H, d)
    v = packed[:, 2 * H * d:].view(T, H, d)
    wide = torch.zeros(T, 2 * H * d, dtype=torch.bfloat16, device="cuda")
    out = wide[:, :H * d].view(T, H, d)
    p = case.pool.cuda().clone()
    kda.chunk_prefill(q, k, v, case.g.cuda(), case.beta.cuda(), case.cu_seqlens.cuda(), p,
                      case.slots.cuda(), out, chunk_size=32)
    torch.cuda.synchronize()
    o_ref, p_ref, _ = gpu_prefill(case)
    assert torch.equal(bits(out.cpu()), bits(o_ref)) and torch.equal(bits(p.cpu()), bits(p_ref))
    assert torch.count_nonzero(wide[:, H * d:]) == 0


def test_prefill_failure_report():
    """KDA_FLAG_DIAG_GIVE_UP makes every output workgroup give up its bounded
    wait at once, as if its producer never published: the call completes
    normally, the real rows come out NaN, the states are computed as usual
    (bit for bit those of a normal call) and the status word reports the
    wait that ran out.  The next normal call on the same workspace clears the
    word and is correct."""
    from gated_delta_rule_42_amd import kda
    case = wl.random_prefill(91, [100, 37, 64], 4, 64, 64, n_slots=6, chunk_size=32,
                             state_std=0.3)
    ws = torch.empty(kda.chunk_prefill_workspace_size(case.num_seqs, case.total_tokens, 4, 64, 64, 32),
                     dtype=torch.uint8, device="cuda")
    dev = lambda t: t.to("cuda")
    pool = dev(case.pool).clone()
    out = torch.zeros(case.v.shape, dtype=case.v.dtype, device="cuda")
    kda.chunk_prefill(dev(case.q), dev(case.k), dev(case.v), dev(case.g), dev(case.beta),
                      dev(case.cu_seqlens), pool, dev(case.slots), out, workspace=ws,
                      chunk_size=32, flags=kda.KDA_FLAG_DIAG_GIVE_UP)
    torch.cuda.synchronize()
    word = kda.chunk_prefill_check(ws)
    say(f"  status after the forced give-up: {word:#x}")
    assert word == 1, f"status {word:#x}, expected the timeout bit alone"
    assert torch.isnan(out.float()).all(), "rows written after a given-up wait must be NaN"
    o_n, p_n, _ = gpu_prefill(case, workspace=ws)     # asserts the word is back to 0
    assert torch.equal(bits(pool.cpu()), bits(p_n)), "states differ from a normal call"
    check_prefill(case, (o_n, p_n, None), label="normal call after the forced give-up")
