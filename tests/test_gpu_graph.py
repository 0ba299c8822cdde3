"""Graph replay: the entry points allocate nothing, synchronise nothing and
record no memset, so a HIP graph captured around them replays the same work
(page "[KK] Prepare B12X Kimi KDA prefill ...", Behavior: prepared bindings
reusable under graph replay with caller-owned scratch).  A prefill, a decode
step and the gated norm are captured once and replayed several times, with
eager work in between; every replay must reproduce the eager results bit for
bit."""
import pytest
import torch

from gated_delta_rule_42_amd import workloads as wl
from tests.gpu_support import DEV, bits, inv_sqrt, say

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def test_graph_replay_prefill_decode_norm():
    from gated_delta_rule_42_amd import kda
    pc = wl.random_prefill(900, [300, 64, 1, 130], 4, 128, 128, n_slots=9, slots=[2, 5, 0, 7],
                           ckpt_interval=64, scale=inv_sqrt(128), state_std=0.3)
    dc = wl.random_decode(901, 6, 4, 128, 128, n_slots=9, slots=[1, 2, 3, 4, 6, 8])
    T = pc.total_tokens
    # Static buffers, allocated before capture.
    q, k, v, g, beta = (t.to(DEV) for t in (pc.q, pc.k, pc.v, pc.g, pc.beta))
    cu, slots = pc.cu_seqlens.to(DEV), pc.slots.to(DEV)
    pool0 = pc.pool.to(DEV)
    pool = pool0.clone()
    ws = torch.empty(kda.chunk_prefill_workspace_size(4, T, 4, 128, 128, 64), dtype=torch.uint8,
                     device=DEV)
    ck = torch.empty((sum(L // 64 for L in pc.lengths), 4, 128, 128), dtype=pool.dtype, device=DEV)
    out = torch.empty_like(v)
    gate = torch.randn(T, 4, 128, generator=torch.Generator().manual_seed(902)).to(BF16).to(DEV)
    y = torch.empty_like(out)
    dq, dk, dv, dg, db = (t.to(DEV) for t in (dc.q, dc.k, dc.v, dc.g, dc.beta))
    dslots = dc.slots.to(DEV)
    dout = torch.empty_like(dv)

    def work():
        kda.chunk_prefill(q, k, v, g, beta, cu, pool, slots, out, workspace=ws, checkpoints=ck,
                          ckpt_interval=64, scale=pc.scale)
        kda.recurrent_decode(dq, dk, dv, dg, db, pool, dslots, dout)
        kda.gated_rmsnorm(out, gate, y)

    # Eager reference.
    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, pool, ck, dout, y)]

    # Capture on a side stream (torch's capture stream), then replay.
    pool.copy_(pool0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        pool.copy_(pool0)                       # eager work between replays
        for t in (out, ck, dout, y):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "pool", "checkpoints", "decode out", "norm"),
                              (out, pool, ck, dout, y), ref):
            assert torch.equal(bits(a.cpu()), bits(b.cpu())), f"replay {rep}: {name} differs"
        say(f"  replay {rep}: prefill, decode and norm bit for bit equal to the eager run")


def test_graph_replay_fused_norm_prefill():
    """The prefill with the norm fused (its o-stored flags are cleared inside
    the launch, like the chain's): captured once and replayed three times with
    eager work in between, each replay bit for bit the eager call."""
    from gated_delta_rule_42_amd import kda
    pc = wl.random_prefill(903, [300, 64, 1, 130], 4, 128, 128, n_slots=9, slots=[2, 5, 0, 7],
                           ckpt_interval=64, scale=inv_sqrt(128), state_std=0.3)
    T = pc.total_tokens
    q, k, v, g, beta = (t.to(DEV) for t in (pc.q, pc.k, pc.v, pc.g, pc.beta))
    cu, slots = pc.cu_seqlens.to(DEV), pc.slots.to(DEV)
    pool0 = pc.pool.to(DEV)
    pool = pool0.clone()
    ws = torch.empty(kda.chunk_prefill_workspace_size(4, T, 4, 128, 128, 64, norm=True),
                     dtype=torch.uint8, device=DEV)
    ck = torch.empty((sum(L // 64 for L in pc.lengths), 4, 128, 128), dtype=pool.dtype, device=DEV)
    out = torch.empty_like(v)
    gate = torch.randn(T, 4, 128, generator=torch.Generator().manual_seed(904)).to(BF16).to(DEV)
    w = (1.0 + 0.2 * torch.randn(128, generator=torch.Generator().manual_seed(905))).to(BF16).to(DEV)
    y = torch.empty_like(out)

    def work():
        kda.chunk_prefill(q, k, v, g, beta, cu, pool, slots, out, workspace=ws, checkpoints=ck,
                          ckpt_interval=64, scale=pc.scale, norm_gate=gate, norm_weight=w,
                          norm_out=y)

    work()
    torch.cuda.synchronize()
    assert kda.chunk_prefill_check(ws) == 0
    ref = [t.clone() for t in (out, pool, ck, y)]
    pool.copy_(pool0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        pool.copy_(pool0)
        for t in (out, ck, y):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert kda.chunk_prefill_check(ws) == 0
        for name, a, b in zip(("out", "pool", "checkpoints", "norm out"), (out, pool, ck, y), ref):
            assert torch.equal(bits(a.cpu()), bits(b.cpu())), f"replay {rep}: {name} differs"
        say(f"  replay {rep}: prefill with the fused norm bit for bit equal to the eager run")
