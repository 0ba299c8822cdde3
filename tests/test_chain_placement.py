"""Placement of the chain kernel's workgroups (host logic, no GPU).

The two workgroups of a state tile -- the state role, which publishes each
chunk's S and D, and the output role, which waits for them -- pass data
through the XCD's L2, so they must run on one XCD, and the producer must be
dispatched before its consumer so that the consumer's bounded wait always
ends.  The GPU deals the workgroups of a launch to its 8 XCDs round-robin by
linear id and dispatches them in linear-id order.  This test checks that the
chain kernel's source launches the grid modelled here, then enumerates that
grid for every shape the tests and the bench launch (and more) and checks
both properties.

The grid is one-dimensional, in blocks of 8 (sequence, head) pairs, the last
block first: the state workgroups of the block's pairs and d/16 tiles, then
their output workgroups, pair fastest in both.  With the gated norm fused the output
workgroups of a pair also wait for one another, so besides the two
properties above a pair's workgroups must all share one XCD and its output
workgroups lie in one block, whose members wait only for each other and for
earlier workgroups: dispatch in id order can then always finish the earliest
unfinished block."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "gated_delta_rule_42_amd", "csrc", "prefill.hip")
XCDS = 8


def chain_grid(num_seqs: int, heads: int, d: int) -> int:
    """Workgroups of the chain kernel's launch: (sequence, head) pairs padded
    to a multiple of 8, times the 16-column tiles of d_v, times the two roles."""
    pairs = (num_seqs * heads + 7) // 8 * 8
    return 2 * pairs * (d // 16)


def grid_decode(L: int, total: int, d: int):
    """(pair, tile, state_role) of linear id L in a grid of `total`
    workgroups, as the kernel computes it (blocks last pair first)."""
    tb = 8 * (d // 16)
    blk = total // (2 * tb) - 1 - L // (2 * tb)
    rb = L % (2 * tb)
    state = rb < tb
    rr = rb if state else rb - tb
    return blk * 8 + rr % 8, rr // 8, state


def test_source_launches_the_modelled_grid():
    src = open(SRC).read()
    assert "const int64_t pairs = ((int64_t)a.num_seqs * a.heads + 7) / 8 * 8;" in src
    assert "const int64_t plane = pairs * (D / 16);" in src
    for norm, pack in (("true", "true"), ("true", "false"), ("false", "true"), ("false", "false")):
        assert re.search(r"chain_kernel<D, BT, AT, ST, %s, %s>\)\s*,\s*dim3\(\(unsigned\)\(2 \* plane\)\)"
                         % (norm, pack), src), f"chain_kernel<..., {norm}, {pack}> launch geometry changed"
    for line in ("constexpr int TB = 8 * (D / 16);",
                 "const int blk = (int)(gridDim.x / (2u * TB)) - 1 - (int)(blockIdx.x / (2u * TB));",
                 "const int rb = (int)(blockIdx.x % (2u * TB));",
                 "const bool state_role = rb < TB;",
                 "const int rr = state_role ? rb : rb - TB;",
                 "const int pair = blk * 8 + rr % 8, tile = rr / 8;"):
        assert line in src, line


SHAPES = sorted({
    (1, 16, 128),    # single-sequence prefill, T=4096 (bench)
    (8, 16, 128),    # varlen batch of 8 sequences: 2,048 workgroups
    (1, 16, 128),    # long-context calls
    (5, 16, 128),    # allocation-free prefill test
    (7, 3, 16), (7, 3, 32), (7, 3, 64), (7, 3, 128),   # small varlen tests: H = 3
    (1, 2, 16), (2, 4, 128), (3, 2, 64), (1, 4, 64),
} | {(n, h, d) for n in (1, 2, 3, 9, 64) for h in (1, 5, 12, 32) for d in (16, 32, 64, 128)})


@pytest.mark.parametrize("n,h,d", SHAPES)
def test_grid_placement(n, h, d):
    total = chain_grid(n, h, d)
    Y = d // 16
    seen = {}
    for L in range(total):
        pair, tile, state = grid_decode(L, total, d)
        assert 0 <= tile < Y and 0 <= pair < total // (2 * Y)
        seen[(pair, tile, state)] = L
    assert len(seen) == total                             # every (pair, tile, role) once
    block = 2 * 8 * Y
    for pair in range(n * h):                             # workgroups past n*h return at once
        ids = [seen[(pair, t, s)] for t in range(Y) for s in (True, False)]
        assert len({L % XCDS for L in ids}) == 1           # one XCD for the whole pair
        for t in range(Y):
            assert seen[(pair, t, True)] < seen[(pair, t, False)]   # producer first
        assert len({L // block for L in ids}) == 1          # one block holds the pair
    # A block is at most 2 x 8 x 8 = 128 workgroups: half of what the
    # chip holds at one chain workgroup per CU.
    assert block <= 128


def test_varlen_batch_grid_size():
    assert chain_grid(8, 16, 128) == 2048
