"""Placement of the chain kernel's workgroups (host logic, no GPU).

The two workgroups of a state tile -- the state role (blockIdx.z = 0), which
publishes each chunk's S and D, and the output role (z = 1), which waits for
them -- pass data through the XCD's L2, so they must run on one XCD, and the
producer must be dispatched before its consumer so that the consumer's
bounded wait always ends.  The GPU deals the workgroups of a launch to its 8
XCDs round-robin by linear id x + X (y + Y z) and dispatches them in
linear-id order.  This test checks that the chain kernel's source launches
the grid modelled here, then enumerates that grid for every shape the tests
and the bench launch (and more) and checks both properties.

With the gated norm fused, the grid is one-dimensional (the state plane, then
the output plane, each in blocks of 8 pairs x d/16 tiles, pair fastest) and
the output workgroups of a pair also wait for one another.  Besides the two
properties above, a pair's workgroups must then all share one XCD and its
output workgroups lie in one block of 8 d/16 consecutive ids, so that the
earliest unfinished block, whose members wait only for each other and for
earlier workgroups, is always dispatched whole."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "gated_delta_rule_42_amd", "csrc", "prefill.hip")
XCDS = 8


def chain_grid(num_seqs: int, heads: int, d: int):
    """(X, Y, Z) of the chain kernel's launch: (sequence, head) pairs padded to
    a multiple of 8, the 16-column tiles of d_v, the two roles."""
    pairs = (num_seqs * heads + 7) // 8 * 8
    return pairs, d // 16, 2


def test_source_launches_the_modelled_grid():
    src = open(SRC).read()
    assert "const int64_t pairs = ((int64_t)a.num_seqs * a.heads + 7) / 8 * 8;" in src
    assert re.search(r"chain_kernel<D, BT, AT, ST, false>\)\s*,\s*dim3\(\(unsigned\)pairs, \(unsigned\)\(D / 16\), 2u\)",
                     src), "chain_kernel launch geometry changed"
    assert "pair = blockIdx.x;" in src
    assert "tile = blockIdx.y;" in src
    assert "state_role = blockIdx.z == 0;" in src
    # The fused-norm grid.
    assert "const int64_t plane = pairs * (D / 16);" in src
    assert re.search(r"chain_kernel<D, BT, AT, ST, true>\)\s*,\s*dim3\(\(unsigned\)\(2 \* plane\)\)", src)
    for line in ("const int plane = (int)(gridDim.x / 2u), id = (int)(blockIdx.x % (unsigned)plane);",
                 "state_role = blockIdx.x < (unsigned)plane;",
                 "const int r = id % (8 * (D / 16));",
                 "pair = id / (8 * (D / 16)) * 8 + r % 8;",
                 "tile = r / 8;"):
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
def test_tile_roles_share_an_xcd_and_the_producer_comes_first(n, h, d):
    X, Y, Z = chain_grid(n, h, d)
    assert X % XCDS == 0
    lin = lambda x, y, z: x + X * (y + Y * z)
    for x in range(n * h):                     # workgroups past n*h return at once
        for y in range(Y):
            producer, consumer = lin(x, y, 0), lin(x, y, 1)
            assert producer % XCDS == consumer % XCDS
            assert producer < consumer


def test_varlen_batch_grid_size():
    X, Y, Z = chain_grid(8, 16, 128)
    assert X * Y * Z == 2048


def norm_grid_decode(L: int, plane: int, d: int):
    """(pair, tile, state_role) of linear id L in the fused-norm grid, as the
    kernel computes it."""
    Y = d // 16
    i = L % plane
    r = i % (8 * Y)
    return i // (8 * Y) * 8 + r % 8, r // 8, L < plane


@pytest.mark.parametrize("n,h,d", SHAPES)
def test_norm_grid_placement(n, h, d):
    X, Y, _ = chain_grid(n, h, d)
    plane = X * Y
    seen = {}
    for L in range(2 * plane):
        pair, tile, state = norm_grid_decode(L, plane, d)
        assert 0 <= tile < Y and 0 <= pair < X
        seen[(pair, tile, state)] = L
    assert len(seen) == 2 * plane                       # every (pair, tile, role) once
    block = 8 * Y
    for pair in range(n * h):
        ids = [seen[(pair, t, s)] for t in range(Y) for s in (True, False)]
        assert len({L % XCDS for L in ids}) == 1           # one XCD for the whole pair
        for t in range(Y):
            assert seen[(pair, t, True)] < seen[(pair, t, False)]   # producer first
        outs = [seen[(pair, t, False)] - plane for t in range(Y)]
        assert len({o // block for o in outs}) == 1        # one block of the output plane
    # Output workgroups wait only on their own block and on earlier ids (the
    # state plane), so dispatch in id order can always finish the earliest
    # unfinished block: it needs 8 d/16 <= 64 slots.
    assert block <= 64
