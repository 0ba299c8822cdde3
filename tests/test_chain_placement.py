"""Placement of the chain kernel's workgroups (host logic, no GPU).

The two workgroups of a state tile -- the state role (blockIdx.z = 0), which
publishes each chunk's S and D, and the output role (z = 1), which waits for
them -- pass data through the XCD's L2, so they must run on one XCD, and the
producer must be dispatched before its consumer so that the consumer's
bounded wait always ends.  The GPU deals the workgroups of a launch to its 8
XCDs round-robin by linear id x + X (y + Y z) and dispatches them in
linear-id order.  This test checks that the chain kernel's source launches
the grid modelled here, then enumerates that grid for every shape the tests
and the bench launch (and more) and checks both properties."""
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
    assert re.search(r"chain_kernel<D, BT, AT, ST>\)\s*,\s*dim3\(\(unsigned\)pairs, \(unsigned\)\(D / 16\), 2u\)",
                     src), "chain_kernel launch geometry changed"
    assert "const int pair = blockIdx.x;" in src
    assert "tile = blockIdx.y" in src
    assert "const bool state_role = blockIdx.z == 0;" in src


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
