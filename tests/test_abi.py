"""The C-ABI library on the CPU: it loads, exports every entry point that
include/kda.h declares, and rejects bad arguments on the host before any
launch.  No call here reaches a kernel (every call either fails validation or
has nothing to do)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    from gated_delta_rule_42_amd import build as kbuild
    srcs = [os.path.join(kbuild.CSRC, s) for s in os.listdir(kbuild.CSRC)] + [HEADER]
    if (not os.path.exists(kbuild.LIBRARY) or
            os.path.getmtime(kbuild.LIBRARY) < max(os.path.getmtime(s) for s in srcs)):
        kbuild.build()
    from gated_delta_rule_42_amd import kda
    return kda._lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("kda_chunk_prefill", "kda_recurrent_decode", "kda_gated_rmsnorm",
                 "kda_causal_conv1d", "kda_chunk_prefill_workspace_size",
                 "kda_conv_chunk_prefill", "kda_gated_rmsnorm_ex", "kda_chunk_prefill_at",
                 "kda_spec_decode", "kda_spec_commit", "kda_chunk_prefill_check",
                 "kda_chunk_prefill_norm", "kda_conv_chunk_prefill_norm",
                 "kda_chunk_prefill_norm_workspace_size",
                 "kda_abi_version", "kda_status_string"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    from gated_delta_rule_42_amd import kda
    out = subprocess.run(["nm", "-D", "--defined-only", kda.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)", out))
    for name in declared_functions():
        assert name in exported, f"{name} not exported"
        assert getattr(lib, name) is not None
    # Exactly those: the library is built with hidden visibility, so no
    # internal function (and no benchmarking aid) is part of the ABI.
    assert exported == set(declared_functions()), sorted(exported ^ set(declared_functions()))


def test_version_and_status_strings(lib):
    from gated_delta_rule_42_amd import kda
    assert kda.abi_version() == 1
    for code in range(7):
        assert kda.status_string(code) and kda.status_string(code) != "unknown status"
    assert kda.status_string(99) == "unknown status"


def test_workspace_size(lib):
    from gated_delta_rule_42_amd import kda
    one = kda.chunk_prefill_workspace_size(1, 64, 1, 128, 128, 64)
    assert one > 0 and one % 256 == 0
    # A 256-byte header (the status word), then per (chunk slot, head) one
    # record and the chain's exchange slots (one per 16-column tile); chunk
    # slots = ceil(T / C) + 2 N (a sequence starting at an absolute position
    # off the chunk grid has a partial chunk at each end).  Then one 32-bit
    # flag per (sequence, head, tile), rounded up to 256 bytes.
    header = 256
    flags = lambda n, h: (n * h * (128 // 16) * 4 + 255) // 256 * 256
    per_slot = (one - header - flags(1, 1)) // 3
    assert per_slot == 74240 + 8 * 16 * (128 + 64) * 2
    assert (kda.chunk_prefill_workspace_size(1, 4096, 16, 128, 128, 64)
            == header + (64 + 2) * 16 * per_slot + flags(1, 16))
    assert kda.chunk_prefill_workspace_size(3, 100, 2, 64, 64, 32) > 0
    for bad in [(1, 64, 1, 48, 48, 64), (1, 64, 1, 128, 64, 64), (1, 64, 1, 128, 128, 48),
                (-1, 64, 1, 128, 128, 64), (1, 64, 0, 128, 128, 64)]:
        assert kda.chunk_prefill_workspace_size(*bad) == 0
        assert kda.chunk_prefill_workspace_size(*bad, norm=True) == 0
    # With the fused norm: a second flag per (sequence, head, tile) right
    # after the first, both in one 256-byte aligned block.
    body = (64 + 2) * 16 * per_slot
    n_flags = 1 * 16 * (128 // 16)
    assert (kda.chunk_prefill_workspace_size(1, 4096, 16, 128, 128, 64, norm=True)
            == header + body + (2 * n_flags * 4 + 255) // 256 * 256)


FAKE = 0x10000   # aligned, never dereferenced: every call below stops in validation


def _prefill(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, act=1, qs=2048, ks=2048, vs=2048, g=FAKE, beta=FAKE,
             cu=FAKE, n=1, T=64, H=16, dk=128, dv=128, pool=FAKE, sdt=0, slots=4, idx=FAKE,
             hi=None, ck=None, cap=0, interval=0, scale=1.0, C=64, flags=0, out=FAKE,
             os=2048, ws=FAKE, wsb=0, stream=None)
    a.update(over)
    return lib.kda_chunk_prefill(
        a["q"], a["k"], a["v"], a["act"], a["qs"], a["ks"], a["vs"], a["g"], a["beta"],
        a["cu"], a["n"], a["T"], a["H"], a["dk"], a["dv"], a["pool"], a["sdt"], a["slots"],
        a["idx"], a["hi"], a["ck"], a["cap"], a["interval"], a["scale"], a["C"], a["flags"],
        a["out"], a["os"], a["ws"], a["wsb"], a["stream"])


def test_prefill_validation(lib):
    from gated_delta_rule_42_amd import kda as K
    assert _prefill(lib, n=0) == K.KDA_OK                              # nothing to do
    assert _prefill(lib, dk=48, dv=48) == K.KDA_ERR_UNSUPPORTED
    assert _prefill(lib, dv=64) == K.KDA_ERR_UNSUPPORTED
    assert _prefill(lib, C=48) == K.KDA_ERR_UNSUPPORTED
    assert _prefill(lib, interval=100) == K.KDA_ERR_UNSUPPORTED       # not a multiple of C
    assert _prefill(lib, act=7) == K.KDA_ERR_INVALID_ARG
    assert _prefill(lib, flags=8) == K.KDA_ERR_INVALID_ARG
    assert _prefill(lib, q=None) == K.KDA_ERR_INVALID_ARG
    assert _prefill(lib, cu=None) == K.KDA_ERR_INVALID_ARG
    assert _prefill(lib, qs=1000) == K.KDA_ERR_INVALID_ARG              # < H * dk
    assert _prefill(lib, qs=2052) == K.KDA_ERR_INVALID_ARG              # not a multiple of 8
    assert _prefill(lib, q=FAKE + 2) == K.KDA_ERR_INVALID_ARG           # misaligned
    assert _prefill(lib, interval=64, cap=4, ck=None) == K.KDA_ERR_INVALID_ARG
    assert _prefill(lib, T=-1) == K.KDA_ERR_INVALID_ARG
    assert _prefill(lib, wsb=100) == K.KDA_ERR_WORKSPACE_TOO_SMALL
    # 2^20 + 2 chunk slots x 16 heads exceeds the first kernel's 1-D grid:
    # refused on the host, before anything is enqueued (no GPU needed).
    assert _prefill(lib, T=1 << 26, wsb=1 << 62) == K.KDA_ERR_LAUNCH
    need = K.chunk_prefill_workspace_size(1, 64, 16, 128, 128, 64)
    assert _prefill(lib, wsb=need, ws=FAKE + 16) == K.KDA_ERR_INVALID_ARG   # 256-B alignment


def _prefill_noalloc(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, act=1, qs=2048, ks=2048, vs=2048, g=FAKE, beta=FAKE,
             cu=FAKE, n=1, T=64, H=16, dk=128, dv=128, pool=FAKE, sdt=0, slots=4, idx=FAKE,
             hi=None, ck=None, cap=0, interval=0, scale=1.0, C=64, flags=0, out=FAKE,
             os=2048, stream=None)
    a.update(over)
    return lib.kda_chunk_prefill_noalloc(*a.values())


def test_prefill_noalloc_validation(lib):
    from gated_delta_rule_42_amd import kda as K
    assert _prefill_noalloc(lib, n=0) == K.KDA_OK                        # nothing to do
    assert _prefill_noalloc(lib, dk=48, dv=48) == K.KDA_ERR_UNSUPPORTED
    assert _prefill_noalloc(lib, q=None) == K.KDA_ERR_INVALID_ARG
    assert _prefill_noalloc(lib, qs=1000) == K.KDA_ERR_INVALID_ARG
    # The fixed area is 128 MiB: the headline call (one 4096-token sequence,
    # 16 heads of d = 128, chunk 64) fits, 20,000 tokens do not and are
    # refused on the host before any HIP call.
    assert K.chunk_prefill_workspace_size(1, 4096, 16, 128, 128, 64) <= (128 << 20)
    assert K.chunk_prefill_workspace_size(1, 20000, 16, 128, 128, 64) > (128 << 20)
    assert _prefill_noalloc(lib, T=20000) == K.KDA_ERR_SCRATCH_LIMIT
    assert K.status_string(K.KDA_ERR_SCRATCH_LIMIT) != "unknown status"


def test_prefill_check_validation(lib):
    from gated_delta_rule_42_amd import kda as K
    word = ctypes.c_uint32(7)
    # Refused on the host (no stream is touched): null or too small workspace.
    assert lib.kda_chunk_prefill_check(None, 1 << 20, ctypes.byref(word), None) == K.KDA_ERR_INVALID_ARG
    assert lib.kda_chunk_prefill_check(FAKE, 3, ctypes.byref(word), None) == K.KDA_ERR_INVALID_ARG
    assert word.value == 7


def _conv_prefill(lib, **over):
    a = dict(x=FAKE, xs=6144, act=1, w=FAKE, b=None, W=4, cflags=1, cpool=FAKE, g=FAKE,
             beta=FAKE, cu=FAKE, n=1, T=64, H=16, dk=128, dv=128, pool=FAKE, sdt=0, slots=4,
             idx=FAKE, hi=None, ck=None, cap=0, interval=0, scale=1.0, C=64, flags=1,
             out=FAKE, os=2048, ws=FAKE, wsb=0, stream=None)
    a.update(over)
    return lib.kda_conv_chunk_prefill(*a.values())


def test_prefill_at_validation(lib):
    from gated_delta_rule_42_amd import kda as K
    need = K.chunk_prefill_workspace_size(1, 64, 16, 128, 128, 64)
    a = dict(q=FAKE, k=FAKE, v=FAKE, act=1, qs=2048, ks=2048, vs=2048, g=FAKE, beta=FAKE,
             cu=FAKE, pos=FAKE + 4, n=1, T=64, H=16, dk=128, dv=128, pool=FAKE, sdt=0, slots=4,
             idx=FAKE, hi=None, ck=None, cap=0, interval=0, scale=1.0, C=64, flags=0, out=FAKE,
             os=2048, ws=FAKE, wsb=need, stream=None)
    assert lib.kda_chunk_prefill_at(*a.values()) == K.KDA_ERR_INVALID_ARG    # misaligned positions
    assert lib.kda_chunk_prefill_at(*dict(a, n=0).values()) == K.KDA_OK
    assert lib.kda_chunk_prefill_at(*dict(a, interval=100).values()) == K.KDA_ERR_UNSUPPORTED
    assert lib.kda_chunk_prefill_at(*dict(a, wsb=100).values()) == K.KDA_ERR_WORKSPACE_TOO_SMALL


def test_conv_prefill_validation(lib):
    from gated_delta_rule_42_amd import kda as K
    need = K.chunk_prefill_workspace_size(1, 64, 16, 128, 128, 64)
    assert _conv_prefill(lib, n=0) == K.KDA_OK                          # nothing to do
    assert _conv_prefill(lib, W=1) == K.KDA_ERR_UNSUPPORTED
    assert _conv_prefill(lib, W=9) == K.KDA_ERR_UNSUPPORTED
    assert _conv_prefill(lib, cflags=2) == K.KDA_ERR_INVALID_ARG
    assert _conv_prefill(lib, act=7) == K.KDA_ERR_INVALID_ARG
    assert _conv_prefill(lib, xs=6000) == K.KDA_ERR_INVALID_ARG         # < 3 H dk
    assert _conv_prefill(lib, xs=6148) == K.KDA_ERR_INVALID_ARG         # not a multiple of 8
    assert _conv_prefill(lib, x=None) == K.KDA_ERR_INVALID_ARG
    assert _conv_prefill(lib, dk=48, dv=48, xs=3 * 16 * 48) == K.KDA_ERR_UNSUPPORTED
    assert _conv_prefill(lib, wsb=100) == K.KDA_ERR_WORKSPACE_TOO_SMALL
    # Past the prefill checks (workspace large enough), the conv arguments.
    assert _conv_prefill(lib, wsb=need, w=None) == K.KDA_ERR_INVALID_ARG
    assert _conv_prefill(lib, wsb=need, w=FAKE + 2) == K.KDA_ERR_INVALID_ARG
    assert _conv_prefill(lib, wsb=need, b=FAKE + 4) == K.KDA_ERR_INVALID_ARG
    assert _conv_prefill(lib, wsb=need, cpool=None) == K.KDA_ERR_INVALID_ARG
    assert _conv_prefill(lib, wsb=need, cpool=FAKE + 8) == K.KDA_ERR_INVALID_ARG


def test_decode_validation(lib):
    from gated_delta_rule_42_amd import kda as K

    def call(**over):
        a = dict(q=FAKE, k=FAKE, v=FAKE, act=1, qs=2048, ks=2048, vs=2048, g=FAKE, beta=FAKE,
                 B=4, H=16, dk=128, dv=128, pool=FAKE, sdt=0, slots=8, idx=FAKE, scale=1.0,
                 flags=0, out=FAKE, os=2048, stream=None)
        a.update(over)
        return lib.kda_recurrent_decode(*a.values())

    assert call(B=0) == K.KDA_OK
    assert call(dk=96, dv=96) == K.KDA_ERR_UNSUPPORTED
    assert call(v=None) == K.KDA_ERR_INVALID_ARG
    assert call(os=100) == K.KDA_ERR_INVALID_ARG
    assert call(pool=FAKE + 4) == K.KDA_ERR_INVALID_ARG
    assert call(sdt=3) == K.KDA_ERR_INVALID_ARG
    assert call(flags=2) == K.KDA_ERR_INVALID_ARG


def test_spec_decode_and_commit_validation(lib):
    from gated_delta_rule_42_amd import kda as K

    def spec(**over):
        a = dict(q=FAKE, k=FAKE, v=FAKE, act=1, qs=2048, ks=2048, vs=2048, g=FAKE, beta=FAKE,
                 B=4, ntok=3, H=16, dk=128, dv=128, pool=FAKE, sdt=0, slots=8, idx=FAKE,
                 ts=FAKE, scale=1.0, flags=0, out=FAKE, os=2048, stream=None)
        a.update(over)
        return lib.kda_spec_decode(*a.values())

    assert spec(B=0) == K.KDA_OK
    assert spec(ntok=0) == K.KDA_ERR_INVALID_ARG
    assert spec(ts=None) == K.KDA_ERR_INVALID_ARG
    assert spec(ts=FAKE + 8) == K.KDA_ERR_INVALID_ARG
    assert spec(dk=48, dv=48) == K.KDA_ERR_UNSUPPORTED
    assert spec(qs=1000) == K.KDA_ERR_INVALID_ARG
    assert spec(flags=4) == K.KDA_ERR_INVALID_ARG

    def commit(**over):
        a = dict(ts=FAKE, B=4, ntok=3, H=16, dk=128, dv=128, acc=FAKE, pool=FAKE, sdt=1,
                 slots=8, idx=FAKE, stream=None)
        a.update(over)
        return lib.kda_spec_commit(*a.values())

    assert commit(B=0) == K.KDA_OK
    assert commit(slots=0) == K.KDA_OK
    assert commit(acc=None) == K.KDA_ERR_INVALID_ARG
    assert commit(ntok=0) == K.KDA_ERR_INVALID_ARG
    assert commit(sdt=5) == K.KDA_ERR_INVALID_ARG
    assert commit(dk=128, dv=64) == K.KDA_ERR_UNSUPPORTED
    assert commit(pool=FAKE + 2) == K.KDA_ERR_INVALID_ARG


def test_norm_and_conv_validation(lib):
    from gated_delta_rule_42_amd import kda as K
    n = lambda **o: lib.kda_gated_rmsnorm(*dict(
        dict(x=FAKE, xs=2048, gate=FAKE, gs=2048, w=None, y=FAKE, ys=2048, dt=1, T=4, H=16,
             dim=128, eps=1e-6, stream=None), **o).values())
    assert n(T=0) == K.KDA_OK
    assert n(dim=100) == K.KDA_ERR_UNSUPPORTED
    assert n(gate=None) == K.KDA_ERR_INVALID_ARG
    assert n(eps=-1.0) == K.KDA_ERR_INVALID_ARG
    assert n(ys=1000) == K.KDA_ERR_INVALID_ARG
    nx = lambda **o: lib.kda_gated_rmsnorm_ex(*dict(
        dict(x=FAKE, xs=2048, gate=FAKE, gs=2048, r=None, rs=0, w=None, b=None, y=FAKE, ys=2048,
             ro=None, ros=0, dt=2, T=4, H=16, dim=128, eps=1e-6, flags=0, stream=None),
        **o).values())
    assert nx(T=0) == K.KDA_OK
    assert nx(dt=3) == K.KDA_ERR_INVALID_ARG
    assert nx(flags=4) == K.KDA_ERR_INVALID_ARG
    assert nx(dim=12) == K.KDA_ERR_UNSUPPORTED
    assert nx(r=FAKE, rs=100) == K.KDA_ERR_INVALID_ARG        # residual stride < H * dim
    assert nx(ro=FAKE, ros=2052) == K.KDA_ERR_INVALID_ARG     # not a multiple of 8
    assert nx(b=FAKE + 2) == K.KDA_ERR_INVALID_ARG            # misaligned bias
    assert nx(ro=FAKE + 8, ros=2048) == K.KDA_ERR_INVALID_ARG
    # fp16 is a norm-only type: the attention entry points reject it.
    assert _prefill(lib, act=2) == K.KDA_ERR_INVALID_ARG
    c = lambda **o: lib.kda_causal_conv1d(*dict(
        dict(x=FAKE, xs=6144, w=FAKE, b=None, st=FAKE, slots=4, cu=FAKE, idx=FAKE, hi=None,
             n=1, T=64, C=6144, W=4, dt=1, flags=1, y=FAKE, ys=6144, stream=None), **o).values())
    assert c(n=0) == K.KDA_OK
    assert c(W=1) == K.KDA_ERR_UNSUPPORTED
    assert c(W=9) == K.KDA_ERR_UNSUPPORTED
    assert c(C=6) == K.KDA_ERR_UNSUPPORTED
    assert c(w=None) == K.KDA_ERR_INVALID_ARG
    assert c(xs=100) == K.KDA_ERR_INVALID_ARG
    assert c(flags=4) == K.KDA_ERR_INVALID_ARG


def _norm_tail(over):
    t = dict(ngate=FAKE, ngs=2048, nw=None, neps=1e-6, nout=FAKE, nos=2048)
    t.update({k: v for k, v in over.items() if k in t})
    return t


def _prefill_norm(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, act=1, qs=2048, ks=2048, vs=2048, g=FAKE, beta=FAKE,
             cu=FAKE, n=1, T=64, H=16, dk=128, dv=128, pool=FAKE, sdt=0, slots=4, idx=FAKE,
             hi=None, ck=None, cap=0, interval=0, scale=1.0, C=64, flags=0, out=FAKE,
             os=2048)
    a.update({k: v for k, v in over.items() if k in a})
    w = dict(ws=FAKE, wsb=0, stream=None)
    w.update({k: v for k, v in over.items() if k in w})
    return lib.kda_chunk_prefill_norm(*a.values(), *_norm_tail(over).values(), *w.values())


def _conv_prefill_norm(lib, **over):
    a = dict(x=FAKE, xs=6144, act=1, w=FAKE, b=None, W=4, cflags=1, cpool=FAKE, g=FAKE,
             beta=FAKE, cu=FAKE, n=1, T=64, H=16, dk=128, dv=128, pool=FAKE, sdt=0, slots=4,
             idx=FAKE, hi=None, ck=None, cap=0, interval=0, scale=1.0, C=64, flags=1,
             out=FAKE, os=2048)
    a.update({k: v for k, v in over.items() if k in a})
    w = dict(ws=FAKE, wsb=0, stream=None)
    w.update({k: v for k, v in over.items() if k in w})
    return lib.kda_conv_chunk_prefill_norm(*a.values(), *_norm_tail(over).values(), *w.values())


def test_prefill_norm_validation(lib):
    from gated_delta_rule_42_amd import kda as K
    plain = K.chunk_prefill_workspace_size(1, 64, 16, 128, 128, 64)
    need = K.chunk_prefill_workspace_size(1, 64, 16, 128, 128, 64, norm=True)
    assert need > plain
    for call in (_prefill_norm, _conv_prefill_norm):
        assert call(lib, n=0) == K.KDA_OK                               # nothing to do
        assert call(lib, dk=48, dv=48, xs=3 * 16 * 48) == K.KDA_ERR_UNSUPPORTED
        # The plain prefill's workspace is not enough for the fused norm.
        assert call(lib, wsb=plain) == K.KDA_ERR_WORKSPACE_TOO_SMALL
        assert call(lib, wsb=need, ngate=None) == K.KDA_ERR_INVALID_ARG
        assert call(lib, wsb=need, nout=None) == K.KDA_ERR_INVALID_ARG
        assert call(lib, wsb=need, ngs=1000) == K.KDA_ERR_INVALID_ARG   # < H * dv
        assert call(lib, wsb=need, nos=2052) == K.KDA_ERR_INVALID_ARG   # not a multiple of 8
        assert call(lib, wsb=need, neps=-1.0) == K.KDA_ERR_INVALID_ARG
        assert call(lib, wsb=need, neps=float("nan")) == K.KDA_ERR_INVALID_ARG
        assert call(lib, wsb=need, nw=FAKE + 4) == K.KDA_ERR_INVALID_ARG   # misaligned
        assert call(lib, wsb=need, nout=FAKE + 8) == K.KDA_ERR_INVALID_ARG
        # 64 rows of out at this stride span 2^31 bytes: past the 32-bit
        # offsets the norm reads out with (the plain prefill takes it).
        assert call(lib, wsb=need, os=1 << 24) == K.KDA_ERR_INVALID_ARG
    # The conv front end's own checks still apply.
    assert _conv_prefill_norm(lib, wsb=need, W=9) == K.KDA_ERR_UNSUPPORTED
    assert _conv_prefill_norm(lib, wsb=need, w=None) == K.KDA_ERR_INVALID_ARG
