"""Pins of the fp64 oracle to facts outside itself.

Each `pin_*` function takes a loaded `oracle.Oracle` and raises AssertionError
when the oracle disagrees with the fact it checks.  tests/test_oracle_pins.py
runs them on the real oracle; tests/test_oracle_mutants.py runs them on
deliberately broken copies and requires every copy to fail at least one pin.

What pins what (the pages print no numeric example, so the facts come from
hand arithmetic, closed forms, invariants, library routines and a second
algorithm):
  hand_worked        three tokens worked in exact fractions (tests/golden)
  beta_zero          beta = 0 leaves pure per-channel decay: S_T = Diag(prod alpha) S_0
  exact_retrieval    alpha = 1, beta = 1, orthonormal keys: reading k_j returns v_j
  delta_invariant    beta = 1, unit key: S_t^T k_t = v_t for any decay and state
  linearity          (S_0, v) -> (o, S_T) is linear for fixed q, k, g, beta
  chunk_form         the chunked algebra (second algorithm) at C = 1..64
  split_calls        one call equals the same tokens split over calls via the pool
  checkpoints        checkpoint j equals the final state of a call cut at j*interval
  checkpoints_absolute with start positions: rows at absolute multiples of the
                     interval, each the state after that prefix; split calls agree
  decode             decode equals one-token prefill
  padding_empty      slot < 0 and empty sequences touch nothing
  has_init           has_initial_state = 0 equals a zeroed slot
  l2norm             flag output is invariant to positive rescaling of q, k
  conv_numpy         conv1d equals numpy.convolve per channel, SiLU from scipy
  conv_state         conv1d state carries across split calls
  rmsnorm_library    gated RMSNorm equals torch rms_norm times silu (float64)
  rmsnorm_variants   residual/prenorm, bias and sigmoid gate vs torch (float64)
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def _frac(x) -> float:
    return float(Fraction(x))


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def _rand_case(rng, T, H, dk, dv, unit=True):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -np.log1p(np.exp(rng.standard_normal((T, H, dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


# --------------------------------------------------------------------------
def pin_hand_worked(orc):
    with open(os.path.join(GOLDEN, "hand_worked_recurrence.json")) as f:
        gold = json.load(f)
    toks = gold["tokens"]
    T = len(toks)
    q = np.array([[[_frac(x) for x in t["q"]]] for t in toks])
    k = np.array([[[_frac(x) for x in t["k"]]] for t in toks])
    v = np.array([[[_frac(x) for x in t["v"]]] for t in toks])
    g = np.log(np.array([[[_frac(x) for x in t["alpha"]]] for t in toks]))
    beta = np.array([[_frac(t["beta"])] for t in toks])
    S0 = np.array([[_frac(x) for x in row] for row in gold["S0"]])
    pool = np.full((3, 1, 2, 1), 7.0)
    pool[1, 0] = S0
    scale = _frac(gold["scale"])
    o, pool2, ck = orc.prefill(q, k, v, g, beta, [0, T], pool, [1], ckpt_interval=1,
                               scale=scale)
    _close(o[:, 0, 0], [_frac(x) for x in gold["expected_o"]], 1e-14, "hand-worked o")
    states = np.array([[[_frac(x) for x in row] for row in st] for st in gold["expected_states"]])
    _close(ck[:, 0], states, 1e-14, "hand-worked states")
    _close(pool2[1, 0], states[-1], 1e-14, "hand-worked final state")
    _close(pool2[[0, 2]], pool[[0, 2]], 0.0, "untouched slots")
    # The same three tokens as three decode steps.
    p = pool.copy()
    for t in range(T):
        od, p = orc.decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1],
                           p, [1], scale=scale)
        _close(od[0, 0, 0], _frac(gold["expected_o"][t]), 1e-14, f"hand-worked decode o{t}")
        _close(p[1, 0], states[t], 1e-14, f"hand-worked decode state {t}")
    z = gold["zero_state_case"]
    zq = np.array([[[_frac(x) for x in z["q"]]]])
    zk = np.array([[[_frac(x) for x in z["k"]]]])
    zv = np.array([[[_frac(x) for x in z["v"]]]])
    zg = np.log(np.array([[[_frac(x) for x in z["alpha"]]]]))
    zb = np.array([[_frac(z["beta"])]])
    o, pz, _ = orc.prefill(zq, zk, zv, zg, zb, [0, 1], np.full((1, 1, 2, 1), 5.0), [0],
                           has_init=[0])
    _close(o[0, 0, 0], _frac(z["expected_o"]), 1e-14, "zero-state o")
    _close(pz[0, 0], [[_frac(x) for x in r] for r in z["expected_state"]], 1e-14,
           "zero-state final state")


def pin_beta_zero(orc):
    rng = np.random.default_rng(101)
    T, H, dk, dv = 9, 2, 5, 3
    q, k, v, g, _ = _rand_case(rng, T, H, dk, dv)
    beta = np.zeros((T, H))
    pool = rng.standard_normal((2, H, dk, dv))
    scale = 0.75
    o, p2, _ = orc.prefill(q, k, v, g, beta, [0, T], pool, [1], scale=scale)
    G = np.cumsum(g, axis=0)                                  # [T, H, dk]
    S0 = pool[1]
    _close(p2[1], np.exp(G[-1])[:, :, None] * S0, 1e-13, "beta=0 final state")
    want = scale * np.einsum("hkv,thk->thv", S0, np.exp(G) * q)
    _close(o, want, 1e-13, "beta=0 outputs")


def pin_exact_retrieval(orc):
    rng = np.random.default_rng(102)
    d, T = 8, 8
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Q.T                                                 # orthonormal rows
    v = rng.standard_normal((T, 1, d))
    k = keys[:, None, :].copy()
    pick = np.array([rng.integers(0, t + 1) for t in range(T)])
    q = keys[pick][:, None, :]
    g = np.zeros((T, 1, d))
    beta = np.ones((T, 1))
    o, p2, _ = orc.prefill(q, k, v, g, beta, [0, T], np.zeros((1, 1, d, d)), [0])
    _close(o[:, 0], v[pick, 0], 1e-12, "retrieval of an earlier key")
    _close(keys @ p2[0, 0], v[:, 0], 1e-12, "final state maps k_j to v_j")
    # A key written twice keeps the latest value.
    k2 = np.concatenate([k, k[2:3]], axis=0)
    v2 = np.concatenate([v, rng.standard_normal((1, 1, d))], axis=0)
    q2 = np.concatenate([q, k[2:3]], axis=0)
    o2, _, _ = orc.prefill(q2, k2, v2, np.zeros((T + 1, 1, d)), np.ones((T + 1, 1)),
                           [0, T + 1], np.zeros((1, 1, d, d)), [0])
    _close(o2[-1, 0], v2[-1, 0], 1e-12, "overwrite with the latest value")


def pin_delta_invariant(orc):
    rng = np.random.default_rng(103)
    T, H, dk, dv = 10, 2, 6, 4
    q, k, v, g, _ = _rand_case(rng, T, H, dk, dv)
    beta = np.ones((T, H))
    pool = rng.standard_normal((1, H, dk, dv))
    o, _, _ = orc.prefill(k, k, v, g, beta, [0, T], pool, [0])
    _close(o, v, 1e-12, "S_t^T k_t = v_t at beta = 1")


def pin_linearity(orc):
    rng = np.random.default_rng(104)
    T, H, dk, dv = 12, 2, 5, 4
    q, k, va, g, beta = _rand_case(rng, T, H, dk, dv)
    vb = rng.standard_normal(va.shape)
    Sa = rng.standard_normal((1, H, dk, dv))
    Sb = rng.standard_normal((1, H, dk, dv))
    a, b = 0.7, -1.3
    oa, pa, _ = orc.prefill(q, k, va, g, beta, [0, T], Sa, [0], scale=0.5)
    ob, pb, _ = orc.prefill(q, k, vb, g, beta, [0, T], Sb, [0], scale=0.5)
    oc, pc, _ = orc.prefill(q, k, a * va + b * vb, g, beta, [0, T], a * Sa + b * Sb, [0],
                            scale=0.5)
    _close(oc, a * oa + b * ob, 1e-12, "linearity of o")
    _close(pc, a * pa + b * pb, 1e-12, "linearity of the state")


def pin_chunk_form(orc):
    from oracle import chunk_form
    rng = np.random.default_rng(105)
    lens = [37, 0, 5, 16]
    T, H, dk, dv = sum(lens), 2, 8, 6
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lens)])
    slots = [3, 0, -1, 1]
    pool = rng.standard_normal((4, H, dk, dv))
    o_tok, p_tok, _ = orc.prefill(q, k, v, g, beta, cu, pool, slots, has_init=[1, 1, 1, 0],
                                  scale=0.3)
    for C in (1, 2, 3, 4, 8, 16, 64):
        o_ch, p_ch = chunk_form.chunk_prefill(q, k, v, g, beta, cu, pool, slots,
                                              has_init=[1, 1, 1, 0], chunk=C, scale=0.3)
        _close(o_tok, o_ch, 1e-12, f"token loop vs chunk form, C={C}: o")
        _close(p_tok, p_ch, 1e-12, f"token loop vs chunk form, C={C}: pool")


def pin_split_calls(orc):
    rng = np.random.default_rng(106)
    T, H, dk, dv = 40, 2, 6, 5
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv)
    pool = rng.standard_normal((2, H, dk, dv))
    o, p, _ = orc.prefill(q, k, v, g, beta, [0, T], pool, [1])
    o1, p1, _ = orc.prefill(q[:13], k[:13], v[:13], g[:13], beta[:13], [0, 13], pool, [1])
    o2, p2, _ = orc.prefill(q[13:], k[13:], v[13:], g[13:], beta[13:], [0, T - 13], p1, [1])
    _close(np.concatenate([o1, o2]), o, 1e-12, "split calls: o")
    _close(p2, p, 1e-12, "split calls: state")


def pin_checkpoints(orc):
    rng = np.random.default_rng(107)
    lens = [10, 3, 8]
    T, H, dk, dv = sum(lens), 2, 4, 3
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lens)])
    pool = rng.standard_normal((3, H, dk, dv))
    slots = [2, 0, 1]
    _, _, ck = orc.prefill(q, k, v, g, beta, cu, pool, slots, ckpt_interval=4)
    assert ck.shape[0] == 2 + 0 + 2, f"checkpoint rows {ck.shape[0]}"
    row = 0
    for i, L in enumerate(lens):
        for j in range(L // 4):
            t0, t1 = cu[i], cu[i] + 4 * (j + 1)
            _, pj, _ = orc.prefill(q[t0:t1], k[t0:t1], v[t0:t1], g[t0:t1], beta[t0:t1],
                                   [0, t1 - t0], pool, [slots[i]])
            _close(ck[row], pj[slots[i]], 1e-13, f"checkpoint {j} of sequence {i}")
            row += 1


def pin_checkpoints_absolute(orc):
    """With start positions, checkpoint rows fall where start + tokens
    processed is a multiple of the interval (rows sequence by sequence), and
    each equals the state after that prefix of the call; a sequence split
    over two calls at a point off the interval grid gives the same
    checkpoints as one call."""
    rng = np.random.default_rng(116)
    lens, start, iv = [11, 6, 9, 0], [3, 0, 13, 5], 4
    T, H, dk, dv = sum(lens), 2, 4, 3
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lens)])
    pool = rng.standard_normal((4, H, dk, dv))
    slots = [1, 3, 0, 2]
    _, _, ck = orc.prefill(q, k, v, g, beta, cu, pool, slots, ckpt_interval=iv, start_pos=start)
    assert ck.shape[0] == 3 + 1 + 2 + 0, f"checkpoint rows {ck.shape[0]}"
    row = 0
    for i, L in enumerate(lens):
        for p in range(start[i] + 1, start[i] + L + 1):
            if p % iv:
                continue
            t0, t1 = cu[i], cu[i] + p - start[i]
            _, pj, _ = orc.prefill(q[t0:t1], k[t0:t1], v[t0:t1], g[t0:t1], beta[t0:t1],
                                   [0, t1 - t0], pool, [slots[i]])
            _close(ck[row], pj[slots[i]], 1e-13, f"checkpoint at position {p} of sequence {i}")
            row += 1
    # Sequence 0 (start 3) as two calls of 5 and 6 tokens.
    _, p1, c1 = orc.prefill(q[:5], k[:5], v[:5], g[:5], beta[:5], [0, 5], pool, [1],
                            ckpt_interval=iv, start_pos=[3])
    _, _, c2 = orc.prefill(q[5:11], k[5:11], v[5:11], g[5:11], beta[5:11], [0, 6], p1, [1],
                           ckpt_interval=iv, start_pos=[8])
    assert c1.shape[0] == 2 and c2.shape[0] == 1
    _close(np.concatenate([c1, c2]), ck[:3], 1e-13, "split calls: same absolute checkpoints")


def pin_decode(orc):
    rng = np.random.default_rng(108)
    B, H, dk, dv = 7, 3, 5, 4
    q, k, v, g, beta = _rand_case(rng, B, H, dk, dv)
    pool = rng.standard_normal((9, H, dk, dv))
    slots = rng.permutation(9)[:B]
    od, pd = orc.decode(q, k, v, g, beta, pool, slots, scale=0.9)
    op, pp, _ = orc.prefill(q, k, v, g, beta, np.arange(B + 1), pool, slots, scale=0.9)
    _close(od, op, 1e-14, "decode vs one-token prefill: o")
    _close(pd, pp, 1e-14, "decode vs one-token prefill: pool")


def pin_padding_empty(orc):
    rng = np.random.default_rng(109)
    lens = [4, 0, 3]
    T, H, dk, dv = 7, 2, 3, 3
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv)
    pool = rng.standard_normal((3, H, dk, dv))
    o, p, _ = orc.prefill(q, k, v, g, beta, [0, 4, 4, 7], pool, [0, 1, -1])
    _close(o[4:], np.zeros((3, H, dv)), 0.0, "padding rows are zero")
    _close(p[1:], pool[1:], 0.0, "empty and padding sequences leave the pool alone")
    od, pd = orc.decode(q[:3], k[:3], v[:3], g[:3], beta[:3], pool, [-1, 2, -1])
    _close(od[[0, 2]], np.zeros((2, H, dv)), 0.0, "decode padding rows are zero")
    _close(pd[:2], pool[:2], 0.0, "decode padding rows leave the pool alone")


def pin_has_init(orc):
    rng = np.random.default_rng(110)
    T, H, dk, dv = 6, 2, 4, 4
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv)
    pool = rng.standard_normal((2, H, dk, dv))
    zeroed = pool.copy()
    zeroed[1] = 0.0
    o1, p1, _ = orc.prefill(q, k, v, g, beta, [0, T], pool, [1], has_init=[0])
    o2, p2, _ = orc.prefill(q, k, v, g, beta, [0, T], zeroed, [1], has_init=[1])
    _close(o1, o2, 0.0, "has_init=0 equals a zeroed slot: o")
    _close(p1[1], p2[1], 0.0, "has_init=0 equals a zeroed slot: state")


def pin_l2norm(orc):
    rng = np.random.default_rng(111)
    T, H, dk, dv = 8, 2, 6, 3
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv)
    pool = rng.standard_normal((1, H, dk, dv))
    o1, p1, _ = orc.prefill(q, k, v, g, beta, [0, T], pool, [0], l2norm_qk=True, l2_eps=0.0)
    o0, p0, _ = orc.prefill(q, k, v, g, beta, [0, T], pool, [0], l2norm_qk=False)
    _close(o1, o0, 1e-12, "unit inputs are fixed points of the normalisation")
    c = rng.uniform(0.1, 10.0, (T, H, 1))
    o2, p2, _ = orc.prefill(c * q, 3.0 * c * k, v, g, beta, [0, T], pool, [0],
                            l2norm_qk=True, l2_eps=0.0)
    _close(o2, o1, 1e-12, "invariance to positive rescaling of q, k: o")
    _close(p2, p1, 1e-12, "invariance to positive rescaling of q, k: state")


def pin_conv_numpy(orc):
    from scipy.special import expit
    rng = np.random.default_rng(112)
    T, C, W = 19, 5, 4
    x = rng.standard_normal((T, C))
    w = rng.uniform(-0.5, 0.5, (C, W))
    y, cp = orc.conv1d(x, w, [0, T], np.full((1, W - 1, C), 9.0), [0], has_init=[0])
    for c in range(C):
        pre = np.convolve(x[:, c], w[c, ::-1])[:T]
        _close(y[:, c], pre * expit(pre), 1e-13, f"conv channel {c} vs numpy.convolve")
    _close(cp[0], x[-(W - 1):], 0.0, "conv state holds the last W-1 inputs")
    e = np.zeros((C, W))
    e[:, W - 1] = 1.0
    y2, _ = orc.conv1d(x, e, [0, T], np.zeros((1, W - 1, C)), [0])
    _close(y2, x * expit(x), 1e-14, "identity filter gives silu(x)")
    y3, _ = orc.conv1d(x, w, [0, T], np.zeros((1, W - 1, C)), [0], silu=False)
    for c in range(C):
        _close(y3[:, c], np.convolve(x[:, c], w[c, ::-1])[:T], 1e-13, "conv without activation")


def pin_conv_state(orc):
    rng = np.random.default_rng(113)
    T, C, W = 23, 6, 4
    x = rng.standard_normal((T, C))
    w = rng.uniform(-0.5, 0.5, (C, W))
    b = rng.standard_normal(C)
    pool = rng.standard_normal((3, W - 1, C))
    y, p = orc.conv1d(x, w, [0, T], pool, [2], bias=b)
    ya, pa = orc.conv1d(x[:2], w, [0, 2], pool, [2], bias=b)   # shorter than W-1
    yb, pb = orc.conv1d(x[2:9], w, [0, 7], pa, [2], bias=b)
    yc, pc = orc.conv1d(x[9:], w, [0, T - 9], pb, [2], bias=b)
    _close(np.concatenate([ya, yb, yc]), y, 1e-13, "conv split calls: y")
    _close(pc, p, 0.0, "conv split calls: state")
    _close(p[:2], pool[:2], 0.0, "conv leaves other slots alone")
    # Varlen with padding: the second sequence is padding, the third empty.
    y4, p4 = orc.conv1d(x[:9], w, [0, 5, 9, 9], pool, [0, -1, 1], bias=b)
    _close(y4[5:], np.zeros((4, C)), 0.0, "conv padding rows are zero")
    _close(p4[1:], pool[1:], 0.0, "conv padding and empty sequences leave state alone")


def pin_rmsnorm_library(orc):
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(114)
    rows, dim, eps = 11, 16, 1e-6
    x = rng.standard_normal((rows, dim))
    gate = rng.standard_normal((rows, dim))
    w = 1.0 + 0.1 * rng.standard_normal(dim)
    y = orc.gated_rmsnorm(x, gate, w, eps)
    xt, gt, wt = (torch.from_numpy(a) for a in (x, gate, w))
    ref = (F.rms_norm(xt, (dim,), wt, eps) * F.silu(gt)).numpy()
    _close(y, ref, 1e-13, "gated RMSNorm vs torch rms_norm * silu")
    cst = np.full((3, dim), 0.25)
    y2 = orc.gated_rmsnorm(cst, gate[:3], None, eps)
    _close(y2, 0.25 / np.sqrt(0.0625 + eps) * F.silu(torch.from_numpy(gate[:3])).numpy(),
           1e-14, "constant rows: c / sqrt(c^2 + eps) * silu(gate)")


def pin_rmsnorm_variants(orc):
    """Residual / prenorm, bias and the sigmoid gate against torch's rms_norm,
    sigmoid and silu in float64; y_silu = y_sigmoid * gate; with weight 0 the
    output is bias * act(gate)."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(115)
    rows, dim, eps = 9, 24, 1e-6
    x, gate, res = (rng.standard_normal((rows, dim)) for _ in range(3))
    w = 1.0 + 0.1 * rng.standard_normal(dim)
    b = 0.3 * rng.standard_normal(dim)
    gt = torch.from_numpy(gate)
    hsum = x + res
    normed = (F.rms_norm(torch.from_numpy(hsum), (dim,), torch.from_numpy(w), eps)
              + torch.from_numpy(b))
    for sig, act in ((False, F.silu(gt)), (True, torch.sigmoid(gt))):
        y, h = orc.gated_rmsnorm_ex(x, gate, w, b, eps, residual=res, sigmoid=sig)
        _close(y, (normed * act).numpy(), 1e-13, f"gated RMSNorm variant sigmoid={sig}")
        _close(h, hsum, 0.0, "prenorm output h = x + residual")
    y_silu, _ = orc.gated_rmsnorm_ex(x, gate, w, b, eps, residual=res)
    y_sig, _ = orc.gated_rmsnorm_ex(x, gate, w, b, eps, residual=res, sigmoid=True)
    _close(y_silu, y_sig * gate, 1e-13, "silu gate = sigmoid gate times gate")
    y0, h0 = orc.gated_rmsnorm_ex(x, gate, np.zeros(dim), b, eps)
    _close(y0, b * (F.silu(gt)).numpy(), 1e-14, "weight 0: bias * act(gate)")
    _close(h0, x, 0.0, "no residual: h = x")
    y1, _ = orc.gated_rmsnorm_ex(x, gate, w, None, eps)
    _close(y1, orc.gated_rmsnorm(x, gate, w, eps), 0.0, "no residual, no bias = plain norm")


def pin_spec_decode(orc):
    """Speculative decode: row b's ntok tokens from pool[slot_b], state after
    each token, pool untouched; commit copies an accepted prefix's state."""
    rng = np.random.default_rng(113)
    B, ntok, H, dk, dv = 4, 3, 2, 5, 4
    q, k, v, g, beta = _rand_case(rng, B * ntok, H, dk, dv)
    pool = rng.standard_normal((6, H, dk, dv))
    slots = np.array([4, -1, 0, 2])
    o, ts = orc.spec_decode(q, k, v, g, beta, pool, slots, ntok, scale=0.8)
    # Closed form with beta = 0: pure decay, outputs read the decayed state.
    o0, ts0 = orc.spec_decode(q, k, v, g, np.zeros_like(beta), pool, slots, ntok, scale=0.8)
    for b in (0, 2, 3):
        G = np.cumsum(g[b * ntok:(b + 1) * ntok], axis=0)        # [ntok, H, dk]
        S0 = pool[slots[b]]
        for t in range(ntok):
            _close(ts0[b, t], np.exp(G[t])[:, :, None] * S0, 1e-13, "spec beta=0 state")
            _close(o0[b * ntok + t], 0.8 * np.einsum("hkv,hk->hv", S0, np.exp(G[t]) * q[b * ntok + t]),
                   1e-13, "spec beta=0 output")
    # The same tokens as a varlen prefill of ntok-token sequences with a
    # checkpoint after every token (a different indexing path).
    cu = np.arange(0, B * ntok + 1, ntok)
    op, _, ck = orc.prefill(q, k, v, g, beta, cu, pool, slots, ckpt_interval=1, scale=0.8)
    real = [b for b in range(B) if slots[b] >= 0]
    rows = np.concatenate([np.arange(b * ntok, (b + 1) * ntok) for b in real])
    _close(o[rows], op[rows], 1e-14, "spec outputs vs prefill")
    for b in real:
        _close(ts[b], ck[b * ntok:(b + 1) * ntok], 1e-14, "spec token states vs checkpoints")
    _close(o[ntok:2 * ntok], np.zeros((ntok, H, dv)), 0.0, "spec padding rows are zero")
    assert np.isnan(ts[1]).all(), "padding rows leave their token states alone"
    # Commit: accepted prefix lengths 2, -, 0, 3.
    acc = np.array([2, 1, 0, 3])
    p2 = orc.spec_commit(ts, acc, pool, slots)
    _close(p2[4], ts[0, 1], 0.0, "commit copies the last accepted state")
    _close(p2[2], ts[3, 2], 0.0, "commit of a full acceptance")
    keep = [s for s in range(6) if s not in (4, 2)]
    _close(p2[keep], pool[keep], 0.0, "zero acceptance, padding and other slots unchanged")
    # Accepting n tokens equals prefilling those n tokens from the same state.
    _, pp, _ = orc.prefill(q[0:2], k[0:2], v[0:2], g[0:2], beta[0:2], [0, 2], pool, [4])
    _close(p2[4], pp[4], 1e-14, "commit of 2 tokens vs a 2-token prefill")


ALL_PINS = [pin_hand_worked, pin_beta_zero, pin_exact_retrieval, pin_delta_invariant,
            pin_linearity, pin_chunk_form, pin_split_calls, pin_checkpoints,
            pin_checkpoints_absolute, pin_decode,
            pin_padding_empty, pin_has_init, pin_l2norm, pin_conv_numpy, pin_conv_state,
            pin_rmsnorm_library, pin_rmsnorm_variants, pin_spec_decode]
