"""Pins for the fp64 oracle: facts fixed outside the oracle itself.

Each ``pin_*`` function takes an oracle module (the real one, or a copy with
a planted mistake) and raises AssertionError if the module disagrees with
the fact.  The facts come from:

* hand-worked values (tests/golden/hand_worked.json),
* exact rational arithmetic (Python ``fractions``) of the token recurrence,
* closed forms (geometric series for all-ones inputs),
* library routines for special cases: ``scipy.signal.lfilter`` is the
  first-order decayed prefix sum, ``numpy.tril``/``cumsum`` the no-decay
  case,
* invariants: the three definitions agree for every block size; splitting a
  sequence and continuing from the state gives the same result; a decode
  step equals the last row of a longer prefill; packing order does not
  matter.
"""

import json
import os
from fractions import Fraction

import numpy as np
import scipy.signal

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol:.1e} * {scale:.3e}"


def _forms(orc, beta_list=(1, 2, 3, 5)):
    """(name, fn(q,k,v,lam,s0) -> (o, s)) for every definition the oracle holds."""
    out = [("quadratic", orc.quadratic), ("quadratic_loops", orc.quadratic_loops),
           ("recurrent", orc.recurrent)]
    for b in beta_list:
        out.append((f"blockwise{b}", (lambda b_: (lambda q, k, v, lam, s0=None:
                                                 orc.blockwise(q, k, v, lam, b_, s0)))(b)))
    return out


def pin_golden(orc):
    g = json.load(open(GOLDEN))
    for case in g["prefill"]:
        q, k, v = (np.array(case[x], dtype=np.float64) for x in "qkv")
        s0 = None if case["s0"] is None else np.array(case["s0"], dtype=np.float64)
        for name, fn in _forms(orc):
            o, s = fn(q, k, v, case["lam"], s0)
            _close(o, case["o"], 0.0, f"golden {case['name']} {name} o")
            _close(s, case["s_final"], 0.0, f"golden {case['name']} {name} state")
    for case in g["decode"]:
        o, s = orc.decode_step(np.array(case["q"], float), np.array(case["k"], float),
                               np.array(case["v"], float), np.array(case["s"], float),
                               case["lam"])
        _close(o, case["o"], 0.0, f"golden decode {case['name']} o")
        _close(s, case["s_new"], 0.0, f"golden decode {case['name']} state")


def _fraction_recurrence(q, k, v, lam, s0):
    """Exact token recurrence over Fractions (the value fp64 must round to)."""
    L, dk = q.shape
    dv = v.shape[1]
    lam = Fraction(lam)
    S = [[Fraction(s0[r][c]) if s0 is not None else Fraction(0) for c in range(dv)]
         for r in range(dk)]
    o = []
    for t in range(L):
        S = [[lam * S[r][c] + Fraction(k[t][r]) * Fraction(v[t][c]) for c in range(dv)]
             for r in range(dk)]
        o.append([sum((Fraction(q[t][r]) * S[r][c] for r in range(dk)), Fraction(0))
                  for c in range(dv)])
    return o, S


def pin_exact_rational(orc):
    """Small integer inputs, lam = 3/4: every form must equal the exact value."""
    rng = _rng(7)
    L, d = 9, 3
    q, k, v = (rng.integers(-3, 4, size=(L, d)).astype(np.float64) for _ in range(3))
    s0 = rng.integers(-2, 3, size=(d, d)).astype(np.float64)
    for use_s0 in (False, True):
        s = s0 if use_s0 else None
        o_ex, s_ex = _fraction_recurrence(q, k, v, 0.75, s)
        o_ex = np.array([[float(x) for x in row] for row in o_ex])
        s_ex = np.array([[float(x) for x in row] for row in s_ex])
        for name, fn in _forms(orc, (1, 2, 4, 9, 20)):
            o, st = fn(q, k, v, 0.75, s)
            _close(o, o_ex, 1e-14, f"exact {name} o s0={use_s0}")
            _close(st, s_ex, 1e-14, f"exact {name} state s0={use_s0}")


def pin_lfilter(orc):
    """The decayed prefix sum of k_t^T v_t is a first-order IIR filter along t.

    scipy.signal.lfilter([1], [1, -lam], x) computes y_t = x_t + lam*y_{t-1},
    which is the state S_t; then o_t = q_t S_t.
    """
    rng = _rng(11)
    L, dk, dv = 40, 5, 4
    q, k = rng.standard_normal((L, dk)), rng.standard_normal((L, dk))
    v = rng.standard_normal((L, dv))
    for lam in (0.9, 0.37, 1.0):
        x = np.einsum("tr,tc->trc", k, v)
        S_all = scipy.signal.lfilter([1.0], [1.0, -lam], x, axis=0)
        o_ref = np.einsum("tr,trc->tc", q, S_all)
        for name, fn in _forms(orc, (1, 7, 16, 64)):
            if name == "quadratic_loops" and lam != 0.9:
                continue
            o, st = fn(q, k, v, lam, None)
            _close(o, o_ref, 1e-11, f"lfilter {name} lam={lam} o")
            _close(st, S_all[-1], 1e-11, f"lfilter {name} lam={lam} state")


def pin_nodecay_library(orc):
    """lam = 1: O = tril(Q K^T) V and S_L = K^T V; with S0, O += Q S0."""
    rng = _rng(13)
    L, d = 50, 6
    q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
    s0 = rng.standard_normal((d, d))
    o_ref = np.tril(q @ k.T) @ v + q @ s0
    s_ref = s0 + k.T @ v
    for name, fn in _forms(orc, (1, 8, 13, 50, 64)):
        if name == "quadratic_loops":
            continue
        o, st = fn(q, k, v, 1.0, s0)
        _close(o, o_ref, 1e-12, f"nodecay {name} o")
        _close(st, s_ref, 1e-12, f"nodecay {name} state")


def pin_geometric(orc):
    """All-ones q, k, v of width d: o_t[c] = d (1 - lam^(t+1)) / (1 - lam),
    S_L[r, c] = (1 - lam^L) / (1 - lam); lam = 1 gives d (t+1) and L."""
    L, d = 37, 4
    ones = np.ones((L, d))
    t = np.arange(L)
    for lam in (0.5, 0.875, 1.0):
        if lam == 1.0:
            o_ref = np.repeat((d * (t + 1.0))[:, None], d, 1)
            s_ref = np.full((d, d), float(L))
        else:
            o_ref = np.repeat((d * (1 - lam ** (t + 1.0)) / (1 - lam))[:, None], d, 1)
            s_ref = np.full((d, d), (1 - lam ** L) / (1 - lam))
        for name, fn in _forms(orc, (1, 4, 10, 37, 40)):
            o, st = fn(ones, ones, ones, lam, None)
            _close(o, o_ref, 1e-13, f"geometric {name} lam={lam} o")
            _close(st, s_ref, 1e-13, f"geometric {name} lam={lam} state")


def pin_three_way(orc, L=256, d=16, betas=(1, 7, 32, 100, 256, 300)):
    """The quadratic, recurrent and blockwise definitions agree for any beta."""
    rng = _rng(17)
    q, k, v = (rng.standard_normal((L, d)) / np.sqrt(d) for _ in range(3))
    s0 = rng.standard_normal((d, d))
    for lam in (1.0, 0.9, 0.3):
        for s in (None, s0):
            o1, s1 = orc.quadratic(q, k, v, lam, s)
            o2, s2 = orc.recurrent(q, k, v, lam, s)
            _close(o2, o1, 1e-12, f"three-way recurrent lam={lam}")
            _close(s2, s1, 1e-12, f"three-way recurrent state lam={lam}")
            for b in betas:
                o3, s3 = orc.blockwise(q, k, v, lam, b, s)
                _close(o3, o1, 1e-12, f"three-way blockwise beta={b} lam={lam}")
                _close(s3, s1, 1e-12, f"three-way blockwise state beta={b} lam={lam}")


def pin_continuation(orc):
    """Prefill of A||B equals prefill of B started from the state after A."""
    rng = _rng(19)
    L, d = 90, 8
    q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
    for lam in (0.95, 1.0):
        o_full, s_full = orc.blockwise(q, k, v, lam, 16)
        for cut in (1, 16, 45, 89):
            o_a, s_a = orc.blockwise(q[:cut], k[:cut], v[:cut], lam, 16)
            o_b, s_b = orc.blockwise(q[cut:], k[cut:], v[cut:], lam, 16, s_a)
            _close(np.concatenate([o_a, o_b]), o_full, 1e-12, f"continuation cut={cut}")
            _close(s_b, s_full, 1e-12, f"continuation state cut={cut}")


def pin_decode_consistency(orc):
    """prefill(x[:L]) then decode(x[L]) equals the last row of prefill(x[:L+1])."""
    rng = _rng(23)
    L, d = 33, 8
    q, k, v = (rng.standard_normal((L + 1, d)) for _ in range(3))
    for lam in (0.8, 1.0):
        _, s = orc.blockwise(q[:L], k[:L], v[:L], lam, 8)
        o1, s1 = orc.decode_step(q[L], k[L], v[L], s, lam)
        o_all, s_all = orc.blockwise(q, k, v, lam, 8)
        _close(o1, o_all[L], 1e-12, "decode vs prefill row")
        _close(s1, s_all, 1e-12, "decode vs prefill state")
        # batch form agrees with the single step
        ob, sb = orc.decode_batch(q[L][None, None], k[L][None, None], v[L][None, None],
                                  s[None, None], np.array([lam]))
        _close(ob[0, 0], o1, 0.0, "decode_batch")
        _close(sb[0, 0], s1, 0.0, "decode_batch state")


def pin_packing(orc):
    """Packed varlen prefill equals per-sequence runs; order of packing does
    not matter; a zero-length sequence returns its initial state; each head
    uses its own decay."""
    rng = _rng(29)
    H, d = 3, 4
    lens = [5, 0, 17, 1, 9]
    decay = np.array([0.9, 1.0, 0.5])
    T = sum(lens)
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    kv0 = rng.standard_normal((len(lens), H, d, d))
    cu = np.concatenate([[0], np.cumsum(lens)])
    for form in ("blockwise", "recurrent", "quadratic"):
        o, kv = orc.prefill_varlen(q, k, v, cu, decay, kv_init=kv0, form=form, beta=4)
        for s in range(len(lens)):
            a, b = cu[s], cu[s + 1]
            for h in range(H):
                o_ref, s_ref = orc.recurrent(q[a:b, h], k[a:b, h], v[a:b, h], decay[h], kv0[s, h])
                _close(o[a:b, h], o_ref, 1e-12, f"packing {form} s={s} h={h}")
                _close(kv[s, h], s_ref, 1e-12, f"packing {form} state s={s} h={h}")
        _close(kv[1], kv0[1], 0.0, "zero-length sequence keeps its state")
    # reverse packing order
    order = list(range(len(lens)))[::-1]
    lens_r = [lens[i] for i in order]
    cu_r = np.concatenate([[0], np.cumsum(lens_r)])
    idx = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in order]).astype(int)
    o_r, kv_r = orc.prefill_varlen(q[idx], k[idx], v[idx], cu_r, decay, kv_init=kv0[order], beta=4)
    o_f, kv_f = orc.prefill_varlen(q, k, v, cu, decay, kv_init=kv0, beta=4)
    _close(o_r, o_f[idx], 1e-12, "packing order o")
    _close(kv_r, kv_f[order], 1e-12, "packing order state")
    # decode batch: each head its own decay
    kv1 = rng.standard_normal((2, H, d, d))
    qd, kd, vd = (rng.standard_normal((2, H, d)) for _ in range(3))
    od, kvd = orc.decode_batch(qd, kd, vd, kv1, decay)
    for b in range(2):
        for h in range(H):
            S = decay[h] * kv1[b, h] + np.outer(kd[b, h], vd[b, h])
            _close(kvd[b, h], S, 1e-14, "decode_batch per-head decay")
            _close(od[b, h], qd[b, h] @ S, 1e-13, "decode_batch per-head o")


def pin_decode_pool(orc):
    """Pool decode, worked by hand with d = 1 and lambda = 1/2 (exact in
    binary): pool [2, 3, 5], slots [2, 0], q [1, 2], k [3, 1], v [1/2, 4].
    Sequence 0 on slot 2: S = 5/2 + 3/2 = 4, o = 4.  Sequence 1 on slot 0:
    S = 1 + 4 = 5, o = 10.  Slot 1 is untouched: pool becomes [5, 3, 4]."""
    pool = np.array([2.0, 3.0, 5.0]).reshape(3, 1, 1, 1)
    q = np.array([1.0, 2.0]).reshape(2, 1, 1)
    k = np.array([3.0, 1.0]).reshape(2, 1, 1)
    v = np.array([0.5, 4.0]).reshape(2, 1, 1)
    o, pool_new = orc.decode_pool(q, k, v, pool, [2, 0], np.array([0.5]))
    _close(o.reshape(-1), np.array([4.0, 10.0]), 0.0, "pool decode o")
    _close(pool_new.reshape(-1), np.array([5.0, 3.0, 4.0]), 0.0, "pool decode states")
    _close(pool.reshape(-1), np.array([2.0, 3.0, 5.0]), 0.0, "input pool unchanged")


def pin_prefill_pool(orc):
    """Pool prefill, worked by hand with d = 1 and lambda = 1/2 (exact in
    binary): pool [2, 3, 5]; sequence 0 (two tokens) on slot 2, sequence 1
    (one token) on slot 0; q [1, 2 | 1], k [3, 1 | 4], v [1/2, 2 | 1].  Sequence 0 from S = 5: S = 5/2 + 3/2 = 4, o = 4; then
    S = 2 + 2 = 4, o = 8.  Sequence 1 from S = 2: S = 1 + 4 = 5, o = 5.
    Slot 1 is untouched: pool becomes [5, 3, 4]; every block size agrees."""
    pool = np.array([2.0, 3.0, 5.0]).reshape(3, 1, 1, 1)
    q = np.array([1.0, 2.0, 1.0]).reshape(3, 1, 1)
    k = np.array([3.0, 1.0, 4.0]).reshape(3, 1, 1)
    v = np.array([0.5, 2.0, 1.0]).reshape(3, 1, 1)
    for beta in (1, 2, 64):
        o, pool_new = orc.prefill_pool(q, k, v, [0, 2, 3], np.array([0.5]), pool, [2, 0], beta=beta)
        _close(o.reshape(-1), np.array([4.0, 8.0, 5.0]), 0.0, f"pool prefill o beta={beta}")
        _close(pool_new.reshape(-1), np.array([5.0, 3.0, 4.0]), 0.0, "pool prefill states")
    _close(pool.reshape(-1), np.array([2.0, 3.0, 5.0]), 0.0, "input pool unchanged")


def pin_backward_autograd(orc):
    """Backward against automatic differentiation: torch (float64, CPU)
    differentiates a token-by-token forward, S_t = lam S_(t-1) + k_t^T v_t,
    o_t = q_t S_t, through the loss sum(O * dO) + sum(S_L * dS_L); both
    oracle backward forms must give the same gradients, also for the initial
    state and with neither initial state nor final-state gradient."""
    import torch

    rng = _rng(31)
    L, dk, dv = 11, 3, 4
    for lam, with_s0, with_g in ((0.8, True, True), (1.0, True, False), (0.5, False, True),
                                 (0.9, False, False)):
        q, k = rng.standard_normal((L, dk)), rng.standard_normal((L, dk))
        v, do = rng.standard_normal((L, dv)), rng.standard_normal((L, dv))
        s0 = rng.standard_normal((dk, dv))
        g = rng.standard_normal((dk, dv))
        if not with_s0:
            s0 = np.zeros((dk, dv))  # ds0 is then the gradient at a zero initial state
        tq, tk, tv, ts0 = (torch.tensor(x, dtype=torch.float64, requires_grad=True)
                           for x in (q, k, v, s0))
        S = ts0
        outs = []
        for t in range(L):
            S = lam * S + torch.outer(tk[t], tv[t])
            outs.append(tq[t] @ S)
        loss = (torch.stack(outs) * torch.tensor(do)).sum()
        if with_g:
            loss = loss + (S * torch.tensor(g)).sum()
        loss.backward()
        ref = [x.grad.numpy() for x in (tq, tk, tv, ts0)]
        for fn in (orc.backward_quadratic, orc.backward_recurrent):
            got = fn(q, k, v, do, lam, s0 if with_s0 else None, g if with_g else None)
            for name, a, b in zip(("dq", "dk", "dv", "ds0"), got, ref):
                _close(a, b, 1e-12, f"{fn.__name__} {name} lam={lam}")


def pin_backward_finite_difference(orc):
    """Central differences of a scalar loss through the oracle's forward
    (quadratic form) on a tiny problem match the backward within the
    difference error."""
    rng = _rng(37)
    L, d, lam, h = 5, 2, 0.7, 1e-6
    q, k, v, do = (rng.standard_normal((L, d)) for _ in range(4))
    s0, g = rng.standard_normal((d, d)), rng.standard_normal((d, d))

    def loss(q_, k_, v_, s0_):
        o, sl = orc.quadratic(q_, k_, v_, lam, s0_)
        return float((o * do).sum() + (sl * g).sum())

    grads = orc.backward_quadratic(q, k, v, do, lam, s0, g)
    for which, arr in enumerate((q, k, v, s0)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            args = [q.copy(), k.copy(), v.copy(), s0.copy()]
            args[which][idx] += h
            up = loss(*args)
            args[which][idx] -= 2 * h
            num[idx] = (up - loss(*args)) / (2 * h)
        _close(grads[which], num, 1e-6, f"finite difference input {which}")


def pin_backward_varlen(orc):
    """Packed-batch backward against automatic differentiation of the packed
    forward: torch (float64, CPU) runs the token recurrence of every
    (sequence, head) of a packed batch -- per-head decays, per-sequence
    initial states, a zero-length sequence -- and differentiates
    sum(O * dO) + sum(S_final * dS_final).  Both backward forms of the varlen
    wrapper must give the same gradients, the zero-length sequence passes its
    final-state gradient straight to its initial state, and packing the
    sequences in reverse order permutes the gradients accordingly."""
    import torch

    rng = _rng(41)
    H, d = 3, 3
    lens = [4, 0, 7, 1]
    decay = np.array([0.9, 1.0, 0.6])
    S = len(lens)
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, do = (rng.standard_normal((T, H, d)) for _ in range(4))
    kv0 = rng.standard_normal((S, H, d, d))
    g = rng.standard_normal((S, H, d, d))

    tq, tk, tv, tkv0 = (torch.tensor(x, dtype=torch.float64, requires_grad=True)
                        for x in (q, k, v, kv0))
    loss = 0.0
    for s in range(S):
        for h in range(H):
            St = tkv0[s, h]
            for t in range(int(cu[s]), int(cu[s + 1])):
                St = float(decay[h]) * St + torch.outer(tk[t, h], tv[t, h])
                loss = loss + (tq[t, h] @ St * torch.tensor(do[t, h])).sum()
            loss = loss + (St * torch.tensor(g[s, h])).sum()
    loss.backward()
    ref = [x.grad.numpy() for x in (tq, tk, tv, tkv0)]
    for form in ("recurrent", "quadratic"):
        got = orc.backward_varlen(q, k, v, do, cu, decay, kv_init=kv0, dkv_final=g, form=form)
        for name, a, b in zip(("dq", "dk", "dv", "dkv_init"), got, ref):
            _close(a, b, 1e-12, f"backward_varlen {form} {name}")
        _close(got[3][1], g[1], 0.0, f"backward_varlen {form} zero-length sequence")
    # reverse packing order: gradients move with their tokens and sequences
    order = list(range(S))[::-1]
    lens_r = [lens[i] for i in order]
    cu_r = np.concatenate([[0], np.cumsum(lens_r)])
    idx = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in order]).astype(int)
    got_r = orc.backward_varlen(q[idx], k[idx], v[idx], do[idx], cu_r, decay,
                                kv_init=kv0[order], dkv_final=g[order])
    for name, a, b in zip(("dq", "dk", "dv"), got_r[:3], ref[:3]):
        _close(a, b[idx], 1e-12, f"backward_varlen reversed packing {name}")
    _close(got_r[3], ref[3][order], 1e-12, "backward_varlen reversed packing dkv_init")


def pin_norm_gate(orc):
    """Output normalisation: hand-worked values (tests/golden), invariants
    of an RMS normalisation (positive scale invariance at eps = 0, odd in o,
    unit mean square with unit weights), each head its own weight and its
    own rows, and the gate as the logistic function (sigmoid(-g) =
    1 - sigmoid(g), limits 0 and 1)."""
    g = json.load(open(GOLDEN))
    for case in g["norm_gate"]:
        o = np.array(case["o"], dtype=np.float64)
        gate = None if case["gate"] is None else np.array(case["gate"], dtype=np.float64)
        y = orc.norm_gate(o, np.array(case["weight"], dtype=np.float64), case["eps"], gate)
        _close(y, case["y"], 1e-15, f"golden norm_gate {case['name']}")
    rng = _rng(43)
    T, H, d = 7, 3, 16
    o = rng.standard_normal((T, H, d)) * rng.uniform(0.1, 10.0, (T, H, 1))
    w1 = np.ones((H, d))
    y = orc.norm_gate(o, w1, 0.0)
    _close(np.mean(y * y, axis=-1), np.ones((T, H)), 1e-13, "norm_gate unit mean square")
    _close(orc.norm_gate(3.7 * o, w1, 0.0), y, 1e-13, "norm_gate scale invariance")
    _close(orc.norm_gate(-o, w1, 0.0), -y, 0.0, "norm_gate odd")
    w = rng.standard_normal((H, d))
    yw = orc.norm_gate(o, w, 1e-3)
    for h in range(H):
        row = o[:, h, :]
        ref = row / np.sqrt(np.mean(row * row, axis=-1, keepdims=True) + 1e-3) * w[h]
        _close(yw[:, h, :], ref, 1e-14, f"norm_gate head {h}")
    gt = rng.standard_normal((T, H, d)) * 3.0
    a = orc.norm_gate(o, w, 1e-3, gt) / yw
    b = orc.norm_gate(o, w, 1e-3, -gt) / yw
    _close(a + b, np.ones_like(a), 1e-12, "gate: sigmoid(g) + sigmoid(-g) = 1")
    big = np.full((T, H, d), 800.0)
    with np.errstate(over="ignore"):  # exp(800) is inf: sigmoid(-800) = 1 / inf = 0
        _close(orc.norm_gate(o, w, 1e-3, big), yw, 1e-15, "gate limit 1")
        _close(orc.norm_gate(o, w, 1e-3, -big), np.zeros_like(yw), 0.0, "gate limit 0")


ALL_PINS = [pin_golden, pin_exact_rational, pin_lfilter, pin_nodecay_library, pin_geometric,
            pin_three_way, pin_continuation, pin_decode_consistency, pin_packing, pin_decode_pool,
            pin_prefill_pool, pin_backward_autograd, pin_backward_finite_difference,
            pin_backward_varlen, pin_norm_gate]
