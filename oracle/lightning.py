"""fp64 reference forms of causal linear attention with per-head decay.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the method computes, per sequence and per head, for row vectors
q_t, k_t, v_t in R^d and a decay lambda in (0, 1]:

* The pages say that Lightning Attention replaces softmax normalisation by
  an element-wise product ([EMZ] 方法要点) and that it is causal linear
  attention computed with the "right product" kernel trick, split into an
  intra-block part and an inter-block part so that the cumsum of causal
  linear attention is avoided ([CSDN] §2.1, [JVY] 一、模型架构, [MZK]
  关键概念清单).  They do not print a formula.
* Reading taken: the element-wise product is a causal decay mask
  M_tj = lambda^(t-j) for t >= j and 0 otherwise, applied to Q K^T.  The
  diagonal (t = j) is included with weight lambda^0 = 1.  There is no
  softmax, no 1/sqrt(d) scale and no normaliser inside the attention core;
  the normalisation of TransNormer's NormAttention ([CSDN] §2.1) belongs
  to the surrounding layer and is not part of this core (``norm_gate`` at
  the end of this file is that normalisation as an optional epilogue, under
  the reading stated there).
* The carried state is the d x d matrix S (rows: key dimension, columns:
  value dimension), the fixed-size "state note" of linear attention
  ([MZK] 三).  An optional initial state S0 continues an earlier prefix.

Inputs are numpy arrays; every computation is done in float64.
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def decay_mask(lam, rows, cols=None):
    """Causal decay mask M[i, j] = lam**(i - j) for i >= j, else 0.

    The element-wise product that replaces softmax ([EMZ] 方法要点), read as
    an exponential decay in the distance between query and key positions.
    """
    cols = rows if cols is None else cols
    i = np.arange(rows)[:, None]
    j = np.arange(cols)[None, :]
    dist = i - j
    return np.where(dist >= 0, float(lam) ** np.maximum(dist, 0).astype(np.float64), 0.0)


def quadratic(q, k, v, lam, s0=None):
    """Explicit quadratic ("left product") form over a whole sequence.

    O = [(Q K^T) * M] V + diag(lam^(t+1)) Q S0, and the final state
    S_L = lam^L S0 + sum_j lam^(L-1-j) k_j^T v_j.

    This is the attention the tiled method must reproduce; inside one
    block the method computes exactly this masked left product ([EMZ]
    方法要点 "standard attention inside a block", [MZK] 关键概念清单
    "intra-block left product").  With S0 = 0 it is
    O = [(Q K^T) * M] V.  Uses an L x L matrix, so keep L modest.

    Returns (o [L, d_v], s_final [d_k, d_v]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    L = q.shape[0]
    dk, dv = k.shape[1], v.shape[1]
    lam = float(lam)
    o = ((q @ k.T) * decay_mask(lam, L)) @ v
    t = np.arange(L, dtype=np.float64)
    key_w = lam ** (L - 1 - t)
    s_final = (k * key_w[:, None]).T @ v
    if s0 is not None:
        s0 = _f64(s0)
        o = o + (lam ** (t + 1))[:, None] * (q @ s0)
        s_final = s_final + lam ** L * s0
    assert s_final.shape == (dk, dv)
    return o, s_final


def quadratic_loops(q, k, v, lam, s0=None):
    """Brute force of the quadratic form with plain Python loops.

    o_t[c] = sum_{j <= t} lam^(t-j) (sum_r q_t[r] k_j[r]) v_j[c]
             + lam^(t+1) sum_r q_t[r] S0[r, c].
    No array arithmetic at all; intended for L, d <= ~64.
    Returns (o, s_final) as nested lists converted to float64 arrays.
    """
    q = _f64(q).tolist()
    k = _f64(k).tolist()
    v = _f64(v).tolist()
    lam = float(lam)
    L = len(q)
    dk = len(k[0]) if L else (0 if s0 is None else len(s0))
    dv = len(v[0]) if L else (0 if s0 is None else len(s0[0]))
    s0l = None if s0 is None else _f64(s0).tolist()
    o = []
    for t in range(L):
        row = [0.0] * dv
        for j in range(t + 1):
            dot = 0.0
            for r in range(dk):
                dot += q[t][r] * k[j][r]
            w = lam ** (t - j) * dot
            for c in range(dv):
                row[c] += w * v[j][c]
        if s0l is not None:
            f = lam ** (t + 1)
            for c in range(dv):
                acc = 0.0
                for r in range(dk):
                    acc += q[t][r] * s0l[r][c]
                row[c] += f * acc
        o.append(row)
    s_final = [[0.0] * dv for _ in range(dk)]
    for j in range(L):
        w = lam ** (L - 1 - j)
        for r in range(dk):
            for c in range(dv):
                s_final[r][c] += w * k[j][r] * v[j][c]
    if s0l is not None:
        f = lam ** L
        for r in range(dk):
            for c in range(dv):
                s_final[r][c] += f * s0l[r][c]
    return np.array(o, dtype=np.float64).reshape(L, dv), np.array(s_final, dtype=np.float64)


def recurrent(q, k, v, lam, s0=None):
    """Token-by-token recurrence: the cumsum form the tiling avoids.

    S_t = lam * S_{t-1} + k_t^T v_t, then o_t = q_t S_t (the update comes
    first, so o_t sees its own token).  This is the per-token prefix sum
    of causal linear attention that [CSDN] §2.1 and [JVY] 一、模型架构 name
    as the bottleneck, and the fixed-size state of [MZK] 三.
    Returns (o [L, d_v], s_final [d_k, d_v]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    L = q.shape[0]
    dk, dv = k.shape[1], v.shape[1]
    lam = float(lam)
    S = np.zeros((dk, dv)) if s0 is None else _f64(s0).copy()
    o = np.zeros((L, dv))
    for t in range(L):
        S = lam * S + np.outer(k[t], v[t])
        o[t] = q[t] @ S
    return o, S


def blockwise(q, k, v, lam, beta, s0=None):
    """The tiled method: intra-block left product + inter-block right product.

    The sequence is cut into blocks of ``beta`` tokens (the last one may be
    shorter, length ell < beta).  With S_b the state entering block b and
    local indices i, j in [0, ell):

      intra  O_b  = [(Q_b K_b^T) * M^(ell)] V_b           (left product)
      inter  O_b += diag(lam^(i+1)) Q_b S_b               (right product)
      state  S_{b+1} = lam^ell S_b + (diag(lam^(ell-1-j)) K_b)^T V_b

    [EMZ] 方法要点 (intra "standard" attention inside a fixed-size block,
    linear attention between blocks), [CSDN] §2.1 and [JVY] 一、模型架构
    (right-product trick, intra/inter split avoids the cumsum), [MZK]
    关键概念清单 (tiling; intra-block left product, inter-block right
    product).  The pages never fix beta; the result does not depend on it.
    Returns (o [L, d_v], s_final [d_k, d_v]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    beta = int(beta)
    if beta < 1:
        raise ValueError("beta must be >= 1")
    L = q.shape[0]
    dk, dv = k.shape[1], v.shape[1]
    lam = float(lam)
    S = np.zeros((dk, dv)) if s0 is None else _f64(s0).copy()
    o = np.zeros((L, dv))
    for b0 in range(0, L, beta):
        ell = min(beta, L - b0)
        Qb = q[b0:b0 + ell]
        Kb = k[b0:b0 + ell]
        Vb = v[b0:b0 + ell]
        loc = np.arange(ell, dtype=np.float64)
        intra = ((Qb @ Kb.T) * decay_mask(lam, ell)) @ Vb
        inter = (lam ** (loc + 1))[:, None] * (Qb @ S)
        o[b0:b0 + ell] = intra + inter
        S = lam ** ell * S + (Kb * (lam ** (ell - 1 - loc))[:, None]).T @ Vb
    return o, S


def decode_step(q, k, v, s, lam):
    """One decode token: S' = lam S + k^T v, then o = q S'.

    The length-1 step that serving runs in its own kernel, apart from the
    length > 1 prefill ([JVY] 二、计算优化: separate prefill and decode,
    two kernels on two streams).  Same order as ``recurrent``.
    Returns (o [d_v], s_new [d_k, d_v]).
    """
    q, k, v, s = _f64(q), _f64(k), _f64(v), _f64(s)
    s_new = float(lam) * s + np.outer(k, v)
    return q @ s_new, s_new


_FORMS = {"blockwise", "recurrent", "quadratic"}


def prefill_varlen(q, k, v, cu_seqlens, decay, kv_init=None, form="blockwise",
                   beta=64, heads=None):
    """Packed variable-length prefill over [T, H, d] inputs.

    Sequences of different lengths are concatenated along the token axis
    (data packing, [CSDN] §3.2, [JVY] 二、计算优化); ``cu_seqlens`` holds the
    S+1 boundaries.  Each (sequence, head) pair is independent; head h uses
    decay[h] for every sequence.  A zero-length sequence produces no output
    rows and its final state equals its initial state.

    ``heads`` restricts the work to a subset of heads (outputs for other
    heads stay zero).  Returns (o [T, H, d_v], kv [S, H, d_k, d_v]).
    """
    if form not in _FORMS:
        raise ValueError(form)
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = [int(x) for x in np.asarray(cu_seqlens).tolist()]
    S = len(cu) - 1
    decay = _f64(decay)
    heads = range(H) if heads is None else heads
    o = np.zeros((T, H, dv))
    kv = np.zeros((S, H, dk, dv))
    for s in range(S):
        a, b = cu[s], cu[s + 1]
        for h in heads:
            s0 = None if kv_init is None else _f64(kv_init[s, h])
            qs, ks, vs = q[a:b, h, :], k[a:b, h, :], v[a:b, h, :]
            if form == "blockwise":
                os_, st = blockwise(qs, ks, vs, decay[h], beta, s0)
            elif form == "recurrent":
                os_, st = recurrent(qs, ks, vs, decay[h], s0)
            else:
                os_, st = quadratic(qs, ks, vs, decay[h], s0)
            o[a:b, h, :] = os_
            kv[s, h] = st
    return o, kv


def prefill_pool(q, k, v, cu_seqlens, decay, pool, slots, beta=64, heads=None):
    """Packed variable-length prefill on a pool of states: sequence s starts
    from ``pool[slots[s]]`` and its final state replaces that entry (a
    serving engine keeps every live sequence's state in one pool, prefills
    new chunks from it and decodes from it, [JVY] 二、计算优化).

    q, k, v [T, H, d]; pool [P, H, d_k, d_v]; slots [S] distinct indices
    into the pool, one per sequence of ``cu_seqlens``.  Each (sequence,
    head) runs the blockwise chain from its pooled state.  Returns
    (o [T, H, d_v], pool_new [P, H, d_k, d_v]); entries that no slot names
    are copied unchanged and the input pool is not modified.
    """
    slots = [int(x) for x in np.asarray(slots).reshape(-1).tolist()]
    cu = [int(x) for x in np.asarray(cu_seqlens).tolist()]
    if len(slots) != len(cu) - 1:
        raise ValueError("one slot per sequence")
    if len(set(slots)) != len(slots):
        raise ValueError("a slot is used twice")
    T, H, dk = q.shape
    dv = v.shape[2]
    decay = _f64(decay)
    heads = range(H) if heads is None else heads
    pool_new = _f64(pool).copy()
    o = np.zeros((T, H, dv))
    for s, sl in enumerate(slots):
        a, b = cu[s], cu[s + 1]
        for h in heads:
            o[a:b, h, :], pool_new[sl, h] = blockwise(q[a:b, h, :], k[a:b, h, :], v[a:b, h, :],
                                                      decay[h], beta, _f64(pool[sl, h]))
    return o, pool_new


def decode_batch(q, k, v, kv, decay, heads=None):
    """Decode step for a batch: q, k, v [B, H, d], kv [B, H, d, d].

    Returns (o [B, H, d_v], kv_new [B, H, d_k, d_v]); the input kv is not
    modified.  ``heads`` restricts the work to a subset of heads.
    """
    B, H, dk = q.shape
    dv = v.shape[2]
    decay = _f64(decay)
    heads = range(H) if heads is None else heads
    o = np.zeros((B, H, dv))
    kv_new = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in heads:
            o[b, h], kv_new[b, h] = decode_step(q[b, h], k[b, h], v[b, h], kv[b, h], decay[h])
    return o, kv_new


def decode_pool(q, k, v, pool, slots, decay, heads=None):
    """Decode step on a pool of states: sequence b reads and updates state
    ``pool[slots[b]]`` (the serving engine keeps every live sequence's state
    in one pool and decodes a subset of them, [JVY] 二、计算优化).

    q, k, v [B, H, d]; pool [P, H, d_k, d_v]; slots [B] distinct indices into
    the pool.  Each step is ``decode_step``.  Returns (o [B, H, d_v],
    pool_new [P, H, d_k, d_v]); entries that no slot names are copied
    unchanged and the input pool is not modified.
    """
    slots = [int(x) for x in np.asarray(slots).reshape(-1).tolist()]
    if len(set(slots)) != len(slots):
        raise ValueError("a slot is used twice")
    B, H, dk = q.shape
    dv = v.shape[2]
    decay = _f64(decay)
    heads = range(H) if heads is None else heads
    pool_new = _f64(pool).copy()
    o = np.zeros((B, H, dv))
    for b, sl in enumerate(slots):
        for h in heads:
            o[b, h], pool_new[sl, h] = decode_step(q[b, h], k[b, h], v[b, h], pool[sl, h],
                                                   decay[h])
    return o, pool_new


# ---------------------------------------------------------------------------
# Backward.  The pages give the forward only; the gradients below follow from
# its definition (the quadratic form above) by the chain rule.  With
# A[t, j] = lam^(t-j) (do_t . v_j) and B[t, j] = lam^(t-j) (q_t . k_j) for
# t >= j (else 0), and the loss seen through dO = dL/dO and dS_L = dL/dS_L:
#   dQ  = A K + diag(lam^(t+1)) dO S0^T
#   dK  = A^T Q + diag(lam^(L-1-j)) V dS_L^T
#   dV  = B^T dO + diag(lam^(L-1-j)) K dS_L
#   dS0 = Q^T diag(lam^(t+1)) dO + lam^L dS_L
# dK and dV gather over t >= j: a chain running backwards in time.
# ---------------------------------------------------------------------------

def backward_quadratic(q, k, v, do, lam, s0=None, ds_final=None):
    """Gradients of ``quadratic`` for the upstream gradients do [L, d_v] of
    the output and ds_final [d_k, d_v] of the final state (None = 0).

    Returns (dq [L, d_k], dk [L, d_k], dv [L, d_v], ds0 [d_k, d_v]); ds0 is
    the gradient with respect to the initial state (defined when s0 is None,
    i.e. a zero initial state).  Uses L x L matrices, so keep L modest.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    L = q.shape[0]
    lam = float(lam)
    m = decay_mask(lam, L)
    a = (do @ v.T) * m
    b = (q @ k.T) * m
    t = np.arange(L, dtype=np.float64)
    dq = a @ k
    dk = a.T @ q
    dv = b.T @ do
    ds0 = (q * (lam ** (t + 1))[:, None]).T @ do
    if s0 is not None:
        dq = dq + (lam ** (t + 1))[:, None] * (do @ _f64(s0).T)
    if ds_final is not None:
        g = _f64(ds_final)
        w = lam ** (L - 1 - t)
        dk = dk + w[:, None] * (v @ g.T)
        dv = dv + w[:, None] * (k @ g)
        ds0 = ds0 + lam ** L * g
    return dq, dk, dv, ds0


def backward_recurrent(q, k, v, do, lam, s0=None, ds_final=None):
    """The same gradients as two token chains.

    Forward in time, the forward state S_t (as in ``recurrent``) gives
    dq_t = S_t do_t.  Backward in time, R_j = lam R_(j+1) + q_j^T do_j with
    R_(L-1) = q_(L-1)^T do_(L-1) + dS_L gives dk_j = R_j v_j and
    dv_j = R_j^T k_j, and dS0 = lam R_0 (dS_L when L = 0).
    Returns (dq, dk, dv, ds0) as ``backward_quadratic``.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    L = q.shape[0]
    dk_, dv_ = k.shape[1], v.shape[1]
    lam = float(lam)
    S = np.zeros((dk_, dv_)) if s0 is None else _f64(s0).copy()
    dq = np.zeros((L, dk_))
    for t in range(L):
        S = lam * S + np.outer(k[t], v[t])
        dq[t] = S @ do[t]
    R = np.zeros((dk_, dv_)) if ds_final is None else _f64(ds_final).copy()
    dk = np.zeros((L, dk_))
    dv = np.zeros((L, dv_))
    for j in range(L - 1, -1, -1):
        if j < L - 1:
            R = lam * R
        R = R + np.outer(q[j], do[j])
        dk[j] = R @ v[j]
        dv[j] = R.T @ k[j]
    ds0 = lam * R if L > 0 else R
    return dq, dk, dv, ds0


def backward_varlen(q, k, v, do, cu_seqlens, decay, kv_init=None, dkv_final=None,
                    form="recurrent", heads=None):
    """Gradients of ``prefill_varlen`` over packed sequences.

    q, k, v, do [T, H, d]; kv_init, dkv_final [S, H, d, d] or None.  Returns
    (dq, dk, dv [T, H, d], dkv_init [S, H, d, d]).  ``heads`` restricts the
    work to a subset of heads (other heads stay zero).
    """
    fn = {"recurrent": backward_recurrent, "quadratic": backward_quadratic}[form]
    T, H, dk_ = q.shape
    dv_ = v.shape[2]
    cu = [int(x) for x in np.asarray(cu_seqlens).tolist()]
    S = len(cu) - 1
    decay = _f64(decay)
    heads = range(H) if heads is None else heads
    dq = np.zeros((T, H, dk_))
    dk = np.zeros((T, H, dk_))
    dv = np.zeros((T, H, dv_))
    dkv0 = np.zeros((S, H, dk_, dv_))
    for s in range(S):
        a, b = cu[s], cu[s + 1]
        for h in heads:
            s0 = None if kv_init is None else _f64(kv_init[s, h])
            g = None if dkv_final is None else _f64(dkv_final[s, h])
            r = fn(q[a:b, h], k[a:b, h], v[a:b, h], do[a:b, h], decay[h], s0, g)
            dq[a:b, h], dk[a:b, h], dv[a:b, h], dkv0[s, h] = r
    return dq, dk, dv, dkv0


# ---------------------------------------------------------------------------
# Output normalisation and gate (the memory-bound epilogue next to the core).
# The pages say the model takes TransNormer's NormAttention ([CSDN] §2.1),
# i.e. a normalisation of the linear-attention output in place of softmax's
# scaling, and that memory-bound kernels around lightning attention are fused
# so that intermediate results are not stored ([JVY] 二、计算优化, [CSDN]
# §3.2).  They do not define the normalisation.  Reading taken: an RMS
# normalisation of each head's output row over its d features with a
# per-(head, feature) weight, y = w_h * o / sqrt(mean(o^2) + eps), optionally
# multiplied element-wise by sigmoid(g) for a caller-supplied gate g of the
# same shape (the gate is not on the pages; it is an option).
# ---------------------------------------------------------------------------

def norm_gate(o, weight, eps, gate=None):
    """Per-head RMS normalisation of o [..., H, d] over its last axis, scaled
    by weight [H, d], then, if gate [..., H, d] is given, multiplied by
    sigmoid(gate).  Returns float64 of o's shape."""
    o = _f64(o)
    w = _f64(weight)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    y = o / np.sqrt(ms + float(eps)) * w
    if gate is not None:
        y = y * (1.0 / (1.0 + np.exp(-_f64(gate))))
    return y
