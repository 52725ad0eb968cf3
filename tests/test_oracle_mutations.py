"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each case copies the oracle's source, plants one plausible mistake (a
dropped term, an off-by-one decay exponent, a transposed operand, a wrong
index, a swapped update order), loads the copy as a fresh module and runs
the pin battery of ``tests/oracle_pins.py`` on it.  At least one pin must
fail; the real oracle passes them all (``test_oracle_pins.py``).
"""

import os
import types

import pytest

from tests import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "lightning.py")

MUTATIONS = {
    "mask_drops_diagonal": ("np.where(dist >= 0,", "np.where(dist > 0,"),
    "mask_wrong_sign": ("np.maximum(dist, 0)", "np.maximum(-dist, 0)"),
    "quadratic_transposed_scores": ("o = ((q @ k.T) * decay_mask", "o = ((k @ q.T) * decay_mask"),
    "quadratic_inter_exponent": ("o = o + (lam ** (t + 1))[:, None]", "o = o + (lam ** t)[:, None]"),
    "quadratic_state_key_weight": ("key_w = lam ** (L - 1 - t)", "key_w = lam ** (L - t)"),
    "loops_off_by_one": ("w = lam ** (t - j) * dot", "w = lam ** (t - j + 1) * dot"),
    "recurrent_read_before_update": (
        "S = lam * S + np.outer(k[t], v[t])\n        o[t] = q[t] @ S",
        "o[t] = q[t] @ S\n        S = lam * S + np.outer(k[t], v[t])"),
    "recurrent_transposed_outer": ("S = lam * S + np.outer(k[t], v[t])\n        o[t] = q[t] @ S",
                                   "S = lam * S + np.outer(v[t], k[t])\n        o[t] = q[t] @ S"),
    "blockwise_inter_exponent": ("inter = (lam ** (loc + 1))", "inter = (lam ** loc)"),
    "blockwise_drops_inter": ("o[b0:b0 + ell] = intra + inter", "o[b0:b0 + ell] = intra"),
    "blockwise_state_decay": ("S = lam ** ell * S +", "S = lam ** (ell - 1) * S +"),
    "blockwise_key_decay": ("(lam ** (ell - 1 - loc))", "(lam ** (ell - loc))"),
    "blockwise_transposed_update": ("(Kb * (lam ** (ell - 1 - loc))[:, None]).T @ Vb",
                                    "((Vb * (lam ** (ell - 1 - loc))[:, None]).T @ Kb)"),
    "blockwise_stale_state": ("inter = (lam ** (loc + 1))[:, None] * (Qb @ S)",
                              "inter = (lam ** (loc + 1))[:, None] * (Qb @ (S * 0))"),
    "decode_no_decay": ("s_new = float(lam) * s + np.outer(k, v)", "s_new = s + np.outer(k, v)"),
    "decode_reads_old_state": ("return q @ s_new, s_new", "return q @ s, s_new"),
    "varlen_wrong_head_decay": ("os_, st = blockwise(qs, ks, vs, decay[h], beta, s0)",
                                "os_, st = blockwise(qs, ks, vs, decay[0], beta, s0)"),
    "varlen_swapped_kv": ("qs, ks, vs = q[a:b, h, :], k[a:b, h, :], v[a:b, h, :]",
                          "qs, ks, vs = q[a:b, h, :], v[a:b, h, :], k[a:b, h, :]"),
    "varlen_ignores_init": ("s0 = None if kv_init is None else _f64(kv_init[s, h])\n            qs, ks",
                            "s0 = None\n            qs, ks"),
    "pool_writes_batch_index": ("o[b, h], pool_new[sl, h] = decode_step(", "o[b, h], pool_new[b, h] = decode_step("),
    "pool_reads_batch_index": ("v[b, h], pool[sl, h],", "v[b, h], pool[b, h],"),
    "prefill_pool_writes_seq_index": ("o[a:b, h, :], pool_new[sl, h] = blockwise(",
                                      "o[a:b, h, :], pool_new[s, h] = blockwise("),
    "prefill_pool_reads_seq_index": ("decay[h], beta, _f64(pool[sl, h]))",
                                     "decay[h], beta, _f64(pool[s, h]))"),
    "bwd_quad_dk_untransposed": ("    dk = a.T @ q\n", "    dk = a @ q\n"),
    "bwd_quad_dv_wrong_scores": ("    dv = b.T @ do\n", "    dv = a.T @ do\n"),
    "bwd_quad_ds0_exponent": ("    ds0 = (q * (lam ** (t + 1))[:, None]).T @ do",
                              "    ds0 = (q * (lam ** t)[:, None]).T @ do"),
    "bwd_quad_drops_final_grad_dk": ("        dk = dk + w[:, None] * (v @ g.T)\n", ""),
    "bwd_quad_s0_untransposed": ("(do @ _f64(s0).T)", "(do @ _f64(s0))"),
    "bwd_rec_reads_before_update": ("        S = lam * S + np.outer(k[t], v[t])\n        dq[t] = S @ do[t]",
                                    "        dq[t] = S @ do[t]\n        S = lam * S + np.outer(k[t], v[t])"),
    "bwd_rec_no_reverse_decay": ("        if j < L - 1:\n            R = lam * R\n", ""),
    "bwd_rec_dv_untransposed": ("        dv[j] = R.T @ k[j]", "        dv[j] = R @ k[j]"),
    "bwd_varlen_first_head_decay": ("r = fn(q[a:b, h], k[a:b, h], v[a:b, h], do[a:b, h], decay[h], s0, g)",
                                    "r = fn(q[a:b, h], k[a:b, h], v[a:b, h], do[a:b, h], decay[0], s0, g)"),
    "bwd_varlen_swapped_state_args": ("r = fn(q[a:b, h], k[a:b, h], v[a:b, h], do[a:b, h], decay[h], s0, g)",
                                      "r = fn(q[a:b, h], k[a:b, h], v[a:b, h], do[a:b, h], decay[h], g, s0)"),
    "bwd_varlen_swapped_dk_dv": ("dq[a:b, h], dk[a:b, h], dv[a:b, h], dkv0[s, h] = r",
                                 "dq[a:b, h], dv[a:b, h], dk[a:b, h], dkv0[s, h] = r"),
    "norm_sum_not_mean": ("ms = np.mean(o * o, axis=-1, keepdims=True)",
                          "ms = np.sum(o * o, axis=-1, keepdims=True)"),
    "norm_drops_eps": ("y = o / np.sqrt(ms + float(eps)) * w", "y = o / np.sqrt(ms) * w"),
    "norm_first_head_weight": ("y = o / np.sqrt(ms + float(eps)) * w", "y = o / np.sqrt(ms + float(eps)) * w[0]"),
    "norm_over_heads": ("ms = np.mean(o * o, axis=-1, keepdims=True)",
                        "ms = np.mean(o * o, axis=-2, keepdims=True)"),
    "gate_wrong_sign": ("y = y * (1.0 / (1.0 + np.exp(-_f64(gate))))",
                        "y = y * (1.0 / (1.0 + np.exp(_f64(gate))))"),
    "gate_ignored": ("        y = y * (1.0 / (1.0 + np.exp(-_f64(gate))))\n", "        pass\n"),
}


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/absent: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(*MUTATIONS[name])
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError) as e:  # shape errors count as caught
            failures.append((pin.__name__, str(e)[:80]))
    assert failures, f"no pin caught mutation {name}"
