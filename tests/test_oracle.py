"""The CPU oracle against its pins, and planted mistakes against the same pins.

CPU only. A planted mistake is an edit of the oracle's source text, applied
to a private copy that is executed as a separate module; the real oracle is
never modified.
"""
from __future__ import annotations

import os
import types

import numpy as np
import pytest

import oracle
from oracle import fljsd_oracle
from tests import oracle_pins

ORACLE_SRC = os.path.join(os.path.dirname(fljsd_oracle.__file__), "fljsd_oracle.py")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(fljsd_oracle)


# (name, text to find, replacement, occurrences expected). Each is a plausible
# slip: a dropped factor, a wrong sign, a transposed or wrong operand, the
# temperature applied in the wrong place, the wrong reduction scale, a missing
# max shift, swapped mixture weights, a dropped tie rule, a per-block scale.
MUTANTS = [
    ("dropped_1_minus_beta", "term_q = np.where(Q > 0, (1.0 - beta) * Q * (logQ - logM), 0.0)",
     "term_q = np.where(Q > 0, Q * (logQ - logM), 0.0)", 1),
    ("wrong_sign_dX_sum", "dA = g - Q * G", "dA = g + Q * G", 1),
    ("missing_dX_sum", "dA = g - Q * G", "dA = g", 1),
    ("no_chain_temperature", "grad = dA * (scale / temperature)", "grad = dA * scale", 1),
    ("temperature_squared", "dZ = dA * (scale / temperature)", "dZ = dA * (scale / temperature ** 2)", 2),
    ("teacher_not_tempered", "B = np.asarray(logits_t, dtype=np.float64) / temperature",
     "B = np.asarray(logits_t, dtype=np.float64)", 1),
    ("batchmean_over_vocab", "return 1.0 / rows\n", "return 1.0 / vocab\n", 1),
    ("no_max_shift", "shifted = a - m", "shifted = a", 1),
    ("swapped_mixture_weights", "logM = np.logaddexp(np.log(beta) + logP, np.log1p(-beta) + logQ)",
     "logM = np.logaddexp(np.log(beta) + logQ, np.log1p(-beta) + logP)", 1),
    ("forward_kl_grad_sign", "        dA = Q - P\n", "        dA = P - Q\n", 1),
    ("reverse_kl_missing_row_term", "dA = np.where(Q > 0, Q * ((logQ - logP) - kl_row), 0.0)",
     "dA = np.where(Q > 0, Q * (logQ - logP), 0.0)", 1),
    ("tie_rule_dropped", "g = np.where(tie, 0.0, g)", "g = g", 1),
    ("grad_W_wrong_operand", "grad_W += dZ.T @ X_s[r0:r1]", "grad_W += dZ.T @ X_t[r0:r1, :X_s.shape[1]]", 1),
    ("grad_X_teacher_weight", "grad_X[r0:r1] = dZ @ W_s", "grad_X[r0:r1] = dZ @ W_t[:, :W_s.shape[1]]", 1),
    ("per_block_scale", "scale = reduction_scale(reduction, BT, V)\n    grad_X",
     "scale = reduction_scale(reduction, min(BT, block_rows), V)\n    grad_X", 1),
    ("forward_kl_swapped_roles", "l = np.where(P > 0, P * (logP - logQ), 0.0)",
     "l = np.where(Q > 0, Q * (logQ - logP), 0.0)", 1),
    ("logprob_forward_grad_sign", "        g = -P\n", "        g = P\n", 1),
    ("logprob_reverse_missing_q", "g = np.where(Q > 0, Q * (logq - logp), 0.0) + Q",
     "g = np.where(Q > 0, Q * (logq - logp), 0.0)", 1),
    ("logprob_dropped_1_minus_beta", "term_q = np.where(Q > 0, (1.0 - beta) * Q * (logq - logM), 0.0)",
     "term_q = np.where(Q > 0, Q * (logq - logM), 0.0)", 1),
    ("logprob_grad_unscaled", "return loss, scale * g", "return loss, g", 1),
    ("logprob_tie_rule_dropped", "g = np.where(tie, 0.0, term_q)", "g = term_q", 1),
    ("tvd_two_way_sign", "grad = scale * 0.5 * np.sign(diff)",
     "grad = scale * 0.5 * np.where(diff > 0, 1.0, -1.0)", 1),
    ("tvd_dropped_half", "elem = 0.5 * np.abs(diff)", "elem = np.abs(diff)", 1),
    ("tvd_grad_wrong_sign", "grad = scale * 0.5 * np.sign(diff)", "grad = -scale * 0.5 * np.sign(diff)", 1),
    ("tvd_grad_unscaled", "grad = scale * 0.5 * np.sign(diff)", "grad = 0.5 * np.sign(diff)", 1),
    ("ce_smoothing_divisor", "(eps / V) * np.sum(logq, axis=-1)", "eps * np.sum(logq, axis=-1)", 1),
    ("ce_onehot_weight", "dz[np.arange(R), yc] -= (1.0 - eps)", "dz[np.arange(R), yc] -= 1.0", 1),
    ("ce_mean_over_rows", 'return 1.0 / n_valid if n_valid > 0 else float("nan")', "return 1.0 / rows", 1),
    ("ce_ignored_rows_kept", "row_loss = np.where(valid, row_loss, 0.0)", "row_loss = row_loss", 1),
    ("ce_grad_unscaled", "dZ = dz * gscale", "dZ = dz", 1),
    ("ce_smoothing_grad_dropped", "dz = np.exp(logq) - eps / V", "dz = np.exp(logq)", 1),
]


def _mutant_module(name, find, replace, count):
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(find) == count, f"mutation {name}: pattern found {src.count(find)} times"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(find, replace), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m[0])
def test_planted_mistake_is_caught(mutant):
    mod = _mutant_module(*mutant)
    failed = oracle_pins.failing_pins(mod)
    assert failed, f"no pin catches the planted mistake {mutant[0]}"


def test_package_exports_oracle():
    assert oracle.generalized_jsd is fljsd_oracle.generalized_jsd
    assert set(oracle.REDUCTIONS) == {"batchmean", "sum", "mean", "none"}


def test_bad_arguments_rejected():
    z = np.zeros((2, 3))
    with pytest.raises(ValueError):
        fljsd_oracle.generalized_jsd(z, z, 1.5, 1.0)
    with pytest.raises(ValueError):
        fljsd_oracle.generalized_jsd(z, z, 0.5, 0.0)
    with pytest.raises(ValueError):
        fljsd_oracle.reduction_scale("avg", 2, 3)
