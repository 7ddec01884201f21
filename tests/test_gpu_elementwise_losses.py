"""GPU parity of the one-pass losses over given distributions against the
oracle: the log-probability JSD (fljsd_jsd_logprob) and the TVD with the
p == q gradient fix (fljsd_tvd), plus the T^2 flag of the fused pass.

Inputs are seeded: log-probabilities are the oracle-independent log-softmax
(scipy) of workloads' logits, rounded to the dtype; probabilities likewise.
The same rounded bits go to the GPU and, widened to fp64, to the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import scipy.special as sps

import oracle
import workloads
from tests.gpu_util import TOL, assert_loss_close, assert_tensor_close, from_device, to_device, \
    to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BETAS = (0.0, 0.1, 0.5, 0.9, 1.0)


@pytest.fixture(scope="module")
def fl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lm_head_distillation_amd import fljsd
    fljsd.load_library()
    return fljsd


def _round(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> the dtype's storage (fp32 values, or bf16 bits, nearest even)."""
    f = np.asarray(a, dtype=np.float32)
    return f if dtype == "f32" else workloads.f32_to_bf16_bits(f)


def _logprobs(seed, R, V, dtype, scale=2.0):
    z = workloads.draw(seed, (R, V), scale, "f32").astype(np.float64)
    return _round(sps.log_softmax(z, axis=-1), dtype)


def _probs(seed, R, V, dtype, scale=2.0):
    z = workloads.draw(seed, (R, V), scale, "f32").astype(np.float64)
    return _round(sps.softmax(z, axis=-1), dtype)


# ---- log-probability JSD ---------------------------------------------------------------

@pytest.mark.parametrize("beta", BETAS)
@pytest.mark.parametrize("reduction", ["batchmean", "sum", "mean", "none"])
def test_logprob_tiny_f32(fl, beta, reduction):
    x = _logprobs(501, 8, 512, "f32")
    y = _logprobs(502, 8, 512, "f32")
    loss, grad = fl.fljsd_jsd_logprob(to_device(x, "f32"), to_device(y, "f32"), beta, reduction)
    torch.cuda.synchronize()
    rl, rg = oracle.jsd_logprob(to_f64(x, "f32"), to_f64(y, "f32"), beta, reduction)
    assert_loss_close(from_device(loss), rl, TOL["f32"])
    assert_tensor_close(from_device(grad), rg, TOL["f32"], "grad_logq")


@pytest.mark.parametrize("beta", [0.001, 0.01, 0.99, 0.999])
@pytest.mark.parametrize("scale", [0.25, 2.0, 8.0])
def test_logprob_extreme_beta_f32(fl, beta, scale):
    """fp32 at mixture weights near 0 and 1, over near-flat (logit std 0.25)
    to sharp (std 8) rows: r = ln(beta e^D + 1 - beta) is then much smaller
    than D, or close to D + ln(beta), where forms that add D to a logarithm
    lose digits. The oracle takes beta as the fp32 value the library gets."""
    x = _logprobs(511, 8, 512, "f32", scale)
    y = _logprobs(512, 8, 512, "f32", scale)
    loss, grad = fl.fljsd_jsd_logprob(to_device(x, "f32"), to_device(y, "f32"), beta, "none")
    torch.cuda.synchronize()
    rl, rg = oracle.jsd_logprob(to_f64(x, "f32"), to_f64(y, "f32"), float(np.float32(beta)), "none")
    assert_loss_close(from_device(loss), rl, TOL["f32"])
    assert_tensor_close(from_device(grad), rg, TOL["f32"], "grad_logq")


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
@pytest.mark.parametrize("R,V", [(64, 40960 + 37), (3, 100), (300, 1000)])
def test_logprob_bf16_shapes(fl, beta, R, V):
    """Several slices per row, ragged tails, rows not a multiple of anything."""
    x = _logprobs(503, R, V, "bf16")
    y = _logprobs(504, R, V, "bf16")
    loss, grad = fl.fljsd_jsd_logprob(to_device(x, "bf16"), to_device(y, "bf16"), beta)
    torch.cuda.synchronize()
    rl, rg = oracle.jsd_logprob(to_f64(x, "bf16"), to_f64(y, "bf16"), beta)
    e0 = assert_loss_close(from_device(loss), rl, TOL["bf16"])
    e1 = assert_tensor_close(from_device(grad), rg, TOL["bf16"], "grad_logq")
    print(f"R={R} V={V} beta={beta}: loss rel {e0:.2e}, grad normwise {e1:.2e}", flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_logprob_ties_and_zero_probabilities(fl, dtype):
    """Equal inputs give loss 0 and (generalized) gradient exactly 0; columns
    that are -inf in both carry nothing; the in-place gradient matches."""
    R, V = 16, 3000
    x = to_f64(_logprobs(505, R, V, dtype), dtype)
    y = to_f64(_logprobs(506, R, V, dtype), dtype)
    y[:4] = x[:4]                         # fully tied rows
    x[:, -50:] = -np.inf                  # zero-probability tail in both
    y[:, -50:] = -np.inf
    xs, ys = _round(x, dtype), _round(y, dtype)
    for beta in BETAS:
        dx = to_device(xs, dtype)
        loss, grad = fl.fljsd_jsd_logprob(dx, to_device(ys, dtype), beta, "none")
        torch.cuda.synchronize()
        rl, rg = oracle.jsd_logprob(to_f64(xs, dtype), to_f64(ys, dtype), beta, "none")
        got_l = from_device(loss)
        got_g = from_device(grad)
        assert np.all(got_l[:4] == 0.0), f"tied rows loss beta={beta}"
        assert np.all(got_g[:, -50:] == 0.0), f"zero-probability columns beta={beta}"
        if 0.0 < beta < 1.0:
            assert np.all(got_g[:4] == 0.0), f"tied rows grad beta={beta}"
        assert_loss_close(got_l[4:], rl[4:], TOL[dtype])
        assert_tensor_close(got_g, rg, TOL[dtype], f"grad beta={beta}")
        # in place over the student log-probabilities
        loss2, g2 = fl.fljsd_jsd_logprob(dx, to_device(ys, dtype), beta, "none", in_place=True)
        torch.cuda.synchronize()
        assert g2.data_ptr() == dx.data_ptr()
        assert np.array_equal(from_device(g2), got_g) and np.array_equal(from_device(loss2), got_l)


# ---- TVD -------------------------------------------------------------------------------

def test_tvd_tie_table(fl):
    """The pages' (8, 512) fp32 batchmean case: p == q everywhere gives a zero
    gradient at all 4096 elements (the fix); untied elements get +-0.0625."""
    p = _probs(507, 8, 512, "f32")
    dp = to_device(p, "f32")
    loss, grad = fl.fljsd_tvd(dp, dp.clone(), "batchmean")
    torch.cuda.synchronize()
    assert float(loss) == 0.0
    assert int(torch.count_nonzero(grad)) == 0
    q = to_f64(p, "f32").copy()
    q[:, ::2] *= 1.5
    q /= q.sum(axis=-1, keepdims=True)
    qs = _round(q, "f32")
    _, grad = fl.fljsd_tvd(dp, to_device(qs, "f32"), "batchmean")
    torch.cuda.synchronize()
    g = from_device(grad)
    pf, qf = to_f64(p, "f32"), to_f64(qs, "f32")
    assert np.all(g[pf < qf] == -0.0625) and np.all(g[pf > qf] == 0.0625)
    assert np.all(g[pf == qf] == 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["batchmean", "sum", "mean", "none"])
def test_tvd_reductions(fl, dtype, reduction):
    R, V = 37, 5003
    p = _probs(508, R, V, dtype)
    q = _probs(509, R, V, dtype)
    q[:5] = p[:5]                          # tied rows (self-distillation)
    loss, grad = fl.fljsd_tvd(to_device(p, dtype), to_device(q, dtype), reduction)
    torch.cuda.synchronize()
    rl, rg = oracle.tvd(to_f64(p, dtype), to_f64(q, dtype), reduction)
    if reduction == "none":
        assert tuple(loss.shape) == (R, V)
        assert_tensor_close(from_device(loss), rl, TOL["f32"], "elementwise tvd")
    else:
        assert_loss_close(from_device(loss), rl, TOL[dtype])
    g = from_device(grad)
    assert np.all(g[:5] == 0.0)
    assert_tensor_close(g, rg, TOL[dtype], "grad_p")


def test_tvd_large_bf16(fl):
    """The pages' forward-benchmark shape family, (4096, 32000) bf16, loss only
    checked on all rows; gradient signs exact."""
    R, V = 1024, 32000
    p = _probs(510, R, V, "bf16")
    q = _probs(511, R, V, "bf16")
    loss, grad = fl.fljsd_tvd(to_device(p, "bf16"), to_device(q, "bf16"), "batchmean")
    torch.cuda.synchronize()
    pf, qf = to_f64(p, "bf16"), to_f64(q, "bf16")
    rl, _ = oracle.tvd(pf, qf, "batchmean")
    assert_loss_close(from_device(loss), rl, TOL["bf16"])
    g = from_device(grad)
    half = 0.5 / R
    assert np.all(np.sign(g) == np.sign(pf - qf))
    assert np.allclose(np.abs(g[pf != qf]), half, rtol=4e-3)


# ---- the T^2 flag of the fused pass ------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_temperature_squared_flag(fl, dtype):
    w = workloads.Workload("t2", 47, 48, 64, 64, 1000, dtype, 0.5, 2.0, "batchmean", "independent")
    inp = workloads.make_inputs(w)
    dev = tuple(to_device(inp[k], dtype) for k in ("X_s", "W_s", "X_t", "W_t"))
    T = 2.0
    for red in ("batchmean", "none"):
        loss, gX, gW = fl.fljsd_forward_backward_ex(*dev, 0.3, T, red, 2,
                                                    flags=fl.FLJSD_TEMPERATURE_SQUARED)
        torch.cuda.synchronize()
        rl, rX, rW = oracle.fused_linear_jsd(*(to_f64(inp[k], dtype) for k in ("X_s", "W_s", "X_t", "W_t")),
                                             0.3, T, red)
        assert_loss_close(from_device(loss), np.asarray(rl) * T * T, TOL[dtype])
        assert_tensor_close(from_device(gX), rX * T * T, TOL[dtype], "grad_input T^2")
        assert_tensor_close(from_device(gW), rW * T * T, TOL[dtype], "grad_weight T^2")
