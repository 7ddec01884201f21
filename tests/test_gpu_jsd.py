"""GPU parity of the loss step alone (fljsd_generalized_jsd) against the oracle.

Inputs are seeded logits drawn by workloads.py; the oracle sees the same
values widened to fp64. Here the logits are exact on both sides, so the only
differences are fp32 arithmetic and, for bf16, the rounding of the gradient
on output; the bounds below are tighter than the pass-level ones.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import assert_loss_close, assert_tensor_close, from_device, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# Loss: fp32 arithmetic on exact inputs. Gradient: one bf16 rounding (2^-8
# relative) plus fp32 arithmetic.
TIGHT = {
    "f32": {"loss_rel": 1e-5, "norm": 1e-5, "elem_rel": 1e-5, "elem_max": 1e-5, "elem_abs": 0.0},
    "bf16": {"loss_rel": 1e-5, "norm": 4e-3, "elem_rel": 2 ** -8, "elem_max": 1e-5, "elem_abs": 0.0},
}


@pytest.fixture(scope="module")
def fl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lm_head_distillation_amd import fljsd
    fljsd.load_library()
    return fljsd


def _logits(seed, BT, V, scale, dtype, ld=None):
    a = workloads.make_logits(seed, BT, V, scale, dtype)
    if ld is not None and ld != V:
        pad = np.zeros((BT, ld), dtype=a.dtype)
        pad[:, :V] = a
        return a, pad
    return a, a


def _run(fl, zs_np, zt_np, V, dtype, beta, T, reduction, **kw):
    zs = to_device(zs_np, dtype)
    zt = to_device(zt_np, dtype)
    if zs_np.shape[1] != V:
        zs = zs[:, :V]
        zt = zt[:, :V]
    loss, grad = fl.fljsd_generalized_jsd(zs, zt, beta, T, reduction, **kw)
    torch.cuda.synchronize()
    return loss, grad, zs


@pytest.mark.parametrize("beta", [0.0, 0.1, 0.5, 0.9, 1.0])
@pytest.mark.parametrize("T", [1.0, 2.0])
@pytest.mark.parametrize("reduction", ["batchmean", "sum", "mean", "none"])
def test_tiny_f32_all_branches(fl, beta, T, reduction):
    zs, _ = _logits(11, 8, 512, 2.0, "f32")
    zt, _ = _logits(12, 8, 512, 2.0, "f32")
    loss, grad, _ = _run(fl, zs, zt, 512, "f32", beta, T, reduction)
    ref_loss, ref_grad = oracle.generalized_jsd(to_f64(zs, "f32"), to_f64(zt, "f32"), beta, T, reduction)
    assert_loss_close(from_device(loss), ref_loss, TIGHT["f32"])
    assert_tensor_close(from_device(grad), ref_grad, TIGHT["f32"], "grad")


@pytest.mark.parametrize("beta", [0.1, 0.5, 0.9])
@pytest.mark.parametrize("V,ld", [(40960, 40960), (40997, 41000)])
def test_multiblock_tail_bf16(fl, beta, V, ld):
    """64 rows x 40960 columns (two 32768-wide blocks of the pages' kernel, the
    second 8192 wide) and a width that leaves a ragged tail in our own slices."""
    zs, zs_pad = _logits(21, 64, V, 2.0, "bf16", ld)
    zt, zt_pad = _logits(22, 64, V, 2.0, "bf16", ld)
    loss, grad, _ = _run(fl, zs_pad, zt_pad, V, "bf16", beta, 1.0, "batchmean")
    ref_loss, ref_grad = oracle.generalized_jsd(to_f64(zs, "bf16"), to_f64(zt, "bf16"), beta, 1.0, "batchmean")
    assert_loss_close(from_device(loss), ref_loss, TIGHT["bf16"])
    assert_tensor_close(from_device(grad), ref_grad, TIGHT["bf16"], "grad")


@pytest.mark.parametrize("BT,V", [(4, 128256), (3000, 1000), (1, 7), (33, 4099)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_row_and_slice_shapes(fl, BT, V, dtype):
    """Few wide rows (many slices per row), many narrow rows (one slice each),
    and odd widths."""
    zs, _ = _logits(31, BT, V, 3.0, dtype)
    zt, _ = _logits(32, BT, V, 3.0, dtype)
    for beta in (0.0, 0.5, 1.0):
        loss, grad, _ = _run(fl, zs, zt, V, dtype, beta, 1.5, "sum")
        ref_loss, ref_grad = oracle.generalized_jsd(to_f64(zs, dtype), to_f64(zt, dtype), beta, 1.5, "sum")
        assert_loss_close(from_device(loss), ref_loss, TIGHT[dtype])
        assert_tensor_close(from_device(grad), ref_grad, TIGHT[dtype], f"grad beta={beta}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_in_place_matches_out_of_place_and_is_deterministic(fl, dtype):
    zs, _ = _logits(41, 16, 20000, 2.0, dtype)
    zt, _ = _logits(42, 16, 20000, 2.0, dtype)
    loss_a, grad_a, _ = _run(fl, zs, zt, 20000, dtype, 0.3, 1.0, "batchmean")
    loss_b, grad_b, _ = _run(fl, zs, zt, 20000, dtype, 0.3, 1.0, "batchmean")
    loss_c, grad_c, zs_dev = _run(fl, zs, zt, 20000, dtype, 0.3, 1.0, "batchmean", in_place=True)
    assert grad_c.data_ptr() == zs_dev.data_ptr()
    assert torch.equal(grad_a, grad_b) and torch.equal(loss_a, loss_b)
    assert torch.equal(grad_a, grad_c) and torch.equal(loss_a, loss_c)
    loss_d, grad_d, _ = _run(fl, zs, zt, 20000, dtype, 0.3, 1.0, "batchmean", want_grad=False)
    assert grad_d is None and torch.equal(loss_a, loss_d)


@pytest.mark.parametrize("beta", [0.0, 0.1, 0.5, 1.0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ties_give_exact_zeros(fl, beta, dtype):
    """Student == teacher: loss and every gradient element exactly zero; slots
    carrying no mass in either distribution get exactly zero gradient."""
    zs, _ = _logits(51, 32, 9000, 3.0, dtype)
    loss, grad, _ = _run(fl, zs, zs.copy(), 9000, dtype, beta, 1.0, "batchmean")
    assert from_device(loss) == 0.0
    assert torch.count_nonzero(grad).item() == 0
    zt, _ = _logits(52, 32, 9000, 3.0, dtype)
    pad_bits = workloads.f32_to_bf16_bits(np.array([workloads.PAD_LOGIT], np.float32))[0]
    pad = np.float32(workloads.PAD_LOGIT) if dtype == "f32" else pad_bits
    zs[:, -64:] = pad
    zt[:, -64:] = pad
    loss, grad, _ = _run(fl, zs, zt, 9000, dtype, beta, 1.0, "batchmean")
    g = from_device(grad)
    assert np.all(g[:, -64:] == 0.0)
    ref_loss, ref_grad = oracle.generalized_jsd(to_f64(zs, dtype), to_f64(zt, dtype), beta, 1.0, "batchmean")
    assert_loss_close(from_device(loss), ref_loss, TIGHT[dtype])
    assert_tensor_close(g, ref_grad, TIGHT[dtype], "grad")


def test_single_column(fl):
    z = np.array([[1.5], [-2.0], [0.0]], dtype=np.float32)
    loss, grad, _ = _run(fl, z, -z, 1, "f32", 0.5, 1.0, "sum")
    assert from_device(loss) == 0.0
    assert np.all(from_device(grad) == 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
def test_single_vocab_entry(fl, dtype, beta):
    """V = 1: P == Q == 1 in every row (an exact tie), so the loss and the
    gradient are exactly 0 in every branch; the oracle agrees."""
    zs, _ = _logits(31, 9, 1, 2.0, dtype)
    zt, _ = _logits(32, 9, 1, 2.0, dtype)
    ref_loss, ref_grad = oracle.generalized_jsd(to_f64(zs, dtype), to_f64(zt, dtype), beta, 2.0, "none")
    assert not np.any(ref_loss) and not np.any(ref_grad)
    loss, grad, _ = _run(fl, zs, zt, 1, dtype, beta, 2.0, "none")
    assert np.all(from_device(loss) == 0.0) and int(torch.count_nonzero(grad)) == 0


@pytest.mark.parametrize("beta", [0.0, 0.1, 0.5, 0.9, 1.0])
def test_peaked_rows_f32(fl, beta):
    """Student rows with one dominant logit (1 - Q_peak from about 1e-2 down to
    1e-7), the teacher peaked at the same column or another one, and two rows
    whose maximum is tied at two columns, over several slices with a ragged
    tail: the dominant element's gradient keeps the fp32 bar."""
    BT, V = 12, 40997
    zs, _ = _logits(61, BT, V, 1.0, "f32")
    zt, _ = _logits(62, BT, V, 1.0, "f32")
    cols = [0, 17, V // 2, V - 1]
    for r in range(BT):
        c = cols[r % 4]
        zs[r, c] = np.float32(16 + r)
        zt[r, c if r % 2 == 0 else cols[(r + 1) % 4]] = np.float32(14 + r)
    for r in (10, 11):   # the maximum tied at two columns
        zs[r, cols[(r + 2) % 4]] = zs[r, cols[r % 4]]
    loss, grad, _ = _run(fl, zs, zt, V, "f32", beta, 1.0, "sum")
    ref_loss, ref_grad = oracle.generalized_jsd(to_f64(zs, "f32"), to_f64(zt, "f32"), beta, 1.0, "sum")
    assert_loss_close(from_device(loss), ref_loss, TIGHT["f32"])
    assert_tensor_close(from_device(grad), ref_grad, TIGHT["f32"], "grad")


@pytest.mark.parametrize("ulps", [1, 4])
@pytest.mark.parametrize("beta", [0.1, 0.5, 0.9])
@pytest.mark.parametrize("T", [1.0, 2.0])
def test_near_ties_bf16(fl, ulps, beta, T):
    """Teacher = student moved by up to `ulps` bf16 ulps per logit: the row
    losses are 1e-6 to 1e-4 and every |D| is small, where an evaluation of
    ln(beta e^D + 1 - beta) that rounds its argument near 1 loses up to 2e-2
    of the row loss (fp32 emulation). Per-row loss within 2e-4 relative (the
    emulated small-argument series reach 4e-5). The gradient elements are
    differences g - Q G of terms O(Q D), whose fp32 evaluation carries an
    absolute error ~1e-7 Q: normwise at the loss-step bound, elementwise with
    1e-3 of the largest element as slack."""
    BT, V = 16, 4096
    zs, _ = _logits(71, BT, V, 2.0, "bf16")
    rng = np.random.default_rng(72)
    zt = (zs.astype(np.int32) + rng.integers(-ulps, ulps + 1, zs.shape)).astype(np.uint16)
    loss, grad, _ = _run(fl, zs, zt, V, "bf16", beta, T, "none")
    ref_loss, ref_grad = oracle.generalized_jsd(to_f64(zs, "bf16"), to_f64(zt, "bf16"), beta, T, "none")
    got = from_device(loss)
    assert np.all(ref_loss > 0)
    rel = np.max(np.abs(got - ref_loss) / ref_loss)
    print(f"row loss {ref_loss.mean():.1e}  max rel {rel:.2e}", flush=True)
    assert rel <= 2e-4
    tol = dict(TIGHT["bf16"], elem_max=1e-3)
    assert_tensor_close(from_device(grad), ref_grad, tol, "grad")


@pytest.mark.parametrize("beta", [0.001, 0.5, 0.999])
@pytest.mark.parametrize("T,scale", [(0.25, 30.0), (20.0, 0.5)])
def test_generalized_bf16_far_and_series(fl, beta, T, scale):
    """The two forms of the bf16 generalized terms at their ends.

    T = 20, logits of std 0.5: nearly every |D| is below 1/16, so nearly every
    element takes the degree-4 series, with beta near 0 and 1 stressing its
    cumulant coefficients. The row losses (~6e-7) are sums of second-order
    terms, each the difference of two first-order ones. At beta near 0 or 1
    the elements past |D| = 1/16 take log2 of an argument within ~1e-4 of 1
    on the side of the small weight, whose fp32 rounding costs that log up to
    ~1e-3 relative, and those errors reach the row loss undiminished (fp32
    emulation: 9e-4 at most): the loss bound is 5e-3. The gradient elements,
    differences g - Q G of first-order terms, take the near-tie bounds.

    T = 0.25, logits of std 30: most log2-probability differences pass 64,
    where 2^t is taken at 64 and the rest of t added back, and the two
    distributions are nearly disjoint one-hot rows. The loss then sits at the
    binary entropy h(beta) and is held to the loss-step bound. The gradient of
    such rows vanishes: its elements are ~1e-17 of their natural scale
    1 / (BT T), and g - Q G, two terms of ~1e-3 Q that cancel, leaves fp32
    noise far above that (the fp32 logit path keeps its terms relative to the
    student's most probable element; the bf16 one does not). There the bound
    is absolute, 1e-6 of the natural scale."""
    BT, V = 48, 12000
    zs, _ = _logits(61, BT, V, scale, "bf16")
    zt, _ = _logits(62, BT, V, scale, "bf16")
    for red in ("batchmean", "none"):
        loss, grad, _ = _run(fl, zs, zt, V, "bf16", beta, T, red)
        ref_loss, ref_grad = oracle.generalized_jsd(to_f64(zs, "bf16"), to_f64(zt, "bf16"), beta, T,
                                                    red)
        got = from_device(grad)
        if T < 1.0:
            assert_loss_close(from_device(loss), ref_loss, dict(TIGHT["bf16"], loss_rel=1e-4))
            natural = (1.0 / BT if red == "batchmean" else 1.0) / T
            err = np.max(np.abs(got - ref_grad)) / natural
            print(f"{red}: max |dZ - ref| = {err:.2e} of 1/(BT T)", flush=True)
            assert err <= 1e-6
        else:
            tol = dict(TIGHT["bf16"], loss_rel=5e-3, elem_max=1e-3)
            assert_loss_close(from_device(loss), ref_loss, tol)
            assert_tensor_close(got, ref_grad, tol, "grad")
