"""GPU parity of the fused-linear cross-entropy (fljsd_flce_forward_backward)
against the oracle: hard labels with ignored and out-of-range rows, label
smoothing, every reduction, chunk counts, ragged shapes, and the degenerate
all-ignored batch."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL, assert_loss_close, assert_tensor_close, from_device, normwise, \
    to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lm_head_distillation_amd import fljsd
    fljsd.load_library()
    return fljsd


def _case(seed, BT, H, V, dtype, ignore=-100):
    w = workloads.Workload("flce", seed, BT, H, H, V, dtype, 0.5, 1.0, "mean", "independent")
    inp = workloads.make_inputs(w)
    rng = np.random.default_rng(seed)
    labels = rng.integers(0, V, size=BT).astype(np.int64)
    if BT >= 4:
        labels[1] = ignore
        labels[BT // 2] = ignore
        labels[-1] = V + 5            # out of range: does not count
    return inp["X_s"], inp["W_s"], labels


def _run(fl, X, W, labels, dtype, ignore, eps, red, nc, **kw):
    out = fl.fljsd_flce_forward_backward(to_device(X, dtype), to_device(W, dtype),
                                         torch.from_numpy(labels).cuda(), ignore, eps, red, nc, **kw)
    torch.cuda.synchronize()
    return out


def _check(dtype, got, ref, what=""):
    loss, gX, gW = got
    rl, rX, rW = ref
    tol = TOL[dtype]
    e0 = assert_loss_close(from_device(loss), rl, tol, f"loss {what}")
    e1 = assert_tensor_close(from_device(gX), rX, tol, f"grad_X {what}")
    e2 = assert_tensor_close(from_device(gW), rW, tol, f"grad_W {what}")
    print(f"{what}: loss {e0:.2e} grad_X {e1:.2e} grad_W {e2:.2e}", flush=True)


@pytest.mark.parametrize("eps", [0.0, 0.1])
@pytest.mark.parametrize("reduction", ["mean", "sum", "none", "batchmean"])
@pytest.mark.parametrize("nc", [1, 3])
def test_tiny_f32(fl, eps, reduction, nc):
    X, W, y = _case(601, 8, 64, 512, "f32")
    got = _run(fl, X, W, y, "f32", -100, eps, reduction, nc)
    ref = oracle.fused_linear_cross_entropy(to_f64(X, "f32"), to_f64(W, "f32"), y, -100, eps,
                                            reduction)
    _check("f32", got, ref, f"{reduction} eps={eps} nc={nc}")


@pytest.mark.parametrize("eps", [0.0, 0.1])
@pytest.mark.parametrize("nc", [1, 4])
def test_multiblock_bf16(fl, eps, nc):
    X, W, y = _case(602, 64, 256, 40960 + 37, "bf16", ignore=7)
    got = _run(fl, X, W, y, "bf16", 7, eps, "mean", nc)
    ref = oracle.fused_linear_cross_entropy(to_f64(X, "bf16"), to_f64(W, "bf16"), y, 7, eps, "mean")
    _check("bf16", got, ref, f"eps={eps} nc={nc}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("BT,H,V,nc", [
    (1, 64, 100, 1), (300, 72, 1000, 7), (513, 264, 5003, 2), (10, 64, 777, 100),
    (256, 1024, 32064, 1),
])
def test_shapes(fl, dtype, BT, H, V, nc):
    X, W, y = _case(603, BT, H, V, dtype)
    got = _run(fl, X, W, y, dtype, -100, 0.05, "mean", nc)
    ref = oracle.fused_linear_cross_entropy(to_f64(X, dtype), to_f64(W, dtype), y, -100, 0.05, "mean")
    _check(dtype, got, ref, f"{BT}x{H}x{V} nc={nc}")


# bf16 shapes with more than 4096 rows, V a multiple of 256 and H of 64, chunks
# of at least 512 rows: the first chunk's logits product also writes W^T and
# grad_X reads both operands along V.
@pytest.mark.parametrize("BT,H,V,nc", [(4160, 64, 768, 1), (4608, 128, 2560, 9), (4601, 192, 1024, 4)])
def test_w_transposed_shapes(fl, BT, H, V, nc):
    X, W, y = _case(612, BT, H, V, "bf16")
    got = _run(fl, X, W, y, "bf16", -100, 0.05, "mean", nc)
    ref = oracle.fused_linear_cross_entropy(to_f64(X, "bf16"), to_f64(W, "bf16"), y, -100, 0.05, "mean")
    _check("bf16", got, ref, f"{BT}x{H}x{V} nc={nc}")


def test_w_transposed_region_is_optional(fl):
    """A workspace short of exactly the W^T region runs grad_X on W as given:
    the same LDS contents and MFMA sequence, so the same bits."""
    BT, H, V, nc = 4160, 128, 2560, 2
    X, W, y = _case(613, BT, H, V, "bf16")
    full = fl.fljsd_flce_workspace_size(BT, H, V, fl.BF16, nc)
    wt = (V * H * 2 + 255) // 256 * 256
    ws_full = torch.empty(full, dtype=torch.uint8, device="cuda")
    ws_short = torch.empty(full - wt, dtype=torch.uint8, device="cuda")
    a = _run(fl, X, W, y, "bf16", -100, 0.05, "mean", nc, workspace=ws_full)
    b = _run(fl, X, W, y, "bf16", -100, 0.05, "mean", nc, workspace=ws_short)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_all_rows_ignored(fl):
    X, W, _ = _case(604, 16, 64, 300, "bf16")
    y = np.full(16, -100, dtype=np.int64)
    loss, gX, gW = _run(fl, X, W, y, "bf16", -100, 0.0, "mean", 2)
    assert np.isnan(float(loss))
    assert int(torch.count_nonzero(gX)) == 0 and int(torch.count_nonzero(gW)) == 0
    loss, gX, gW = _run(fl, X, W, y, "bf16", -100, 0.0, "sum", 2)
    assert float(loss) == 0.0 and int(torch.count_nonzero(gX)) == 0


def test_optional_gradients(fl):
    X, W, y = _case(605, 40, 128, 2000, "bf16")
    full = _run(fl, X, W, y, "bf16", -100, 0.0, "mean", 2)
    only_loss = _run(fl, X, W, y, "bf16", -100, 0.0, "mean", 2, grad_input=False, grad_weight=False)
    assert only_loss[1] is None and only_loss[2] is None
    assert float(only_loss[0]) == float(full[0])
    only_w = _run(fl, X, W, y, "bf16", -100, 0.0, "mean", 2, grad_input=False)
    assert torch.equal(only_w[2].view(torch.int16), full[2].view(torch.int16))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_vocab_entry(fl, dtype):
    """V = 1: the softmax is 1 at the only label, so every counted row's
    gradient is exactly 0 and its loss is 0 up to the rounding of
    (1 - eps) z + eps z against z."""
    X, W, _ = _case(606, 21, 64, 1, dtype)
    y = np.zeros(21, dtype=np.int64)
    y[3] = -100
    for eps in (0.0, 0.1):
        loss, gX, gW = _run(fl, X, W, y, dtype, -100, eps, "none", 2)
        rl, _, _ = oracle.fused_linear_cross_entropy(to_f64(X, dtype), to_f64(W, dtype), y, -100, eps,
                                                     "none")
        assert not np.any(rl)
        assert np.all(np.abs(from_device(loss)) <= 1e-6), f"eps={eps}"
        assert int(torch.count_nonzero(gX)) == 0 and int(torch.count_nonzero(gW)) == 0, f"eps={eps}"


@pytest.mark.slow
def test_beyond_2g_logit_elements(fl):
    """17000 x 256 x 128256 bf16, one chunk: the logits and dZ^T hold 2.18e9
    elements, past 2^31. Sampled rows on both sides of element 2^31 against
    the oracle's per-row cross-entropy; all rows through
    <grad_W, W> = <dZ, Z> = <grad_X, X>."""
    BT, H, V = 17000, 256, 128256
    X, W, y = _case(607, BT, H, V, "bf16")
    rows = np.array([0, 1, 8500, 16743, 16744, 16745, BT - 1])
    Xr = to_f64(X, "bf16")[rows]
    Wf = to_f64(W, "bf16")
    ref_loss, ref_dz, valid = oracle.cross_entropy_rows(Xr @ Wf.T, y[rows], -100, 0.1)
    loss, gX, gW = _run(fl, X, W, y, "bf16", -100, 0.1, "none", 1)
    assert_loss_close(from_device(loss)[rows], ref_loss, TOL["bf16"], "per-row loss")
    got_rows = from_device(gX[torch.as_tensor(rows, device=gX.device)])
    assert_tensor_close(got_rows, ref_dz @ Wf, TOL["bf16"], "grad_X rows")
    Xd, Wd = to_device(X, "bf16"), to_device(W, "bf16")
    lhs = float((gW.double() * Wd.double()).sum())
    rhs = float((gX.double() * Xd.double()).sum())
    assert abs(lhs - rhs) <= 2e-2 * max(abs(lhs), abs(rhs)), f"{lhs} vs {rhs}"


# ---- fp32 weight gradient (Liger-Kernel PR #1429, Details) and adding to an existing one --

def _ex(fl, X, W, y, nc, **kw):
    out = fl.fljsd_flce_forward_backward_ex(to_device(X, "bf16"), to_device(W, "bf16"),
                                            torch.from_numpy(y).cuda(), -100, 0.05, "mean", nc, **kw)
    torch.cuda.synchronize()
    return out


@pytest.fixture(scope="module")
def flce_bf16_case():
    # Several 256-wide vocabulary tiles with a ragged last one, a ragged
    # hidden tile, and chunks down to 4 rows.
    X, W, y = _case(611, 64, 264, 5003, "bf16")
    ref = oracle.fused_linear_cross_entropy(to_f64(X, "bf16"), to_f64(W, "bf16"), y, -100, 0.05, "mean")
    return X, W, y, ref


@pytest.mark.parametrize("nc", [1, 4, 16])
def test_flce_fp32_grad_w_matches_oracle(fl, flce_bf16_case, nc):
    X, W, y, ref = flce_bf16_case
    loss, gX, gW = _ex(fl, X, W, y, nc, grad_w_dtype=torch.float32)
    assert gW.dtype == torch.float32 and gX.dtype == torch.bfloat16
    _check("bf16", (loss, gX, gW), ref, f"fp32 grad_W nc={nc}")


def test_flce_fp32_grad_w_does_not_depend_on_chunks(fl, flce_bf16_case):
    """dZ rows do not depend on the chunking, so the fp32 sums over 1, 4 and 16
    chunks differ only by fp32 rounding; the bf16 result carries one bf16
    rounding per chunk."""
    X, W, y, _ = flce_bf16_case
    f32 = {nc: from_device(_ex(fl, X, W, y, nc, grad_w_dtype=torch.float32)[2]) for nc in (1, 4, 16)}
    b16 = {nc: from_device(_ex(fl, X, W, y, nc)[2]) for nc in (1, 16)}
    for nc in (4, 16):
        e = normwise(f32[nc], f32[1])
        assert e <= 1e-5, f"fp32 grad_W nc={nc} vs nc=1: {e:.3e}"
    print(f"fp32 nc=16 vs 1: {normwise(f32[16], f32[1]):.2e}; "
          f"bf16 nc=16 vs 1: {normwise(b16[16], b16[1]):.2e}", flush=True)


def test_flce_fp32_one_chunk_rounds_to_the_bf16_mode(fl, flce_bf16_case):
    """With one chunk the fp32 grad_W is the unrounded product; rounding it to
    bf16 gives the bf16 mode's bits."""
    X, W, y, _ = flce_bf16_case
    f32 = _ex(fl, X, W, y, 1, grad_w_dtype=torch.float32)[2]
    b16 = _ex(fl, X, W, y, 1)[2]
    assert torch.equal(f32.to(torch.bfloat16).view(torch.int16), b16.view(torch.int16))


@pytest.mark.parametrize("gw_dtype", [torch.bfloat16, torch.float32])
def test_flce_accumulate_into_existing_grad_w(fl, flce_bf16_case, gw_dtype):
    """FLJSD_ACCUMULATE_GRAD_W: the call adds its gradient to the grad_W it is
    given (micro-batch sums), in every chunk, the first included."""
    X, W, y, ref = flce_bf16_case
    rng = np.random.default_rng(612)
    base = (rng.standard_normal((W.shape[0], W.shape[1])) * float(np.std(ref[2]))).astype(np.float32)
    gW = torch.from_numpy(base).cuda().to(gw_dtype)
    start = from_device(gW)
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    gX = torch.empty(X.shape, dtype=torch.bfloat16, device="cuda")
    _ex(fl, X, W, y, 3, grad_w_dtype=gw_dtype, flags=fl.FLJSD_ACCUMULATE_GRAD_W, out=(loss, gX, gW))
    assert_tensor_close(from_device(gW), start + ref[2], TOL["bf16"], "grad_W added")


def test_flce_accumulate_fp32_inputs(fl):
    X, W, y = _case(613, 24, 64, 700, "f32")
    ref = oracle.fused_linear_cross_entropy(to_f64(X, "f32"), to_f64(W, "f32"), y, -100, 0.05, "mean")
    g0 = workloads.draw(9003, W.shape, float(np.std(ref[2])), "f32")
    out = (torch.empty(1, dtype=torch.float32, device="cuda"),
           torch.empty(X.shape, dtype=torch.float32, device="cuda"), to_device(g0, "f32"))
    fl.fljsd_flce_forward_backward_ex(to_device(X, "f32"), to_device(W, "f32"), torch.from_numpy(y).cuda(),
                                      -100, 0.05, "mean", 5, flags=fl.FLJSD_ACCUMULATE_GRAD_W, out=out)
    torch.cuda.synchronize()
    tol = TOL["f32"]
    assert_loss_close(from_device(out[0]), ref[0], tol)
    assert_tensor_close(from_device(out[1]), ref[1], tol, "grad_input")
    assert_tensor_close(from_device(out[2]), to_f64(g0, "f32") + ref[2], tol, "grad_weight + existing")


def test_flce_plain_entry_point_is_the_ex_default(fl, flce_bf16_case):
    X, W, y, _ = flce_bf16_case
    a = _run(fl, X, W, y, "bf16", -100, 0.05, "mean", 4)
    b = _ex(fl, X, W, y, 4)
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v)


def test_flce_ex_rejects_on_device(fl, flce_bf16_case):
    X, W, y, _ = flce_bf16_case
    with pytest.raises(fl.FljsdError):
        _ex(fl, X, W, y, 2, grad_w_dtype=torch.float16)
    with pytest.raises(ValueError):
        _ex(fl, X, W, y, 2, flags=fl.FLJSD_ACCUMULATE_GRAD_W)
