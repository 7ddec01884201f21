"""GPU parity of the whole pass (fljsd_forward_backward) against the oracle.

Workloads and seeds come from workloads.py. The oracle takes the same input
bits widened to fp64 and keeps every intermediate in fp64; the GPU rounds the
logits and dZ to the input dtype, which the bf16 tolerances cover.
"""
from __future__ import annotations

import functools
import time

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import (TOL, assert_loss_close, assert_tensor_close, from_device, normwise,
                            to_device, to_f64)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lm_head_distillation_amd import fljsd
    fljsd.load_library()
    return fljsd


@functools.lru_cache(maxsize=4)
def _inputs(key, BT=None, V=None, H_s=None, H_t=None):
    w = workloads.WORKLOADS[key]
    return w, workloads.make_inputs(w, BT=BT, V=V, H_s=H_s, H_t=H_t)


@functools.lru_cache(maxsize=8)
def _oracle(key, beta, T, reduction, BT=None, V=None, H_s=None, H_t=None):
    w, inp = _inputs(key, BT, V, H_s, H_t)
    d = w.dtype
    return oracle.fused_linear_jsd(to_f64(inp["X_s"], d), to_f64(inp["W_s"], d),
                                   to_f64(inp["X_t"], d), to_f64(inp["W_t"], d),
                                   beta, T, reduction)


def _device_inputs(inp, dtype):
    return tuple(to_device(inp[k], dtype) for k in ("X_s", "W_s", "X_t", "W_t"))


def _run(fl, dev, beta, T, reduction, nc, **kw):
    loss, gX, gW = fl.fljsd_forward_backward(*dev, beta, T, reduction, nc, **kw)
    torch.cuda.synchronize()
    return loss, gX, gW


def _compare(dtype, got, ref, tol=None):
    loss, gX, gW = got
    rl, rX, rW = ref
    tol = TOL[dtype] if tol is None else tol
    e0 = assert_loss_close(from_device(loss), rl, tol)
    e1 = assert_tensor_close(from_device(gX), rX, tol, "grad_input")
    e2 = assert_tensor_close(from_device(gW), rW, tol, "grad_weight")
    print(f"loss rel {e0:.2e}  grad_input normwise {e1:.2e}  grad_weight normwise {e2:.2e}", flush=True)


@pytest.mark.parametrize("beta", [0.0, 0.1, 0.5, 0.9, 1.0])
@pytest.mark.parametrize("T", [1.0, 2.0])
@pytest.mark.parametrize("reduction", ["batchmean", "sum", "mean", "none"])
@pytest.mark.parametrize("nc", [1, 3])
def test_tiny_f32(fl, beta, T, reduction, nc):
    """8 x 64 x 512 fp32 (the pages' (8, 512) tie-test shape) at the 1e-5 bar."""
    w, inp = _inputs("tiny_f32")
    got = _run(fl, _device_inputs(inp, "f32"), beta, T, reduction, nc)
    _compare("f32", got, _oracle("tiny_f32", beta, T, reduction))


def _scaled(inp, dtype, factor):
    """The inputs with both hidden-state matrices times a power of two (exact in
    fp32 and bf16), so the logits, and what the temperature makes of them, are
    far from the default workloads' small values."""
    out = dict(inp)
    for k in ("X_s", "X_t"):
        if dtype == "f32":
            out[k] = (inp[k] * np.float32(factor)).astype(np.float32)
        else:
            out[k] = workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(inp[k]) * np.float32(factor))
    return out


@pytest.mark.parametrize("beta", [0.0, 0.001, 0.1, 0.5, 0.9, 0.999, 1.0])
@pytest.mark.parametrize("T", [0.25, 0.5, 4.0])
@pytest.mark.parametrize("factor", [8.0, 16.0])
@pytest.mark.parametrize("nc", [1, 3])
def test_temperature_extremes_f32(fl, beta, T, factor, nc):
    """8 x 64 x 512 fp32 with 8x and 16x hidden states (logit std ~1.2 and
    ~2.5): at T = 0.25 the rows are close to one-hot (std of z / T ~4.9 and
    ~9.8; many rows put nearly all of the student's mass where the teacher has
    almost none, so the divergence is near its maximum and the gradient is a
    small difference of large terms), at T = 4 nearly flat; all at the 1e-5
    bar, in one chunk and in three (ragged: 3 + 3 + 2 rows). The oracle takes
    beta as the fp32 value the library receives (0.999 rounds to
    0.99900001, which moves 1 - beta by 1.3e-5 relative)."""
    w, inp = _inputs("tiny_f32")
    inp = _scaled(inp, "f32", factor)
    got = _run(fl, _device_inputs(inp, "f32"), beta, T, "batchmean", nc)
    _compare("f32", got, _oracle_of(inp, "f32", float(np.float32(beta)), T, "batchmean"))


@pytest.mark.parametrize("beta", [0.1, 0.5, 0.9])
@pytest.mark.parametrize("T", [0.5, 4.0])
def test_temperature_extremes_bf16(fl, beta, T):
    """64 x 256 x 5003 bf16 with 8x hidden states, two chunks. The logits are
    stored in bf16, and a rounding error dz of a logit moves the distribution
    as dz / T does, so below T = 1 the bf16 bounds widen by 1 / T."""
    inp = _scaled(_adhoc(31, 64, 256, 256, 5003, "bf16"), "bf16", 8.0)
    got = _run(fl, _device_inputs(inp, "bf16"), beta, T, "batchmean", 2)
    f = max(1.0, 1.0 / T)
    tol = {k: v * f for k, v in TOL["bf16"].items()}
    _compare("bf16", got, _oracle_of(inp, "bf16", beta, T, "batchmean"), tol)


@pytest.mark.parametrize("beta", [0.1, 0.5, 0.9])
@pytest.mark.parametrize("nc", [1, 4])
def test_multiblock_tail(fl, beta, nc):
    """64 x 256 x 40960 bf16: the pages' multi-block shape, partial trailing block."""
    w, inp = _inputs("multiblock_tail")
    got = _run(fl, _device_inputs(inp, "bf16"), beta, 1.0, "batchmean", nc)
    _compare("bf16", got, _oracle("multiblock_tail", beta, 1.0, "batchmean"))


def test_ties_self_distillation(fl):
    """Teacher bit-identical to student: loss and every gradient element are 0."""
    w, inp = _inputs("ties_self")
    loss, gX, gW = _run(fl, _device_inputs(inp, "bf16"), w.beta, w.temperature, w.reduction, 1)
    assert from_device(loss) == 0.0
    assert torch.count_nonzero(gX).item() == 0
    assert torch.count_nonzero(gW).item() == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("beta,T", [(0.5, 1.0), (0.1, 2.0), (0.0, 1.0), (1.0, 0.7)])
def test_shifted_teacher_rows(fl, dtype, beta, T):
    """Teacher logits equal to the student's plus a constant per row, exactly:
    integer features and weights make every logit a small integer (exact in
    bf16), and the teacher's extra feature column, against an all-ones weight
    column, adds the row's constant (seven zero columns more keep H_t a whole
    number of 16-byte vectors). The softmax ignores a shift of its row,
    so the two distributions are equal element by element (exact ties, PR
    #1374) and the loss and every gradient element are exactly 0, across
    several vocabulary tiles and the merge of their row statistics."""
    rng = np.random.default_rng(41)
    BT, H, V = 300, 64, 1000
    X_s = rng.integers(-1, 2, size=(BT, H)).astype(np.float32)
    W_s = rng.integers(-1, 2, size=(V, H)).astype(np.float32)
    shift = rng.integers(-60, 61, size=(BT, 1)).astype(np.float32)
    X_t = np.concatenate([X_s, shift, np.zeros((BT, 7), np.float32)], axis=1)
    W_t = np.concatenate([W_s, np.ones((V, 1), np.float32), np.zeros((V, 7), np.float32)], axis=1)
    arrays = (X_s, W_s, X_t, W_t)
    if dtype == "bf16":  # small integers: the fp32 pattern's top half is exact
        arrays = tuple((a.view(np.uint32) >> 16).astype(np.uint16) for a in arrays)
    dev = tuple(to_device(a, dtype) for a in arrays)
    for reduction, nc in (("batchmean", 1), ("sum", 3), ("none", 2)):
        loss, gX, gW = _run(fl, dev, beta, T, reduction, nc)
        assert np.all(from_device(loss) == 0.0), f"{reduction} nc={nc}"
        assert torch.count_nonzero(gX).item() == 0, f"{reduction} nc={nc}"
        assert torch.count_nonzero(gW).item() == 0, f"{reduction} nc={nc}"


def test_ties_padded_vocabulary(fl):
    """Padded vocabulary rows carry zero mass in both models: their grad_W rows
    are exactly 0, and everything else matches the oracle."""
    w, inp = _inputs("ties_padded")
    got = _run(fl, _device_inputs(inp, "bf16"), w.beta, w.temperature, w.reduction, 1)
    gW = from_device(got[2])
    assert np.all(gW[-workloads.PAD_ROWS:] == 0.0)
    _compare("bf16", got, _oracle("ties_padded", w.beta, w.temperature, w.reduction))


@pytest.fixture(scope="module")
def llama3_device():
    w, inp = _inputs("llama3_head")
    return w, _device_inputs(inp, "bf16")


@pytest.mark.slow
@pytest.mark.parametrize("nc", [1, 8, 32])
def test_llama3_head_full(fl, llama3_device, nc):
    """1024 x 4096 x 128256 bf16 against the full oracle, per chunk count."""
    w, dev = llama3_device
    got = _run(fl, dev, w.beta, w.temperature, w.reduction, nc)
    _compare("bf16", got, _oracle("llama3_head", w.beta, w.temperature, w.reduction))


@pytest.fixture(scope="module")
def large_batch():
    w, inp = _inputs("large_batch")
    return w, inp, _device_inputs(inp, "bf16")


@pytest.fixture(scope="module")
def large_batch_oracle(large_batch):
    """The oracle over the whole 8192 x 4096 x 128256 workload, once per module
    (about a minute on 16 host threads, ~20 GB of host memory at its peak)."""
    w, _inp, _dev = large_batch
    t0 = time.perf_counter()
    ref = _oracle("large_batch", w.beta, w.temperature, w.reduction)
    print(f"large_batch oracle: {time.perf_counter() - t0:.1f} s", flush=True)
    return ref


@pytest.mark.slow
@pytest.mark.timeout(1200)
@pytest.mark.parametrize("nc", [1, 8, 32])
def test_large_batch_full(fl, large_batch, large_batch_oracle, nc):
    """8192 x 4096 x 128256 bf16, T = 2 (the pages' B*T = 8192 benchmark shape):
    loss, every grad_input element and every grad_W element against the full
    oracle, per chunk count."""
    w, _inp, dev = large_batch
    print(f"large_batch nc={nc}", flush=True)
    got = _run(fl, dev, w.beta, w.temperature, w.reduction, nc)
    _compare("bf16", got, large_batch_oracle)


@pytest.mark.slow
def test_large_batch_sampled_and_properties(fl, large_batch):
    """8192 x 4096 x 128256 bf16, T = 2. Sampled rows (chunk edges included)
    against the oracle one by one; grad_W through chunk-count invariance and the
    identity <grad_W, W_s> = <dZ, Z_s> = <grad_X, X_s>."""
    w, inp, dev = large_batch
    d = w.dtype
    rows = np.array([0, 1, 255, 256, 1023, 1024, 4097, 8191])
    Xs = to_f64(inp["X_s"], d)
    Ws = to_f64(inp["W_s"], d)
    Xt = to_f64(inp["X_t"], d)
    Wt = to_f64(inp["W_t"], d)
    ref_rows_loss, ref_rows_gX = oracle.fused_linear_jsd_rows(Xs, Ws, Xt, Wt, rows, w.beta,
                                                              w.temperature, w.reduction)
    del Wt
    results = {}
    for nc in (1, 8, 32):
        loss, gX, gW = _run(fl, dev, w.beta, w.temperature, w.reduction, nc)
        results[nc] = (from_device(loss), from_device(gX[torch.as_tensor(rows, device=gX.device)]),
                       gW)
        # <grad_W, W_s> == <grad_X, X_s>, both in fp64 from the GPU outputs.
        lhs = float((gW.double() * dev[1].double()).sum())
        rhs = float((gX.double() * dev[0].double()).sum())
        assert abs(lhs - rhs) <= 2e-2 * max(abs(lhs), abs(rhs)), f"nc={nc}: {lhs} vs {rhs}"
        assert torch.isfinite(gW).all() and torch.isfinite(gX).all()
        assert_tensor_close(results[nc][1], ref_rows_gX, TOL[d], f"grad_input rows nc={nc}")
    loss_none, _, _ = _run(fl, dev, w.beta, w.temperature, "none", 1, grad_input=False,
                           grad_weight=False)
    row_losses = from_device(loss_none)
    assert_loss_close(row_losses[rows], ref_rows_loss, TOL[d], "per-row loss")
    for nc in (1, 8, 32):
        assert_loss_close(results[nc][0], row_losses.mean(), {"loss_rel": 1e-5}, f"loss nc={nc}")
    ref_gW = results[1][2].double()
    for nc in (8, 32):
        nw = float(torch.linalg.vector_norm(results[nc][2].double() - ref_gW) / torch.linalg.vector_norm(ref_gW))
        assert nw <= TOL[d]["norm"], f"grad_W nc={nc} vs nc=1 normwise {nw:.3e}"


# ---- edge cases -------------------------------------------------------------------------

def _adhoc(seed, BT, H_s, H_t, V, dtype):
    w = workloads.Workload("adhoc", seed, BT, H_s, H_t, V, dtype, 0.5, 1.0, "batchmean", "independent")
    return workloads.make_inputs(w)


def _oracle_of(inp, dtype, beta, T, reduction):
    return oracle.fused_linear_jsd(*(to_f64(inp[k], dtype) for k in ("X_s", "W_s", "X_t", "W_t")),
                                   beta, T, reduction)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("BT,H_s,H_t,V,nc", [
    (1, 64, 64, 100, 1),          # one row
    (300, 72, 72, 1000, 1),       # ragged M, N and K tiles
    (200, 264, 264, 5003, 2),     # 100-row chunks: 128-row tiles with ragged rows
    (300, 72, 72, 1000, 3),       # ragged chunks
    (300, 72, 72, 1000, 7),
    (64, 128, 256, 3000, 2),      # teacher hidden size differs
    (10, 64, 64, 777, 100),       # more chunks asked than rows
    (513, 264, 136, 5003, 2),     # odd everything
    (2100, 264, 264, 3000, 2),    # 1050-row chunks: 256-row read-add-write tiles, partial K-tile
])
def test_shapes(fl, dtype, BT, H_s, H_t, V, nc):
    inp = _adhoc(7, BT, H_s, H_t, V, dtype)
    for beta, T in ((0.5, 1.0), (0.0, 2.0), (1.0, 1.5)):
        got = _run(fl, _device_inputs(inp, dtype), beta, T, "batchmean", nc)
        _compare(dtype, got, _oracle_of(inp, dtype, beta, T, "batchmean"))


# bf16 shapes whose vocabulary tiles by 256, H_s by 64, with more than 4096
# rows and chunks of at least 512: the first chunk's student logits product
# also writes W_s^T, and grad_input reads both operands along V.
@pytest.mark.parametrize("BT,H_s,H_t,V,nc", [
    (4160, 64, 64, 768, 1),       # one chunk, a ragged last M-tile (4160 = 16 * 256 + 64)
    (4608, 128, 128, 2560, 9),    # 512-row chunks: split-K grad_input over K-contiguous operands
    (4601, 192, 320, 1024, 4),    # H_t differs; chunks of 1151 and 1148 rows (ragged M-tiles)
    (235108, 64, 64, 256, 460),   # 512-row chunks; last chunk 100 rows (128-row tiles)
    (235061, 64, 64, 256, 460),   # last chunk 53 rows (64-row tiles)
])
def test_w_transposed_shapes(fl, BT, H_s, H_t, V, nc):
    inp = _adhoc(13, BT, H_s, H_t, V, "bf16")
    dev = _device_inputs(inp, "bf16")
    # Hundreds of chunks: grad_W summed in fp32 (a bf16 sum rounds once per
    # chunk, ~2^-9 each, beyond the bf16 tolerance after 460 roundings).
    kw = {"grad_w_dtype": torch.float32} if nc > 64 else {}
    for beta, T in ((0.5, 1.0), (0.0, 2.0), (1.0, 1.5)):
        got = fl.fljsd_forward_backward_ex(*dev, beta, T, "batchmean", nc, **kw)
        torch.cuda.synchronize()
        _compare("bf16", got, _oracle_of(inp, "bf16", beta, T, "batchmean"))


def test_w_transposed_region_is_optional(fl):
    """A workspace short of exactly the W_s^T region runs grad_input on W_s as
    given. The two layouts put the same values in LDS and run the same MFMA
    sequence, so every output is bit-identical."""
    BT, H, V, nc = 4160, 128, 2560, 2
    inp = _adhoc(14, BT, H, H, V, "bf16")
    dev = _device_inputs(inp, "bf16")
    full = fl.fljsd_workspace_size(BT, H, H, V, fl.BF16, nc)
    wst = (V * H * 2 + 255) // 256 * 256
    assert fl.fljsd_workspace_size(BT, H, H, V + 8, fl.BF16, nc) < full   # V + 8: no region
    # 4096 rows: no region; 4104: the region (and 8 more rows)
    assert (fl.fljsd_workspace_size(4104, H, H, V, fl.BF16, 1)
            - fl.fljsd_workspace_size(4096, H, H, V, fl.BF16, 1)) >= wst
    ws_full = torch.empty(full, dtype=torch.uint8, device="cuda")
    ws_short = torch.empty(full - wst, dtype=torch.uint8, device="cuda")
    a = _run(fl, dev, 0.5, 1.0, "batchmean", nc, workspace=ws_full)
    b = _run(fl, dev, 0.5, 1.0, "batchmean", nc, workspace=ws_short)
    assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])
    assert torch.equal(a[1], b[1])
    _compare("bf16", b, _oracle_of(inp, "bf16", 0.5, 1.0, "batchmean"))
    _compare("bf16", a, _oracle_of(inp, "bf16", 0.5, 1.0, "batchmean"))
    with pytest.raises(fl.FljsdError):
        fl.fljsd_forward_backward(*dev, 0.5, 1.0, "batchmean", nc,
                                  workspace=ws_short[:full - wst - 256])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_optional_gradients_and_determinism(fl, dtype):
    inp = _adhoc(8, 200, 128, 128, 4000, dtype)
    dev = _device_inputs(inp, dtype)
    full = _run(fl, dev, 0.3, 1.0, "batchmean", 2)
    again = _run(fl, dev, 0.3, 1.0, "batchmean", 2)
    for a, b in zip(full, again):
        assert torch.equal(a, b), "two identical calls differ"
    only_x = _run(fl, dev, 0.3, 1.0, "batchmean", 2, grad_weight=False)
    only_w = _run(fl, dev, 0.3, 1.0, "batchmean", 2, grad_input=False)
    neither = _run(fl, dev, 0.3, 1.0, "batchmean", 2, grad_input=False, grad_weight=False)
    assert only_x[2] is None and only_w[1] is None
    assert torch.equal(only_x[1], full[1]) and torch.equal(only_w[2], full[2])
    assert torch.equal(only_w[0], full[0])
    # Without a weight gradient (or any gradient) the loss terms are summed in
    # pass 2 instead of pass 3 (bf16): the same terms in another order.
    for r in (only_x, neither):
        if dtype == "f32":
            assert torch.equal(r[0], full[0])
        else:
            assert abs(float(r[0]) - float(full[0])) <= 1e-6 * abs(float(full[0]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["sum", "mean", "none"])
def test_reductions(fl, dtype, reduction):
    inp = _adhoc(9, 96, 64, 64, 2500, dtype)
    got = _run(fl, _device_inputs(inp, dtype), 0.7, 1.3, reduction, 3)
    _compare(dtype, got, _oracle_of(inp, dtype, 0.7, 1.3, reduction))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_output_element_written(fl, dtype):
    """Outputs prefilled with NaN come back finite: the first chunk overwrites
    grad_W and the loop writes every element (PR #1429 Summary)."""
    inp = _adhoc(10, 130, 64, 64, 1500, dtype)
    dev = _device_inputs(inp, dtype)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    gX = torch.full(dev[0].shape, float("nan"), dtype=tdt, device="cuda")
    gW = torch.full(dev[1].shape, float("nan"), dtype=tdt, device="cuda")
    _run(fl, dev, 0.5, 1.0, "batchmean", 4, out=(loss, gX, gW))
    assert torch.isfinite(loss).all() and torch.isfinite(gX).all() and torch.isfinite(gW).all()
    _compare(dtype, (loss[0], gX, gW), _oracle_of(inp, dtype, 0.5, 1.0, "batchmean"))


def test_policy_picks_chunks_for_workspace(fl):
    inp = _adhoc(11, 256, 64, 64, 3000, "bf16")
    dev = _device_inputs(inp, "bf16")
    need3 = fl.fljsd_workspace_size(256, 64, 64, 3000, fl.BF16, 3)
    assert fl.fljsd_plan_num_chunks(256, 64, 64, 3000, fl.BF16, need3) == 3
    ws = torch.empty(need3, dtype=torch.uint8, device="cuda")
    auto = _run(fl, dev, 0.5, 1.0, "batchmean", 0, workspace=ws)
    explicit = _run(fl, dev, 0.5, 1.0, "batchmean", 3)
    for a, b in zip(auto, explicit):
        assert torch.equal(a, b)


def test_status_codes_on_device(fl):
    inp = _adhoc(12, 16, 64, 64, 300, "bf16")
    dev = _device_inputs(inp, "bf16")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(fl.FljsdError) as e:
        fl.fljsd_forward_backward(*dev, 0.5, 1.0, "batchmean", 1, workspace=small)
    assert e.value.code == -3
    with pytest.raises(fl.FljsdError) as e:
        fl.fljsd_forward_backward(*dev, 1.5, 1.0, "batchmean", 1)
    assert e.value.code == -1


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_vocab_entry(fl, dtype):
    """V = 1, the method's degenerate case: both distributions are the point
    mass on the one entry (P == Q == 1, an exact tie), so the loss and every
    gradient are exactly 0 under every reduction and chunking."""
    inp = _adhoc(611, 37, 64, 64, 1, dtype)
    dev = _device_inputs(inp, dtype)
    ref = _oracle_of(inp, dtype, 0.5, 2.0, "batchmean")
    assert float(ref[0]) == 0.0 and not np.any(ref[1]) and not np.any(ref[2])
    for red in ("batchmean", "sum", "mean", "none"):
        for nc in (1, 3):
            loss, gX, gW = _run(fl, dev, 0.5, 2.0, red, nc)
            assert np.all(from_device(loss) == 0.0), f"{red} nc={nc}"
            assert int(torch.count_nonzero(gX)) == 0 and int(torch.count_nonzero(gW)) == 0, f"{red} nc={nc}"


@pytest.mark.slow
def test_beyond_2g_logit_elements(fl):
    """17000 x 256 x 128256 bf16, one chunk: each logits buffer (and dZ^T)
    holds 2.18e9 elements, past 2^31, so every flat offset into them must be
    64-bit. Sampled rows on both sides of element 2^31 (row 16744 starts past
    it) against the oracle one by one; all rows through the identity
    <grad_W, W_s> = <dZ, Z_s> = <grad_X, X_s>."""
    BT, H, V = 17000, 256, 128256
    assert BT * V > 2 ** 31
    w = workloads.Workload("beyond_2g", 621, BT, H, H, V, "bf16", 0.5, 2.0, "batchmean",
                           "independent")
    inp = workloads.make_inputs(w)
    dev = _device_inputs(inp, "bf16")
    rows = np.array([0, 1, 8500, 16743, 16744, 16745, BT - 1])
    ref_loss, ref_gX = oracle.fused_linear_jsd_rows(
        *(to_f64(inp[k], "bf16") for k in ("X_s", "W_s", "X_t", "W_t")), rows, w.beta,
        w.temperature, w.reduction)
    loss, gX, gW = _run(fl, dev, w.beta, w.temperature, w.reduction, 1)
    got_rows = from_device(gX[torch.as_tensor(rows, device=gX.device)])
    assert_tensor_close(got_rows, ref_gX, TOL["bf16"], "grad_input rows")
    lhs = float((gW.double() * dev[1].double()).sum())
    rhs = float((gX.double() * dev[0].double()).sum())
    assert abs(lhs - rhs) <= 2e-2 * max(abs(lhs), abs(rhs)), f"{lhs} vs {rhs}"
    assert torch.isfinite(gW).all() and torch.isfinite(gX).all()
    del gX, gW
    row_loss, _, _ = _run(fl, dev, w.beta, w.temperature, "none", 1, grad_input=False,
                          grad_weight=False)
    rl = from_device(row_loss)
    assert_loss_close(rl[rows], ref_loss, TOL["bf16"], "per-row loss")
    assert_loss_close(from_device(loss), rl.mean(), {"loss_rel": 1e-5}, "batchmean = mean of rows")


def test_binding_rejects_mismatched_outputs(fl):
    """Caller-supplied outputs whose dtype, size or layout differ from what the
    kernels write are refused before any launch: an fp32 grad_W asked for into
    a bf16 tensor, a one-element loss for reduction "none", a gradient tensor
    of another dtype with the logits' strides."""
    inp = _adhoc(13, 16, 64, 64, 300, "bf16")
    dev = _device_inputs(inp, "bf16")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    gX = torch.empty_like(dev[0])
    gW_bf16 = torch.empty_like(dev[1])
    with pytest.raises(ValueError, match="grad_W_s"):
        fl.fljsd_forward_backward_ex(*dev, 0.5, 1.0, "batchmean", 1, grad_w_dtype=torch.float32,
                                     out=(loss, gX, gW_bf16))
    with pytest.raises(ValueError, match="loss"):
        fl.fljsd_forward_backward(*dev, 0.5, 1.0, "none", 1, out=(loss, gX, gW_bf16))
    with pytest.raises(ValueError, match="grad_X_s"):
        fl.fljsd_forward_backward(*dev, 0.5, 1.0, "batchmean", 1,
                                  out=(loss, gX[:8], gW_bf16))
    zs = torch.randn(16, 300, device="cuda")
    zt = torch.randn(16, 300, device="cuda")
    bad = torch.empty_strided(zs.shape, zs.stride(), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="dtype"):
        fl.fljsd_generalized_jsd(zs, zt, 0.5, 1.0, grad=bad)
    with pytest.raises(ValueError, match="dtype"):
        fl.fljsd_jsd_logprob(zs, zt, 0.5, grad=bad)
    torch.cuda.synchronize()
