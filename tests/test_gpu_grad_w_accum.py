"""GPU tests of fljsd_forward_backward_ex: fp32 weight-gradient accumulation
over chunks and adding to an existing weight gradient.

The fp32 mode follows Liger-Kernel PR #1429, Details (the accum_dtype=float32
path: per-chunk products summed in fp32). The oracle's grad_W is fp64; adding
to an existing gradient is checked against that value plus the oracle's.
"""
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


def _inputs(seed, BT, H_s, H_t, V, dtype):
    w = workloads.Workload("accum", seed, BT, H_s, H_t, V, dtype, 0.5, 1.0, "batchmean",
                           "independent")
    inp = workloads.make_inputs(w)
    dev = tuple(to_device(inp[k], dtype) for k in ("X_s", "W_s", "X_t", "W_t"))
    ref = oracle.fused_linear_jsd(*(to_f64(inp[k], dtype) for k in ("X_s", "W_s", "X_t", "W_t")),
                                  0.5, 1.0, "batchmean")
    return dev, ref


@pytest.fixture(scope="module")
def bf16_case():
    # Several 256-wide vocabulary tiles with a ragged last one, a ragged hidden
    # tile, and chunks down to 4 rows.
    return _inputs(41, 64, 264, 136, 5003, "bf16")


def _ex(fl, dev, nc, **kw):
    out = fl.fljsd_forward_backward_ex(*dev, 0.5, 1.0, "batchmean", nc, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("nc", [1, 4, 16])
def test_fp32_grad_w_matches_oracle(fl, bf16_case, nc):
    dev, (rl, rX, rW) = bf16_case
    loss, gX, gW = _ex(fl, dev, nc, grad_w_dtype=torch.float32)
    assert gW.dtype == torch.float32 and gX.dtype == torch.bfloat16
    tol = TOL["bf16"]
    assert_loss_close(from_device(loss), rl, tol)
    assert_tensor_close(from_device(gX), rX, tol, "grad_input")
    e = assert_tensor_close(from_device(gW), rW, tol, "grad_weight fp32")
    print(f"nc={nc}: fp32 grad_W normwise {e:.2e}", flush=True)


def test_fp32_grad_w_does_not_depend_on_chunks(fl, bf16_case):
    """dZ rows do not depend on the chunking, so the fp32 sums over 1, 4 and
    16 chunks differ only by fp32 rounding; the bf16 result carries one bf16
    rounding per chunk and differs by far more."""
    dev, _ = bf16_case
    f32 = {nc: from_device(_ex(fl, dev, nc, grad_w_dtype=torch.float32)[2]) for nc in (1, 4, 16)}
    b16 = {nc: from_device(_ex(fl, dev, nc)[2]) for nc in (1, 16)}
    for nc in (4, 16):
        e = normwise(f32[nc], f32[1])
        assert e <= 1e-5, f"fp32 grad_W nc={nc} vs nc=1: {e:.3e}"
    print(f"fp32 nc=16 vs 1: {normwise(f32[16], f32[1]):.2e}; "
          f"bf16 nc=16 vs 1: {normwise(b16[16], b16[1]):.2e}", flush=True)


def test_single_chunk_fp32_rounds_to_the_bf16_result(fl, bf16_case):
    """With one chunk both modes take the same fp32 product; bf16 mode rounds
    it once (to nearest even), so rounding the fp32 result gives the same bits."""
    dev, _ = bf16_case
    g32 = _ex(fl, dev, 1, grad_w_dtype=torch.float32)[2]
    g16 = _ex(fl, dev, 1)[2]
    assert torch.equal(g32.to(torch.bfloat16).view(torch.int16), g16.view(torch.int16))


@pytest.mark.parametrize("gw", ["f32", "bf16"])
@pytest.mark.parametrize("nc", [1, 3])
def test_accumulate_into_existing_grad_w(fl, bf16_case, gw, nc):
    dev, (rl, rX, rW) = bf16_case
    V, H = dev[1].shape
    g0 = workloads.draw(9001, (V, H), float(np.std(rW)), gw)
    g0_dev = to_device(g0, gw)
    g0_f64 = to_f64(g0, gw)
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    gX = torch.empty_like(dev[0])
    out = (loss, gX, g0_dev.clone())
    _, _, gW = _ex(fl, dev, nc, grad_w_dtype=torch.float32 if gw == "f32" else None,
                   flags=fl.FLJSD_ACCUMULATE_GRAD_W, out=out)
    assert gW.data_ptr() == out[2].data_ptr()
    tol = TOL["bf16"]
    assert_loss_close(from_device(loss), rl, tol)
    assert_tensor_close(from_device(gX), rX, tol, "grad_input")
    assert_tensor_close(from_device(gW), g0_f64 + rW, tol, "grad_weight + existing")
    if gw == "f32":
        fresh = from_device(_ex(fl, dev, nc, grad_w_dtype=torch.float32)[2])
        e = normwise(from_device(gW) - g0_f64, fresh)
        assert e <= 1e-5, f"added part differs from a fresh fp32 result: {e:.3e}"


@pytest.fixture(scope="module")
def long_chunk_case():
    # Chunks of 1050 rows: the weight-gradient product of each chunk has
    # K = 1050 (> 1024), so it runs on 256-row tiles with the staged
    # read-add-write epilogue and a partial last K-tile; V = 3000 and H = 264
    # give interior and ragged tiles in both directions.
    return _inputs(44, 2100, 264, 136, 3000, "bf16")


@pytest.mark.parametrize("gw", ["f32", "bf16"])
@pytest.mark.parametrize("accumulate", [False, True])
def test_long_chunks(fl, long_chunk_case, gw, accumulate):
    dev, (rl, rX, rW) = long_chunk_case
    V, H = dev[1].shape
    kw = {"grad_w_dtype": torch.float32} if gw == "f32" else {}
    expect = rW
    if accumulate:
        g0 = workloads.draw(9003, (V, H), float(np.std(rW)), gw)
        out = (torch.empty(1, dtype=torch.float32, device="cuda"), torch.empty_like(dev[0]),
               to_device(g0, gw))
        kw.update(flags=fl.FLJSD_ACCUMULATE_GRAD_W, out=out)
        expect = to_f64(g0, gw) + rW
    loss, gX, gW = _ex(fl, dev, 2, **kw)
    tol = TOL["bf16"]
    assert_loss_close(from_device(loss), rl, tol)
    assert_tensor_close(from_device(gX), rX, tol, "grad_input")
    e = assert_tensor_close(from_device(gW), expect, tol, f"grad_weight {gw}")
    print(f"1050-row chunks, {gw}, accumulate={accumulate}: grad_W normwise {e:.2e}", flush=True)


def test_accumulate_fp32_inputs(fl):
    dev, (rl, rX, rW) = _inputs(43, 24, 64, 64, 700, "f32")
    V, H = dev[1].shape
    g0 = workloads.draw(9002, (V, H), float(np.std(rW)), "f32")
    out = (torch.empty(1, dtype=torch.float32, device="cuda"), torch.empty_like(dev[0]),
           to_device(g0, "f32"))
    loss, gX, gW = _ex(fl, dev, 5, flags=fl.FLJSD_ACCUMULATE_GRAD_W, out=out)
    tol = TOL["f32"]
    assert_loss_close(from_device(loss), rl, tol)
    assert_tensor_close(from_device(gX), rX, tol, "grad_input")
    assert_tensor_close(from_device(gW), to_f64(g0, "f32") + rW, tol, "grad_weight + existing")


def test_plain_entry_point_is_the_ex_default(fl, bf16_case):
    dev, _ = bf16_case
    a = fl.fljsd_forward_backward(*dev, 0.5, 1.0, "batchmean", 4)
    b = _ex(fl, dev, 4)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def test_ex_rejects_on_device(fl, bf16_case):
    dev, _ = bf16_case
    with pytest.raises(fl.FljsdError):
        _ex(fl, dev, 2, grad_w_dtype=torch.float16)
    with pytest.raises(ValueError):
        _ex(fl, dev, 2, flags=fl.FLJSD_ACCUMULATE_GRAD_W)
