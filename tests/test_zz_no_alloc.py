"""GPU check of fljsd_generalized_jsd_noalloc, the entry point that allocates
nothing: called through the C ABI, its loss and gradient must equal those of
fljsd_generalized_jsd (same kernels, caller-owned workspace) bit for bit, on
consecutive calls that share the library's scratch array, the later ones
smaller than the first."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL, assert_loss_close, assert_tensor_close, from_device, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lm_head_distillation_amd import fljsd
    fljsd.load_library()
    return fljsd


def _logits(seed, BT, V, dtype, ld=None):
    """Seeded logits with the spread of the pages' workloads (std ~1.3)."""
    ld = V if ld is None else ld
    zs = workloads.draw(seed, (BT, ld), 1.3, dtype)
    zt = workloads.draw(seed + 1, (BT, ld), 1.3, dtype)
    return zs, zt


def _call_workspace(fl, zs, zt, beta, T, red, V, ld, in_place):
    lib = fl.load_library()
    BT = zs.shape[0]
    dt = fl._dtype_code(zs)
    ws = torch.empty(fl.fljsd_generalized_jsd_workspace_size(BT, V, dt), dtype=torch.uint8,
                     device="cuda")
    loss = torch.empty(BT if red == "none" else 1, dtype=torch.float32, device="cuda")
    grad = zs if in_place else torch.empty_like(zs)
    rc = lib.fljsd_generalized_jsd(zs.data_ptr(), zt.data_ptr(), BT, V, ld, dt, beta, T,
                                   fl.REDUCTIONS[red], loss.data_ptr(), grad.data_ptr(),
                                   ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, lib.fljsd_last_error()
    return loss, grad


def _call_noalloc(fl, zs, zt, beta, T, red, V, ld, in_place):
    lib = fl.load_library()
    BT = zs.shape[0]
    dt = fl._dtype_code(zs)
    loss = torch.empty(BT if red == "none" else 1, dtype=torch.float32, device="cuda")
    grad = zs if in_place else torch.empty_like(zs)
    rc = lib.fljsd_generalized_jsd_noalloc(zs.data_ptr(), zt.data_ptr(), BT, V, ld, dt, beta, T,
                                           fl.REDUCTIONS[red], loss.data_ptr(), grad.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
    assert rc == 0, lib.fljsd_last_error()
    return loss, grad


# Consecutive calls on the one scratch array: the first fills it with a large
# problem's statistics and partial sums, the later ones are smaller and must
# not see any of it.
SEQUENCE = [
    # (seed, BT, V, ld, dtype, beta, T, reduction, in_place)
    (101, 3000, 32064, 32064, "bf16", 0.5, 1.0, "batchmean", False),
    (102, 64, 200000, 200000, "bf16", 0.5, 1.0, "sum", False),   # 32 slices per row
    (103, 37, 7001, 7008, "bf16", 0.1, 2.0, "batchmean", True),
    (105, 600, 5003, 5003, "f32", 0.9, 0.5, "none", False),
    (107, 8, 512, 512, "f32", 0.0, 1.0, "sum", False),
    (109, 5, 1000, 1000, "f32", 1.0, 1.5, "mean", True),
]


def test_noalloc_matches_workspace_entry_point(fl):
    for seed, BT, V, ld, dt, beta, T, red, in_place in SEQUENCE:
        print(f"noalloc case seed={seed} BT={BT} V={V} ld={ld} {dt} beta={beta} T={T} {red} "
              f"in_place={in_place}", flush=True)
        zs_np, zt_np = _logits(seed, BT, V, dt, ld)
        zs_a, zt = to_device(zs_np, dt), to_device(zt_np, dt)
        zs_b = zs_a.clone()
        ref_loss, ref_grad = _call_workspace(fl, zs_a, zt, beta, T, red, V, ld, in_place)
        got_loss, got_grad = _call_noalloc(fl, zs_b, zt, beta, T, red, V, ld, in_place)
        torch.cuda.synchronize()
        assert torch.equal(got_loss, ref_loss), f"seed {seed}: loss differs"
        assert torch.equal(got_grad[:, :V], ref_grad[:, :V]), f"seed {seed}: gradient differs"
        # And the oracle, at the parity bar, for the small cases.
        if BT * V <= 4_000_000:
            ref = oracle.generalized_jsd(workloads.to_f64(zs_np[:, :V], dt),
                                         workloads.to_f64(zt_np[:, :V], dt), beta, T, red)
            assert_loss_close(from_device(got_loss) if red == "none" else float(got_loss[0]),
                              ref[0], TOL[dt])
            assert_tensor_close(from_device(got_grad[:, :V]), ref[1], TOL[dt], "grad_logits")


def test_noalloc_rejects_oversized_shape(fl):
    lib = fl.load_library()
    BT, V = 400_000, 1000
    need = fl.fljsd_generalized_jsd_workspace_size(BT, V, fl.BF16)
    assert need > fl.NOALLOC_SCRATCH_BYTES
    rc = lib.fljsd_generalized_jsd_noalloc(ctypes.c_void_p(16), ctypes.c_void_p(16), BT, V, V,
                                           fl.BF16, 0.5, 1.0, 0, ctypes.c_void_p(16), None, None)
    assert rc == -3
    assert b"scratch" in lib.fljsd_last_error()
