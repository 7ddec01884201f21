"""The C ABI on the CPU: the library loads, exports every declared symbol, its
pure-host planning functions compute what the header promises, and every
invalid argument is rejected with its status code before any device work.

Every call here carries at least one invalid argument (or is a pure host
function), so no kernel can be reached even when a GPU is present.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fljsd.h")
LIB = os.path.join(ROOT, "lm_head_distillation_amd", "libfljsd.so")

OK, EINVAL, EDTYPE, EWORKSPACE, EALIGN, EHIP, EDEVICE = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
FAKE = 0x10000  # a 16-byte aligned address; never dereferenced in these tests


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:int|size_t|const char\*)\s+(fljsd_\w+)\s*\(", text, re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libfljsd.so is not built; run `python -m lm_head_distillation_amd.build`")
    from lm_head_distillation_amd import fljsd
    return fljsd.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fljsd_forward_backward", "fljsd_forward_backward_ex", "fljsd_generalized_jsd",
              "fljsd_jsd_logprob", "fljsd_tvd", "fljsd_flce_forward_backward",
              "fljsd_flce_workspace_size", "fljsd_flce_plan_num_chunks", "fljsd_workspace_size",
              "fljsd_generalized_jsd_workspace_size", "fljsd_plan_num_chunks", "fljsd_strerror",
              "fljsd_last_error", "fljsd_profile_enable", "fljsd_profile_read",
              "fljsd_generalized_jsd_noalloc", "fljsd_flce_forward_backward_ex"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fljsd_\w+)", out))
    for n in declared_functions():
        assert n in exported, f"{n} declared but not exported"
        getattr(lib, n)
    # Nothing else with the prefix leaks out.
    assert exported == set(declared_functions())


def test_header_compiles_as_c():
    src = ('#include "fljsd.h"\n'
           'int (*fb)(const void*, const void*, const void*, const void*, int64_t, int64_t, int64_t,'
           ' int64_t, int, float, float, int, int, float*, void*, void*, void*, size_t, void*)'
           ' = fljsd_forward_backward;\n'
           'int (*fbx)(const void*, const void*, const void*, const void*, int64_t, int64_t, int64_t,'
           ' int64_t, int, float, float, int, int, float*, void*, void*, int, unsigned, void*, size_t,'
           ' void*) = fljsd_forward_backward_ex;\n'
           'int main(void){return (fb == 0 || fbx == 0) && FLJSD_KCLASS_COUNT == 12 '
           '&& FLJSD_ACCUMULATE_GRAD_W == 1u;}\n')
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", "-",
                          "-I", os.path.join(ROOT, "include")], input=src, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_strerror_and_last_error(lib):
    for code in (OK, EINVAL, EDTYPE, EWORKSPACE, EALIGN, EHIP, EDEVICE):
        assert lib.fljsd_strerror(code)
    assert lib.fljsd_strerror(12345) == b"unknown status code"


# ---- pure host planning ------------------------------------------------------------------

def cdiv(a, b):
    return -(-a // b)


def test_policy_ignores_the_w_transposed_region(lib):
    # 8192 x 4096 x 128256 tiles evenly: W_s^T (V * H_s * 2 bytes) is counted
    # in the workspace size but never makes the policy pick more chunks.
    BT, H, V = 8192, 4096, 128256
    wst = a256(V * H * 2)
    one = lib.fljsd_workspace_size(BT, H, H, V, BF16, 1)
    assert lib.fljsd_plan_num_chunks(BT, H, H, V, BF16, one) == 1
    assert lib.fljsd_plan_num_chunks(BT, H, H, V, BF16, one - wst) == 1
    assert lib.fljsd_plan_num_chunks(BT, H, H, V, BF16, one - wst - 1) == 2
    # Chunks of fewer than 512 rows take no W_s^T region.
    small = lib.fljsd_workspace_size(BT, H, H, V, BF16, 64)        # 128-row chunks
    assert lib.fljsd_plan_num_chunks(BT, H, H, V, BF16, small) == 64
    assert small < wst


def a256(x):
    return (x + 255) // 256 * 256


def test_workspace_size_accounts_for_each_buffer(lib):
    BT, H, V = 1000, 64, 1003
    ldz = cdiv(V, 8) * 8
    for dtype, es in ((F32, 4), (BF16, 2)):
        for nc in (1, 3, 1000):
            C = cdiv(BT, nc)
            got = lib.fljsd_workspace_size(BT, H, H, V, dtype, nc)
            logits = 2 * a256(C * ldz * es)
            # logits chunks + per-row loss + (stats, partial sums) + optional split-K
            # (+ bf16: dZ^T may need more than the teacher chunk, and X_s^T)
            assert got >= logits + a256(BT * 4) + a256(C * 16) + a256(C * 8)
            if dtype == BF16:
                ldt = cdiv(C, 8) * 8
                assert got >= (2 * a256(C * ldz * es) + a256(V * ldt * es) + a256(H * ldt * es)
                               + a256(2 * C * cdiv(V, 256) * 8))
            assert got <= logits + a256(BT * 4) + 64 * (a256(C * 16) + a256(C * 8)) + 4096 * C * H * 4 + 4096


def test_workspace_size_rejects_bad_arguments(lib):
    assert lib.fljsd_workspace_size(0, 64, 64, 10, BF16, 1) == 0
    assert lib.fljsd_workspace_size(8, 64, 64, 10, BF16, 0) == 0
    assert lib.fljsd_workspace_size(8, 64, 64, 10, 7, 1) == 0
    assert lib.fljsd_generalized_jsd_workspace_size(8, 0, BF16) == 0
    assert lib.fljsd_generalized_jsd_workspace_size(8, 100, BF16) >= 8 * 4


def test_large_shapes_workspace(lib):
    # 8192 x 4096 x 128256 bf16 in one chunk: both logits chunks dominate; the
    # transposed X_s chunk for the grad_W product adds C * H_s * 2 bytes, and
    # (V a multiple of 256, H_s of 64) W_s^T for the grad_input product
    # V * H_s * 2.
    one = lib.fljsd_workspace_size(8192, 4096, 4096, 128256, BF16, 1)
    xt = 8192 * 4096 * 2                   # X_s^T
    dzt = 128256 * 8192 * 2                # dZ^T, written by the gradient pass
    wst = 4096 * 128256 * 2                # W_s^T, written by the first logits product
    spart = 2 * 8192 * 501 * 8             # the logits GEMMs' row-statistic partials
    base = 2 * 8192 * 128256 * 2 + xt + dzt + wst + spart
    assert base <= one < base + 64 * 2**20
    eight = lib.fljsd_workspace_size(8192, 4096, 4096, 128256, BF16, 8)
    assert eight < one / 3
    # A vocabulary that does not tile by 256 takes no W_s^T region.
    odd = lib.fljsd_workspace_size(8192, 4096, 4096, 128256 + 8, BF16, 1)
    assert odd < one - wst + 64 * 2**20


def test_policy_smallest_count_that_fits(lib):
    BT, H, V = 8192, 4096, 4096 * 31 + 1
    sizes = {nc: lib.fljsd_workspace_size(BT, H, H, V, BF16, nc) for nc in (1, 2, 3, 8)}
    assert lib.fljsd_plan_num_chunks(BT, H, H, V, BF16, sizes[1]) == 1
    assert lib.fljsd_plan_num_chunks(BT, H, H, V, BF16, 10**15) == 1
    assert lib.fljsd_plan_num_chunks(BT, H, H, V, BF16, sizes[1] - 1) == 2
    nc = lib.fljsd_plan_num_chunks(BT, H, H, V, BF16, sizes[3])
    assert nc <= 3 and lib.fljsd_workspace_size(BT, H, H, V, BF16, nc) <= sizes[3]
    assert lib.fljsd_workspace_size(BT, H, H, V, BF16, nc - 1) > sizes[3] if nc > 1 else True
    assert lib.fljsd_plan_num_chunks(BT, H, H, V, BF16, 1000) == EWORKSPACE
    assert lib.fljsd_plan_num_chunks(0, H, H, V, BF16, 10**12) == EINVAL
    assert lib.fljsd_plan_num_chunks(BT, H, H, V, 5, 10**12) == EDTYPE


# ---- argument checks before any device work --------------------------------------------

# Valid arguments of each entry point (fake, never dereferenced pointers).
FB_ARGS = dict(X_s=FAKE, W_s=FAKE, X_t=FAKE, W_t=FAKE, BT=8, H_s=64, H_t=64, V=512, dtype=BF16,
             beta=0.5, T=1.0, reduction=0, nc=1, loss=FAKE, gX=FAKE, gW=FAKE, ws=FAKE,
             ws_bytes=1 << 30, stream=None)
FBX_ARGS = dict(X_s=FAKE, W_s=FAKE, X_t=FAKE, W_t=FAKE, BT=8, H_s=64, H_t=64, V=512, dtype=BF16,
             beta=0.5, T=1.0, reduction=0, nc=1, loss=FAKE, gX=FAKE, gW=FAKE, gw_dtype=BF16,
             flags=0, ws=FAKE, ws_bytes=1 << 30, stream=None)
JSD_ARGS = dict(zs=FAKE, zt=FAKE, BT=8, V=512, ld=512, dtype=BF16, beta=0.5, T=1.0, reduction=0,
             loss=FAKE, grad=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None)
NOALLOC_ARGS = dict(zs=FAKE, zt=FAKE, BT=8, V=512, ld=512, dtype=BF16, beta=0.5, T=1.0, reduction=0,
             loss=FAKE, grad=FAKE, stream=None)
ELEM_ARGS = dict(a=FAKE, b=FAKE, BT=8, V=512, ld=512, dtype=BF16, beta=0.5, reduction=0,
             loss=FAKE, grad=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None)
FLCE_ARGS = dict(X=FAKE, W=FAKE, labels=FAKE, BT=8, H=64, V=512, dtype=BF16, ignore=-100, eps=0.0,
             reduction=2, nc=1, loss=FAKE, gX=FAKE, gW=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None)

# Invalid-argument cases: (overrides of a valid call, status code). The host-only
# sanitizer test runs the same cases through the checks built under ASan/UBSan.
FB_CASES = [
    (dict(X_s=None), EINVAL), (dict(W_t=None), EINVAL), (dict(loss=None), EINVAL),
    (dict(BT=0), EINVAL), (dict(V=-3), EINVAL), (dict(H_t=0), EINVAL),
    (dict(beta=1.5), EINVAL), (dict(beta=-0.1), EINVAL), (dict(beta=float("nan")), EINVAL),
    (dict(T=0.0), EINVAL), (dict(T=-1.0), EINVAL), (dict(T=float("inf")), EINVAL),
    (dict(T=float("nan")), EINVAL), (dict(nc=-1), EINVAL),
    (dict(dtype=2), EDTYPE), (dict(reduction=4), EDTYPE), (dict(reduction=-1), EDTYPE),
    (dict(X_s=FAKE + 2), EALIGN), (dict(gW=FAKE + 8), EALIGN), (dict(ws=FAKE + 4), EALIGN),
    (dict(H_s=60), EALIGN), (dict(dtype=F32, H_t=66), EALIGN),
    (dict(ws_bytes=100), EWORKSPACE), (dict(nc=0, ws_bytes=100), EWORKSPACE),
    (dict(ws=None), EINVAL),
]

FBX_CASES = [
    (dict(gw_dtype=2), EDTYPE), (dict(gw_dtype=-1), EDTYPE),
    (dict(dtype=F32, gw_dtype=BF16), EDTYPE),
    (dict(flags=4), EINVAL), (dict(flags=0x80000001), EINVAL), (dict(flags=3, X_s=None), EINVAL),
    (dict(gw_dtype=F32, X_s=None), EINVAL), (dict(gw_dtype=F32, flags=1, ws_bytes=100), EWORKSPACE),
    (dict(gw_dtype=F32, gW=FAKE + 8), EALIGN),
]

JSD_CASES = [
    (dict(zs=None), EINVAL), (dict(loss=None), EINVAL), (dict(BT=0), EINVAL),
    (dict(V=0), EINVAL), (dict(ld=511), EINVAL), (dict(beta=2.0), EINVAL), (dict(T=0.0), EINVAL),
    (dict(dtype=9), EDTYPE), (dict(reduction=7), EDTYPE), (dict(zt=FAKE + 1), EALIGN),
    (dict(grad=FAKE + 2), EALIGN), (dict(ws_bytes=8), EWORKSPACE), (dict(ws=None), EINVAL),
]

NOALLOC_CASES = [
    (dict(zs=None), EINVAL), (dict(loss=None), EINVAL), (dict(BT=0), EINVAL),
    (dict(V=0), EINVAL), (dict(ld=511), EINVAL), (dict(beta=2.0), EINVAL), (dict(T=0.0), EINVAL),
    (dict(dtype=9), EDTYPE), (dict(reduction=7), EDTYPE), (dict(zt=FAKE + 1), EALIGN),
    (dict(grad=FAKE + 2), EALIGN),
    # Past the 8 MiB scratch array: 400,000 rows need 19.2 MB of row statistics.
    (dict(BT=400_000, V=1000, ld=1000), EWORKSPACE),
]

ELEM_CASES = [
    (dict(a=None), EINVAL), (dict(b=None), EINVAL), (dict(loss=None), EINVAL), (dict(BT=0), EINVAL),
    (dict(V=-1), EINVAL), (dict(ld=100), EINVAL), (dict(dtype=3), EDTYPE),
    (dict(reduction=9), EDTYPE), (dict(b=FAKE + 2), EALIGN), (dict(grad=FAKE + 4), EALIGN),
    (dict(ws_bytes=8), EWORKSPACE), (dict(ws=None), EINVAL),
]

FLCE_CASES = [
    (dict(X=None), EINVAL), (dict(labels=None), EINVAL), (dict(loss=None), EINVAL),
    (dict(BT=0), EINVAL), (dict(H=-1), EINVAL), (dict(V=0), EINVAL), (dict(eps=-0.1), EINVAL),
    (dict(eps=1.5), EINVAL), (dict(eps=float("nan")), EINVAL), (dict(nc=-2), EINVAL),
    (dict(dtype=5), EDTYPE), (dict(reduction=4), EDTYPE), (dict(X=FAKE + 8), EALIGN),
    (dict(labels=FAKE + 4), EALIGN), (dict(gW=FAKE + 2), EALIGN), (dict(H=60), EALIGN),
    (dict(ws_bytes=64), EWORKSPACE), (dict(nc=0, ws_bytes=64), EWORKSPACE), (dict(ws=None), EINVAL),
]


def fb(lib, **over):
    """A call to fljsd_forward_backward with fake pointers; callers always
    override at least one argument to make it invalid."""
    a = dict(FB_ARGS)
    a.update(over)
    return lib.fljsd_forward_backward(a["X_s"], a["W_s"], a["X_t"], a["W_t"], a["BT"], a["H_s"],
                                      a["H_t"], a["V"], a["dtype"], a["beta"], a["T"],
                                      a["reduction"], a["nc"], a["loss"], a["gX"], a["gW"], a["ws"],
                                      a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", FB_CASES)
def test_forward_backward_rejects(lib, over, code):
    assert fb(lib, **over) == code
    assert lib.fljsd_last_error()


def fbx(lib, **over):
    """fljsd_forward_backward_ex with fake pointers; always at least one
    invalid argument."""
    a = dict(FBX_ARGS)
    a.update(over)
    return lib.fljsd_forward_backward_ex(a["X_s"], a["W_s"], a["X_t"], a["W_t"], a["BT"], a["H_s"],
                                         a["H_t"], a["V"], a["dtype"], a["beta"], a["T"],
                                         a["reduction"], a["nc"], a["loss"], a["gX"], a["gW"],
                                         a["gw_dtype"], a["flags"], a["ws"], a["ws_bytes"],
                                         a["stream"])


@pytest.mark.parametrize("over,code", FBX_CASES)
def test_forward_backward_ex_rejects(lib, over, code):
    assert fbx(lib, **over) == code
    assert lib.fljsd_last_error()


def jsd(lib, **over):
    a = dict(JSD_ARGS)
    a.update(over)
    return lib.fljsd_generalized_jsd(a["zs"], a["zt"], a["BT"], a["V"], a["ld"], a["dtype"],
                                     a["beta"], a["T"], a["reduction"], a["loss"], a["grad"],
                                     a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", JSD_CASES)
def test_generalized_jsd_rejects(lib, over, code):
    assert jsd(lib, **over) == code


def jsd_noalloc(lib, **over):
    a = dict(NOALLOC_ARGS)
    a.update(over)
    return lib.fljsd_generalized_jsd_noalloc(a["zs"], a["zt"], a["BT"], a["V"], a["ld"], a["dtype"],
                                             a["beta"], a["T"], a["reduction"], a["loss"], a["grad"],
                                             a["stream"])


@pytest.mark.parametrize("over,code", NOALLOC_CASES)
def test_generalized_jsd_noalloc_rejects(lib, over, code):
    """The no-allocation entry point checks everything, its scratch bound
    included, before any HIP call (so these run without a GPU)."""
    assert jsd_noalloc(lib, **over) == code
    assert lib.fljsd_last_error()


def test_noalloc_scratch_bound_matches_header(lib):
    text = open(HEADER).read()
    m = re.search(r"#define FLJSD_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == 8 << 20
    from lm_head_distillation_amd import fljsd
    assert fljsd.NOALLOC_SCRATCH_BYTES == 8 << 20
    # The largest batch of a bf16 / fp32 row stride that fits, and the next one out.
    assert lib.fljsd_generalized_jsd_workspace_size(174_000, 1000, BF16) <= 8 << 20
    assert jsd_noalloc(lib, BT=175_000, V=1000, ld=1000) == EWORKSPACE


def elem(lib, fn, **over):
    a = dict(ELEM_ARGS)
    a.update(over)
    if fn == "logprob":
        return lib.fljsd_jsd_logprob(a["a"], a["b"], a["BT"], a["V"], a["ld"], a["dtype"], a["beta"],
                                     a["reduction"], a["loss"], a["grad"], a["ws"], a["ws_bytes"],
                                     a["stream"])
    return lib.fljsd_tvd(a["a"], a["b"], a["BT"], a["V"], a["ld"], a["dtype"], a["reduction"],
                         a["loss"], a["grad"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("fn", ["logprob", "tvd"])
@pytest.mark.parametrize("over,code", ELEM_CASES)
def test_elementwise_losses_reject(lib, fn, over, code):
    assert elem(lib, fn, **over) == code
    assert lib.fljsd_last_error()


def flce(lib, **over):
    a = dict(FLCE_ARGS)
    a.update(over)
    return lib.fljsd_flce_forward_backward(a["X"], a["W"], a["labels"], a["BT"], a["H"], a["V"],
                                           a["dtype"], a["ignore"], a["eps"], a["reduction"], a["nc"],
                                           a["loss"], a["gX"], a["gW"], a["ws"], a["ws_bytes"],
                                           a["stream"])


@pytest.mark.parametrize("over,code", FLCE_CASES)
def test_flce_rejects(lib, over, code):
    assert flce(lib, **over) == code
    assert lib.fljsd_last_error()


FLCEX_ARGS = dict(FLCE_ARGS, gw_dtype=BF16, flags=0)
FLCEX_CASES = [
    (dict(gw_dtype=2), EDTYPE), (dict(dtype=F32, gw_dtype=BF16), EDTYPE), (dict(flags=2), EINVAL),
    (dict(flags=0x80000001), EINVAL), (dict(gw_dtype=F32, X=None), EINVAL),
    (dict(gw_dtype=F32, flags=1, ws_bytes=64), EWORKSPACE), (dict(gw_dtype=F32, gW=FAKE + 8), EALIGN),
]


def flcex(lib, **over):
    a = dict(FLCEX_ARGS)
    a.update(over)
    return lib.fljsd_flce_forward_backward_ex(a["X"], a["W"], a["labels"], a["BT"], a["H"], a["V"],
                                              a["dtype"], a["ignore"], a["eps"], a["reduction"],
                                              a["nc"], a["loss"], a["gX"], a["gW"], a["gw_dtype"],
                                              a["flags"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", FLCE_CASES + FLCEX_CASES)
def test_flce_ex_rejects(lib, over, code):
    assert flcex(lib, **over) == code
    assert lib.fljsd_last_error()


def test_flce_workspace_and_policy(lib):
    BT, H, V = 8192, 4096, 128256
    one = lib.fljsd_flce_workspace_size(BT, H, V, BF16, 1)
    # logits chunk + dZ^T + X^T dominate, plus W^T (V * H * 2) for grad_X
    wt = a256(V * H * 2)
    base = BT * V * 2 * 2 + BT * H * 2 + wt
    assert base <= one < base + 64 * 2**20
    assert lib.fljsd_flce_workspace_size(BT, H, V, 7, 1) == 0
    assert lib.fljsd_flce_workspace_size(BT, H, V, BF16, 0) == 0
    assert lib.fljsd_flce_plan_num_chunks(BT, H, V, BF16, one) == 1
    assert lib.fljsd_flce_plan_num_chunks(BT, H, V, BF16, one - wt) == 1   # W^T costs no chunk
    nc = lib.fljsd_flce_plan_num_chunks(BT, H, V, BF16, one // 3)
    assert nc > 1 and lib.fljsd_flce_workspace_size(BT, H, V, BF16, nc) - wt <= one // 3
    # No region at 4096 rows.
    assert (lib.fljsd_flce_workspace_size(4104, H, V, BF16, 1)
            - lib.fljsd_flce_workspace_size(4096, H, V, BF16, 1)) >= wt
    assert lib.fljsd_flce_plan_num_chunks(BT, H, V, BF16, 100) == EWORKSPACE


def test_logprob_rejects_beta(lib):
    assert elem(lib, "logprob", beta=1.5) == EINVAL
    assert elem(lib, "logprob", beta=float("nan")) == EINVAL


def test_profile_interface_without_work(lib):
    n = 10
    ms = (ctypes.c_double * n)()
    launches = (ctypes.c_int64 * n)()
    assert lib.fljsd_profile_enable(1) == OK
    assert lib.fljsd_profile_read(ms, launches, None, None, n) == OK
    assert all(x == 0 for x in launches)
    assert lib.fljsd_profile_enable(0) == OK


# ---- the Python binding ----------------------------------------------------------------

def test_binding_rejects_host_tensors(lib):
    import torch
    from lm_head_distillation_amd import fljsd
    x = torch.zeros(4, 64)
    w = torch.zeros(10, 64)
    with pytest.raises(ValueError):
        fljsd.fljsd_forward_backward(x, w, x, w, 0.5, 1.0)
    with pytest.raises(ValueError):
        fljsd.fljsd_generalized_jsd(w, w, 0.5, 1.0)


def test_binding_checks_caller_outputs():
    """Outputs the caller passes in must be what the kernels write (dtype,
    element count, layout, device), or the binding refuses them before the
    library sees a pointer: a bf16 tensor where fp32 grad_W is asked for, a
    one-element loss for reduction "none", a strided gradient."""
    import torch
    from lm_head_distillation_amd import fljsd
    dev = torch.device("cpu")
    with pytest.raises(ValueError, match="float32"):
        fljsd._check_out(torch.empty(16, 8, dtype=torch.bfloat16), torch.float32, 128, dev, "grad_W_s")
    with pytest.raises(ValueError, match="hold 8 elements"):
        fljsd._check_out(torch.empty(1, dtype=torch.float32), torch.float32, 8, dev, "loss")
    with pytest.raises(ValueError, match="contiguous"):
        fljsd._check_out(torch.empty(8, 16, dtype=torch.float32).t(), torch.float32, 128, dev, "grad")
    with pytest.raises(ValueError, match="live on"):
        fljsd._check_out(torch.empty(4, dtype=torch.float32), torch.float32, 4, dev, "loss")
    with pytest.raises(ValueError, match="contiguous tensor"):
        fljsd._check_workspace(torch.empty(64, dtype=torch.uint8), dev)


def test_binding_fails_loudly_without_library(tmp_path):
    code = ("import lm_head_distillation_amd.fljsd as f; f._LIB_PATH = '/nonexistent/libfljsd.so'\n"
            "try:\n    f.load_library()\nexcept ImportError as e:\n    print('IMPORTERROR', e)\n")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "IMPORTERROR" in res.stdout, res.stderr


def test_product_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "lm_head_distillation_amd")
    for dirpath, _dirs, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, re.M), f
                assert "oracle/" not in text, f
