"""Pins that tie the CPU oracle to facts outside itself.

Each pin takes the oracle module as its argument and raises AssertionError
when the module disagrees with the pages, a closed form, a library routine,
finite differences or an invariant. The same pins run against copies of the
oracle with planted mistakes, to show that a plausible slip fails one of them.
No pin retypes an oracle formula.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special as sps

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BETAS = (0.0, 0.1, 0.5, 0.9, 1.0)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _logits(seed, R, V, scale=1.0):
    return _rng(seed).standard_normal((R, V)) * scale


def _h(beta):
    """Binary entropy in nats: the value of JSD_beta at disjoint supports."""
    return -beta * math.log(beta) - (1 - beta) * math.log(1 - beta)


def pin_log_softmax_library(o):
    """log_softmax equals scipy's routine, also at large offsets; shift invariant."""
    a = _logits(1, 5, 37, 3.0) + 800.0      # exp(800) overflows without a max shift
    ref = sps.log_softmax(a, axis=-1)
    got = o.log_softmax(a)
    assert np.all(np.isfinite(got)), "log_softmax overflowed"
    assert np.allclose(got, ref, rtol=0, atol=1e-12), "log_softmax != scipy"
    assert np.allclose(o.log_softmax(a - 1234.5), got, rtol=0, atol=1e-12), "not shift invariant"


def pin_batchmean_scale_golden(o):
    """PR #1374's tie table fixes batchmean = 1/rows."""
    g = _golden("tvd_tie_batchmean.json")
    rows, vocab = g["rows"], g["vocab"]
    assert rows * vocab == g["elements"]
    page_scale = g["gradient_at_tie_before_fix"] / g["per_element_slope_before_fix"]
    assert abs(o.reduction_scale("batchmean", rows, vocab) - page_scale) < 1e-15
    assert o.reduction_scale("sum", rows, vocab) == 1.0


def pin_self_distillation_exact_zero(o):
    """Student == teacher: loss exactly 0 and every gradient exactly 0 (PR #1374)."""
    z = _logits(2, 6, 50, 2.0)
    for beta in BETAS:
        for T in (1.0, 2.0):
            for red in ("batchmean", "sum", "mean"):
                loss, grad = o.generalized_jsd(z, z.copy(), beta, T, red)
                assert loss == 0.0, f"self loss {loss} at beta={beta}"
                assert np.all(grad == 0.0), f"self grad nonzero at beta={beta}, T={T}"
    X = _rng(3).standard_normal((5, 7))
    W = _rng(4).standard_normal((11, 7)) * 0.3
    for beta in BETAS:
        loss, gX, gW = o.fused_linear_jsd(X, W, X.copy(), W.copy(), beta, 1.5, "batchmean", block_rows=2)
        assert loss == 0.0 and np.all(gX == 0.0) and np.all(gW == 0.0), f"fused self beta={beta}"


def pin_disjoint_support_closed_form(o):
    """Disjoint supports give JSD_beta = h(beta) exactly (ln 2 at beta = 0.5)."""
    V = 8
    zs = np.full((2, V), -1e4)
    zt = np.full((2, V), -1e4)
    zs[0, 0] = 0.0
    zt[0, 5] = 0.0
    zs[1, :4] = 0.0      # uniform over the first half
    zt[1, 4:] = 0.0      # uniform over the second half
    for beta in (0.1, 0.5, 0.9):
        loss, _ = o.generalized_jsd(zs, zt, beta, 1.0, "none")
        assert np.allclose(loss, _h(beta), rtol=1e-12, atol=0), f"beta={beta}: {loss} vs {_h(beta)}"
    loss, _ = o.generalized_jsd(zs, zt, 0.5, 1.0, "none")
    assert np.allclose(loss, math.log(2.0), rtol=1e-12)


def pin_bounds(o):
    """0 <= JSD_beta <= h(beta) per row; JSD_0.5 <= ln 2."""
    zs = _logits(5, 40, 30, 4.0)
    zt = _logits(6, 40, 30, 4.0)
    for beta in (0.1, 0.5, 0.9):
        loss, _ = o.generalized_jsd(zs, zt, beta, 1.0, "none")
        assert np.all(loss >= 0) and np.all(loss <= _h(beta) + 1e-12), f"bounds beta={beta}"


def pin_role_swap(o):
    """Swapping student and teacher maps beta to 1-beta (symmetric at 0.5)."""
    zs = _logits(7, 4, 25, 2.0)
    zt = _logits(8, 4, 25, 2.0)
    for beta in (0.1, 0.3, 0.5):
        a, _ = o.generalized_jsd(zs, zt, beta, 1.0, "none")
        b, _ = o.generalized_jsd(zt, zs, 1.0 - beta, 1.0, "none")
        assert np.allclose(a, b, rtol=1e-12, atol=1e-15), f"role swap beta={beta}"
    a, _ = o.generalized_jsd(zs, zt, 0.5, 1.0, "sum")
    b, _ = o.generalized_jsd(zt, zs, 0.5, 1.0, "sum")
    assert abs(a - b) <= 1e-12 * abs(a)


def _kl_rows(p, q):
    return np.sum(sps.rel_entr(p, q), axis=-1)


def pin_kl_endpoints_library(o):
    """beta=0 is KL(teacher||student), beta=1 is KL(student||teacher) (PR #1352)."""
    g = _golden("beta_branches.json")
    kinds = {b["beta"]: b["kind"] for b in g["branches"]}
    zs = _logits(9, 6, 33, 2.0)
    zt = _logits(10, 6, 33, 2.0)
    for T in (1.0, 3.0):
        Q = sps.softmax(zs / T, axis=-1)
        P = sps.softmax(zt / T, axis=-1)
        assert kinds[0.0] == "forward_kl" and kinds[1.0] == "reverse_kl"
        fwd, _ = o.generalized_jsd(zs, zt, 0.0, T, "none")
        rev, _ = o.generalized_jsd(zs, zt, 1.0, T, "none")
        assert np.allclose(fwd, _kl_rows(P, Q), rtol=1e-10, atol=1e-14), "beta=0 != KL(P||Q)"
        assert np.allclose(rev, _kl_rows(Q, P), rtol=1e-10, atol=1e-14), "beta=1 != KL(Q||P)"


def pin_jsd_half_library(o):
    """beta = 1/2 is the symmetric Jensen-Shannon divergence: the square of
    scipy's Jensen-Shannon distance (natural log), per row, at two temperatures."""
    from scipy.spatial.distance import jensenshannon
    zs = _logits(41, 5, 37, 2.0)
    zt = _logits(42, 5, 37, 2.0)
    for T in (1.0, 2.0):
        Q = sps.softmax(zs / T, axis=-1)
        P = sps.softmax(zt / T, axis=-1)
        ref = jensenshannon(P, Q, axis=-1) ** 2
        got, _ = o.generalized_jsd(zs, zt, 0.5, T, "none")
        assert np.allclose(got, ref, rtol=1e-9, atol=1e-15), f"beta=0.5 != JS distance^2 (T={T})"


def pin_jsd_entropy_identity(o):
    """For every beta, JSD_beta = H(M) - beta H(P) - (1-beta) H(Q) with
    M = beta P + (1-beta) Q (Shannon entropies from scipy.stats.entropy): the
    entropy form of the divergence, independent of the KL-sum definition."""
    from scipy.stats import entropy
    zs = _logits(43, 6, 29, 2.0)
    zt = _logits(44, 6, 29, 2.0)
    for T in (1.0, 1.7):
        Q = sps.softmax(zs / T, axis=-1)
        P = sps.softmax(zt / T, axis=-1)
        for beta in (0.1, 0.3, 0.7, 0.9):
            M = beta * P + (1.0 - beta) * Q
            ref = entropy(M, axis=-1) - beta * entropy(P, axis=-1) - (1.0 - beta) * entropy(Q, axis=-1)
            got, _ = o.generalized_jsd(zs, zt, beta, T, "none")
            assert np.allclose(got, ref, rtol=1e-9, atol=1e-14), f"entropy identity beta={beta} T={T}"


def pin_kl_limits(o):
    """JSD_b / b -> KL(P||Q) as b -> 0 and JSD_b / (1-b) -> KL(Q||P) as b -> 1."""
    zs = _logits(11, 3, 20, 1.5)
    zt = _logits(12, 3, 20, 1.5)
    Q = sps.softmax(zs, axis=-1)
    P = sps.softmax(zt, axis=-1)
    eps = 1e-7
    lo, _ = o.generalized_jsd(zs, zt, eps, 1.0, "none")
    hi, _ = o.generalized_jsd(zs, zt, 1.0 - eps, 1.0, "none")
    assert np.allclose(lo / eps, _kl_rows(P, Q), rtol=1e-5), "beta->0 limit"
    assert np.allclose(hi / eps, _kl_rows(Q, P), rtol=1e-5), "beta->1 limit"


def _fd_grad_logits(o, zs, zt, beta, T, red, h=1e-6):
    g = np.zeros_like(zs)
    for idx in np.ndindex(*zs.shape):
        zp = zs.copy()
        zm = zs.copy()
        zp[idx] += h
        zm[idx] -= h
        lp, _ = o.generalized_jsd(zp, zt, beta, T, red)
        lm, _ = o.generalized_jsd(zm, zt, beta, T, red)
        g[idx] = (lp - lm) / (2 * h)
    return g


def pin_finite_differences_logits(o):
    """Gradient w.r.t. student logits equals central differences of the loss."""
    zs = _logits(13, 3, 9, 1.5)
    zt = _logits(14, 3, 9, 1.5)
    for beta in BETAS:
        for T in (1.0, 2.0):
            for red in ("batchmean", "sum", "mean"):
                _, grad = o.generalized_jsd(zs, zt, beta, T, red)
                fd = _fd_grad_logits(o, zs, zt, beta, T, red)
                err = np.max(np.abs(grad - fd))
                assert err <= 1e-7 * max(1.0, np.max(np.abs(fd))), \
                    f"FD logits beta={beta} T={T} {red}: err {err}"


def pin_finite_differences_fused(o):
    """grad_input and grad_W equal central differences of the fused loss."""
    rng = _rng(15)
    BT, H, V = 3, 4, 7
    X_s = rng.standard_normal((BT, H))
    W_s = rng.standard_normal((V, H)) * 0.7
    X_t = rng.standard_normal((BT, H + 1))
    W_t = rng.standard_normal((V, H + 1)) * 0.7
    h = 1e-6
    for beta in (0.0, 0.5, 1.0):
        for T in (1.0, 2.0):
            _, gX, gW = o.fused_linear_jsd(X_s, W_s, X_t, W_t, beta, T, "batchmean", block_rows=2)
            for name, M, G in (("X_s", X_s, gX), ("W_s", W_s, gW)):
                fd = np.zeros_like(M)
                for idx in np.ndindex(*M.shape):
                    Mp = M.copy()
                    Mm = M.copy()
                    Mp[idx] += h
                    Mm[idx] -= h
                    if name == "X_s":
                        lp = o.fused_linear_jsd(Mp, W_s, X_t, W_t, beta, T, "batchmean")[0]
                        lm = o.fused_linear_jsd(Mm, W_s, X_t, W_t, beta, T, "batchmean")[0]
                    else:
                        lp = o.fused_linear_jsd(X_s, Mp, X_t, W_t, beta, T, "batchmean")[0]
                        lm = o.fused_linear_jsd(X_s, Mm, X_t, W_t, beta, T, "batchmean")[0]
                    fd[idx] = (lp - lm) / (2 * h)
                err = np.max(np.abs(G - fd))
                assert err <= 1e-7 * max(1.0, np.max(np.abs(fd))), \
                    f"FD {name} beta={beta} T={T}: err {err}"


def pin_temperature_identity(o):
    """loss(z, T) == loss(z/T, 1); grad(z, T) == grad(z/T, 1) / T."""
    zs = _logits(16, 4, 21, 3.0)
    zt = _logits(17, 4, 21, 3.0)
    for beta in BETAS:
        for T in (0.5, 2.0, 3.0):
            la, ga = o.generalized_jsd(zs, zt, beta, T, "batchmean")
            lb, gb = o.generalized_jsd(zs / T, zt / T, beta, 1.0, "batchmean")
            assert abs(la - lb) <= 1e-12 * max(1.0, abs(lb)), f"T loss beta={beta} T={T}"
            assert np.allclose(ga, gb / T, rtol=1e-10, atol=1e-15), f"T grad beta={beta} T={T}"


def pin_gradient_rows_sum_to_zero(o):
    """Softmax shift invariance: each row of the logit gradient sums to zero."""
    zs = _logits(18, 5, 40, 2.0)
    zt = _logits(19, 5, 40, 2.0)
    for beta in BETAS:
        _, g = o.generalized_jsd(zs, zt, beta, 1.7, "sum")
        assert np.all(np.abs(g.sum(axis=-1)) <= 1e-14 * 40), f"row sums beta={beta}"


def pin_block_invariance_and_reductions(o):
    """Row blocking changes nothing; none/sum/mean/batchmean scale consistently."""
    rng = _rng(20)
    BT, H, V = 7, 5, 13
    X_s, X_t = rng.standard_normal((BT, H)), rng.standard_normal((BT, H))
    W_s, W_t = rng.standard_normal((V, H)) * 0.5, rng.standard_normal((V, H)) * 0.5
    for beta in (0.0, 0.4, 1.0):
        ref = o.fused_linear_jsd(X_s, W_s, X_t, W_t, beta, 1.3, "batchmean", block_rows=BT)
        for br in (1, 3):
            got = o.fused_linear_jsd(X_s, W_s, X_t, W_t, beta, 1.3, "batchmean", block_rows=br)
            for a, b in zip(got, ref):
                assert np.allclose(a, b, rtol=1e-12, atol=1e-15), f"block_rows={br} beta={beta}"
        l_none, gX_none, gW_none = o.fused_linear_jsd(X_s, W_s, X_t, W_t, beta, 1.3, "none", block_rows=3)
        l_sum, gX_sum, gW_sum = o.fused_linear_jsd(X_s, W_s, X_t, W_t, beta, 1.3, "sum", block_rows=3)
        l_mean, gX_mean, _ = o.fused_linear_jsd(X_s, W_s, X_t, W_t, beta, 1.3, "mean", block_rows=3)
        assert l_none.shape == (BT,)
        assert abs(l_none.sum() - l_sum) <= 1e-12 * abs(l_sum)
        assert abs(ref[0] * BT - l_sum) <= 1e-12 * abs(l_sum)
        assert abs(l_mean * BT * V - l_sum) <= 1e-12 * abs(l_sum)
        assert np.allclose(gX_none, gX_sum, rtol=1e-13, atol=0)
        assert np.allclose(gW_none, gW_sum, rtol=1e-13, atol=0)
        assert np.allclose(gX_mean * BT * V, gX_sum, rtol=1e-12, atol=1e-15)
        rows = [0, 4, 6]
        lr, gXr = o.fused_linear_jsd_rows(X_s, W_s, X_t, W_t, rows, beta, 1.3, "batchmean")
        assert np.allclose(lr, l_none[rows], rtol=1e-12, atol=1e-15)
        assert np.allclose(gXr, ref[1][rows], rtol=1e-12, atol=1e-15)


def pin_padded_slots_exact_zero(o):
    """Slots with zero mass in both distributions get exactly zero gradient."""
    rng = _rng(21)
    BT, H, V, pad = 4, 6, 20, 5
    X_s, X_t = rng.standard_normal((BT, H)), rng.standard_normal((BT, H))
    W_s, W_t = rng.standard_normal((V, H)) * 0.5, rng.standard_normal((V, H)) * 0.5
    for X in (X_s, X_t):
        X[:, H - 1] = 1.0
    for W in (W_s, W_t):
        W[V - pad:, :] = 0.0
        W[V - pad:, H - 1] = -9984.0
    for beta in (0.5, 0.1):
        _, gX, gW = o.fused_linear_jsd(X_s, W_s, X_t, W_t, beta, 1.0, "batchmean")
        assert np.all(gW[V - pad:] == 0.0), f"padded grad_W rows beta={beta}"
        zs, zt = X_s @ W_s.T, X_t @ W_t.T
        _, g = o.generalized_jsd(zs, zt, beta, 1.0, "batchmean")
        assert np.all(g[:, V - pad:] == 0.0), f"padded logit grads beta={beta}"


# ---- the log-probability JSD and the TVD -------------------------------------------------

def pin_logprob_kl_library(o):
    """Over normalized log-probabilities, beta=0 is KL(P||Q) and beta=1 is
    KL(Q||P) (scipy's rel_entr), as in the logit path (PR #1352 Testing Done)."""
    logq = sps.log_softmax(_logits(21, 5, 29, 2.0), axis=-1)
    logp = sps.log_softmax(_logits(22, 5, 29, 2.0), axis=-1)
    Q, P = np.exp(logq), np.exp(logp)
    fwd, _ = o.jsd_logprob(logq, logp, 0.0, "none")
    rev, _ = o.jsd_logprob(logq, logp, 1.0, "none")
    assert np.allclose(fwd, _kl_rows(P, Q), rtol=1e-10, atol=1e-14), "logprob beta=0 != KL(P||Q)"
    assert np.allclose(rev, _kl_rows(Q, P), rtol=1e-10, atol=1e-14), "logprob beta=1 != KL(Q||P)"
    # beta = 1/2: the square of scipy's Jensen-Shannon distance; other betas:
    # the entropy form H(M) - beta H(P) - (1-beta) H(Q).
    from scipy.spatial.distance import jensenshannon
    from scipy.stats import entropy
    half, _ = o.jsd_logprob(logq, logp, 0.5, "none")
    assert np.allclose(half, jensenshannon(P, Q, axis=-1) ** 2, rtol=1e-9, atol=1e-15), \
        "logprob beta=0.5 != JS distance^2"
    for beta in (0.2, 0.8):
        M = beta * P + (1.0 - beta) * Q
        ref = entropy(M, axis=-1) - beta * entropy(P, axis=-1) - (1.0 - beta) * entropy(Q, axis=-1)
        got, _ = o.jsd_logprob(logq, logp, beta, "none")
        assert np.allclose(got, ref, rtol=1e-9, atol=1e-14), f"logprob entropy identity beta={beta}"


def pin_logprob_disjoint_closed_form(o):
    """Disjoint supports give h(beta) exactly; swapping roles maps beta to 1-beta."""
    logq = np.full((1, 6), -1e4)
    logp = np.full((1, 6), -1e4)
    logq[0, 1] = 0.0
    logp[0, 4] = 0.0
    for beta in (0.1, 0.5, 0.9):
        loss, _ = o.jsd_logprob(logq, logp, beta, "none")
        assert np.allclose(loss, _h(beta), rtol=1e-12, atol=0), f"logprob disjoint beta={beta}"
    a = sps.log_softmax(_logits(23, 3, 17, 2.0), axis=-1)
    b = sps.log_softmax(_logits(24, 3, 17, 2.0), axis=-1)
    for beta in (0.2, 0.5):
        x, _ = o.jsd_logprob(a, b, beta, "none")
        y, _ = o.jsd_logprob(b, a, 1.0 - beta, "none")
        assert np.allclose(x, y, rtol=1e-12, atol=1e-15), f"logprob role swap beta={beta}"


def pin_logprob_finite_differences(o):
    """grad = d loss / d logq elementwise, by central differences, for
    arbitrary (also unnormalized) log-probabilities and every reduction."""
    rng = _rng(25)
    logq = rng.standard_normal((3, 6)) - 2.0
    logp = rng.standard_normal((3, 6)) - 2.0
    h = 1e-6
    for beta in BETAS:
        for red in ("batchmean", "sum", "mean"):
            _, g = o.jsd_logprob(logq, logp, beta, red)
            fd = np.zeros_like(logq)
            for idx in np.ndindex(*logq.shape):
                xp = logq.copy()
                xm = logq.copy()
                xp[idx] += h
                xm[idx] -= h
                fd[idx] = (o.jsd_logprob(xp, logp, beta, red)[0] -
                           o.jsd_logprob(xm, logp, beta, red)[0]) / (2 * h)
            assert np.allclose(g, fd, rtol=1e-6, atol=1e-10), f"logprob fd beta={beta} {red}"


def pin_logprob_ties_and_logit_path(o):
    """Equal inputs: loss 0 and, in the generalized branch, gradient exactly 0
    (PR #1374). Over log_softmax outputs at T = 1 the loss equals the logit
    path's loss."""
    a = sps.log_softmax(_logits(26, 4, 21, 2.0), axis=-1)
    for beta in BETAS:
        loss, g = o.jsd_logprob(a, a.copy(), beta, "batchmean")
        assert loss == 0.0, f"logprob self loss beta={beta}"
        if 0.0 < beta < 1.0:
            assert np.all(g == 0.0), f"logprob self grad beta={beta}"
    zs = _logits(27, 4, 21, 2.0)
    zt = _logits(28, 4, 21, 2.0)
    for beta in BETAS:
        x, _ = o.jsd_logprob(sps.log_softmax(zs, axis=-1), sps.log_softmax(zt, axis=-1), beta, "sum")
        y, _ = o.generalized_jsd(zs, zt, beta, 1.0, "sum")
        assert abs(x - y) <= 1e-12 * max(1.0, abs(y)), f"logprob vs logit path beta={beta}"


def pin_tvd_golden_ties(o):
    """PR #1374's tie table at (8, 512) fp32, batchmean: with p == q everywhere
    every gradient element is 0.0 (after the fix); the page's pre-fix value
    -0.0625 is the p < q slope, which untied elements with p < q still get."""
    g = _golden("tvd_tie_batchmean.json")
    R, V = g["rows"], g["vocab"]
    p = sps.softmax(_logits(29, R, V), axis=-1)
    loss, grad = o.tvd(p, p.copy(), "batchmean")
    assert loss == 0.0
    assert np.count_nonzero(grad) == 0 and grad.size == g["elements"]
    assert np.all(grad == g["gradient_at_tie_after_fix"])
    q = p.copy()
    q[:, ::2] *= 1.5          # p < q on even columns, p > q on odd ones after renormalizing
    q /= q.sum(axis=-1, keepdims=True)
    _, grad = o.tvd(p, q, "batchmean")
    assert np.all(grad[p < q] == g["gradient_at_tie_before_fix"])
    assert np.all(grad[p > q] == -g["gradient_at_tie_before_fix"])


def pin_tvd_library_and_closed_form(o):
    """Row TVD is half the L1 distance (numpy's norm); disjoint rows give 1;
    reductions scale the total as batchmean 1/rows, mean 1/(rows V), sum 1."""
    p = sps.softmax(_logits(30, 5, 23), axis=-1)
    q = sps.softmax(_logits(31, 5, 23), axis=-1)
    elem, _ = o.tvd(p, q, "none")
    assert elem.shape == p.shape
    rows = np.array([0.5 * np.linalg.norm(p[r] - q[r], ord=1) for r in range(5)])
    assert np.allclose(elem.sum(axis=-1), rows, rtol=1e-14, atol=0)
    tot = rows.sum()
    assert abs(o.tvd(p, q, "sum")[0] - tot) <= 1e-14
    assert abs(o.tvd(p, q, "batchmean")[0] - tot / 5) <= 1e-14
    assert abs(o.tvd(p, q, "mean")[0] - tot / (5 * 23)) <= 1e-15
    a = np.zeros((2, 4))
    b = np.zeros((2, 4))
    a[0, 0] = b[0, 3] = 1.0
    a[1, :2] = b[1, 2:] = 0.5
    assert np.allclose(o.tvd(a, b, "none")[0].sum(axis=-1), 1.0, rtol=0, atol=1e-15)


def pin_tvd_finite_differences(o):
    """Away from ties, grad = d loss / d p by central differences."""
    rng = _rng(32)
    p = rng.random((3, 7))
    q = rng.random((3, 7))
    h = 1e-7
    for red in ("batchmean", "sum", "mean"):
        _, g = o.tvd(p, q, red)
        for idx in np.ndindex(*p.shape):
            pp = p.copy()
            pm = p.copy()
            pp[idx] += h
            pm[idx] -= h
            fd = (o.tvd(pp, q, red)[0] - o.tvd(pm, q, red)[0]) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-7, f"tvd fd {red} {idx}"


# ---- fused-linear cross-entropy ------------------------------------------------------------

def _ce_case(seed, R=9, V=13, H=6, ignore=-100):
    rng = _rng(seed)
    X = rng.standard_normal((R, H))
    W = rng.standard_normal((V, H)) * 0.5
    y = rng.integers(0, V, size=R)
    y[1] = ignore
    y[-1] = ignore
    return X, W, y


def pin_ce_torch_library(o):
    """Row losses and every reduction equal torch's fp64 CPU cross_entropy,
    with ignored labels and label smoothing."""
    import torch
    import torch.nn.functional as F
    X, W, y = _ce_case(41)
    Z = X @ W.T
    for eps in (0.0, 0.1, 0.7):
        rows, _, valid = o.cross_entropy_rows(Z, y, -100, eps)
        ref = F.cross_entropy(torch.from_numpy(Z), torch.from_numpy(y), ignore_index=-100,
                              label_smoothing=eps, reduction="none").numpy()
        assert np.allclose(rows, ref, rtol=1e-12, atol=1e-14), f"rows eps={eps}"
        for red in ("mean", "sum", "none"):
            loss, _, _ = o.fused_linear_cross_entropy(X, W, y, -100, eps, red, block_rows=4)
            ref = F.cross_entropy(torch.from_numpy(Z), torch.from_numpy(y), ignore_index=-100,
                                  label_smoothing=eps, reduction=red).numpy()
            assert np.allclose(loss, ref, rtol=1e-12, atol=1e-14), f"{red} eps={eps}"
        assert valid.sum() == len(y) - 2


def pin_ce_autograd(o):
    """grad_X and grad_W equal torch autograd of linear + cross_entropy (fp64)."""
    import torch
    import torch.nn.functional as F
    X, W, y = _ce_case(42)
    for eps in (0.0, 0.2):
        for red in ("mean", "sum"):
            tX = torch.from_numpy(X.copy()).requires_grad_(True)
            tW = torch.from_numpy(W.copy()).requires_grad_(True)
            F.cross_entropy(tX @ tW.T, torch.from_numpy(y), ignore_index=-100, label_smoothing=eps,
                            reduction=red).backward()
            _, gX, gW = o.fused_linear_cross_entropy(X, W, y, -100, eps, red, block_rows=3)
            assert np.allclose(gX, tX.grad.numpy(), rtol=1e-11, atol=1e-14), f"gX {red} {eps}"
            assert np.allclose(gW, tW.grad.numpy(), rtol=1e-11, atol=1e-14), f"gW {red} {eps}"


def pin_ce_finite_differences(o):
    """Gradients by central differences of the summed loss on a tiny case."""
    X, W, y = _ce_case(43, R=4, V=5, H=3, ignore=7)
    h = 1e-6
    _, gX, gW = o.fused_linear_cross_entropy(X, W, y, 7, 0.3, "sum", block_rows=2)
    for A, G in ((X, gX), (W, gW)):
        for idx in np.ndindex(*A.shape):
            Ap = A.copy()
            Am = A.copy()
            Ap[idx] += h
            Am[idx] -= h
            args_p = (Ap, W) if A is X else (X, Ap)
            args_m = (Am, W) if A is X else (X, Am)
            fd = (o.fused_linear_cross_entropy(*args_p, y, 7, 0.3, "sum")[0] -
                  o.fused_linear_cross_entropy(*args_m, y, 7, 0.3, "sum")[0]) / (2 * h)
            assert abs(fd - G[idx]) <= 1e-7 * max(1.0, abs(fd)), f"fd {idx}"


def pin_ce_closed_forms(o):
    """Uniform logits give log V per counted row; each row of dz sums to 0;
    with no counted row the sum is 0, the mean nan, and the gradients 0."""
    V = 11
    Z = np.zeros((3, V))
    rows, dz, _ = o.cross_entropy_rows(Z, np.array([0, 4, 10]), -100, 0.25)
    assert np.allclose(rows, math.log(V), rtol=1e-14)
    rows, dz, _ = o.cross_entropy_rows(_logits(44, 5, V, 3.0), np.array([1, 2, 3, 4, -100]), -100, 0.1)
    assert np.allclose(dz.sum(axis=-1), 0.0, atol=1e-15)
    X, W, _ = _ce_case(45)
    y = np.full(X.shape[0], -100)
    loss, gX, gW = o.fused_linear_cross_entropy(X, W, y, -100, 0.0, "sum")
    assert loss == 0.0 and np.all(gX == 0.0) and np.all(gW == 0.0)
    loss, gX, gW = o.fused_linear_cross_entropy(X, W, y, -100, 0.0, "mean")
    assert math.isnan(loss) and np.all(gX == 0.0) and np.all(gW == 0.0)


def pin_ce_blocks_and_batchmean(o):
    """Results do not depend on the row blocking; batchmean divides by all rows."""
    X, W, y = _ce_case(46, R=10)
    a = o.fused_linear_cross_entropy(X, W, y, -100, 0.1, "sum", block_rows=1)
    b = o.fused_linear_cross_entropy(X, W, y, -100, 0.1, "sum", block_rows=256)
    for u, v in zip(a, b):
        assert np.allclose(u, v, rtol=1e-13, atol=1e-15)
    bm = o.fused_linear_cross_entropy(X, W, y, -100, 0.1, "batchmean")[0]
    assert abs(bm - a[0] / 10) <= 1e-14


ALL_PINS = [
    pin_log_softmax_library,
    pin_batchmean_scale_golden,
    pin_self_distillation_exact_zero,
    pin_disjoint_support_closed_form,
    pin_bounds,
    pin_role_swap,
    pin_kl_endpoints_library,
    pin_jsd_half_library,
    pin_jsd_entropy_identity,
    pin_kl_limits,
    pin_finite_differences_logits,
    pin_finite_differences_fused,
    pin_temperature_identity,
    pin_gradient_rows_sum_to_zero,
    pin_block_invariance_and_reductions,
    pin_padded_slots_exact_zero,
    pin_logprob_kl_library,
    pin_logprob_disjoint_closed_form,
    pin_logprob_finite_differences,
    pin_logprob_ties_and_logit_path,
    pin_tvd_golden_ties,
    pin_tvd_library_and_closed_form,
    pin_tvd_finite_differences,
    pin_ce_torch_library,
    pin_ce_autograd,
    pin_ce_finite_differences,
    pin_ce_closed_forms,
    pin_ce_blocks_and_batchmean,
]


def failing_pins(module):
    """Names of the pins the module fails (any exception counts as a failure)."""
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(module)
        except Exception:   # noqa: BLE001 - any failure marks the pin
            failed.append(pin.__name__)
    return failed
