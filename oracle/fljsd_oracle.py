"""Plain fp64 CPU oracle for the fused-linear generalized-JSD distillation pass.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run this module; the product path
never does. It shares no code with the HIP library and imports nothing from it.

What it computes, and where the pages fix it:
  * Logits are the lm_head products Z_s = X_s W_s^T and Z_t = X_t W_t^T
    (Liger-Kernel PR #1352, "Fuse log-softmax into fused_linear_jsd kernel",
    Details: the GEMM produces the logits the loss kernel reads).
  * Both logits are divided by the temperature once, with no T^2 factor on the
    loss (PR #1352, Open question 2).
  * log-softmax is materialized here, on purpose: the fused kernel's online
    softmax (PR #1352, Details, first bullet) is an exact reorganisation of it,
    so the oracle is the plain definition and differs only in rounding.
  * The generalized JSD with beta mixing and its two endpoint branches
    (PR #1352, Testing Done: 0.0 is forward KL, 0.1 and 0.5 generalized, 1.0
    reverse KL). The formula is not printed on the pages; the reading used is
        JSD_beta = beta KL(P||M) + (1-beta) KL(Q||M),  M = beta P + (1-beta) Q,
    with P the teacher and Q the student distribution. It is the only
    assignment under which the generalized loss tends to the labelled
    endpoints: JSD_beta / beta -> KL(P||Q) as beta -> 0 and
    JSD_beta / (1-beta) -> KL(Q||P) as beta -> 1.
  * The student-logit gradient through the log-softmax (the chain rule the
    fused kernel applies in-kernel, PR #1352 Summary), including the
    cross-column term dX_sum (PR #1352, Details).
  * Exact ties p == q contribute zero (PR #1374, "Fix TVD gradient at
    p == q", Summary): where P == Q exactly the element's loss is 0 and, in
    the generalized branch, its gradient term is 0.
  * grad_input = dZ W_s and grad_W = dZ^T X_s, accumulated over row chunks
    (PR #1429 "write the weight-gradient product directly into grad_weight",
    Summary); the oracle accumulates in fp64.
  * Two adjacent public losses over given distributions: the generalized
    JSD in log-probability space (PR #1352, Open question 3) and the total
    variation distance with the p == q gradient fix (PR #1374).
  * The fused-linear cross-entropy that PR #1352 (Details) names as the
    pattern the JSD path follows: lm_head logits, a two-pass online softmax,
    hard labels with an ignore index, optional label smoothing, and
    grad_input / grad_weight products as above.
  * Reductions: batchmean divides by the number of rows. PR #1374's tie table
    prints -0.0625 at (8, 512) for a -0.5 per-element TVD slope, i.e. a scale
    of 1/8 = 1/rows. sum uses 1, mean uses 1/(rows*V), none returns per-row
    losses and uses scale 1 for the gradient.

Every function is pinned by tests that do not retype its formulas (closed
forms, library routines, finite differences, invariants, and planted-mistake
checks); see the test suite's oracle pin module.
"""
from __future__ import annotations

import numpy as np

REDUCTIONS = ("batchmean", "sum", "mean", "none")


def reduction_scale(reduction: str, rows: int, vocab: int) -> float:
    """Scale applied to the summed per-element loss and to the gradient.

    batchmean = 1/rows (PR #1374 tie table: -0.0625 = -0.5 * 1/8 at 8 rows),
    sum = 1, mean = 1/(rows*vocab) (elementwise mean), none = 1.
    """
    if reduction == "batchmean":
        return 1.0 / rows
    if reduction == "sum":
        return 1.0
    if reduction == "mean":
        return 1.0 / (rows * vocab)
    if reduction == "none":
        return 1.0
    raise ValueError(f"unknown reduction {reduction!r}")


def log_softmax(a: np.ndarray) -> np.ndarray:
    """Row-wise log-softmax along the last axis, max-subtracted, in fp64."""
    a = np.asarray(a, dtype=np.float64)
    m = np.max(a, axis=-1, keepdims=True)
    shifted = a - m
    return shifted - np.log(np.sum(np.exp(shifted), axis=-1, keepdims=True))


def jsd_rows(logits_s: np.ndarray, logits_t: np.ndarray, beta: float,
             temperature: float):
    """Per-row generalized JSD and its gradient w.r.t. the scaled student logits.

    Returns (row_loss[R], dA[R, V]) where A = logits_s / temperature and
    row_loss[r] = sum_v l[r, v]. dA is the gradient of row_loss w.r.t. A
    (no reduction scale, no 1/T factor yet).

    Branches (PR #1352, Testing Done):
      beta == 0: forward KL(P||Q); l = P (log P - log Q); dA = Q - P.
      beta == 1: reverse KL(Q||P); l = Q (log Q - log P);
                 dA = Q ((log Q - log P) - KL_row).
      otherwise: l = beta P (log P - log M) + (1-beta) Q (log Q - log M);
                 g = (1-beta) Q (log Q - log M);  dA = g - Q * sum_v g.
    Tie rule (PR #1374): where P == Q exactly, l = 0, and g = 0 in the
    generalized branch. 0 log 0 is taken as 0 throughout.
    """
    if temperature <= 0:
        raise ValueError("temperature must be > 0")
    if not 0.0 <= beta <= 1.0:
        raise ValueError("beta must be in [0, 1]")
    A = np.asarray(logits_s, dtype=np.float64) / temperature
    B = np.asarray(logits_t, dtype=np.float64) / temperature
    logQ = log_softmax(A)
    logP = log_softmax(B)
    Q = np.exp(logQ)
    P = np.exp(logP)
    tie = P == Q

    if beta == 0.0:
        l = np.where(P > 0, P * (logP - logQ), 0.0)
        dA = Q - P
    elif beta == 1.0:
        l = np.where(Q > 0, Q * (logQ - logP), 0.0)
        l = np.where(tie, 0.0, l)
        kl_row = np.sum(l, axis=-1, keepdims=True)
        dA = np.where(Q > 0, Q * ((logQ - logP) - kl_row), 0.0)
    else:
        # log M = log(beta P + (1-beta) Q), evaluated from the log-probs so it
        # stays finite where P and Q underflow together.
        logM = np.logaddexp(np.log(beta) + logP, np.log1p(-beta) + logQ)
        term_p = np.where(P > 0, beta * P * (logP - logM), 0.0)
        term_q = np.where(Q > 0, (1.0 - beta) * Q * (logQ - logM), 0.0)
        l = term_p + term_q
        g = term_q
        g = np.where(tie, 0.0, g)
        G = np.sum(g, axis=-1, keepdims=True)   # dX_sum, the cross-column term
        dA = g - Q * G
    l = np.where(tie, 0.0, l)
    return np.sum(l, axis=-1), dA


def generalized_jsd(logits_s, logits_t, beta: float, temperature: float,
                    reduction: str = "batchmean"):
    """Loss and student-logit gradient over given logits.

    Returns (loss, grad_logits_s): loss is a scalar (or per-row array for
    reduction "none"); grad_logits_s = (scale / T) * dA.
    """
    logits_s = np.asarray(logits_s, dtype=np.float64)
    R, V = logits_s.shape
    scale = reduction_scale(reduction, R, V)
    row_loss, dA = jsd_rows(logits_s, logits_t, beta, temperature)
    grad = dA * (scale / temperature)
    loss = row_loss if reduction == "none" else scale * np.sum(row_loss)
    return loss, grad


def jsd_logprob(logq, logp, beta: float, reduction: str = "batchmean"):
    """Generalized JSD over given log-probabilities, with the gradient w.r.t.
    the student's log-probabilities (the log-space contract of the public JSD
    op that PR #1352, Open question 3, keeps apart from the fused path).

    logq: student log-probabilities [R, V]; logp: teacher log-probabilities.
    Element terms, with Q = exp(logq), P = exp(logp), taken as given (no
    renormalization; each element is an independent variable):
      beta == 0: l = P (logp - logq);             g = dl/dlogq = -P
      beta == 1: l = Q (logq - logp);             g = Q (logq - logp) + Q
      otherwise: M = beta P + (1-beta) Q,
                 l = beta P (logp - log M) + (1-beta) Q (logq - log M),
                 g = (1-beta) Q (logq - log M)
    (in the generalized branch the derivatives of log M cancel against the
    mixture weights, leaving g). Tie rule (PR #1374): where P == Q exactly,
    l = 0 and, in the generalized branch, g = 0. 0 log 0 is taken as 0.
    Returns (loss, grad): loss = scale * sum l (per-row sums for "none"),
    grad = scale * g.
    """
    if not 0.0 <= beta <= 1.0:
        raise ValueError("beta must be in [0, 1]")
    logq = np.asarray(logq, dtype=np.float64)
    logp = np.asarray(logp, dtype=np.float64)
    R, V = logq.shape
    scale = reduction_scale(reduction, R, V)
    Q = np.exp(logq)
    P = np.exp(logp)
    tie = P == Q
    if beta == 0.0:
        l = np.where(P > 0, P * (logp - logq), 0.0)
        g = -P
    elif beta == 1.0:
        l = np.where(Q > 0, Q * (logq - logp), 0.0)
        g = np.where(Q > 0, Q * (logq - logp), 0.0) + Q
    else:
        logM = np.logaddexp(np.log(beta) + logp, np.log1p(-beta) + logq)
        term_p = np.where(P > 0, beta * P * (logp - logM), 0.0)
        term_q = np.where(Q > 0, (1.0 - beta) * Q * (logq - logM), 0.0)
        l = term_p + term_q
        g = np.where(tie, 0.0, term_q)
    l = np.where(tie, 0.0, l)
    row_loss = np.sum(l, axis=-1)
    loss = row_loss if reduction == "none" else scale * np.sum(row_loss)
    return loss, scale * g


def tvd(p, q, reduction: str = "batchmean"):
    """Total variation distance between given distributions, with the
    gradient w.r.t. p (PR #1374 "Fix TVD gradient at p == q", Summary).

    Element loss 0.5 |p - q|; its derivative w.r.t. p is +0.5 where p > q,
    -0.5 where p < q, and 0 at an exact tie p == q (the fix: a three-way
    sign). Returns (loss, grad): loss = scale * sum over all elements, or the
    elementwise [R, V] losses for "none" (the plain elementwise reading of the
    page's reference torch.abs(p - q) / 2); grad = scale * derivative.
    """
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    R, V = p.shape
    scale = reduction_scale(reduction, R, V)
    diff = p - q
    elem = 0.5 * np.abs(diff)
    grad = scale * 0.5 * np.sign(diff)
    loss = elem if reduction == "none" else scale * np.sum(elem)
    return loss, grad


def fused_linear_jsd(X_s, W_s, X_t, W_t, beta: float, temperature: float,
                     reduction: str = "batchmean", block_rows: int = 256):
    """Loss, grad_input and grad_weight of the whole fused-linear JSD pass.

    Rows are processed in blocks of ``block_rows`` only to bound memory; the
    scale always uses the global row count, and grad_W accumulates over
    blocks in fp64.
    Returns (loss, grad_X_s [BT, H_s], grad_W_s [V, H_s]).
    """
    X_s = np.asarray(X_s, dtype=np.float64)
    W_s = np.asarray(W_s, dtype=np.float64)
    X_t = np.asarray(X_t, dtype=np.float64)
    W_t = np.asarray(W_t, dtype=np.float64)
    BT = X_s.shape[0]
    V = W_s.shape[0]
    if X_t.shape[0] != BT or W_t.shape[0] != V:
        raise ValueError("student and teacher shapes disagree")
    scale = reduction_scale(reduction, BT, V)
    grad_X = np.empty_like(X_s)
    grad_W = np.zeros_like(W_s)
    row_loss = np.empty(BT, dtype=np.float64)
    for r0 in range(0, BT, block_rows):
        r1 = min(BT, r0 + block_rows)
        Z_s = X_s[r0:r1] @ W_s.T
        Z_t = X_t[r0:r1] @ W_t.T
        loss_rows, dA = jsd_rows(Z_s, Z_t, beta, temperature)
        dZ = dA * (scale / temperature)
        grad_X[r0:r1] = dZ @ W_s
        grad_W += dZ.T @ X_s[r0:r1]
        row_loss[r0:r1] = loss_rows
    loss = row_loss if reduction == "none" else scale * np.sum(row_loss)
    return loss, grad_X, grad_W


def cross_entropy_rows(logits, labels, ignore_index: int = -100,
                       label_smoothing: float = 0.0):
    """Per-row cross-entropy with hard labels and its gradient w.r.t. the
    logits, unscaled (the cross-entropy the fused-linear pattern of PR #1352,
    Details, comes from: a two-pass online softmax over the lm_head logits).

    With q = softmax(z) over the row and eps = label_smoothing:
        loss_r = -(1 - eps) log q[y] - (eps / V) sum_v log q[v]
        dz_r   = q - (1 - eps) onehot(y) - eps / V
    Rows whose label is ignore_index, or outside [0, V), are ignored: loss 0,
    gradient 0. Returns (row_loss[R], dz[R, V], valid[R] bool).
    """
    if not 0.0 <= label_smoothing <= 1.0:
        raise ValueError("label_smoothing must be in [0, 1]")
    z = np.asarray(logits, dtype=np.float64)
    y = np.asarray(labels, dtype=np.int64)
    R, V = z.shape
    valid = (y != ignore_index) & (y >= 0) & (y < V)
    logq = log_softmax(z)
    yc = np.where(valid, y, 0)
    logq_y = logq[np.arange(R), yc]
    eps = label_smoothing
    row_loss = -(1.0 - eps) * logq_y - (eps / V) * np.sum(logq, axis=-1)
    dz = np.exp(logq) - eps / V
    dz[np.arange(R), yc] -= (1.0 - eps)
    row_loss = np.where(valid, row_loss, 0.0)
    dz = np.where(valid[:, None], dz, 0.0)
    return row_loss, dz, valid


def ce_reduction_scale(reduction: str, rows: int, n_valid: int) -> float:
    """mean: 1 / (number of rows whose label counts), the usual cross-entropy
    mean (nan when no row counts); batchmean: 1 / rows; sum and none: 1."""
    if reduction == "mean":
        return 1.0 / n_valid if n_valid > 0 else float("nan")
    if reduction == "batchmean":
        return 1.0 / float(rows)
    if reduction in ("sum", "none"):
        return 1.0
    raise ValueError(f"unknown reduction {reduction!r}")


def fused_linear_cross_entropy(X, W, labels, ignore_index: int = -100,
                               label_smoothing: float = 0.0, reduction: str = "mean",
                               block_rows: int = 256):
    """Loss, grad_input and grad_weight of the fused-linear cross-entropy:
    Z = X W^T, cross-entropy over each row of Z (cross_entropy_rows), then
    grad_X = dZ W and grad_W = dZ^T X with dZ = scale * dz. Rows are processed
    in blocks only to bound memory; grad_W accumulates in fp64. With no
    counted row, the mean is nan and the gradients are 0.
    Returns (loss, grad_X [BT, H], grad_W [V, H]); loss is per-row for "none".
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    y = np.asarray(labels, dtype=np.int64)
    BT = X.shape[0]
    V = W.shape[0]
    n_valid = int(np.sum((y != ignore_index) & (y >= 0) & (y < V)))
    scale = ce_reduction_scale(reduction, BT, n_valid)
    gscale = scale if n_valid > 0 else 0.0
    grad_X = np.empty_like(X)
    grad_W = np.zeros_like(W)
    row_loss = np.empty(BT, dtype=np.float64)
    for r0 in range(0, BT, block_rows):
        r1 = min(BT, r0 + block_rows)
        Z = X[r0:r1] @ W.T
        loss_rows, dz, _ = cross_entropy_rows(Z, y[r0:r1], ignore_index, label_smoothing)
        dZ = dz * gscale
        grad_X[r0:r1] = dZ @ W
        grad_W += dZ.T @ X[r0:r1]
        row_loss[r0:r1] = loss_rows
    loss = row_loss if reduction == "none" else scale * np.sum(row_loss)
    return loss, grad_X, grad_W


def fused_linear_jsd_rows(X_s, W_s, X_t, W_t, rows, beta: float,
                          temperature: float, reduction: str = "batchmean"):
    """Per-row loss and grad_input for selected rows only.

    Each row's loss and grad_input depend on that row alone (the scale uses
    the global row count), so a sample of rows can be checked at full size
    one by one. Returns (row_loss[len(rows)], grad_X_rows [len(rows), H_s]).
    """
    X_s = np.asarray(X_s)
    BT = X_s.shape[0]
    V = W_s.shape[0]
    scale = reduction_scale(reduction, BT, V)
    rows = np.asarray(rows, dtype=np.int64)
    Ws = np.asarray(W_s, dtype=np.float64)
    Wt = np.asarray(W_t, dtype=np.float64)
    Z_s = np.asarray(X_s[rows], dtype=np.float64) @ Ws.T
    Z_t = np.asarray(np.asarray(X_t)[rows], dtype=np.float64) @ Wt.T
    loss_rows, dA = jsd_rows(Z_s, Z_t, beta, temperature)
    dZ = dA * (scale / temperature)
    return loss_rows, dZ @ Ws
