"""Magnitude of the terms that form each output of one pass (TEST
INFRASTRUCTURE; used only by the parity gate).

Every output of the pass is a sum: a contraction c_ij = sum_k a_ik b_kj, an
all-reduce sum of partials plus bias and residual, a column sum over rows,
or a linear combination inside the LayerNorm backward. For each element the
oracle gives a magnitude M >= |value| such that u * M bounds what the
element moves by when each tensor it is formed from is off by a relative
u, the storage format's unit roundoff: the pages' mixed precision (overview
page, section 2) stores the layer's intermediates in 16 bits, so an element
whose terms cancel carries their rounding, not its own.

An operand that comes out of an earlier product carries an error spread
over its whole vector (each of its elements sums many rounded terms), so the
rule for a product is normwise: if the rows a_i and columns b_j are known to
a relative accuracy u in the 2-norm, c_ij moves by at most
u * ||a_i||_2 ||b_j||_2 (Cauchy-Schwarz), and
M_ij = ||a_i||_2 ||b_j||_2 >= sum_k |a_ik| |b_kj| >= |c_ij|.

Rules, applied in the order the pass computes:
* a product: M = ||row of A|| ||column of B|| from the operands' values;
* a sum of tensors adds their magnitudes (an input, weight or stand-in peer
  contributes |value|; a partial or an earlier output its own M);
* the LayerNorm backward's combination rstd * (g - mean(g) - xhat mean(g xhat))
  adds the magnitudes of its three terms, g taken with the incoming M;
* a column sum over rows is the product with a vector of ones:
  M = sqrt(rows) * ||column||, and the LayerNorm weight gradient
  sum_n d_nj xhat_nj is the product of its two columns:
  M = ||M_d[:, j]|| ||xhat[:, j]||;
* the loss statistics: with M_l[n, j] = ||H_n|| ||E_j|| the magnitude of
  logit (n, j), the row max carries M_l of its logit, the shard's
  log-sum-exp its own magnitude plus the softmax-weighted M_l (its
  derivative), the target logit M_l of that logit;
* the attention backward's score gradient dS = P (dP - delta) cancels
  (its rows sum to zero), so its magnitude P (|dP| + |delta|) is carried
  into dQ = dS K / sqrt(d) and dK = dS^T Q / sqrt(d) (normwise products of
  that magnitude), and those M of dqkv, not its values, are the operand of
  the products and sums that take dqkv (the QKV weight, bias and input
  gradients);
* the loss gradient dl = g (softmax(l) - onehot) carries, besides |dl|, what
  the logits' own magnitudes move it by through the exponential:
  g * softmax(l) * (M_l + M_lse), since exp turns an absolute change of a
  logit into a relative change of its probability. The products dl E and
  dl^T H take that M of dl as their dl operand.
"""
from __future__ import annotations

import numpy as np

__all__ = ["product", "ln_bwd", "logit_stats", "sum_rows", "col_product", "attention_grad", "softmax_weighted",
           "loss_grad"]


def _norms(a, axis):
    """2-norms of the rows (axis=1) or columns (axis=0) of a matrix."""
    a = np.asarray(a, np.float64)
    return np.sqrt(np.einsum("ij,ij->i" if axis == 1 else "ij,ij->j", a, a))


def product(a, b):
    """M of the contraction A @ B: ||A[i, :]||_2 * ||B[:, j]||_2."""
    return np.outer(_norms(a, 1), _norms(b, 0))


def sum_rows(m):
    """M of a column sum over rows (the bias gradients, the LayerNorm shift
    gradient): the product with a ones vector, sqrt(rows) * ||m[:, j]||_2."""
    m = np.asarray(m, np.float64)
    return np.sqrt(m.shape[0]) * _norms(m, 0)


def col_product(m_a, b):
    """M of sum_n a_nj b_nj (the LayerNorm scale gradient): ||m_a[:, j]|| ||b[:, j]||."""
    return _norms(m_a, 0) * _norms(b, 0)


def ln_bwd(m_d, xhat, rstd, gamma):
    """M of the LayerNorm backward d_in = rstd * (g - mean(g) - xhat * mean(g * xhat))
    with g = d * gamma, given M of the incoming gradient d (rows of h)."""
    g = np.asarray(m_d, np.float64) * np.abs(np.asarray(gamma, np.float64))
    ax = np.abs(xhat)
    return rstd[:, None] * (g + g.mean(-1, keepdims=True) + ax * (g * ax).mean(-1, keepdims=True))


def attention_grad(q, k, v, o, probs, do):
    """M of one head's (dQ, dK, dV) given its forward (q, k, v, o = P v,
    probs P) and the output gradient do: M_dS = P (|do v^T| + |rowsum(do o)|),
    dQ = dS k / sqrt(d), dK = dS^T q / sqrt(d), dV = P^T do as products."""
    q, k, v, o, do = (np.asarray(a, np.float64) for a in (q, k, v, o, do))
    d = q.shape[1]
    m_ds = probs * (np.abs(do @ v.T) + np.abs((do * o).sum(axis=1, keepdims=True)))
    return product(m_ds, k) / np.sqrt(d), product(m_ds.T, q) / np.sqrt(d), product(probs.T, do)


def _logit_norms(hidden, emb):
    """||H_n|| and ||E_j||: the magnitude of logit (n, j) is their product."""
    return _norms(hidden, 1), _norms(emb, 1)


def logit_stats(hidden, emb, logits, lse_local, targets, v0):
    """M of one vocabulary shard's statistics in the form the parity gate
    compares them: (row max, the shard's log-sum-exp m + ln se, target logit).
    Returns [N, 3]."""
    hn, en = _logit_norms(hidden, emb)
    logits = np.asarray(logits, np.float64)
    n, vr = logits.shape
    m_max = hn * en[logits.argmax(axis=1)]
    lse_local = np.asarray(lse_local, np.float64)
    p = np.exp(logits - lse_local[:, None])
    m_lse = np.abs(lse_local) + hn * (p @ en)
    t = np.asarray(targets, np.int64) - v0
    inside = (t >= 0) & (t < vr)
    m_tl = np.zeros(n)
    m_tl[inside] = hn[inside] * en[t[inside]]
    return np.stack([m_max, m_lse, m_tl], axis=1)


def softmax_weighted(hidden, emb, logits, lse):
    """One shard's share of M of the full log-sum-exp: sum_j exp(l_j - lse) M_l[j]."""
    hn, en = _logit_norms(hidden, emb)
    p = np.exp(np.asarray(logits, np.float64) - np.asarray(lse, np.float64)[:, None])
    return hn * (p @ en)


def loss_grad(dl, hidden, emb, logits, lse, m_lse, g):
    """M of the loss gradient dl = g_n (exp(l - lse_n) - onehot) of one shard:
    |dl| + g_n exp(l - lse_n) (M_l + M_lse_n)."""
    hn, en = _logit_norms(hidden, emb)
    m = np.outer(hn, en)
    m += np.asarray(m_lse, np.float64)[:, None]
    m *= np.exp(np.asarray(logits, np.float64) - np.asarray(lse, np.float64)[:, None])
    m *= np.asarray(g, np.float64)[:, None]
    m += np.abs(np.asarray(dl, np.float64))
    return m
