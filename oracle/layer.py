"""Float64 reference of one Megatron-LM transformer layer, restricted to any
subset of heads / ffn columns / vocabulary rows, forward and backward, plus the
vocabulary-parallel cross-entropy.  TEST INFRASTRUCTURE ONLY (see package doc).

Conventions (readings where the pages are silent; each listed in the design notes):
* rows are batch-major: row n = b*seq + s;
* weights use the nn.Linear layout W[out, in], so y = x @ W.T + b;
* a parameter dict ``p`` holds the blocks of the heads / ffn columns / vocab
  rows under study, stacked in global order (see synth.oracle_params). With
  every rank's blocks it is the unsharded layer; with one rank's it is that
  rank's restriction -- the same definition over a smaller index set;
* pre-LN placement (podcast page, Outline: LayerNorm/residual placement fixes
  large-BERT training), LN eps = cfg.ln_eps, biased variance, affine;
* GeLU is the exact form u * Phi(u) (the pages only name GeLU);
* attention scale 1/sqrt(d); causal = key j visible to query i iff j <= i;
* dropout rate 0 (the pages give no rate).
"""
from __future__ import annotations

import math
import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "layernorm_fwd", "layernorm_bwd", "gelu", "gelu_prime", "linear",
    "attention_head_fwd", "attention_head_bwd",
    "attn_block_fwd", "attn_block_bwd_shard", "mlp_block_fwd", "mlp_block_bwd_shard",
    "block_bwd_replicated", "partial_sum", "layer_fwd", "layer_bwd",
    "xent_logits", "xent_local_stats", "xent_finish", "xent_full", "xent_bwd_local",
    "embedding_fwd_shard", "embedding_bwd_shard",
    "layer_flops",
]

F64 = np.float64


def _f(a):
    return np.asarray(a, dtype=F64)


# ---------------------------------------------------------------------------
# elementary operations

def linear(x, w, b=None):
    """y = x W^T (+ b): the dense contraction of every parallel linear layer
    (guide page, section 1.2: tensor parallelism splits a single matrix product)."""
    y = _f(x) @ _f(w).T
    return y if b is None else y + _f(b)


def layernorm_fwd(v, gamma, beta, eps):
    """Row-wise LayerNorm (podcast page, Key concepts: layer normalisation;
    replicated on every rank per the Outline). Returns (out, mu, rstd, xhat)."""
    v = _f(v)
    mu = v.mean(axis=-1, keepdims=True)
    var = ((v - mu) ** 2).mean(axis=-1, keepdims=True)          # biased variance
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (v - mu) * rstd
    return _f(gamma) * xhat + _f(beta), mu[..., 0], rstd[..., 0], xhat


def layernorm_bwd(dout, xhat, rstd, gamma):
    """Gradient of layernorm_fwd: returns (d_in, d_gamma, d_beta).

    With g = dout*gamma: d_in = rstd * (g - mean(g) - xhat * mean(g*xhat))."""
    dout = _f(dout)
    g = dout * _f(gamma)
    d_in = rstd[:, None] * (g - g.mean(-1, keepdims=True) - xhat * (g * xhat).mean(-1, keepdims=True))
    return d_in, (dout * xhat).sum(0), dout.sum(0)


def gelu(u):
    """Exact GeLU u*Phi(u) (podcast page, Key concepts: GeLU, applied per shard)."""
    u = _f(u)
    return 0.5 * u * (1.0 + _erf(u / math.sqrt(2.0)))


def gelu_prime(u):
    """d/du of u*Phi(u) = Phi(u) + u*phi(u)."""
    u = _f(u)
    return 0.5 * (1.0 + _erf(u / math.sqrt(2.0))) + u * np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)


# ---------------------------------------------------------------------------
# attention of one head over one sequence (podcast page, Outline and Key
# concepts: self-attention parallelised over heads; guide page, section 3.2)

def attention_head_fwd(q, k, v, causal):
    """softmax(q k^T / sqrt(d) + mask) v for one head; returns (o, lse, probs).

    Masked scores are excluded exactly (probability 0)."""
    q, k, v = _f(q), _f(k), _f(v)
    s, d = q.shape
    scores = (q @ k.T) / math.sqrt(d)
    if causal:
        scores = np.where(np.tril(np.ones((s, s), dtype=bool)), scores, -np.inf)
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    z = e.sum(axis=-1, keepdims=True)
    probs = e / z
    return probs @ v, (m + np.log(z))[:, 0], probs


def attention_head_bwd(q, k, v, o, probs, do):
    """Gradient of attention_head_fwd w.r.t. q, k, v given do = dL/do."""
    q, k, v, o, do = _f(q), _f(k), _f(v), _f(o), _f(do)
    d = q.shape[1]
    dv = probs.T @ do
    dp = do @ v.T
    rowdot = (do * o).sum(axis=-1, keepdims=True)     # sum_j P_ij dP_ij
    ds = probs * (dp - rowdot)
    return ds @ k / math.sqrt(d), ds.T @ q / math.sqrt(d), dv


# ---------------------------------------------------------------------------
# blocks. "partial" = the block's row-parallel product over the given heads /
# columns, before the all-reduce, without the row-parallel bias or residual.

def _seq_slices(n_rows, seq):
    for b in range(n_rows // seq):
        yield b, slice(b * seq, (b + 1) * seq)


def attn_block_fwd(x, p, seq, causal, eps):
    """Attention block of one rank (or the full layer): pre-LN, column-parallel
    QKV, per-head attention, row-parallel output projection -> partial.

    podcast page Outline (K/Q/V parallelised by heads; 2 all-reduces per
    module); guide page sections 3.2 (QKV split by heads, output projection
    split by rows)."""
    d = p["head_dim"]
    y, mu, rstd, xhat = layernorm_fwd(x, p["ln1_g"], p["ln1_b"], eps)
    q = linear(y, p["wq"], p["bq"])
    k = linear(y, p["wk"], p["bk"])
    v = linear(y, p["wv"], p["bv"])
    n_heads = q.shape[1] // d
    ctx = np.zeros_like(q)
    lse = np.zeros((x.shape[0] // seq, n_heads, seq))
    probs = {}
    for b, rows in _seq_slices(x.shape[0], seq):
        for g in range(n_heads):
            cols = slice(g * d, (g + 1) * d)
            o, l, pr = attention_head_fwd(q[rows, cols], k[rows, cols], v[rows, cols], causal)
            ctx[rows, cols] = o
            lse[b, g] = l
            probs[b, g] = pr
    partial = linear(ctx, p["wo"])        # = sum over heads of O_g W_o[:, g]^T
    cache = dict(x=_f(x), y=y, mu=mu, rstd=rstd, xhat=xhat, q=q, k=k, v=v, ctx=ctx,
                 lse=lse, probs=probs, seq=seq)
    return partial, cache


def attn_block_bwd_shard(dy, p, cache):
    """Rank-local backward of the attention block up to the gradient w.r.t. the
    LayerNorm output (the quantity the backward all-reduce sums).

    Returns d_ln_partial [N, h] and grads {d_w_qkv, d_b_qkv, d_w_o} plus the
    intermediates dctx and dqkv [N, 3*h_sub] ([dQ | dK | dV])."""
    dy = _f(dy)
    d, seq = p["head_dim"], cache["seq"]
    dctx = dy @ p["wo"]
    d_wo = dy.T @ cache["ctx"]
    q, k, v, ctx = cache["q"], cache["k"], cache["v"], cache["ctx"]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b, rows in _seq_slices(dy.shape[0], seq):
        for g in range(q.shape[1] // d):
            cols = slice(g * d, (g + 1) * d)
            dq[rows, cols], dk[rows, cols], dv[rows, cols] = attention_head_bwd(
                q[rows, cols], k[rows, cols], v[rows, cols], ctx[rows, cols],
                cache["probs"][b, g], dctx[rows, cols])
    y = cache["y"]
    grads = {
        "d_w_qkv": np.concatenate([dq.T @ y, dk.T @ y, dv.T @ y], axis=0),
        "d_b_qkv": np.concatenate([dq.sum(0), dk.sum(0), dv.sum(0)]),
        "d_w_o": d_wo,
    }
    d_ln = dq @ p["wq"] + dk @ p["wk"] + dv @ p["wv"]
    return d_ln, grads, {"dctx": dctx, "dqkv": np.concatenate([dq, dk, dv], axis=1)}


def mlp_block_fwd(h1, p, eps):
    """MLP block of one rank: pre-LN, then the column-parallel first linear
    layer with its bias, GeLU applied to this rank's columns, then the
    row-parallel second linear layer on those columns -> partial (guide page
    "From Transformer splitting to communication optimisation", section 3.1:
    the first layer is split by columns so GeLU needs no exchange, the second
    by rows so it consumes the local columns directly; the ffn is four times
    the hidden width there)."""
    z, mu, rstd, xhat = layernorm_fwd(h1, p["ln2_g"], p["ln2_b"], eps)
    u = linear(z, p["w1"], p["b1"])
    a = gelu(u)
    partial = linear(a, p["w2"])          # = sum over ffn columns c of a_c W_2[:, c]^T
    return partial, dict(x=_f(h1), z=z, mu=mu, rstd=rstd, xhat=xhat, u=u, a=a)


def mlp_block_bwd_shard(dy, p, cache):
    """Rank-local MLP backward up to the gradient w.r.t. the LayerNorm output."""
    dy = _f(dy)
    du = (dy @ p["w2"]) * gelu_prime(cache["u"])
    grads = {"d_w_2": dy.T @ cache["a"], "d_w_1": du.T @ cache["z"], "d_b_1": du.sum(0)}
    return du @ p["w1"], grads, {"du": du}


def block_bwd_replicated(dy, d_ln_sum, cache, gamma):
    """Replicated tail of a block's backward (podcast page Outline: LayerNorm and
    residual are duplicated on every rank): given the all-reduced gradient
    w.r.t. the LN output, dx = dy (residual path) + LN_bwd(d_ln_sum).

    Returns dx and {d_ln_g, d_ln_b, d_b_out} where d_b_out = sum_n dy is the
    gradient of the row-parallel bias added after the all-reduce."""
    d_in, dg, db = layernorm_bwd(d_ln_sum, cache["xhat"], cache["rstd"], gamma)
    dy = _f(dy)
    return dy + d_in, {"d_ln_g": dg, "d_ln_b": db, "d_b_out": dy.sum(0)}


def partial_sum(partials, bias=None, residual=None):
    """The all-reduce (podcast page, Key concepts: all-reduce sums across the
    group) followed by the row-parallel bias and the residual, added once."""
    out = sum(_f(t) for t in partials)
    if bias is not None:
        out = out + _f(bias)
    if residual is not None:
        out = out + _f(residual)
    return out


def layer_fwd(x, p, seq, causal, eps):
    """Whole layer over the heads/columns in ``p`` (the unsharded layer when p
    holds every rank): out = h1 + MLP(LN2(h1)) + b2, h1 = x + Attn(LN1(x)) + b_o."""
    pa, ca = attn_block_fwd(x, p, seq, causal, eps)
    h1 = partial_sum([pa], p["b_o"], x)
    pm, cm = mlp_block_fwd(h1, p, eps)
    out = partial_sum([pm], p["b_2"], h1)
    return out, {"attn": ca, "mlp": cm, "h1": h1, "attn_partial": pa, "mlp_partial": pm}


def layer_bwd(dout, p, cache):
    """Backward of layer_fwd; returns dx and every parameter gradient."""
    dz, g_mlp, _ = mlp_block_bwd_shard(dout, p, cache["mlp"])
    dh1, g_mlp_r = block_bwd_replicated(dout, dz, cache["mlp"], p["ln2_g"])
    dyln, g_attn, _ = attn_block_bwd_shard(dh1, p, cache["attn"])
    dx, g_attn_r = block_bwd_replicated(dh1, dyln, cache["attn"], p["ln1_g"])
    grads = dict(g_attn)
    grads.update(g_mlp)
    grads.update({"d_ln1_g": g_attn_r["d_ln_g"], "d_ln1_b": g_attn_r["d_ln_b"],
                  "d_b_o": g_attn_r["d_b_out"], "d_ln2_g": g_mlp_r["d_ln_g"],
                  "d_ln2_b": g_mlp_r["d_ln_b"], "d_b_2": g_mlp_r["d_b_out"]})
    return dx, grads


# ---------------------------------------------------------------------------
# vocabulary-parallel output embedding + cross-entropy (guide page section 3.3:
# output embedding split along the vocabulary, gather deferred and fused with
# the loss; podcast page Outline: same)

def xent_logits(hidden, emb):
    """logits over the given vocabulary rows: H E^T."""
    return _f(hidden) @ _f(emb).T


def xent_local_stats(logits, targets, v0):
    """Per-row statistics of one vocabulary shard with global ids [v0, v0+V_r):
    m = max_j l_j, se = sum_j exp(l_j - m), tl = l[target - v0] if the target
    lies in the shard else 0. Returns [N, 3]."""
    logits = _f(logits)
    n, vr = logits.shape
    m = logits.max(axis=1)
    se = np.exp(logits - m[:, None]).sum(axis=1)
    t = np.asarray(targets, np.int64) - v0
    inside = (t >= 0) & (t < vr)
    tl = np.zeros(n)
    tl[inside] = logits[np.nonzero(inside)[0], t[inside]]
    return np.stack([m, se, tl], axis=1)


def xent_finish(stats_list, mask=None):
    """Combine the shards' statistics into the full-vocabulary loss:
    M = max_r m_r, S = sum_r se_r exp(m_r - M), lse = M + ln S,
    loss_n = lse - sum_r tl_r, mean over rows with mask 1.
    Returns (lse [N], loss_rows [N] (0 where masked out), mean loss, count)."""
    st = np.stack([_f(s) for s in stats_list])            # [t, N, 3]
    big_m = st[:, :, 0].max(axis=0)
    big_s = (st[:, :, 1] * np.exp(st[:, :, 0] - big_m)).sum(axis=0)
    lse = big_m + np.log(big_s)
    loss_rows = lse - st[:, :, 2].sum(axis=0)
    w = np.ones_like(lse) if mask is None else np.asarray(mask, F64)
    count = w.sum()
    loss_rows = loss_rows * w
    return lse, loss_rows, loss_rows.sum() / count, count


def xent_full(hidden, emb, targets, mask=None):
    """Plain (unsplit) cross-entropy: mean over masked rows of
    logsumexp(l_n) - l_n[target_n]. Returns (mean loss, lse, logits)."""
    logits = xent_logits(hidden, emb)
    m = logits.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(logits - m).sum(axis=1, keepdims=True)))[:, 0]
    loss_rows = lse - logits[np.arange(len(targets)), np.asarray(targets, np.int64)]
    w = np.ones_like(lse) if mask is None else np.asarray(mask, F64)
    return (loss_rows * w).sum() / w.sum(), lse, logits


def xent_bwd_local(logits, lse, targets, v0, mask, dloss, hidden, emb):
    """Backward of the mean loss for one vocabulary shard:
    dl = g_n (exp(l - lse_n) - [j == target_n - v0]), g_n = dloss*mask_n/sum(mask);
    d_hidden (partial over the shard) = dl E_r; d_emb = dl^T H.
    Returns (dlogits, d_hidden_partial, d_emb)."""
    logits = _f(logits)
    n, vr = logits.shape
    w = np.ones(n) if mask is None else np.asarray(mask, F64)
    g = dloss * w / w.sum()
    dl = np.exp(logits - _f(lse)[:, None])
    t = np.asarray(targets, np.int64) - v0
    inside = np.nonzero((t >= 0) & (t < vr))[0]
    dl[inside, t[inside]] -= 1.0
    dl *= g[:, None]
    return dl, dl @ _f(emb), dl.T @ _f(hidden)


# ---------------------------------------------------------------------------
# vocabulary-parallel input embedding (guide page section 3.3: the input
# layer is split along the vocabulary and the ranks' outputs are summed by an
# all-reduce)

def embedding_fwd_shard(tokens, emb_in, v0):
    """This rank's partial of the input embedding: row n is E_in[tok_n - v0]
    when the id lies in the rank's range [v0, v0 + V_r), else zero. The sum of
    the ranks' partials (the all-reduce) is the full lookup E_in[tok_n]."""
    emb_in = _f(emb_in)
    vr = emb_in.shape[0]
    t = np.asarray(tokens, np.int64) - v0
    out = np.zeros((len(t), emb_in.shape[1]))
    inside = np.nonzero((t >= 0) & (t < vr))[0]
    out[inside] = emb_in[t[inside]]
    return out


def embedding_bwd_shard(tokens, d_out, v0, vr):
    """Gradient of this rank's rows of E_in given the (replicated) gradient of
    the summed embedding output: d_E[v] = sum of d_out[n] over the rows n whose
    id is v0 + v (a scatter-add; ids outside the range contribute nothing)."""
    d_out = _f(d_out)
    t = np.asarray(tokens, np.int64) - v0
    grad = np.zeros((vr, d_out.shape[1]))
    inside = np.nonzero((t >= 0) & (t < vr))[0]
    np.add.at(grad, t[inside], d_out[inside])
    return grad


# ---------------------------------------------------------------------------
# algorithmic work (for throughput figures)

def layer_flops(cfg, rank_local=True):
    """Contraction flops of one rank's layer shard, forward + backward
    (= 3 x forward: dgrad and wgrad each repeat the forward product).
    Causal attention counts only the s(s+1)/2 visible query-key pairs.
    Returns dict(layer=..., xent=..., xent_rows=...)."""
    t = cfg.tp if rank_local else 1
    n, h = cfg.rows, cfg.hidden
    hr, fr, vr = cfg.hidden // t, cfg.ffn // t, cfg.vocab // t
    a_r, d, s, b = cfg.heads // t, cfg.head_dim, cfg.seq, cfg.micro_batch
    pairs = s * (s + 1) // 2 if cfg.causal else s * s
    fwd = 2 * n * h * 3 * hr            # QKV
    fwd += 2 * 2 * b * a_r * pairs * d  # QK^T and PV
    fwd += 2 * n * hr * h               # output projection
    fwd += 2 * n * h * fr * 2           # fc1 and fc2
    xrows = n if cfg.mask_rows is None else cfg.mask_rows
    return {"layer": 3 * fwd, "xent": 3 * 2 * xrows * vr * h, "xent_rows": xrows}
