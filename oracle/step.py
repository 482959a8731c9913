"""Float64 reference of one whole pass of the hot path (TEST INFRASTRUCTURE).

Same sequence as the GPU pass: attention block -> all-reduce -> MLP block ->
all-reduce -> vocabulary-parallel cross-entropy forward and backward ->
all-reduce of the hidden-state gradient (plus the extra upstream term R of
J = loss + sum(out*R)) -> MLP backward -> all-reduce -> LN backward ->
attention backward -> all-reduce -> LN backward. Each rank's contribution
is the oracle's block definition restricted to that rank's heads / columns /
vocabulary rows; ranks not computed here contribute fixed stand-in tensors.
"""
from __future__ import annotations

import numpy as np

from . import magnitude as MG
from .layer import (attn_block_bwd_shard, attn_block_fwd, block_bwd_replicated, mlp_block_bwd_shard,
                    mlp_block_fwd, partial_sum, xent_bwd_local, xent_finish, xent_local_stats, xent_logits)

__all__ = ["step_reference"]


def _attention_grad_mag(cache, dctx, d):
    """M of the attention block's dqkv = [dQ | dK | dV], head by head and
    sequence by sequence in the layout the oracle's attention backward uses."""
    q, k, v, ctx, seq = cache["q"], cache["k"], cache["v"], cache["ctx"], cache["seq"]
    m = np.zeros((q.shape[0], 3 * q.shape[1]))
    hs = q.shape[1]
    for b in range(q.shape[0] // seq):
        rows = slice(b * seq, (b + 1) * seq)
        for g in range(hs // d):
            cols = slice(g * d, (g + 1) * d)
            mq, mk, mv = MG.attention_grad(q[rows, cols], k[rows, cols], v[rows, cols], ctx[rows, cols],
                                           cache["probs"][b, g], dctx[rows, cols])
            m[rows, g * d:(g + 1) * d] = mq
            m[rows, hs + g * d:hs + (g + 1) * d] = mk
            m[rows, 2 * hs + g * d:2 * hs + (g + 1) * d] = mv
    return m


def step_reference(params_by_rank: dict, x, R, targets, mask, *, seq, causal, eps, tp, vocab_r,
                   peers=(), peer_stats=(), use_mask=False, dloss=1.0, mags: dict | None = None) -> dict:
    """params_by_rank: {rank: oracle parameter dict restricted to that rank}
    (the replicated LayerNorm / bias vectors are read from any of them).
    Returns every quantity the GPU pass produces, keyed like LayerStep.results():
    shared tensors by name, per-rank ones as "name@rank".

    mags: if a dict is given it is filled, under the same keys, with the
    magnitude of the terms forming each output (oracle.magnitude); the loss
    statistics' entry holds the magnitudes of (row max, the shard's
    log-sum-exp, target logit)."""
    ranks = sorted(params_by_rank)
    p0 = params_by_rank[ranks[0]]
    x = np.asarray(x, np.float64)
    peers = [np.asarray(p, np.float64) for p in peers]
    want = mags is not None
    M = mags if want else {}
    abs_peers = sum(np.abs(p) for p in peers) if peers else 0.0
    out = {}
    caches_a, caches_m = {}, {}

    parts = []
    for r in ranks:
        pa, caches_a[r] = attn_block_fwd(x, params_by_rank[r], seq, causal, eps)
        out[f"part_attn@{r}"] = pa
        parts.append(pa)
        if want:
            M[f"part_attn@{r}"] = MG.product(caches_a[r]["ctx"], params_by_rank[r]["wo"].T)
    h1 = partial_sum(parts + peers, p0["b_o"], x)
    if want:
        M["h1"] = np.abs(x) + np.abs(p0["b_o"]) + sum(M[f"part_attn@{r}"] for r in ranks) + abs_peers
    parts = []
    for r in ranks:
        pm, caches_m[r] = mlp_block_fwd(h1, params_by_rank[r], eps)
        out[f"part_mlp@{r}"] = pm
        parts.append(pm)
        if want:
            M[f"part_mlp@{r}"] = MG.product(caches_m[r]["a"], params_by_rank[r]["w2"].T)
    y = partial_sum(parts + peers, p0["b_2"], h1)
    out.update(h1=h1, out=y)
    if want:
        M["out"] = M["h1"] + np.abs(p0["b_2"]) + sum(M[f"part_mlp@{r}"] for r in ranks) + abs_peers

    # cross-entropy over the vocabulary shards
    logits, stats_by_rank = {}, {}
    for r in ranks:
        logits[r] = xent_logits(y, params_by_rank[r]["emb"])
        stats_by_rank[r] = xent_local_stats(logits[r], targets, r * vocab_r)
        out[f"stats@{r}"] = stats_by_rank[r]
        if want:
            st = stats_by_rank[r]
            M[f"stats@{r}"] = MG.logit_stats(y, params_by_rank[r]["emb"], logits[r], st[:, 0] + np.log(st[:, 1]),
                                             targets, r * vocab_r)
    it = iter(peer_stats)
    all_stats = [stats_by_rank[r] if r in stats_by_rank else np.asarray(next(it), np.float64) for r in range(tp)]
    m = mask if use_mask else None
    lse, loss_rows, loss, count = xent_finish(all_stats, m)
    out.update(lse=lse, loss_rows=loss_rows, loss=np.array([loss, count]))
    if want:
        w = np.ones_like(lse) if m is None else np.asarray(m, np.float64)
        M["lse"] = np.abs(lse) + sum(MG.softmax_weighted(y, params_by_rank[r]["emb"], logits[r], lse) for r in ranks)
        tl_all = sum(np.asarray(s_, np.float64)[:, 2] for s_ in all_stats)
        M["loss_rows"] = (M["lse"] + np.abs(tl_all) + sum(M[f"stats@{r}"][:, 2] for r in ranks)) * w
        M["loss"] = np.array([M["loss_rows"].sum() / count, count])   # the row count is exact
        g_rows = dloss * w / count
    dparts = []
    for r in ranks:
        dl, dh, de = xent_bwd_local(logits[r], lse, targets, r * vocab_r, m, dloss, y, params_by_rank[r]["emb"])
        out[f"dH@{r}"] = dh
        out[f"d_emb@{r}"] = de
        dparts.append(dh)
        if want:
            m_dl = MG.loss_grad(dl, y, params_by_rank[r]["emb"], logits[r], lse, M["lse"], g_rows)
            M[f"dH@{r}"] = MG.product(m_dl, params_by_rank[r]["emb"])
            M[f"d_emb@{r}"] = MG.product(m_dl.T, y)
            del m_dl
    dout = partial_sum(dparts + peers, None, R)
    out["dout"] = dout
    if want:
        M["dout"] = np.abs(np.asarray(R, np.float64)) + sum(M[f"dH@{r}"] for r in ranks) + abs_peers

    # layer backward
    dparts = []
    for r in ranks:
        dz, g, inter = mlp_block_bwd_shard(dout, params_by_rank[r], caches_m[r])
        out[f"dln_mlp@{r}"] = dz
        out[f"d_w_1@{r}"], out[f"d_b_1@{r}"], out[f"d_w_2@{r}"] = g["d_w_1"], g["d_b_1"], g["d_w_2"]
        dparts.append(dz)
        if want:
            du = inter["du"]
            M[f"dln_mlp@{r}"] = MG.product(du, params_by_rank[r]["w1"])
            M[f"d_w_1@{r}"] = MG.product(du.T, caches_m[r]["z"])
            M[f"d_b_1@{r}"] = MG.sum_rows(du)
            M[f"d_w_2@{r}"] = MG.product(dout.T, caches_m[r]["a"])
    dz_sum = partial_sum(dparts + peers)
    cm = caches_m[ranks[0]]
    dh1, gr = block_bwd_replicated(dout, dz_sum, cm, p0["ln2_g"])
    out.update(dz_sum=dz_sum, dh1=dh1, d_ln2_g=gr["d_ln_g"], d_ln2_b=gr["d_ln_b"], d_b_2=gr["d_b_out"])
    if want:
        M["dz_sum"] = sum(M[f"dln_mlp@{r}"] for r in ranks) + abs_peers
        M["dh1"] = M["dout"] + MG.ln_bwd(M["dz_sum"], cm["xhat"], cm["rstd"], p0["ln2_g"])
        M["d_ln2_g"] = MG.col_product(M["dz_sum"], cm["xhat"])
        M["d_ln2_b"] = MG.sum_rows(M["dz_sum"])
        M["d_b_2"] = MG.sum_rows(M["dout"])
    dparts = []
    for r in ranks:
        dyl, g, inter = attn_block_bwd_shard(dh1, params_by_rank[r], caches_a[r])
        out[f"dln_attn@{r}"] = dyl
        out[f"d_w_qkv@{r}"], out[f"d_b_qkv@{r}"], out[f"d_w_o@{r}"] = g["d_w_qkv"], g["d_b_qkv"], g["d_w_o"]
        dparts.append(dyl)
        if want:
            pr, c = params_by_rank[r], caches_a[r]
            m_dqkv = _attention_grad_mag(c, inter["dctx"], pr["head_dim"])
            M[f"dln_attn@{r}"] = MG.product(m_dqkv, np.concatenate([pr["wq"], pr["wk"], pr["wv"]], axis=0))
            M[f"d_w_qkv@{r}"] = MG.product(m_dqkv.T, c["y"])
            M[f"d_b_qkv@{r}"] = MG.sum_rows(m_dqkv)
            M[f"d_w_o@{r}"] = MG.product(dh1.T, c["ctx"])
    dy_sum = partial_sum(dparts + peers)
    ca = caches_a[ranks[0]]
    dx, gr = block_bwd_replicated(dh1, dy_sum, ca, p0["ln1_g"])
    out.update(dy_sum=dy_sum, dx=dx, d_ln1_g=gr["d_ln_g"], d_ln1_b=gr["d_ln_b"], d_b_o=gr["d_b_out"])
    if want:
        M["dy_sum"] = sum(M[f"dln_attn@{r}"] for r in ranks) + abs_peers
        M["dx"] = M["dh1"] + MG.ln_bwd(M["dy_sum"], ca["xhat"], ca["rstd"], p0["ln1_g"])
        M["d_ln1_g"] = MG.col_product(M["dy_sum"], ca["xhat"])
        M["d_ln1_b"] = MG.sum_rows(M["dy_sum"])
        M["d_b_o"] = MG.sum_rows(M["dh1"])
    return out
