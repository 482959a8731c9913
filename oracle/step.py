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

from .layer import (attn_block_bwd_shard, attn_block_fwd, block_bwd_replicated, mlp_block_bwd_shard,
                    mlp_block_fwd, partial_sum, xent_bwd_local, xent_finish, xent_local_stats, xent_logits)

__all__ = ["step_reference"]


def step_reference(params_by_rank: dict, x, R, targets, mask, *, seq, causal, eps, tp, vocab_r,
                   peers=(), peer_stats=(), use_mask=False, dloss=1.0) -> dict:
    """params_by_rank: {rank: oracle parameter dict restricted to that rank}
    (the replicated LayerNorm / bias vectors are read from any of them).
    Returns every quantity the GPU pass produces, keyed like LayerStep.results():
    shared tensors by name, per-rank ones as "name@rank"."""
    ranks = sorted(params_by_rank)
    p0 = params_by_rank[ranks[0]]
    x = np.asarray(x, np.float64)
    peers = [np.asarray(p, np.float64) for p in peers]
    out = {}
    caches_a, caches_m = {}, {}

    parts = []
    for r in ranks:
        pa, caches_a[r] = attn_block_fwd(x, params_by_rank[r], seq, causal, eps)
        out[f"part_attn@{r}"] = pa
        parts.append(pa)
    h1 = partial_sum(parts + peers, p0["b_o"], x)
    parts = []
    for r in ranks:
        pm, caches_m[r] = mlp_block_fwd(h1, params_by_rank[r], eps)
        out[f"part_mlp@{r}"] = pm
        parts.append(pm)
    y = partial_sum(parts + peers, p0["b_2"], h1)
    out.update(h1=h1, out=y)

    # cross-entropy over the vocabulary shards
    logits, stats_by_rank = {}, {}
    for r in ranks:
        logits[r] = xent_logits(y, params_by_rank[r]["emb"])
        stats_by_rank[r] = xent_local_stats(logits[r], targets, r * vocab_r)
        out[f"stats@{r}"] = stats_by_rank[r]
    it = iter(peer_stats)
    all_stats = [stats_by_rank[r] if r in stats_by_rank else np.asarray(next(it), np.float64) for r in range(tp)]
    m = mask if use_mask else None
    lse, loss_rows, loss, count = xent_finish(all_stats, m)
    out.update(lse=lse, loss_rows=loss_rows, loss=np.array([loss, count]))
    dparts = []
    for r in ranks:
        _, dh, de = xent_bwd_local(logits[r], lse, targets, r * vocab_r, m, dloss, y, params_by_rank[r]["emb"])
        out[f"dH@{r}"] = dh
        out[f"d_emb@{r}"] = de
        dparts.append(dh)
    dout = partial_sum(dparts + peers, None, R)
    out["dout"] = dout

    # layer backward
    dparts = []
    for r in ranks:
        dz, g, _ = mlp_block_bwd_shard(dout, params_by_rank[r], caches_m[r])
        out[f"dln_mlp@{r}"] = dz
        out[f"d_w_1@{r}"], out[f"d_b_1@{r}"], out[f"d_w_2@{r}"] = g["d_w_1"], g["d_b_1"], g["d_w_2"]
        dparts.append(dz)
    dz_sum = partial_sum(dparts + peers)
    dh1, gr = block_bwd_replicated(dout, dz_sum, caches_m[ranks[0]], p0["ln2_g"])
    out.update(dz_sum=dz_sum, dh1=dh1, d_ln2_g=gr["d_ln_g"], d_ln2_b=gr["d_ln_b"], d_b_2=gr["d_b_out"])
    dparts = []
    for r in ranks:
        dyl, g, _ = attn_block_bwd_shard(dh1, params_by_rank[r], caches_a[r])
        out[f"dln_attn@{r}"] = dyl
        out[f"d_w_qkv@{r}"], out[f"d_b_qkv@{r}"], out[f"d_w_o@{r}"] = g["d_w_qkv"], g["d_b_qkv"], g["d_w_o"]
        dparts.append(dyl)
    dy_sum = partial_sum(dparts + peers)
    dx, gr = block_bwd_replicated(dh1, dy_sum, caches_a[ranks[0]], p0["ln1_g"])
    out.update(dy_sum=dy_sum, dx=dx, d_ln1_g=gr["d_ln_g"], d_ln1_b=gr["d_ln_b"], d_b_o=gr["d_b_out"])
    return out
