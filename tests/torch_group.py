"""A TP group's pass written directly as a torch graph (test helper, CPU).

Forward + autograd backward of J = mean CE(out) + sum(out * R) for the ranks
in `shards` (rank -> synth.RankShard), with stand-ins for the other ranks:

* every rank's branch is its own torch sub-graph (F.linear,
  F.scaled_dot_product_attention, F.gelu, F.layer_norm) on its own slice of
  the weights, and its row-parallel output enters the residual stream as a
  summand (podcast page, Outline: attention split by heads, MLP by columns
  then rows, two all-reduces per block; guide page sections 3.1-3.2);
* ranks not computed here enter as fixed stand-in tensors P: the forward
  adds sum(P) to the attention and MLP outputs, and the backward all-reduces
  (loss gradient, the two LayerNorm-output gradients) receive sum(P) through
  extra objective terms sum(v * sum(P)) on the tensors they are the
  gradient of (out, LN2 output, LN1 output);
* the output embedding is split along the vocabulary with the loss fused in
  (guide page section 3.3): the stand-in ranks' statistics (m, se, tl) enter
  the log-sum-exp as the extra entries m + ln se, and their target logits as
  constants.

`cdt` is the compute dtype: float64 gives the exact model that pins the
oracle; bfloat16 gives an independent mixed-precision implementation
(torch's CPU kernels, every intermediate stored in bf16, parameters and
their gradients kept in float64 leaves) that the parity gate must accept.
`slip` plants one mistake, for checks that the gate rejects it.
Returns a dict keyed like oracle.step_reference's result (float64 arrays).
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

SLIPS = ("peers_dropped_from_mlp_sum", "no_causal_mask", "r_missing_from_dout", "b1_dropped",
         "attention_scale_off")


def T(a, grad=False):
    t = torch.tensor(np.asarray(a, np.float64), dtype=torch.float64)
    return t.requires_grad_() if grad else t


def torch_group(cfg, rep, shards, peers, peer_stats, cdt=torch.float64, slip=None):
    assert slip is None or slip in SLIPS, slip
    N, h, s, b, d = cfg.rows, cfg.hidden, cfg.seq, cfg.micro_batch, cfg.head_dim
    ar, vr = cfg.heads_r, cfg.vocab_r
    eps = cfg.ln_eps
    ranks = sorted(shards)
    P = sum((T(p) for p in peers), torch.zeros(N, h, dtype=torch.float64))
    x = T(rep.x, True)
    ln1_g, ln1_b, ln2_g, ln2_b = (T(getattr(rep, k), True) for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b"))
    b_o, b_2 = T(rep.b_o, True), T(rep.b_2, True)
    W = {r: {k: T(getattr(shards[r], k), True) for k in ("wq", "wk", "wv", "bq", "bk", "bv", "wo", "w1", "b1",
                                                        "w2", "emb")} for r in ranks}
    c = lambda t: t.to(cdt)
    keep = {}

    def heads(t):   # [N, ar*d] -> [b, ar, s, d]
        return t.reshape(b, s, ar, d).permute(0, 2, 1, 3)

    y = F.layer_norm(c(x), (h,), c(ln1_g), c(ln1_b), eps)
    y.retain_grad()
    h1 = c(x) + c(b_o) + c(P)
    for r in ranks:
        w = W[r]
        y_r = y * 1.0                       # rank r's own use of the replicated LN output
        y_r.retain_grad()
        keep[f"y@{r}"] = y_r
        q, k, v = (F.linear(y_r, c(w[a]), c(w[bb])) for a, bb in (("wq", "bq"), ("wk", "bk"), ("wv", "bv")))
        causal = bool(cfg.causal) and slip != "no_causal_mask"
        scale = (1.0 / d ** 0.5) * (1.1 if slip == "attention_scale_off" else 1.0)
        o = F.scaled_dot_product_attention(heads(q), heads(k), heads(v), is_causal=causal, scale=scale)
        ctx = o.permute(0, 2, 1, 3).reshape(N, ar * d)
        part = F.linear(ctx, c(w["wo"]))
        keep[f"part_attn@{r}"] = part
        h1 = h1 + part
    h1.retain_grad()
    z = F.layer_norm(h1, (h,), c(ln2_g), c(ln2_b), eps)
    z.retain_grad()
    out = h1 + c(b_2) + (0.0 if slip == "peers_dropped_from_mlp_sum" else c(P))
    for r in ranks:
        w = W[r]
        z_r = z * 1.0
        z_r.retain_grad()
        keep[f"z@{r}"] = z_r
        b1 = None if slip == "b1_dropped" else c(w["b1"])
        part = F.linear(F.gelu(F.linear(z_r, c(w["w1"]), b1), approximate="none"), c(w["w2"]))
        keep[f"part_mlp@{r}"] = part
        out = out + part
    out.retain_grad()

    # loss over the vocabulary shards (in float64 from the stored logits):
    # this GPU's logits plus the stand-ins' (m + ln se) entries
    tg = torch.tensor(np.asarray(rep.targets, np.int64))
    logits = {r: out @ c(W[r]["emb"]).T for r in ranks}
    for r in ranks:
        logits[r].retain_grad()
    others = [q for q in range(cfg.tp) if q not in ranks]
    ps = {r: T(st) for r, st in zip(others, peer_stats)}
    cols = [logits[r].double() for r in ranks] + [(p[:, 0] + torch.log(p[:, 1]))[:, None] for p in ps.values()]
    lse = torch.logsumexp(torch.cat(cols, dim=1), dim=1)
    tl = torch.zeros(N, dtype=torch.float64)
    for r in ranks:
        inside = (tg >= r * vr) & (tg < (r + 1) * vr)
        loc = torch.where(inside, tg - r * vr, torch.zeros_like(tg))
        tl = tl + torch.where(inside, logits[r].double().gather(1, loc[:, None])[:, 0], torch.zeros(N).double())
    for p in ps.values():
        tl = tl + p[:, 2]
    w_rows = T(rep.mask) if cfg.mask_rows is not None else torch.ones(N, dtype=torch.float64)
    loss_rows = (lse - tl) * w_rows
    loss = loss_rows.sum() / w_rows.sum()
    # J plus the stand-in ranks' contributions to the three backward all-reduces
    R = T(rep.dout) * (0.0 if slip == "r_missing_from_dout" else 1.0)
    J = loss + (out.double() * (R + P)).sum() + (z.double() * P).sum() + (y.double() * P).sum()
    J.backward()

    res = {"h1": h1, "out": out, "lse": lse, "loss_rows": loss_rows,
           "loss": torch.tensor([loss.item(), w_rows.sum().item()], dtype=torch.float64),
           "dout": out.grad, "dz_sum": z.grad, "dh1": h1.grad, "dy_sum": y.grad, "dx": x.grad,
           "d_ln1_g": ln1_g.grad, "d_ln1_b": ln1_b.grad, "d_ln2_g": ln2_g.grad, "d_ln2_b": ln2_b.grad,
           "d_b_o": b_o.grad, "d_b_2": b_2.grad}
    for r in ranks:
        w = W[r]
        lg = logits[r].detach().double()
        m = lg.max(dim=1).values
        inside = (tg >= r * vr) & (tg < (r + 1) * vr)
        loc = torch.where(inside, tg - r * vr, torch.zeros_like(tg))
        res[f"stats@{r}"] = torch.stack([m, torch.exp(lg - m[:, None]).sum(1),
                                         torch.where(inside, lg.gather(1, loc[:, None])[:, 0],
                                                     torch.zeros(N).double())], 1)
        res[f"dH@{r}"] = logits[r].grad @ c(w["emb"]).detach()
        res[f"d_emb@{r}"] = w["emb"].grad
        res[f"part_attn@{r}"] = keep[f"part_attn@{r}"]
        res[f"part_mlp@{r}"] = keep[f"part_mlp@{r}"]
        res[f"dln_attn@{r}"] = keep[f"y@{r}"].grad
        res[f"dln_mlp@{r}"] = keep[f"z@{r}"].grad
        res[f"d_w_qkv@{r}"] = torch.cat([w["wq"].grad, w["wk"].grad, w["wv"].grad])
        res[f"d_b_qkv@{r}"] = torch.cat([w["bq"].grad, w["bk"].grad, w["bv"].grad])
        res[f"d_w_o@{r}"] = w["wo"].grad
        res[f"d_w_1@{r}"], res[f"d_b_1@{r}"], res[f"d_w_2@{r}"] = w["w1"].grad, w["b1"].grad, w["w2"].grad
    return {k: (np.zeros(W[ranks[0]]["b1"].shape) if v is None else v.detach().double().numpy())
            for k, v in res.items()}
