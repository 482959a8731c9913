"""Pins of the CPU oracle to things other than itself (CPU only).

Each check uses an independent source of truth: a library routine (torch
LayerNorm / SDPA / MultiheadAttention / GeLU / cross_entropy, math.erf), a
brute-force loop, a closed form, an invariant the pages state, or central
finite differences. A plausible slip in the oracle (dropped term, wrong sign,
transposed operand, wrong index) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
torch.set_default_dtype(torch.float64)


def T(a):
    return torch.tensor(np.asarray(a, np.float64))


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- elementary

def test_linear_matches_triple_loop():
    g = rng(1)
    x, w, b = g.standard_normal((3, 5)), g.standard_normal((4, 5)), g.standard_normal(4)
    want = np.zeros((3, 4))
    for i in range(3):
        for j in range(4):
            acc = b[j]
            for k in range(5):
                acc += x[i, k] * w[j, k]
            want[i, j] = acc
    np.testing.assert_allclose(O.linear(x, w, b), want, rtol=1e-14, atol=1e-14)


def test_layernorm_matches_torch_and_closed_forms():
    g = rng(2)
    x = g.standard_normal((6, 10)) * 3 + 1
    gam, bet = g.standard_normal(10), g.standard_normal(10)
    out, mu, rstd, xhat = O.layernorm_fwd(x, gam, bet, 1e-5)
    ref = F.layer_norm(T(x), (10,), T(gam), T(bet), 1e-5).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mu, x.mean(1), rtol=1e-13)
    np.testing.assert_allclose(1 / rstd ** 2 - 1e-5, x.var(1), rtol=1e-10)
    # a constant row normalises to 0, so the output is beta exactly
    c = np.full((1, 10), 7.25)
    np.testing.assert_array_equal(O.layernorm_fwd(c, gam, bet, 1e-5)[0][0], bet)


def test_layernorm_bwd_matches_autograd():
    g = rng(3)
    x, gam, bet, dy = (g.standard_normal((5, 9)), g.standard_normal(9), g.standard_normal(9),
                       g.standard_normal((5, 9)))
    _, _, rstd, xhat = O.layernorm_fwd(x, gam, bet, 1e-5)
    dx, dg, db = O.layernorm_bwd(dy, xhat, rstd, gam)
    xt, gt, bt = T(x).requires_grad_(), T(gam).requires_grad_(), T(bet).requires_grad_()
    F.layer_norm(xt, (9,), gt, bt, 1e-5).backward(T(dy))
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_gelu_exact_form():
    xs = np.linspace(-6, 6, 97)
    want = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in xs])
    np.testing.assert_allclose(O.gelu(xs), want, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(O.gelu(xs), F.gelu(T(xs), approximate="none").numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(O.gelu(xs) - O.gelu(-xs), xs, rtol=1e-13, atol=1e-14)  # u*Phi(u) - (-u)*Phi(-u) = u
    assert O.gelu(0.0) == 0.0 and O.gelu_prime(0.0) == 0.5
    h = 1e-6
    fd = (O.gelu(xs + h) - O.gelu(xs - h)) / (2 * h)
    np.testing.assert_allclose(O.gelu_prime(xs), fd, rtol=1e-8, atol=1e-9)
    # the tanh approximation is a different function: the exact form must not match it
    tanh_form = F.gelu(T(xs), approximate="tanh").numpy()
    assert np.abs(O.gelu(xs) - tanh_form).max() > 1e-4


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("causal", [True, False])
def test_attention_matches_sdpa(causal):
    g = rng(4)
    q, k, v = (g.standard_normal((7, 8)) for _ in range(3))
    o, lse, probs = O.attention_head_fwd(q, k, v, causal)
    ref = F.scaled_dot_product_attention(T(q)[None], T(k)[None], T(v)[None], is_causal=causal)[0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(probs.sum(1), 1.0, rtol=1e-14)
    scores = T(q) @ T(k).T / math.sqrt(8)
    if causal:
        scores = scores.masked_fill(torch.triu(torch.ones(7, 7, dtype=torch.bool), 1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(scores, -1).numpy(), rtol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_attention_closed_forms(causal):
    g = rng(5)
    k, v = g.standard_normal((6, 4)), g.standard_normal((6, 4))
    o, lse, _ = O.attention_head_fwd(np.zeros((6, 4)), k, v, causal)   # uniform weights
    want = np.cumsum(v, 0) / np.arange(1, 7)[:, None] if causal else np.broadcast_to(v.mean(0), v.shape)
    np.testing.assert_allclose(o, want, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(np.arange(1, 7)) if causal else np.full(6, math.log(6)), rtol=1e-13)
    o1, _, _ = O.attention_head_fwd(g.standard_normal((1, 4)), k[:1], v[:1], causal)   # s = 1
    np.testing.assert_allclose(o1, v[:1], rtol=1e-15)


def test_attention_causality():
    g = rng(6)
    q, k, v = (g.standard_normal((8, 4)) for _ in range(3))
    o, _, _ = O.attention_head_fwd(q, k, v, True)
    k2, v2 = k.copy(), v.copy()
    k2[5] += 3.0
    v2[5] -= 2.0
    o2, _, _ = O.attention_head_fwd(q, k2, v2, True)
    np.testing.assert_array_equal(o[:5], o2[:5])
    assert np.abs(o[5:] - o2[5:]).max() > 1e-3


@pytest.mark.parametrize("causal", [True, False])
def test_attention_bwd_matches_autograd(causal):
    g = rng(7)
    q, k, v, do = (g.standard_normal((6, 4)) for _ in range(4))
    o, _, probs = O.attention_head_fwd(q, k, v, causal)
    dq, dk, dv = O.attention_head_bwd(q, k, v, o, probs, do)
    qt, kt, vt = (T(a).requires_grad_() for a in (q, k, v))
    F.scaled_dot_product_attention(qt[None], kt[None], vt[None], is_causal=causal)[0].backward(T(do))
    for mine, ref in ((dq, qt), (dk, kt), (dv, vt)):
        np.testing.assert_allclose(mine, ref.grad.numpy(), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- whole layer vs torch modules

def _tiny_inputs(cfg):
    rep = synth.replicated_inputs(cfg)
    shards = [synth.rank_shard(cfg, r) for r in range(cfg.tp)]
    return rep, shards, synth.oracle_params(cfg, shards, rep)


def _torch_layer(cfg, p, x, targets, mask, with_loss=True):
    """Pre-LN transformer layer + output embedding + mean cross-entropy from
    torch.nn library modules (fp64), independent of the oracle's code
    (with_loss=False: the layer only, loss None)."""
    h, a, s, b = cfg.hidden, cfg.heads, cfg.seq, cfg.micro_batch
    ln1, ln2 = torch.nn.LayerNorm(h, eps=cfg.ln_eps), torch.nn.LayerNorm(h, eps=cfg.ln_eps)
    mha = torch.nn.MultiheadAttention(h, a, bias=True, batch_first=True)
    fc1, fc2 = torch.nn.Linear(h, cfg.ffn), torch.nn.Linear(cfg.ffn, h)
    emb = torch.nn.Parameter(T(p["emb"]))
    with torch.no_grad():
        ln1.weight.copy_(T(p["ln1_g"])); ln1.bias.copy_(T(p["ln1_b"]))
        ln2.weight.copy_(T(p["ln2_g"])); ln2.bias.copy_(T(p["ln2_b"]))
        mha.in_proj_weight.copy_(T(np.concatenate([p["wq"], p["wk"], p["wv"]])))
        mha.in_proj_bias.copy_(T(np.concatenate([p["bq"], p["bk"], p["bv"]])))
        mha.out_proj.weight.copy_(T(p["wo"])); mha.out_proj.bias.copy_(T(p["b_o"]))
        fc1.weight.copy_(T(p["w1"])); fc1.bias.copy_(T(p["b1"]))
        fc2.weight.copy_(T(p["w2"])); fc2.bias.copy_(T(p["b_2"]))
    xt = T(x).reshape(b, s, h).requires_grad_()
    am = torch.triu(torch.ones(s, s, dtype=torch.bool), 1) if cfg.causal else None
    y = ln1(xt)
    h1 = xt + mha(y, y, y, attn_mask=am, need_weights=False)[0]
    out = h1 + fc2(F.gelu(fc1(ln2(h1)), approximate="none"))
    out.retain_grad()
    mods = dict(ln1=ln1, ln2=ln2, mha=mha, fc1=fc1, fc2=fc2, emb=emb)
    if not with_loss:
        return xt, out, None, mods
    logits = out.reshape(-1, h) @ emb.T
    rows = torch.tensor(np.nonzero(mask)[0])
    loss = F.cross_entropy(logits[rows], torch.tensor(targets, dtype=torch.long)[rows])
    return xt, out, loss, mods


@pytest.mark.parametrize("causal,mask_rows", [(True, None), (False, 4)])
def test_layer_and_loss_match_torch_modules(causal, mask_rows):
    cfg = synth.tiny_config(causal=causal, mask_rows=mask_rows, seq=5, micro_batch=2, heads=2,
                            head_dim=8, hidden=16, ffn=64, vocab=12, tp=1)
    rep, shards, p = _tiny_inputs(cfg)
    out, cache = O.layer_fwd(rep.x, p, cfg.seq, cfg.causal, cfg.ln_eps)
    loss, lse, logits = O.xent_full(out, p["emb"], rep.targets, rep.mask)

    xt, out_t, loss_t, m = _torch_layer(cfg, p, rep.x, rep.targets, rep.mask)
    np.testing.assert_allclose(out, out_t.detach().reshape(-1, cfg.hidden).numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(loss, loss_t.item(), rtol=1e-12)

    # backward: J = loss + sum(out * R); oracle chain vs torch autograd
    R = rng(8).standard_normal(out.shape)
    (loss_t + (out_t.reshape(-1, cfg.hidden) * T(R)).sum()).backward()
    st = np.stack([O.xent_local_stats(logits, rep.targets, 0)])
    lse2, _, _, _ = O.xent_finish(st, rep.mask)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)
    _, dH, dE = O.xent_bwd_local(logits, lse2, rep.targets, 0, rep.mask, 1.0, out, p["emb"])
    dx, g = O.layer_bwd(dH + R, p, cache)
    tol = dict(rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dx, xt.grad.reshape(-1, cfg.hidden).numpy(), **tol)
    np.testing.assert_allclose(dE, m["emb"].grad.numpy(), **tol)
    np.testing.assert_allclose(g["d_w_qkv"], m["mha"].in_proj_weight.grad.numpy(), **tol)
    np.testing.assert_allclose(g["d_b_qkv"], m["mha"].in_proj_bias.grad.numpy(), **tol)
    np.testing.assert_allclose(g["d_w_o"], m["mha"].out_proj.weight.grad.numpy(), **tol)
    np.testing.assert_allclose(g["d_b_o"], m["mha"].out_proj.bias.grad.numpy(), **tol)
    np.testing.assert_allclose(g["d_w_1"], m["fc1"].weight.grad.numpy(), **tol)
    np.testing.assert_allclose(g["d_b_1"], m["fc1"].bias.grad.numpy(), **tol)
    np.testing.assert_allclose(g["d_w_2"], m["fc2"].weight.grad.numpy(), **tol)
    np.testing.assert_allclose(g["d_b_2"], m["fc2"].bias.grad.numpy(), **tol)
    for ln, key in (("ln1", "1"), ("ln2", "2")):
        np.testing.assert_allclose(g["d_ln%s_g" % key], m[ln].weight.grad.numpy(), **tol)
        np.testing.assert_allclose(g["d_ln%s_b" % key], m[ln].bias.grad.numpy(), **tol)


def test_layer_backward_finite_differences():
    """Central differences of J = sum(out*R) + L on a tiny shape, for the input
    and sampled entries of every parameter."""
    cfg = synth.tiny_config(seq=4, micro_batch=2, hidden=8, heads=2, head_dim=4, ffn=16, vocab=12)
    rep, shards, p = _tiny_inputs(cfg)
    R = rng(9).standard_normal((cfg.rows, cfg.hidden))
    x = np.asarray(rep.x, np.float64)

    def J(xv, pv):
        out, _ = O.layer_fwd(xv, pv, cfg.seq, cfg.causal, cfg.ln_eps)
        return (out * R).sum() + O.xent_full(out, pv["emb"], rep.targets)[0]

    out, cache = O.layer_fwd(x, p, cfg.seq, cfg.causal, cfg.ln_eps)
    _, lse, logits = O.xent_full(out, p["emb"], rep.targets)
    _, dH, dE = O.xent_bwd_local(logits, lse, rep.targets, 0, None, 1.0, out, p["emb"])
    dx, g = O.layer_bwd(dH + R, p, cache)
    qkv = lambda name: np.concatenate([p["wq"], p["wk"], p["wv"]]) if name == "w" else None
    h = 1e-6
    pick = rng(10)

    def fd_param(key, idx):
        pp = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
        pp[key][idx] += h
        jp = J(x, pp)
        pp[key][idx] -= 2 * h
        return (jp - J(x, pp)) / (2 * h)

    for _ in range(6):
        i = tuple(pick.integers(0, s) for s in x.shape)
        xp, xm = x.copy(), x.copy()
        xp[i] += h
        xm[i] -= h
        assert abs((J(xp, p) - J(xm, p)) / (2 * h) - dx[i]) <= 1e-6 * max(1.0, abs(dx[i]))
    hr = cfg.hidden
    checks = {
        "wq": lambda i: g["d_w_qkv"][i], "wk": lambda i: g["d_w_qkv"][(i[0] + hr, i[1])],
        "wv": lambda i: g["d_w_qkv"][(i[0] + 2 * hr, i[1])], "bq": lambda i: g["d_b_qkv"][i],
        "bv": lambda i: g["d_b_qkv"][(i[0] + 2 * hr,)], "wo": lambda i: g["d_w_o"][i],
        "w1": lambda i: g["d_w_1"][i], "b1": lambda i: g["d_b_1"][i], "w2": lambda i: g["d_w_2"][i],
        "ln1_g": lambda i: g["d_ln1_g"][i], "ln1_b": lambda i: g["d_ln1_b"][i],
        "ln2_g": lambda i: g["d_ln2_g"][i], "ln2_b": lambda i: g["d_ln2_b"][i],
        "b_o": lambda i: g["d_b_o"][i], "b_2": lambda i: g["d_b_2"][i], "emb": lambda i: dE[i],
    }
    for key, grad_of in checks.items():
        for _ in range(3):
            i = tuple(int(pick.integers(0, s)) for s in p[key].shape)
            fd = fd_param(key, i)
            assert abs(fd - grad_of(i)) <= 1e-6 * max(1.0, abs(fd)), (key, i, fd, grad_of(i))


# ---------------------------------------------------------------- sharding identities (the pages' claims)

@pytest.mark.parametrize("tp", [1, 2, 4])
def test_row_parallel_partials_sum_to_unsharded(tp):
    """Sum over ranks of each rank's restricted partial equals the unsharded
    product (podcast page Outline: MLP split by columns then rows, attention by
    heads; the all-reduce sums the partials)."""
    cfg = synth.tiny_config(tp=tp, heads=4, head_dim=4, hidden=16, ffn=32, vocab=16, seq=6)
    rep, shards, p_full = _tiny_inputs(cfg)
    x = np.asarray(rep.x, np.float64)
    pa_full, _ = O.attn_block_fwd(x, p_full, cfg.seq, cfg.causal, cfg.ln_eps)
    pm_full, _ = O.mlp_block_fwd(x, p_full, cfg.ln_eps)
    pa = [O.attn_block_fwd(x, synth.oracle_params(cfg, [s], rep), cfg.seq, cfg.causal, cfg.ln_eps)[0]
          for s in shards]
    pm = [O.mlp_block_fwd(x, synth.oracle_params(cfg, [s], rep), cfg.ln_eps)[0] for s in shards]
    np.testing.assert_allclose(sum(pa), pa_full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sum(pm), pm_full, rtol=1e-12, atol=1e-13)
    # GeLU of a column block equals the column block of the GeLU: no exchange before it
    u_full = O.linear(O.layernorm_fwd(x, rep.ln2_g, rep.ln2_b, cfg.ln_eps)[0], p_full["w1"], p_full["b1"])
    fr = cfg.ffn_r
    for r in range(tp):
        np.testing.assert_array_equal(O.gelu(u_full)[:, r * fr:(r + 1) * fr], O.gelu(u_full[:, r * fr:(r + 1) * fr]))
    # backward: rank-local LN-output gradients also sum to the unsharded one
    dy = rng(11).standard_normal(x.shape)
    _, ca_full = O.attn_block_fwd(x, p_full, cfg.seq, cfg.causal, cfg.ln_eps)
    d_full = O.attn_block_bwd_shard(dy, p_full, ca_full)[0]
    d_parts = []
    for s in shards:
        ps = synth.oracle_params(cfg, [s], rep)
        d_parts.append(O.attn_block_bwd_shard(dy, ps, O.attn_block_fwd(x, ps, cfg.seq, cfg.causal, cfg.ln_eps)[1])[0])
    np.testing.assert_allclose(sum(d_parts), d_full, rtol=1e-11, atol=1e-12)


def test_head_permutation_equivariance():
    cfg = synth.tiny_config(heads=4, head_dim=4, hidden=16)
    rep, shards, p = _tiny_inputs(cfg)
    perm = [2, 0, 3, 1]
    d = cfg.head_dim
    idx = np.concatenate([np.arange(g * d, (g + 1) * d) for g in perm])
    pp = dict(p)
    for k in ("wq", "wk", "wv"):
        pp[k] = p[k][idx]
    for k in ("bq", "bk", "bv"):
        pp[k] = p[k][idx]
    pp["wo"] = p["wo"][:, idx]
    a = O.attn_block_fwd(rep.x, p, cfg.seq, cfg.causal, cfg.ln_eps)[0]
    b = O.attn_block_fwd(rep.x, pp, cfg.seq, cfg.causal, cfg.ln_eps)[0]
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- cross-entropy

def test_uniform_logits_give_ln_v():
    golden = json.load(open(os.path.join(GOLDEN, "xent_uniform_logits.json")))
    for case in golden["cases"]:
        V = case["vocab"]
        n, h, t = 5, 8, 4 if V % 4 == 0 else 1
        H = rng(12).standard_normal((n, h))
        tg = rng(13).integers(0, V, n)
        E = np.zeros((V, h))
        vr = V // t
        stats = [O.xent_local_stats(O.xent_logits(H, E[r * vr:(r + 1) * vr]), tg, r * vr) for r in range(t)]
        _, _, loss, _ = O.xent_finish(stats)
        assert abs(loss - case["loss"]) <= 1e-12 * case["loss"]


@pytest.mark.parametrize("t", [1, 2, 3])
def test_vocab_parallel_equals_full_and_torch(t):
    g = rng(14)
    n, h, V = 9, 6, 12
    H, E = g.standard_normal((n, h)), g.standard_normal((V, h))
    tg = g.integers(0, V, n)
    mask = (g.random(n) < 0.6).astype(np.uint8)
    mask[0] = 1
    vr = V // t
    stats = [O.xent_local_stats(O.xent_logits(H, E[r * vr:(r + 1) * vr]), tg, r * vr) for r in range(t)]
    lse, rows, loss, count = O.xent_finish(stats, mask)
    full, lse_full, _ = O.xent_full(H, E, tg, mask)
    assert count == mask.sum()
    np.testing.assert_allclose(lse, lse_full, rtol=1e-14)
    assert abs(loss - full) <= 1e-13
    sel = np.nonzero(mask)[0]
    ref = F.cross_entropy(T(H @ E.T)[sel], torch.tensor(tg[sel]))
    assert abs(loss - ref.item()) <= 1e-13
    np.testing.assert_array_equal(rows[mask == 0], 0.0)
    # an all-ones mask is the same as no mask
    assert O.xent_finish(stats, np.ones(n, np.uint8))[2] == O.xent_finish(stats)[2]
    # backward: shard pieces of dlogits reassemble the full softmax gradient,
    # each row sums to 0 and matches autograd; d_hidden partials sum to the full
    Ht, Et = T(H).requires_grad_(), T(E).requires_grad_()
    F.cross_entropy((Ht @ Et.T)[sel], torch.tensor(tg[sel])).backward()
    dl_parts, dH, dE = [], 0, []
    for r in range(t):
        lg = O.xent_logits(H, E[r * vr:(r + 1) * vr])
        dl, dh, de = O.xent_bwd_local(lg, lse, tg, r * vr, mask, 1.0, H, E[r * vr:(r + 1) * vr])
        dl_parts.append(dl)
        dH = dH + dh
        dE.append(de)
    dl = np.concatenate(dl_parts, axis=1)
    np.testing.assert_allclose(dl.sum(1), 0.0, atol=1e-15)
    np.testing.assert_allclose(dH, Ht.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.concatenate(dE), Et.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_local_stats_brute_force():
    g = rng(15)
    lg = g.standard_normal((4, 7)) * 5
    tg = np.array([3, 9, 0, 6])
    st = O.xent_local_stats(lg, tg, 3)
    for i in range(4):
        m = max(lg[i])
        se = sum(math.exp(v - m) for v in lg[i])
        tl = lg[i][tg[i] - 3] if 3 <= tg[i] < 10 else 0.0
        assert st[i, 0] == m and abs(st[i, 1] - se) < 1e-13 and st[i, 2] == tl


@pytest.mark.parametrize("causal", [False, True])
def test_flop_count_matches_torch_counter(causal):
    """layer_flops against counts it does not compute itself: torch's
    FlopCounterMode over a forward + backward of the torch-module layer (it
    counts the projection and MLP products, forward and both gradients; the
    fused attention kernel is not counted), plus the attention products
    counted per visible (query, key) pair by brute force: QK^T and PV each
    2d flops per pair, three times for forward, dgrad and the other operand's
    gradient."""
    from torch.utils.flop_counter import FlopCounterMode
    cfg = synth.tiny_config(causal=causal, mask_rows=None, seq=7, micro_batch=2, heads=2, head_dim=8, hidden=16,
                            ffn=64, vocab=12, tp=1)
    rep, shards, p = _tiny_inputs(cfg)
    counter = FlopCounterMode(display=False)
    with counter:
        xt, out, _, _ = _torch_layer(cfg, p, rep.x, rep.targets, rep.mask, with_loss=False)
        (out * T(rng(3).standard_normal(tuple(out.shape)))).sum().backward()
    visible = sum(1 for i in range(cfg.seq) for j in range(cfg.seq) if not cfg.causal or j <= i)
    attention = 3 * cfg.micro_batch * cfg.heads * visible * 2 * (2 * cfg.head_dim)
    assert O.layer_flops(cfg)["layer"] == counter.get_total_flops() + attention


def test_flop_count_of_the_gpt2_layer():
    # 3 x forward flops of the GPT-2 355M layer at 8 x 1024 tokens (one TP rank of one), causal
    # attention over visible pairs only: 670.1 GFLOP
    assert round(O.layer_flops(synth.get_config("gpt2_355m_t1"))["layer"] / 1e9, 1) == 670.1


# ---------------------------------------------------------------------------
# vocabulary-parallel input embedding (guide page section 3.3)

@pytest.mark.parametrize("t", [1, 2, 4])
def test_embedding_partials_sum_to_the_lookup(t):
    """Each rank looks up only its vocabulary rows; the all-reduce of the
    partials is torch's embedding lookup over the whole table, exactly."""
    g = np.random.default_rng(7)
    V, h, n = 64, 24, 200
    E = g.standard_normal((V, h))
    tok = g.integers(0, V, size=n)
    tok[:10] = tok[10]                      # repeated ids
    ref = F.embedding(torch.from_numpy(tok), torch.from_numpy(E)).numpy()
    vr = V // t
    parts = [O.embedding_fwd_shard(tok, E[r * vr:(r + 1) * vr], r * vr) for r in range(t)]
    np.testing.assert_array_equal(sum(parts), ref)
    # a row is non-zero on exactly the rank that owns its id
    owner = tok // vr
    for r, p in enumerate(parts):
        assert np.all(np.any(p != 0, axis=1) == (owner == r))


@pytest.mark.parametrize("t", [1, 4])
def test_embedding_bwd_matches_autograd(t):
    g = np.random.default_rng(8)
    V, h, n = 48, 16, 300
    E = torch.from_numpy(g.standard_normal((V, h))).requires_grad_(True)
    tok = g.integers(0, 12, size=n)          # heavily repeated ids
    tok[-5:] = g.integers(12, V, size=5)
    G = g.standard_normal((n, h))
    (F.embedding(torch.from_numpy(tok), E) * torch.from_numpy(G)).sum().backward()
    vr = V // t
    grads = [O.embedding_bwd_shard(tok, G, r * vr, vr) for r in range(t)]
    np.testing.assert_allclose(np.concatenate(grads), E.grad.numpy(), rtol=1e-13, atol=1e-13)


def test_embedding_bwd_brute_force_and_out_of_range_ids():
    g = np.random.default_rng(9)
    vr, h, v0 = 6, 5, 6
    tok = np.array([6, 7, 6, 11, 0, 12, -1, 6, 9, 100])
    G = g.standard_normal((len(tok), h))
    want = np.zeros((vr, h))
    for i, tid in enumerate(tok):
        if v0 <= tid < v0 + vr:
            for c in range(h):
                want[tid - v0, c] += G[i, c]
    np.testing.assert_allclose(O.embedding_bwd_shard(tok, G, v0, vr), want, rtol=0, atol=1e-15)
    E = g.standard_normal((vr, h))
    out = O.embedding_fwd_shard(tok, E, v0)
    assert np.all(out[[4, 5, 6, 9]] == 0)     # ids outside [v0, v0+vr) give zero rows
    np.testing.assert_array_equal(out[0], E[0])
