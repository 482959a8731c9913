"""Pins of the parity gate's rounding allowance (CPU only).

oracle.magnitude gives, for every output of the pass, the magnitude M of
the terms that form it; the bf16 gate admits |g - r| <= atol * min(1, rms(r)) +
rtol * |r| + 2^-8 * M on every element. Pinned here:

* each magnitude rule against a brute-force loop over the terms it names,
  and the bound it states (Cauchy-Schwarz for products, the LayerNorm and
  attention backward's values within their magnitudes);
* M >= |r| for every output of whole passes (triangle inequality), with
  stand-in ranks and a masked loss included;
* the gate accepts an independent mixed-precision implementation of the
  pass -- torch's CPU kernels with every intermediate stored in bf16
  (tests/torch_group.py) -- on every element of every output, while
  without the allowance it would not;
* the same bf16 implementation with a planted mistake (a stand-in left out
  of a sum, the causal mask off, R missing from the loss gradient, the fc1
  bias dropped, a wrong attention scale) is rejected.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle import magnitude as MG
import synth
from torch_group import torch_group


def rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ rules vs loops

def _norm(xs):
    return math.sqrt(sum(x * x for x in xs))


def test_product_and_column_sums_brute_force():
    g = rng(1)
    a, b = g.standard_normal((3, 5)), g.standard_normal((5, 4))
    m = MG.product(a, b)
    for i in range(3):
        for j in range(4):
            want = _norm(a[i, :]) * _norm(b[:, j])
            assert math.isclose(m[i, j], want, rel_tol=1e-13)
            # Cauchy-Schwarz: at least the componentwise magnitude, hence at least |value|
            assert m[i, j] >= sum(abs(a[i, k] * b[k, j]) for k in range(5)) * (1 - 1e-13)
    # a relative change u of a row in the 2-norm moves the product by at most u * M
    d = g.standard_normal((3, 5))
    d *= 1e-3 * np.linalg.norm(a, axis=1, keepdims=True) / np.linalg.norm(d, axis=1, keepdims=True)
    assert np.all(np.abs(d @ b) <= 1e-3 * m * (1 + 1e-12))
    cs = MG.sum_rows(a)
    for j in range(5):
        assert math.isclose(cs[j], math.sqrt(3) * _norm(a[:, j]), rel_tol=1e-13)
        assert cs[j] >= sum(abs(a[i, j]) for i in range(3)) * (1 - 1e-13)
    c = g.standard_normal((3, 5))
    cp = MG.col_product(a, c)
    for j in range(5):
        assert math.isclose(cp[j], _norm(a[:, j]) * _norm(c[:, j]), rel_tol=1e-13)


def test_layernorm_backward_magnitude_brute_force():
    g = rng(2)
    n, h = 3, 6
    md, xhat, rstd, gam = np.abs(g.standard_normal((n, h))), g.standard_normal((n, h)), 1 + g.random(n), \
        g.standard_normal(h)
    m = MG.ln_bwd(md, xhat, rstd, gam)
    for i in range(n):
        gg = [md[i, j] * abs(gam[j]) for j in range(h)]
        mean_g = sum(gg) / h
        mean_gx = sum(gg[j] * abs(xhat[i, j]) for j in range(h)) / h
        for j in range(h):
            assert math.isclose(m[i, j], rstd[i] * (gg[j] + mean_g + abs(xhat[i, j]) * mean_gx), rel_tol=1e-13)
    # it bounds the LayerNorm backward it describes: |LN_bwd(d)| <= M(|d|)
    d = g.standard_normal((n, h))
    din, _, _ = O.layernorm_bwd(d, xhat, rstd, gam)
    assert np.all(np.abs(din) <= MG.ln_bwd(np.abs(d), xhat, rstd, gam) * (1 + 1e-12))


def test_attention_gradient_magnitude_brute_force():
    g = rng(5)
    s, d = 5, 4
    q, k, v, do = (g.standard_normal((s, d)) for _ in range(4))
    o, _, probs = O.attention_head_fwd(q, k, v, True)
    mq, mk, mv = MG.attention_grad(q, k, v, o, probs, do)
    dp = do @ v.T
    delta = (do * o).sum(1)
    mds = [[probs[i, j] * (abs(dp[i, j]) + abs(delta[i])) for j in range(s)] for i in range(s)]
    for i in range(s):
        for c in range(d):
            assert math.isclose(mq[i, c], _norm(mds[i]) * _norm(k[:, c]) / math.sqrt(d), rel_tol=1e-12)
            assert math.isclose(mk[i, c], _norm([mds[r][i] for r in range(s)]) * _norm(q[:, c]) / math.sqrt(d),
                                rel_tol=1e-12)
            assert math.isclose(mv[i, c], _norm(probs[:, i]) * _norm(do[:, c]), rel_tol=1e-12)
    dq, dk, dv = O.attention_head_bwd(q, k, v, o, probs, do)
    for got, m in ((dq, mq), (dk, mk), (dv, mv)):
        assert np.all(np.abs(got) <= m * (1 + 1e-12))


def test_logit_statistics_magnitudes_brute_force():
    g = rng(3)
    n, h, vr, v0 = 4, 5, 6, 6
    H, E = g.standard_normal((n, h)), g.standard_normal((vr, h))
    tg = np.array([6, 13, 8, 2])
    lg = H @ E.T
    lse_local = np.log(np.exp(lg).sum(1))
    m = MG.logit_stats(H, E, lg, lse_local, tg, v0)
    for i in range(n):
        ml = [_norm(H[i]) * _norm(E[j]) for j in range(vr)]
        assert math.isclose(m[i, 0], ml[int(np.argmax(lg[i]))], rel_tol=1e-13)
        p = np.exp(lg[i] - lse_local[i])
        assert math.isclose(m[i, 1], abs(lse_local[i]) + sum(p[j] * ml[j] for j in range(vr)), rel_tol=1e-13)
        t = tg[i] - v0
        assert m[i, 2] == (pytest.approx(ml[t], rel=1e-13) if 0 <= t < vr else 0.0)
    sw = MG.softmax_weighted(H, E, lg, lse_local)
    assert np.allclose(sw, m[:, 1] - np.abs(lse_local), rtol=1e-13)


def test_loss_gradient_magnitude_brute_force():
    g = rng(4)
    n, h, vr = 5, 3, 4
    H, E = g.standard_normal((n, h)), g.standard_normal((vr, h))
    lg = H @ E.T
    lse = np.log(np.exp(lg).sum(1)) + 0.3              # a shard of a larger vocabulary
    w = np.array([1.0, 0.0, 1.0, 1.0, 0.0])
    gr = w / w.sum()
    dl = np.exp(lg - lse[:, None]) * gr[:, None]
    dl[0, 2] -= gr[0]
    m_lse = np.abs(g.standard_normal(n))
    m = MG.loss_grad(dl, H, E, lg, lse, m_lse, gr)
    for i in range(n):
        for j in range(vr):
            ml = _norm(H[i]) * _norm(E[j])
            want = abs(dl[i, j]) + gr[i] * math.exp(lg[i, j] - lse[i]) * (ml + m_lse[i])
            assert math.isclose(m[i, j], want, rel_tol=1e-13, abs_tol=1e-300)


# ------------------------------------------------------------------ whole passes

def _case(tp, ranks, causal=True, mask_rows=None, hidden=256, heads=4, head_dim=64, ffn=1024, seq=128,
          micro_batch=2, vocab=2048, index=95):
    cfg = synth.tiny_config("bf16", hidden=hidden, heads=heads, head_dim=head_dim, ffn=ffn, tp=tp, seq=seq,
                            micro_batch=micro_batch, vocab=vocab, causal=causal, sigma_w=0.02, mask_rows=mask_rows,
                            index=index)
    rep = synth.replicated_inputs(cfg)
    shards = {r: synth.rank_shard(cfg, r) for r in ranks}
    n_peers = tp - len(ranks)
    peers = synth.peer_partials(cfg, n_peers) if n_peers else []
    pst = [synth.peer_stats(cfg, r) for r in range(tp) if r not in ranks]
    return cfg, rep, shards, peers, pst


def _oracle(cfg, rep, shards, peers, pst):
    prs = {r: synth.oracle_params(cfg, [s], rep) for r, s in shards.items()}
    mags = {}
    ref = O.step_reference(prs, rep.x, rep.dout, rep.targets, rep.mask, seq=cfg.seq, causal=cfg.causal,
                           eps=cfg.ln_eps, tp=cfg.tp, vocab_r=cfg.vocab_r, peers=peers, peer_stats=pst,
                           use_mask=cfg.mask_rows is not None, mags=mags)
    return ref, mags


CASES = {
    "t2_all_ranks_causal": dict(tp=2, ranks=[0, 1]),
    "t4_rank1_stand_ins_bidirectional_masked": dict(tp=4, ranks=[1], causal=False, mask_rows=40),
    "t2_head96_ragged": dict(tp=2, ranks=[0, 1], hidden=384, heads=4, head_dim=96, ffn=768, seq=77, vocab=528,
                             index=96),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_magnitudes_bound_every_output(name):
    ref, mags = _oracle(*_case(**CASES[name]))
    cols = O.compare.stats_columns
    for k, r in ref.items():
        m = mags[k]
        if k.startswith("stats@"):
            rc = cols(r)
            for j, c in enumerate(("max", "lse", "tl")):
                assert np.all(m[:, j] >= np.abs(rc[c]) * (1 - 1e-12)), (k, c)
            continue
        assert m.shape == np.shape(r), k
        assert np.all(m >= np.abs(r) * (1 - 1e-12) - 1e-300), k


@pytest.mark.parametrize("name", sorted(CASES))
def test_gate_accepts_an_independent_bf16_pass(name):
    case = _case(**CASES[name])
    ref, mags = _oracle(*case)
    got = torch_group(*case, cdt=torch.bfloat16)
    rep = O.compare.compare_all(got, ref, "bf16", mags)
    bad = {k: v for k, v in rep.items() if not v["ok"]}
    assert not bad, O.compare.format_report(bad)
    # the rounding allowance is what admits it: the stated band alone rejects outputs formed by cancellation
    plain = O.compare.compare_all(got, ref, "bf16", None)
    assert any(not v["ok_band"] for v in plain.values())


SLIP_CASES = [("t4_rank1_stand_ins_bidirectional_masked", s) for s in
              ("peers_dropped_from_mlp_sum", "r_missing_from_dout", "b1_dropped", "attention_scale_off")] + \
             [("t2_all_ranks_causal", s) for s in ("no_causal_mask", "r_missing_from_dout", "b1_dropped",
                                                   "attention_scale_off")]


@pytest.mark.parametrize("name,slip", SLIP_CASES)
def test_gate_rejects_a_planted_mistake(name, slip):
    case = _case(**CASES[name])
    ref, mags = _oracle(*case)
    got = torch_group(*case, cdt=torch.bfloat16, slip=slip)
    rep = O.compare.compare_all(got, ref, "bf16", mags)
    assert any(not v["ok"] for v in rep.values()), slip
