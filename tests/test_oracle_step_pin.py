"""Pin of the oracle's whole-pass composition (oracle.step_reference) against
torch autograd in float64 (CPU only).

step_reference chains the oracle's blocks the way the GPU pass does: each
rank's restricted partials, the five all-reduce stand-ins (attention output,
MLP output, loss gradient + R, each block's LayerNorm-output gradient), the
vocabulary shards' statistics combined by log-sum-exp, and the replicated
LayerNorm backward. tests/torch_group.py writes the same objective directly
as a torch graph of one TP group (each rank's branch its own sub-graph of
torch library ops, stand-in ranks as constants added to the sums, the
stand-in statistics as extra log-sum-exp entries), in float64 here.

Every gradient is then torch.autograd's, so the five sums (each peer exactly
once, R in the loss gradient), the vocabulary offsets and the replicated
phase are checked against code that shares nothing with the oracle. The
mutation test plants slips in the composition and asserts the pin catches
each of them.
"""
import math

import numpy as np
import pytest

import oracle as O
import oracle.step as OS
import synth
from torch_group import torch_group as _torch_group


def _case(tp, ranks, causal=True, mask_rows=None):
    cfg = synth.tiny_config(hidden=16, heads=4, head_dim=4, ffn=32, tp=tp, seq=5, micro_batch=2, vocab=24,
                            causal=causal, sigma_w=0.3, mask_rows=mask_rows, index=91 + tp)
    rep = synth.replicated_inputs(cfg)
    shards = {r: synth.rank_shard(cfg, r) for r in ranks}
    n_peers = tp - len(ranks)
    peers = synth.peer_partials(cfg, n_peers, scale=0.3) if n_peers else []
    peer_stats = [synth.peer_stats(cfg, r) for r in range(tp) if r not in ranks]
    return cfg, rep, shards, peers, peer_stats


def _oracle(cfg, rep, shards, peers, peer_stats):
    prs = {r: synth.oracle_params(cfg, [s], rep) for r, s in shards.items()}
    return O.step_reference(prs, rep.x, rep.dout, rep.targets, rep.mask, seq=cfg.seq, causal=cfg.causal,
                            eps=cfg.ln_eps, tp=cfg.tp, vocab_r=cfg.vocab_r, peers=peers, peer_stats=peer_stats,
                            use_mask=cfg.mask_rows is not None)


def _mismatches(ref, got):
    bad = []
    for k in ref:
        if k not in got:
            bad.append(k)
            continue
        a, b = np.asarray(got[k], np.float64), np.asarray(ref[k], np.float64)
        if a.shape != b.shape or not np.allclose(a, b, rtol=1e-9, atol=1e-11 * max(1.0, np.abs(b).max())):
            bad.append(k)
    return bad


CASES = [
    pytest.param(2, [0, 1], True, None, id="t2_all_ranks_causal"),
    pytest.param(2, [0, 1], False, 4, id="t2_all_ranks_bidirectional_masked_loss"),
    pytest.param(4, [1], True, None, id="t4_rank1_with_stand_ins"),
    pytest.param(4, [3], False, 3, id="t4_rank3_with_stand_ins_bidirectional_masked_loss"),
]


@pytest.mark.parametrize("tp,ranks,causal,mask_rows", CASES)
def test_step_reference_matches_torch_autograd(tp, ranks, causal, mask_rows):
    cfg, rep, shards, peers, peer_stats = _case(tp, ranks, causal, mask_rows)
    ref = _torch_group(cfg, rep, shards, peers, peer_stats)
    got = _oracle(cfg, rep, shards, peers, peer_stats)
    assert set(got) == set(ref), sorted(set(got) ^ set(ref))
    assert not _mismatches(ref, got), _mismatches(ref, got)


def test_all_ranks_equal_the_unsharded_layer():
    """With every rank of t = 2 present, the summed partials and the gradients
    of the replicated parameters are the plain layer's (torch MultiheadAttention
    and Linear modules in the oracle pins use the same unsharded weights)."""
    cfg, rep, shards, peers, peer_stats = _case(2, [0, 1])
    got = _oracle(cfg, rep, shards, peers, peer_stats)
    p_full = synth.oracle_params(cfg, [shards[0], shards[1]], rep)
    out, cache = O.layer_fwd(rep.x, p_full, cfg.seq, cfg.causal, cfg.ln_eps)
    np.testing.assert_allclose(got["out"], out, rtol=1e-12, atol=1e-13)
    loss, _, _ = O.xent_full(out, p_full["emb"], rep.targets)
    assert abs(got["loss"][0] - loss) <= 1e-12 * abs(loss)


# ------------------------------------------------------------------ planted slips

def _mutate_sum(call_to_break, how):
    """A partial_sum that misbehaves on its n-th call (0-based):
    'twice' adds the stand-in peers a second time, 'drop_residual' drops
    the residual term (R for the loss-gradient sum), 'drop_peers' leaves
    the stand-ins out."""
    real = O.partial_sum
    calls = {"n": 0}

    def fake(partials, bias=None, residual=None):
        n = calls["n"]
        calls["n"] += 1
        if n != call_to_break:
            return real(partials, bias, residual)
        partials = list(partials)
        if how == "twice":
            return real(partials + partials[-1:], bias, residual)
        if how == "drop_residual":
            return real(partials, bias, None)
        if how == "drop_peers":
            return real(partials[:1], bias, residual)
        raise ValueError(how)
    return fake


SLIPS = [("sum", i, how) for i in range(5) for how in ("twice", "drop_peers")] + [("sum", 2, "drop_residual"),
                                                                                  ("vocab_offset", 0, None),
                                                                                  ("mask_ignored", 0, None)]


@pytest.mark.parametrize("kind,i,how", SLIPS, ids=lambda v: str(v))
def test_planted_slips_are_caught(kind, i, how, monkeypatch):
    """Each slip in the composition -- a stand-in added twice to one of the
    five sums or left out of it, R left out of the loss gradient, the wrong
    vocabulary offset, the loss mask ignored -- makes the pin above fail."""
    cfg, rep, shards, peers, peer_stats = _case(4, [1], mask_rows=6)
    ref = _torch_group(cfg, rep, shards, peers, peer_stats)
    if kind == "sum":
        monkeypatch.setattr(OS, "partial_sum", _mutate_sum(i, how))
    elif kind == "vocab_offset":
        real = OS.xent_local_stats
        monkeypatch.setattr(OS, "xent_local_stats", lambda lg, tg, v0: real(lg, tg, 0))
    elif kind == "mask_ignored":
        real_finish = OS.xent_finish
        monkeypatch.setattr(OS, "xent_finish", lambda st, m=None: real_finish(st, None))
    got = _oracle(cfg, rep, shards, peers, peer_stats)
    assert _mismatches(ref, got), "slip not caught"


def test_loss_gradient_carries_r_once():
    """dout = R + sum of the ranks' dH (+ stand-ins): with the loss gradient
    scaled to zero the oracle's dout is R + sum(P) exactly."""
    cfg, rep, shards, peers, peer_stats = _case(4, [2])
    prs = {r: synth.oracle_params(cfg, [s], rep) for r, s in shards.items()}
    got = O.step_reference(prs, rep.x, rep.dout, rep.targets, rep.mask, seq=cfg.seq, causal=cfg.causal,
                           eps=cfg.ln_eps, tp=cfg.tp, vocab_r=cfg.vocab_r, peers=peers, peer_stats=peer_stats,
                           dloss=0.0)
    want = np.asarray(rep.dout, np.float64) + sum(np.asarray(p, np.float64) for p in peers)
    np.testing.assert_allclose(got["dout"], want, rtol=1e-15, atol=1e-15)
    assert math.isfinite(got["loss"][0])
