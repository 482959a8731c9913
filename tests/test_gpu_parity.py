"""Whole-pass parity of the HIP path against the oracle, per workload (GPU).

Each case runs one pass (layer forward, vocabulary-parallel loss forward and
backward, layer backward) through the C ABI and compares every output --
partials, sums, statistics, loss, activation gradients, weight gradients --
with the float64 oracle on the same seeded inputs, under the gate of
oracle/compare.py: fp32 1e-4; bf16 2e-2 relative with a 1e-2 RMS-relative
floor, every element within the band widened by one bf16 rounding of the
terms that form it (the oracle's magnitudes), no element out of band.
Full-size workloads are computed whole by the oracle.
"""
import dataclasses

import numpy as np
import pytest

import synth
from parity_util import build_case, check_case, run_gpu

pytestmark = pytest.mark.gpu

# Small shapes that cover ragged tiles, every head size, both masks, the
# loss mask, a single-token sequence and an all-ranks TP group.
SMALL = [
    synth.tiny_config("f32", hidden=128, heads=2, head_dim=64, ffn=512, tp=1, seq=70, micro_batch=2,
                      vocab=96, causal=True, sigma_w=0.05, index=50, name="small_f32_ragged"),
    synth.tiny_config("bf16", hidden=256, heads=4, head_dim=64, ffn=1024, tp=2, seq=100, micro_batch=3,
                      vocab=1040, causal=True, sigma_w=0.05, index=51, name="small_bf16_t2_ragged"),
    synth.tiny_config("bf16", hidden=192, heads=2, head_dim=96, ffn=768, tp=1, seq=77, micro_batch=2,
                      vocab=264, causal=False, sigma_w=0.05, mask_rows=40, index=52, name="small_bf16_d96_bidir"),
    synth.tiny_config("bf16", hidden=256, heads=2, head_dim=128, ffn=1024, tp=2, seq=130, micro_batch=1,
                      vocab=512, causal=True, sigma_w=0.05, index=53, name="small_bf16_d128"),
    synth.tiny_config("bf16", hidden=128, heads=2, head_dim=64, ffn=512, tp=1, seq=1, micro_batch=5,
                      vocab=64, causal=True, sigma_w=0.05, index=54, name="small_bf16_seq1"),
    synth.tiny_config("f32", hidden=192, heads=2, head_dim=96, ffn=384, tp=2, seq=75, micro_batch=2,
                      vocab=144, causal=False, sigma_w=0.05, index=59, name="small_f32_d96_bidir"),
    synth.tiny_config("f32", hidden=256, heads=2, head_dim=128, ffn=512, tp=1, seq=130, micro_batch=1,
                      vocab=128, causal=True, sigma_w=0.05, index=60, name="small_f32_d128"),
]


def _assert_ok(report):
    bad = {k: v for k, v in report.items() if not v["ok"]}
    assert not bad, f"parity failures: {sorted(bad)}"


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small_shapes(cfg):
    report, st = check_case(cfg)
    _assert_ok(report)


@pytest.mark.parametrize("name,ranks", [
    ("tiny_f32_t2", None),
    ("gpt2_355m_t1", None),
    ("gpt_8p3b_t8", [0]),
    ("gpt_8p3b_t8", [7]),
    ("bert_3p9b_t4", [0]),
    ("gpt_175b_t8", [0]),
])
def test_workload(name, ranks):
    cfg = synth.get_config(name)
    report, st = check_case(cfg, ranks)
    _assert_ok(report)
    # four all-reduce stand-ins per layer forward+backward, plus one for the loss gradient
    assert st.exchanges == 5


def test_bitwise_repeatable():
    cfg = synth.get_config("gpt2_355m_t1")
    small = dataclasses.replace(cfg, micro_batch=2, name="gpt2_mb2")
    rep, shards, peers, pstats = build_case(small)
    a, _ = run_gpu(small, rep, shards, peers, pstats)
    b, _ = run_gpu(small, rep, shards, peers, pstats)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


@pytest.mark.parametrize("cfg", [SMALL[0], SMALL[1], synth.CONFIGS["gpt2_355m_t1"]], ids=lambda c: c.name)
def test_recompute_backward_matches_stash(cfg):
    """Activation recomputation: with every forward stash overwritten after
    the forward, the recomputing backward gives bitwise the stash-based
    results."""
    import torch
    from tensor_transformer_layer_03_amd.step import LayerStep
    rep, shards, peers, peer_stats = build_case(cfg)
    dev = {r: synth.device_shard(cfg, s) for r, s in shards.items()}
    a = LayerStep(cfg, rep, dev, peers, peer_stats)
    a.step()
    b = LayerStep(cfg, rep, dev, peers, peer_stats, recompute=True)
    b.forward()
    b.xent_forward()
    b.xent_backward()
    b.poison_saved()
    b.backward()
    torch.cuda.synchronize()
    ra, rb = a.results(), b.results()
    for k in ra:
        assert np.array_equal(ra[k], rb[k], equal_nan=True), k


@pytest.mark.parametrize("name,ranks", [("gpt2_355m_t1", None), ("gpt_175b_t8", [0])])
def test_recompute_backward_matches_oracle(name, ranks):
    """Activation recomputation (overview page section 3: checkpointing):
    the backward that rebuilds each block's forward stash from the block
    input, run after every stash was overwritten, against the oracle."""
    cfg = synth.get_config(name)
    report, st = check_case(cfg, ranks, recompute=True)
    _assert_ok(report)
    assert st.exchanges == 5


@pytest.mark.parametrize("split,bwd_pair", [("0", "0"), ("1", "0"), ("1", "1")])
@pytest.mark.parametrize("cfg", [SMALL[1], SMALL[2], SMALL[3]], ids=lambda c: c.name)
def test_attention_wave_forms(cfg, split, bwd_pair, monkeypatch):
    """Both attention kernel forms on every head size: four waves per 128
    rows, and eight waves with the looped tiles dealt over two wave groups
    (chosen automatically when the grid is small; forced here), the latter's
    backward as two launches or as the two roles of one launch."""
    monkeypatch.setenv("TPL_ATTN_SPLIT", split)
    monkeypatch.setenv("TPL_ATTN_BWD_PAIR", bwd_pair)
    report, st = check_case(cfg)
    _assert_ok(report)


# 2200 rows, hidden 1152 (4.5 tiles of 256), ffn 2432 (9.5 tiles): deep enough over the
# tokens that every paired weight gradient splits over K in two, the QKV and fc1 activation
# gradients split too, so the launch after each pair runs its slice sums and its bias-gradient
# column work (partials after the QKV pair, the final sum after the fc2 pair) on ragged tiles
PAIR_SPLITS = synth.tiny_config("bf16", hidden=1152, heads=9, head_dim=128, ffn=2432, tp=1, seq=1100,
                                micro_batch=2, vocab=256, causal=True, sigma_w=0.02, index=61,
                                name="small_bf16_pair_splits")


@pytest.mark.parametrize("pair,tile", [("0", "256"), ("1", "256"), ("1", "128")])
@pytest.mark.parametrize("cfg", [SMALL[1], SMALL[2], SMALL[3], PAIR_SPLITS], ids=lambda c: c.name)
def test_paired_backward_products(cfg, pair, tile, monkeypatch):
    """Each block's activation- and weight-gradient products in one launch
    (chosen automatically where it fills the CUs better, e.g. the 175B rank;
    forced on and off here on ragged shapes, on 256x256 tiles and, for the
    pairs without an epilogue, on 128x128 tiles, with the fc2 pair's GeLU'
    epilogue and bias-gradient column partials, and with splits over K and
    the follow-on launch's sums on the deeper case)."""
    monkeypatch.setenv("TPL_GEMM_PAIR", pair)
    monkeypatch.setenv("TPL_GEMM_PAIR_TILE", tile)
    report, st = check_case(cfg)
    _assert_ok(report)


WIDE = [
    synth.tiny_config("f32", hidden=768, heads=12, head_dim=64, ffn=1536, tp=2, seq=40, micro_batch=2,
                      vocab=128, causal=True, sigma_w=0.05, index=56, name="small_f32_wide_rows"),
    # weights at the workloads' scale: with N(0, 0.05) at this width the logits have std ~3 and the
    # bf16-rounded logits alone put the loss gradient ~1.5% off the float64 oracle
    synth.tiny_config("bf16", hidden=1280, heads=10, head_dim=128, ffn=2560, tp=2, seq=33, micro_batch=2,
                      vocab=256, causal=False, sigma_w=0.02, index=57, name="small_bf16_wide_rows"),
    # 23 heads x 96: the output projection's input gradient ([128, 2208], K = 2208) splits over K in
    # two, the last split 1056 deep, so its last K-tile is ragged at a moved base
    synth.tiny_config("bf16", hidden=2208, heads=23, head_dim=96, ffn=4416, tp=1, seq=64, micro_batch=2,
                      vocab=256, causal=True, sigma_w=0.02, index=58, name="small_bf16_split_ragged_k"),
]


@pytest.mark.parametrize("cfg", WIDE, ids=lambda c: c.name)
def test_wide_rows(cfg):
    """Hidden sizes past two 16-B chunks per lane (fp32 > 512, bf16 > 1024):
    LayerNorm forward and backward rows run one four-wave workgroup per row,
    here with a row that leaves part of the workgroup's threads idle."""
    report, st = check_case(cfg)
    _assert_ok(report)
