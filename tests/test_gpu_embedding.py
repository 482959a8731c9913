"""Parity of the vocabulary-parallel input embedding (guide page section 3.3)
through the C ABI against the oracle: the rank's masked lookup exactly, the
scatter-add gradient within the fp32 tolerance, bitwise repeatable (GPU).
The gradient's documented summation order (each vocabulary row adds its
gradient rows in ascending row order, in fp32) is checked bit for bit
against that sum done row by row in numpy, which fails if the sort behind it
is not stable. The cases cover the one-workgroup in-LDS sort (up to 8192
rows) and the multi-pass sort beyond it."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tensor_transformer_layer_03_amd import binding as B

pytestmark = pytest.mark.gpu

CASES = [
    # (config, ranks, skew): skew > 0 draws ids from the first `skew` ids only
    (synth.CONFIGS["tiny_f32_t2"], [0, 1], 0),
    (synth.tiny_config("bf16", hidden=256, heads=4, head_dim=64, ffn=768, tp=2, seq=77, micro_batch=3, vocab=1040,
                       index=71, name="small_bf16_t2_ragged"), [0, 1], 0),
    (synth.tiny_config("bf16", hidden=128, heads=2, head_dim=64, ffn=512, tp=2, seq=300, micro_batch=2, vocab=4096,
                       index=72, name="small_bf16_skewed"), [0, 1], 3),
    (synth.CONFIGS["gpt2_355m_t1"], [0], 0),
    (synth.CONFIGS["gpt2_355m_t1"], [0], 40),
    (synth.CONFIGS["gpt_8p3b_t8"], [0, 7], 0),
    # 8000 rows, 8 per thread of the in-LDS sort, two ids only: long runs of equal keys
    (synth.tiny_config("bf16", hidden=128, heads=2, head_dim=64, ffn=256, tp=2, seq=1000, micro_batch=8, vocab=4096,
                       index=73, name="small_bf16_8000_rows_skewed"), [0, 1], 2),
    # 9216 rows: beyond the in-LDS sort
    (synth.tiny_config("bf16", hidden=128, heads=2, head_dim=64, ffn=256, tp=2, seq=1024, micro_batch=9, vocab=4096,
                       index=74, name="small_bf16_9216_rows"), [0, 1], 0),
    (synth.tiny_config("bf16", hidden=128, heads=2, head_dim=64, ffn=256, tp=2, seq=1024, micro_batch=9, vocab=4096,
                       index=75, name="small_bf16_9216_rows_skewed"), [0, 1], 5),
    (synth.tiny_config("f32", hidden=64, heads=1, head_dim=64, ffn=64, tp=1, seq=1, micro_batch=1, vocab=16,
                       index=76, name="one_row"), [0], 0),
]


def _ascending_sum(tok, dout, v0, vr):
    """fp32 sum of each vocabulary row's gradient rows, in ascending row order."""
    acc = np.zeros((vr, dout.shape[1]), np.float32)
    for i, t in enumerate(tok):
        if v0 <= t < v0 + vr:
            acc[t - v0] += dout[i]
    return acc


def _dev(a, dtype):
    a = np.ascontiguousarray(a, np.float32)
    if dtype == "bf16":
        return torch.from_numpy(synth.bf16_bits(a)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _run(cfg, r, tok, emb, dout):
    desc = B.make_desc(cfg.hidden, cfg.heads, cfg.head_dim, cfg.ffn, cfg.tp, r, cfg.seq, cfg.micro_batch, cfg.vocab,
                       cfg.causal, cfg.dtype)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    t_tok = torch.from_numpy(tok).cuda()
    part = torch.full((cfg.rows, cfg.hidden), float("nan"), dtype=dt, device="cuda")
    grad = torch.full((cfg.vocab_r, cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.vocab_parallel_embedding_ws_bytes(desc), dtype=torch.uint8, device="cuda")
    B.vocab_parallel_embedding_fwd(desc, t_tok, _dev(emb, cfg.dtype), part)
    B.vocab_parallel_embedding_bwd(desc, t_tok, _dev(dout, cfg.dtype), grad, ws)
    torch.cuda.synchronize()
    return part.float().cpu().numpy(), grad.cpu().numpy()


@pytest.mark.parametrize("cfg,ranks,skew", CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_embedding(cfg, ranks, skew):
    tok = synth.input_tokens(cfg, skew)
    tok[::97] = cfg.vocab + 5                      # ids outside [0, V) contribute nothing
    tok[1::101] = -3
    dout = synth.embedding_grad_in(cfg)
    parts = []
    for r in ranks:
        emb = synth.input_emb_shard(cfg, r)
        got_p, got_g = _run(cfg, r, tok, emb, dout)
        want_p = O.embedding_fwd_shard(tok, emb, r * cfg.vocab_r)
        np.testing.assert_array_equal(got_p, want_p)     # a copy: exact
        want_g = O.embedding_bwd_shard(tok, dout, r * cfg.vocab_r, cfg.vocab_r)
        rep = O.compare.compare_tensor(got_g, want_g, "f32")
        print(cfg.name, r, rep)
        assert rep["ok"], rep
        stored = synth.round_to_bf16(dout) if cfg.dtype == "bf16" else np.asarray(dout, np.float32)
        assert np.array_equal(got_g, _ascending_sum(tok, stored, r * cfg.vocab_r, cfg.vocab_r))
        parts.append(got_p)
        # deterministic: a second run is bitwise equal
        got_p2, got_g2 = _run(cfg, r, tok, emb, dout)
        assert np.array_equal(got_g, got_g2) and np.array_equal(got_p, got_p2)
    if len(ranks) == cfg.tp:   # all ranks present: the all-reduce of the partials is the whole lookup
        full = np.concatenate([synth.input_emb_shard(cfg, r) for r in range(cfg.tp)])
        ok = (tok >= 0) & (tok < cfg.vocab)
        want = np.zeros((cfg.rows, cfg.hidden))
        want[ok] = full[tok[ok]]
        np.testing.assert_array_equal(sum(parts), want)
