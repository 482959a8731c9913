"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module holds the workload table and the input generators ONLY. It contains
none of the method's arithmetic (no normalisation, projection, attention, GeLU
or loss); it draws random numbers, rounds them to the storage type, and lays
the per-rank weight shards out in the two shapes the consumers want:

* ``oracle_params``: the oracle's view -- per-head / per-column blocks stacked
  in global order (the full layer when every rank is included);
* ``device_shard``: the C-ABI view -- one rank's contiguous buffers, the fused
  QKV weight being ``[Q rows of its heads; K rows; V rows]``.

Sharding follows the Megatron-LM pages: attention is split by heads (podcast
page, Outline: "Self-Attention ... K, Q, V"; rkmt.cn guide, section 3.2), the
first MLP linear by output columns and the second by input rows (rkmt.cn guide,
section 3.1), the output embedding along the vocabulary (rkmt.cn guide,
section 3.3). Rank r owns the contiguous block r of heads, ffn columns and
vocabulary ids.

Every tensor is drawn from its own PCG64 stream keyed by
(1000 + config index, tensor id, rank), so a rank's shard is identical whether
or not the other ranks are generated.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "Config", "CONFIGS", "CONFIG_ORDER", "get_config", "tiny_config",
    "round_to_bf16", "bf16_bits", "ReplicatedInputs", "RankShard",
    "replicated_inputs", "rank_shard", "oracle_params", "device_shard",
    "peer_stats", "peer_partials",
]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    index: int
    dtype: str            # "f32" or "bf16" (storage); accumulation is fp32
    hidden: int
    heads: int
    head_dim: int
    ffn: int
    tp: int
    seq: int
    micro_batch: int
    vocab: int
    causal: bool
    sigma_w: float
    mask_rows: int | None = None   # rows that carry the loss (None = every row)
    all_ranks: bool = True         # run every rank of the TP group on one GPU
    ln_eps: float = 1e-5

    @property
    def rows(self) -> int:
        return self.seq * self.micro_batch

    @property
    def heads_r(self) -> int:
        return self.heads // self.tp

    @property
    def hidden_r(self) -> int:
        return self.hidden // self.tp

    @property
    def ffn_r(self) -> int:
        return self.ffn // self.tp

    @property
    def vocab_r(self) -> int:
        return self.vocab // self.tp

    @property
    def seed(self) -> int:
        return 1000 + self.index

    def ranks(self) -> list[int]:
        """Ranks exercised for this workload: all of them, or (one-rank mode) rank 0."""
        return list(range(self.tp)) if self.all_ranks else [0]


# The five workloads: shapes, sharding, data scales and masks.
CONFIGS = {
    "tiny_f32_t2": Config("tiny_f32_t2", 0, "f32", 256, 4, 64, 1024, 2, 128, 2, 4096,
                          True, 0.02, None, True),
    "gpt2_355m_t1": Config("gpt2_355m_t1", 1, "bf16", 1024, 16, 64, 4096, 1, 1024, 8, 51200,
                           True, 0.02, None, True),
    "gpt_8p3b_t8": Config("gpt_8p3b_t8", 2, "bf16", 3072, 32, 96, 12288, 8, 1024, 4, 51200,
                          True, 0.02, None, False),
    "bert_3p9b_t4": Config("bert_3p9b_t4", 3, "bf16", 2560, 40, 64, 10240, 4, 512, 16, 32768,
                           False, 0.02, 1229, False),
    "gpt_175b_t8": Config("gpt_175b_t8", 4, "bf16", 12288, 96, 128, 49152, 8, 2048, 1, 51200,
                          True, 0.006, None, False),
}
CONFIG_ORDER = list(CONFIGS)


def get_config(name: str) -> Config:
    return CONFIGS[name]


def tiny_config(dtype="f32", hidden=16, heads=2, head_dim=8, ffn=32, tp=1, seq=5,
                micro_batch=2, vocab=12, causal=True, sigma_w=0.3, mask_rows=None,
                index=90, name="tiny") -> Config:
    """Small shapes for brute-force and finite-difference checks."""
    return Config(name, index, dtype, hidden, heads, head_dim, ffn, tp, seq, micro_batch,
                  vocab, causal, sigma_w, mask_rows, True)


# ---------------------------------------------------------------------------
# storage rounding (bit manipulation only)

def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of bf16-representable float32 values."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# random streams

_TENSOR_IDS = {
    "x": 1, "dout": 2, "targets": 3, "mask": 4, "ln1_g": 5, "ln1_b": 6, "ln2_g": 7,
    "ln2_b": 8, "b_o": 9, "b_2": 10, "wq": 11, "wk": 12, "wv": 13, "bq": 14, "bk": 15,
    "bv": 16, "wo": 17, "w1": 18, "b1": 19, "w2": 20, "emb": 21, "h1": 22,
    "dsum_attn": 23, "dsum_mlp": 24, "peer_stats": 25, "peer_partials": 26,
    "tokens": 27, "emb_in": 28, "dx_emb": 29,
}


def _rng(cfg: Config, tensor: str, rank: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([cfg.seed, _TENSOR_IDS[tensor], rank])
    return np.random.Generator(np.random.PCG64(ss))


def _normal(cfg, tensor, shape, scale=1.0, mean=0.0, rank=0) -> np.ndarray:
    a = _rng(cfg, tensor, rank).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    if mean != 0.0:
        a += np.float32(mean)
    return round_to_bf16(a) if cfg.dtype == "bf16" else a


@dataclasses.dataclass
class ReplicatedInputs:
    x: np.ndarray          # [N, h] layer input
    dout: np.ndarray       # [N, h] upstream gradient of the layer output
    targets: np.ndarray    # [N] int32 global vocabulary ids
    mask: np.ndarray       # [N] uint8 (1 = row carries the loss)
    ln1_g: np.ndarray
    ln1_b: np.ndarray
    ln2_g: np.ndarray
    ln2_b: np.ndarray
    b_o: np.ndarray        # row-parallel biases, added once after the partial sum
    b_2: np.ndarray


def replicated_inputs(cfg: Config) -> ReplicatedInputs:
    N, h, sw = cfg.rows, cfg.hidden, cfg.sigma_w
    targets = _rng(cfg, "targets").integers(0, cfg.vocab, size=N, dtype=np.int64).astype(np.int32)
    mask = np.ones(N, np.uint8)
    if cfg.mask_rows is not None:
        mask[:] = 0
        pick = _rng(cfg, "mask").choice(N, size=cfg.mask_rows, replace=False)
        mask[pick] = 1
    return ReplicatedInputs(
        x=_normal(cfg, "x", (N, h)),
        dout=_normal(cfg, "dout", (N, h)),
        targets=targets, mask=mask,
        ln1_g=_normal(cfg, "ln1_g", (h,), sw, 1.0), ln1_b=_normal(cfg, "ln1_b", (h,), sw),
        ln2_g=_normal(cfg, "ln2_g", (h,), sw, 1.0), ln2_b=_normal(cfg, "ln2_b", (h,), sw),
        b_o=_normal(cfg, "b_o", (h,), sw), b_2=_normal(cfg, "b_2", (h,), sw),
    )


@dataclasses.dataclass
class RankShard:
    rank: int
    wq: np.ndarray   # [h_r, h]  rows of this rank's heads, head-major, d rows per head
    wk: np.ndarray
    wv: np.ndarray
    bq: np.ndarray   # [h_r]
    bk: np.ndarray
    bv: np.ndarray
    wo: np.ndarray   # [h, h_r]  columns of this rank's heads
    w1: np.ndarray   # [f_r, h]
    b1: np.ndarray   # [f_r]
    w2: np.ndarray   # [h, f_r]
    emb: np.ndarray  # [V_r, h]  vocabulary rows [rank*V_r, (rank+1)*V_r)


def rank_shard(cfg: Config, r: int, with_emb: bool = True) -> RankShard:
    h, hr, fr, vr, sw = cfg.hidden, cfg.hidden_r, cfg.ffn_r, cfg.vocab_r, cfg.sigma_w
    return RankShard(
        rank=r,
        wq=_normal(cfg, "wq", (hr, h), sw, rank=r), wk=_normal(cfg, "wk", (hr, h), sw, rank=r),
        wv=_normal(cfg, "wv", (hr, h), sw, rank=r),
        bq=_normal(cfg, "bq", (hr,), sw, rank=r), bk=_normal(cfg, "bk", (hr,), sw, rank=r),
        bv=_normal(cfg, "bv", (hr,), sw, rank=r),
        wo=_normal(cfg, "wo", (h, hr), sw, rank=r),
        w1=_normal(cfg, "w1", (fr, h), sw, rank=r), b1=_normal(cfg, "b1", (fr,), sw, rank=r),
        w2=_normal(cfg, "w2", (h, fr), sw, rank=r),
        emb=_normal(cfg, "emb", (vr, h), sw, rank=r) if with_emb else None,
    )


def synthetic_block_inputs(cfg: Config) -> dict:
    """Stand-ins for the values a one-rank run would receive from its peers.

    ``h1``: the MLP block's input (the attention block's all-reduced output);
    ``dsum_attn`` / ``dsum_mlp``: the all-reduced gradients w.r.t. each block's
    LayerNorm output. Drawn N(0,1) (h1) and N(0, 0.05) (gradient sums).
    """
    N, h = cfg.rows, cfg.hidden
    return {
        "h1": _normal(cfg, "h1", (N, h)),
        "dsum_attn": _normal(cfg, "dsum_attn", (N, h), 0.05),
        "dsum_mlp": _normal(cfg, "dsum_mlp", (N, h), 0.05),
    }


def peer_partials(cfg: Config, n: int, scale: float = 0.05) -> list[np.ndarray]:
    """Stand-in partial sums from ``n`` peer ranks, each [N, h]."""
    return [_normal(cfg, "peer_partials", (cfg.rows, cfg.hidden), scale, rank=i) for i in range(n)]


def peer_stats(cfg: Config, rank: int) -> np.ndarray:
    """Plausible per-row cross-entropy statistics (m, se, tl) of another rank's
    vocabulary shard, [N, 3] float32: m ~ 3 + N(0, 0.5), se in [1, V_r],
    tl = 0 except for rows whose target lies in that rank's id range."""
    N, vr = cfg.rows, cfg.vocab_r
    g = _rng(cfg, "peer_stats", rank)
    m = (3.0 + 0.5 * g.standard_normal(N)).astype(np.float32)
    se = (1.0 + (vr - 1.0) * g.random(N)).astype(np.float32)
    tgt = replicated_inputs_targets(cfg)
    inside = (tgt >= rank * vr) & (tgt < (rank + 1) * vr)
    tl = np.where(inside, m - 1.0 - g.random(N), 0.0).astype(np.float32)
    return np.stack([m, se, tl], axis=1)


def replicated_inputs_targets(cfg: Config) -> np.ndarray:
    return _rng(cfg, "targets").integers(0, cfg.vocab, size=cfg.rows, dtype=np.int64).astype(np.int32)


# ---------------------------------------------------------------------------
# layouts

def oracle_params(cfg: Config, shards: list[RankShard], rep: ReplicatedInputs) -> dict:
    """Stack rank shards in global order (full layer if every rank is given).

    Returns float64 arrays: wq/wk/wv [n*h_r, h], bq/bk/bv, wo [h, n*h_r], w1, b1,
    w2, emb [n*V_r, h], LayerNorm and row-parallel bias vectors, and the list of
    ranks plus vocabulary offsets of each included shard.
    """
    f = lambda a: np.asarray(a, np.float64)
    cat0 = lambda name: f(np.concatenate([getattr(s, name) for s in shards], axis=0))
    p = {
        "wq": cat0("wq"), "wk": cat0("wk"), "wv": cat0("wv"),
        "bq": cat0("bq"), "bk": cat0("bk"), "bv": cat0("bv"),
        "wo": f(np.concatenate([s.wo for s in shards], axis=1)),
        "w1": cat0("w1"), "b1": cat0("b1"),
        "w2": f(np.concatenate([s.w2 for s in shards], axis=1)),
        "ln1_g": f(rep.ln1_g), "ln1_b": f(rep.ln1_b), "ln2_g": f(rep.ln2_g), "ln2_b": f(rep.ln2_b),
        "b_o": f(rep.b_o), "b_2": f(rep.b_2),
        "head_dim": cfg.head_dim, "ranks": [s.rank for s in shards],
    }
    if shards[0].emb is not None:
        p["emb"] = cat0("emb")
        p["vocab_offsets"] = [s.rank * cfg.vocab_r for s in shards]
    return p


def device_shard(cfg: Config, s: RankShard) -> dict:
    """One rank's buffers in the C-ABI layout (host arrays in the storage dtype).

    bf16 tensors are returned as uint16 bit patterns, fp32 as float32.
    """
    conv = bf16_bits if cfg.dtype == "bf16" else (lambda a: np.ascontiguousarray(a, np.float32))
    out = {
        "w_qkv": conv(np.concatenate([s.wq, s.wk, s.wv], axis=0)),
        "b_qkv": conv(np.concatenate([s.bq, s.bk, s.bv], axis=0)),
        "w_o": conv(s.wo),
        "w_1": conv(s.w1), "b_1": conv(s.b1), "w_2": conv(s.w2),
    }
    if s.emb is not None:
        out["emb"] = conv(s.emb)
    return out


def storage(cfg: Config, a: np.ndarray) -> np.ndarray:
    """Host array in the storage dtype (uint16 bits for bf16, float32 otherwise)."""
    return bf16_bits(a) if cfg.dtype == "bf16" else np.ascontiguousarray(a, np.float32)


# ---------------------------------------------------------------------------
# vocabulary-parallel input embedding (guide page section 3.3)

def input_tokens(cfg: Config, skew: int = 0) -> np.ndarray:
    """[N] int32 input ids, uniform in [0, V); with skew > 0 drawn from the
    first `skew` ids only (many repeated ids, for the gradient's scatter-add)."""
    hi = cfg.vocab if skew <= 0 else min(skew, cfg.vocab)
    return _rng(cfg, "tokens").integers(0, hi, size=cfg.rows, dtype=np.int64).astype(np.int32)


def input_emb_shard(cfg: Config, r: int) -> np.ndarray:
    """E_in rows [r*V_r, (r+1)*V_r) of the input embedding, [V_r, h], N(0, sigma_w)."""
    return _normal(cfg, "emb_in", (cfg.vocab_r, cfg.hidden), cfg.sigma_w, rank=r)


def embedding_grad_in(cfg: Config) -> np.ndarray:
    """Upstream gradient of the embedding output, [N, h], N(0, 1)."""
    return _normal(cfg, "dx_emb", (cfg.rows, cfg.hidden))
