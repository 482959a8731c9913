"""One pass of the hot path -- a tensor-parallel layer shard forward+backward
with the vocabulary-parallel cross-entropy -- sequenced through the C ABI.

The sequence for one layer (podcast page, Outline: two all-reduces per module,
four per layer forward+backward; guide page 3.3 for the loss):

  fwd ATTN (each rank) -> sum #1 -> fwd MLP (each rank) -> sum #2
  -> xent LOCAL (each rank) -> stats gather -> xent FINISH
  -> xent bwd (each rank) -> sum (d hidden, + the extra upstream term R)
  -> bwd MLP SHARD (each rank) -> sum #3 -> bwd MLP REPLICATED
  -> bwd ATTN SHARD (each rank) -> sum #4 -> bwd ATTN REPLICATED

On one GPU the TP group is either run whole (every rank's calls in turn, the
sum kernel standing in for the all-reduce), or one rank is run at its real
shape with the other ranks' contributions supplied as fixed stand-in tensors
("peers"). The objective whose gradient is propagated is
J = mean cross-entropy(out) + sum(out * R), R a fixed tensor.

This module only allocates device buffers and calls the library; every
arithmetic step runs in the HIP kernels.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import binding as B


def _dev(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Host array in storage layout (uint16 bf16 bits or float32) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def _bits(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
        return (u >> np.uint32(16)).astype(np.uint16)   # values are already bf16-representable
    return np.ascontiguousarray(a, dtype=np.float32)


@dataclasses.dataclass
class RankState:
    rank: int
    desc: B.TplDesc
    attn: B.TplBlockParams
    mlp: B.TplBlockParams
    tensors: dict   # device tensors (params, saved buffers, outputs, grads)


class LayerStep:
    """Device state of one workload (one rank or a whole TP group on one GPU).

    cfg: a workload description with fields dtype, hidden, heads, head_dim,
    ffn, tp, seq, micro_batch, vocab, causal, ln_eps.
    rep: replicated host inputs (x, dout=R, targets, mask, LN params, b_o, b_2).
    shards: {rank: host buffers in the C-ABI layout (w_qkv, b_qkv, w_o, w_1,
    b_1, w_2, emb)} for the ranks run here.
    peers: stand-in [N, h] host tensors for the ranks not run here (t-1 of
    them in one-rank mode, none otherwise); peer_stats: their [N, 3] xent
    statistics.
    """

    def __init__(self, cfg, rep, shards: dict, peers=(), peer_stats=(), device="cuda", recompute=False):
        self.cfg = cfg
        self.recompute = recompute   # backward rebuilds each block's forward stash from its input
        # optional callable hook(kind, thunk) that runs every library call of a
        # pass; kind is "layer" (the rank's own layer calls), "sum" (the
        # all-reduce stand-in) or "loss" (the vocabulary-parallel loss calls).
        # Timing code uses it to bracket the calls; it must call thunk() once.
        self.hook = None
        self.device = torch.device(device)
        dt = cfg.dtype
        self.tdtype = torch.bfloat16 if dt == "bf16" else torch.float32
        self.N = cfg.seq * cfg.micro_batch
        N, h = self.N, cfg.hidden
        D = lambda a: _dev(_bits(a, dt), dt, self.device)
        z = lambda *shape, dtype=None: torch.empty(shape, dtype=dtype or self.tdtype, device=self.device)
        self.ranks = sorted(shards)
        self.shared = {
            "x": D(rep.x), "R": D(rep.dout),
            "targets": torch.from_numpy(rep.targets.astype(np.int32)).to(self.device),
            "mask": torch.from_numpy(rep.mask.astype(np.uint8)).to(self.device),
            "ln1_g": D(rep.ln1_g), "ln1_b": D(rep.ln1_b), "ln2_g": D(rep.ln2_g), "ln2_b": D(rep.ln2_b),
            "b_o": D(rep.b_o), "b_2": D(rep.b_2),
            "h1": z(N, h), "out": z(N, h), "dout": z(N, h), "dz_sum": z(N, h), "dh1": z(N, h),
            "dy_sum": z(N, h), "dx": z(N, h),
            "lse": z(N, dtype=torch.float32), "loss_rows": z(N, dtype=torch.float32),
            "loss": torch.zeros(4, dtype=torch.float32, device=self.device),
            "d_ln1_g": z(h, dtype=torch.float32), "d_ln1_b": z(h, dtype=torch.float32),
            "d_b_o": z(h, dtype=torch.float32), "d_ln2_g": z(h, dtype=torch.float32),
            "d_ln2_b": z(h, dtype=torch.float32), "d_b_2": z(h, dtype=torch.float32),
        }
        # A masked loss runs on its rows only: their index list (from the
        # batch's mask) gathers them, the loss sees a descriptor of that many
        # rows, and dH is expanded back to every row with zeros elsewhere.
        self.loss_idx = None
        self.NL = N
        if cfg.mask_rows is not None:
            idx = np.nonzero(rep.mask)[0].astype(np.int32)
            pos = np.full(N, -1, np.int32)
            pos[idx] = np.arange(len(idx), dtype=np.int32)
            self.loss_idx = idx
            self.NL = len(idx)
            self.shared.update({
                "loss_rows_idx": torch.from_numpy(idx).to(self.device),
                "loss_rows_pos": torch.from_numpy(pos).to(self.device),
                "out_l": z(self.NL, h), "targets_l": torch.empty(self.NL, dtype=torch.int32, device=self.device),
                "lse": z(self.NL, dtype=torch.float32), "loss_rows": z(self.NL, dtype=torch.float32),
            })
        self.peers = [D(p) for p in peers]
        self.peer_stats = [torch.from_numpy(np.ascontiguousarray(s, np.float32)).to(self.device) for s in peer_stats]
        if self.loss_idx is not None:   # the stand-in ranks' statistics of the loss rows
            self.peer_stats = [self._gather(ps, N, 12, torch.empty(self.NL, 3, dtype=torch.float32, device=self.device))
                               for ps in self.peer_stats]
        self.states: list[RankState] = []
        for r in self.ranks:
            hs = shards[r]
            desc = B.make_desc(cfg.hidden, cfg.heads, cfg.head_dim, cfg.ffn, cfg.tp, r, cfg.seq, cfg.micro_batch,
                               cfg.vocab, cfg.causal, dt, cfg.ln_eps)
            xdesc = desc if self.loss_idx is None else B.make_desc(
                cfg.hidden, cfg.heads, cfg.head_dim, cfg.ffn, cfg.tp, r, self.NL, 1, cfg.vocab, cfg.causal, dt,
                cfg.ln_eps)   # the loss's rows
            hr, fr, vr = cfg.hidden // cfg.tp, cfg.ffn // cfg.tp, cfg.vocab // cfg.tp
            t = {k: _dev(v, dt, self.device) for k, v in hs.items()}
            sa = B.tp_layer_saved_bytes(desc, B.TPL_BLOCK_ATTN)
            sm = B.tp_layer_saved_bytes(desc, B.TPL_BLOCK_MLP)
            sx = B.vocab_parallel_xent_stats_bytes(xdesc)
            if sa == 0 or sm == 0 or sx == 0:
                raise ValueError(f"workload rejected by tp_layer_saved_bytes (rank {r})")
            f32 = torch.float32
            t.update({
                "saved_attn": torch.empty(sa, dtype=torch.uint8, device=self.device),
                "saved_mlp": torch.empty(sm, dtype=torch.uint8, device=self.device),
                "part_attn": z(N, h), "part_mlp": z(N, h), "dln_attn": z(N, h), "dln_mlp": z(N, h),
                "logits": z(self.NL, vr), "stats_buf": z(sx // 4, dtype=f32), "dH": z(N, h),
                "dH_l": z(self.NL, h) if self.loss_idx is not None else None,
                "d_w_qkv": z(3 * hr, h, dtype=f32), "d_b_qkv": z(3 * hr, dtype=f32), "d_w_o": z(h, hr, dtype=f32),
                "d_w_1": z(fr, h, dtype=f32), "d_b_1": z(fr, dtype=f32), "d_w_2": z(h, fr, dtype=f32),
                "d_emb": z(vr, h, dtype=f32),
            })
            sh = self.shared
            attn = B.block_params(sh["ln1_g"], sh["ln1_b"], t["w_qkv"], t["b_qkv"], t["w_o"])
            t["stats"] = t["stats_buf"][:self.NL * 3].view(self.NL, 3)   # the exchanged part; the rest is scratch
            t["xdesc"] = xdesc
            mlp = B.block_params(sh["ln2_g"], sh["ln2_b"], t["w_1"], t["b_1"], t["w_2"])
            self.states.append(RankState(r, desc, attn, mlp, t))
        self.exchanges = 0
        self.dloss = 1.0

    def _call(self, kind, fn, *args, **kw):
        if self.hook is None:
            return fn(*args, **kw)
        return self.hook(kind, lambda: fn(*args, **kw))

    def _gather(self, src, n_src, row_bytes, dst, stream=None):
        self._call("loss", B.tpl_rows_gather, src, n_src, self.shared["loss_rows_idx"], self.NL, row_bytes, dst, stream)
        return dst

    # -------------------------------------------------------------- exchanges
    def _sum(self, key, bias, residual, out, stream=None):
        """All-reduce stand-in: out = residual + bias + sum of every rank's `key`
        tensor (this GPU's ranks, then the stand-in peers)."""
        parts = [st.tensors[key] for st in self.states] + self.peers
        self._call("sum", B.shard_partial_sum, self.states[0].desc, parts, bias, residual, out, self.N, self.cfg.hidden, stream)
        self.exchanges += 1

    # -------------------------------------------------------------- passes
    def forward(self, stream=None):
        sh = self.shared
        for st in self.states:
            self._call("layer", B.tp_layer_shard_fwd, st.desc, B.TPL_BLOCK_ATTN, sh["x"], st.attn, st.tensors["part_attn"],
                                 st.tensors["saved_attn"], stream)
        self._sum("part_attn", sh["b_o"], sh["x"], sh["h1"], stream)
        for st in self.states:
            self._call("layer", B.tp_layer_shard_fwd, st.desc, B.TPL_BLOCK_MLP, sh["h1"], st.mlp, st.tensors["part_mlp"],
                                 st.tensors["saved_mlp"], stream)
        self._sum("part_mlp", sh["b_2"], sh["h1"], sh["out"], stream)

    def _loss_inputs(self):
        """(hidden, targets) of the loss's rows: the whole batch, or the masked
        rows gathered (a NULL mask then: the mean over them is the masked mean)."""
        sh = self.shared
        if self.loss_idx is None:
            return sh["out"], sh["targets"]
        return sh["out_l"], sh["targets_l"]

    def xent_forward(self, stream=None):
        sh = self.shared
        if self.loss_idx is not None:
            es = 2 if self.cfg.dtype == "bf16" else 4
            self._gather(sh["out"], self.N, self.cfg.hidden * es, sh["out_l"], stream)
            self._gather(sh["targets"], self.N, 4, sh["targets_l"], stream)
        hidden, targets = self._loss_inputs()
        for st in self.states:
            self._call("loss", B.vocab_parallel_xent_fwd, st.tensors["xdesc"], B.TPL_XENT_LOCAL, hidden=hidden, emb=st.tensors["emb"],
                                      targets=targets, loss_mask=None, logits=st.tensors["logits"],
                                      stats=st.tensors["stats"], stream=stream)
        all_stats = self._stats_in_rank_order()
        self._call("loss", B.vocab_parallel_xent_fwd, self.states[0].tensors["xdesc"], B.TPL_XENT_FINISH, targets=targets,
                                  loss_mask=None, all_stats=all_stats, lse=sh["lse"], loss_rows=sh["loss_rows"],
                                  loss=sh["loss"], stream=stream)

    def _stats_in_rank_order(self):
        mine = {st.rank: st.tensors["stats"] for st in self.states}
        peers = iter(self.peer_stats)
        return [mine[r] if r in mine else next(peers) for r in range(self.cfg.tp)]

    def xent_backward(self, stream=None):
        sh = self.shared
        hidden, targets = self._loss_inputs()
        for st in self.states:
            t = st.tensors
            dh = t["dH"] if self.loss_idx is None else t["dH_l"]
            self._call("loss", B.vocab_parallel_xent_bwd, t["xdesc"], hidden, t["emb"], targets, None, t["logits"], sh["lse"],
                                      sh["loss"], self.dloss, dh, t["d_emb"], stream)
            if self.loss_idx is not None:   # dH of the loss rows back to every row, zeros elsewhere
                es = 2 if self.cfg.dtype == "bf16" else 4
                self._call("loss", B.tpl_rows_expand, dh, self.NL, sh["loss_rows_pos"], self.N, self.cfg.hidden * es, t["dH"], stream)
        self._sum("dH", None, sh["R"], sh["dout"], stream)

    def poison_saved(self):
        """Overwrite every forward stash (as another layer reusing the buffer
        would); only a recomputing backward can still be right."""
        for st in self.states:
            st.tensors["saved_attn"].fill_(0xFF)
            st.tensors["saved_mlp"].fill_(0xFF)

    def backward(self, stream=None):
        sh = self.shared
        shard = B.TPL_BWD_SHARD_RECOMPUTE if self.recompute else B.TPL_BWD_SHARD
        for st in self.states:
            t = st.tensors
            self._call("layer", B.tp_layer_shard_bwd, st.desc, B.TPL_BLOCK_MLP, shard, sh["dout"], None, sh["h1"], st.mlp,
                                 t["saved_mlp"], t["dln_mlp"], None,
                                 B.block_grads(t["d_w_1"], t["d_b_1"], t["d_w_2"]), stream)
        self._sum("dln_mlp", None, None, sh["dz_sum"], stream)
        st0 = self.states[0]   # the replicated part is identical on every rank: run it once
        self._call("layer", B.tp_layer_shard_bwd, st0.desc, B.TPL_BLOCK_MLP, B.TPL_BWD_REPLICATED, sh["dout"], sh["dz_sum"], sh["h1"],
                             st0.mlp, st0.tensors["saved_mlp"], None, sh["dh1"],
                             B.block_grads(d_ln_g=sh["d_ln2_g"], d_ln_b=sh["d_ln2_b"], d_b_out=sh["d_b_2"]), stream)
        for st in self.states:
            t = st.tensors
            self._call("layer", B.tp_layer_shard_bwd, st.desc, B.TPL_BLOCK_ATTN, shard, sh["dh1"], None, sh["x"], st.attn,
                                 t["saved_attn"], t["dln_attn"], None,
                                 B.block_grads(t["d_w_qkv"], t["d_b_qkv"], t["d_w_o"]), stream)
        self._sum("dln_attn", None, None, sh["dy_sum"], stream)
        self._call("layer", B.tp_layer_shard_bwd, st0.desc, B.TPL_BLOCK_ATTN, B.TPL_BWD_REPLICATED, sh["dh1"], sh["dy_sum"], sh["x"],
                             st0.attn, st0.tensors["saved_attn"], None, sh["dx"],
                             B.block_grads(d_ln_g=sh["d_ln1_g"], d_ln_b=sh["d_ln1_b"], d_b_out=sh["d_b_o"]), stream)

    def step(self, stream=None):
        """One whole pass: layer forward, loss forward+backward, layer backward."""
        self.forward(stream)
        self.xent_forward(stream)
        self.xent_backward(stream)
        self.backward(stream)

    # -------------------------------------------------------------- results
    def results(self) -> dict:
        """Every output of the pass as host float64 numpy arrays."""
        f = lambda t: t.detach().float().cpu().numpy().astype(np.float64)
        skip = ("targets", "mask", "loss_rows_idx", "loss_rows_pos", "out_l", "targets_l")
        out = {k: f(v) for k, v in self.shared.items() if k not in skip}
        for st in self.states:
            for k, v in st.tensors.items():
                if (k.startswith(("d_", "part_", "dln_")) or k in ("dH", "stats")) and v is not None:
                    out[f"{k}@{st.rank}"] = f(v)
        return out
