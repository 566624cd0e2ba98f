"""Per-rank weights in the library's layout, and drivers that run one rank (or
every rank in turn, on one GPU) through the C ABI.

Weight preparation is load-time data movement, not a step of the hot path:
each rank keeps only its own contiguous shard, stored in nn.Linear layout
[out, in] so both operands of every product are contiguous along the
reduction dimension.  The pages write weights as [in, out] (``Y = X A``), so a
rank's weight is the transpose of its block:

* column-parallel A (section "Matmul split"): rank i holds columns
  [i n/t, (i+1) n/t) of A  ->  those rows of A^T;
* row-parallel B: rank i holds rows [i n/t, (i+1) n/t) of B  ->  B_i^T;
* SwiGLU (section "MLP"): W1 and W3 are each split by columns and the rank's
  two blocks are packed [W1_i^T ; W3_i^T], so gate and up slices stay matched
  (packing the whole tensors first and then cutting one contiguous block would
  hand a rank the tail of one and the head of the other);
* attention (section "Self-attention"): rank i holds query heads
  [i a/t, (i+1) a/t) and the KV heads they use (query head j uses KV head
  j // (a/kv)), which replicates a KV head on several ranks when kv < t.

Model-level rules raise ``ValueError`` before anything is sharded: t must
divide the query heads, kv must divide the query heads, and KV heads must
split evenly over ranks or ranks evenly over KV heads.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import tpshard as tp


def _check_split(n: int, t: int, what: str) -> int:
    if t <= 0 or n % t:
        raise ValueError(f"t={t} must divide {what}={n}")
    return n // t


def colwise_weight(a: torch.Tensor, t: int, rank: int) -> torch.Tensor:
    """Rank's block of a column-parallel weight A [in, out], as [out/t, in]."""
    w = _check_split(a.shape[1], t, "output features")
    return a[:, rank * w:(rank + 1) * w].t().contiguous()


def rowwise_weight(b: torch.Tensor, t: int, rank: int) -> torch.Tensor:
    """Rank's block of a row-parallel weight B [in, out], as [out, in/t]."""
    w = _check_split(b.shape[0], t, "input features")
    return b[rank * w:(rank + 1) * w, :].t().contiguous()


def packed_gate_up(w1: torch.Tensor, w3: torch.Tensor, t: int, rank: int) -> torch.Tensor:
    """[W1_i^T ; W3_i^T]: the rank's gate block then its up block, [2 f/t, h]."""
    if w1.shape != w3.shape:
        raise ValueError("gate and up projections differ in shape")
    return torch.cat([colwise_weight(w1, t, rank), colwise_weight(w3, t, rank)], dim=0).contiguous()


def attn_heads(heads: int, kv_heads: int, t: int, rank: int) -> tuple[list[int], list[int]]:
    """(query heads, KV heads) of a rank."""
    hq = _check_split(heads, t, "query heads")
    if kv_heads <= 0 or heads % kv_heads:
        raise ValueError(f"{kv_heads} KV heads do not divide {heads} query heads")
    if kv_heads % t and t % kv_heads:
        raise ValueError(f"{kv_heads} KV heads cannot be split or replicated over t={t} ranks")
    group = heads // kv_heads
    q = list(range(rank * hq, (rank + 1) * hq))
    kv = sorted({j // group for j in q})
    return q, kv


@dataclass
class AttnRank:
    w_qkv: torch.Tensor  # [(hq + 2 hkv) d, h]
    w_o: torch.Tensor    # [h, hq d]
    hq: int
    hkv: int


def attn_rank(wq, wk, wv, wo, heads: int, kv_heads: int, head_dim: int, t: int, rank: int) -> AttnRank:
    q, kv = attn_heads(heads, kv_heads, t, rank)
    d = head_dim
    qcols = slice(q[0] * d, (q[-1] + 1) * d)
    kvcols = slice(kv[0] * d, (kv[-1] + 1) * d)
    w_qkv = torch.cat([wq[:, qcols].t(), wk[:, kvcols].t(), wv[:, kvcols].t()], dim=0).contiguous()
    w_o = wo[qcols, :].t().contiguous()
    return AttnRank(w_qkv, w_o, len(q), len(kv))


# --------------------------------------------------------------------------
# drivers
# --------------------------------------------------------------------------


class MLPShards:
    """All t ranks of an MLP layer on one device, run one after another."""

    def __init__(self, x, weights: dict, t: int, act: str, dtype: str = "bf16"):
        self.t, self.act, self.dt = t, act, dtype
        self.x = x
        self.m, self.h = x.shape
        if act == "gelu":
            a, b = weights["A"], weights["B"]
            self.w_in = [colwise_weight(a, t, r) for r in range(t)]
            self.w_out = [rowwise_weight(b, t, r) for r in range(t)]
        elif act == "swiglu":
            self.w_in = [packed_gate_up(weights["W1"], weights["W3"], t, r) for r in range(t)]
            self.w_out = [rowwise_weight(weights["W2"], t, r) for r in range(t)]
        else:
            raise ValueError(act)
        self.f_shard = self.w_out[0].shape[1]
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        self.act_ws = torch.empty(self.m, self.f_shard, dtype=tdt, device=x.device)
        self.group_ws = None
        self.partials = torch.empty(t, self.m, self.h, dtype=torch.float32, device=x.device)
        self.out = torch.empty(self.m, self.h, dtype=torch.float32, device=x.device)

    def rank(self, r: int, x=None, stream=None) -> None:
        tp.tp_shard_mlp(self.act, self.dt, self.m, self.h, self.f_shard, self.x if x is None else x,
                        self.w_in[r], self.w_out[r], self.act_ws, self.partials[r], stream)

    def colwise(self, r: int, x=None, stream=None) -> None:
        tp.tp_colwise(self.act, self.dt, self.m, self.h, self.f_shard, self.x if x is None else x,
                      self.w_in[r], self.act_ws, stream)

    def rowwise(self, r: int, stream=None) -> None:
        tp.tp_rowwise(self.dt, self.m, self.f_shard, self.h, self.act_ws, self.w_out[r],
                      self.partials[r], stream)

    def all_ranks_grouped(self, x=None, stream=None) -> None:
        """Every rank's MLP in one pair of launches (one workspace per rank)."""
        if self.group_ws is None:
            self.group_ws = torch.empty(self.t, self.m, self.f_shard, dtype=self.act_ws.dtype,
                                        device=self.act_ws.device)
        tp.tp_shard_mlp_group(self.act, self.dt, self.t, self.m, self.h, self.f_shard,
                              self.x if x is None else x, self.w_in, self.w_out,
                              list(self.group_ws), list(self.partials), stream)

    def reduce(self, residual=None, residual_dt="f32", stream=None) -> None:
        tp.tp_shard_sum(self.t, self.m * self.h, list(self.partials), residual, residual_dt, self.out, stream)

    def forward(self, x=None, residual=None, residual_dt="f32", stream=None, grouped=False):
        if grouped:
            self.all_ranks_grouped(x, stream)
        else:
            for r in range(self.t):
                self.rank(r, x, stream)
        self.reduce(residual, residual_dt, stream)
        return self.out


class AttnShards:
    """All t ranks of an attention layer on one device, run one after another."""

    def __init__(self, x, weights: dict, case, t: int | None = None, causal: bool = True):
        self.t = case.t if t is None else t
        self.case, self.causal = case, causal
        self.x = x
        self.batch, self.seq, self.h = case.batch, case.seq, case.hidden
        self.d = case.head_dim
        self.ranks = [attn_rank(weights["Wq"], weights["Wk"], weights["Wv"], weights["Wo"],
                                case.heads, case.kv_heads, case.head_dim, self.t, r)
                      for r in range(self.t)]
        hq, hkv = self.ranks[0].hq, max(rk.hkv for rk in self.ranks)
        self.ws_bytes = tp.tp_shard_attn_workspace_bytes(self.batch, self.seq, hq, hkv, self.d)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=x.device)
        m = self.batch * self.seq
        self.partials = torch.empty(self.t, m, self.h, dtype=torch.float32, device=x.device)
        self.out = torch.empty(m, self.h, dtype=torch.float32, device=x.device)

    def rank(self, r: int, x=None, stream=None) -> None:
        rk = self.ranks[r]
        tp.tp_shard_attn(self.batch, self.seq, self.h, rk.hq, rk.hkv, self.d, self.case.rope_base,
                         self.causal, self.x if x is None else x, rk.w_qkv, rk.w_o, self.ws,
                         self.ws_bytes, self.partials[r], stream)

    def reduce(self, residual=None, residual_dt="f32", stream=None) -> None:
        m = self.batch * self.seq
        tp.tp_shard_sum(self.t, m * self.h, list(self.partials), residual, residual_dt, self.out, stream)

    def forward(self, x=None, residual=None, residual_dt="f32", stream=None):
        for r in range(self.t):
            self.rank(r, x, stream)
        self.reduce(residual, residual_dt, stream)
        return self.out


class BlockShards:
    """Pre-norm block, every rank on one device:
    h1 = X + sum_i Attn_i(RMSNorm(X)); Z = h1 + sum_i MLP_i(RMSNorm(h1)).

    ``forward`` is the replicated form ("f and g": every rank sums and
    normalises the whole activation; the sum after attention and the norm
    before the MLP run as one pass).  ``forward_sp`` is the sequence-parallel
    form ("Sequence parallelism"): rank r normalises only its Shard(1) slice
    of every sequence, the sums after each sublayer are reduce-scatters onto
    those slices, and the slices are gathered before the tensor-parallel
    layers.  On one device every rank's slice lands in the one shared buffer,
    which is the all-gather."""

    def __init__(self, x, weights: dict, case, t: int | None = None):
        self.case = case
        self.t = case.t if t is None else t
        self.x = x
        m, h = x.shape
        self.m, self.h = m, h
        self.xn = torch.empty(m, h, dtype=torch.bfloat16, device=x.device)
        self.hn = torch.empty(m, h, dtype=torch.bfloat16, device=x.device)
        self.g_attn = weights.get("g_attn")
        self.g_mlp = weights.get("g_mlp")
        self.attn = AttnShards(self.xn, weights, case.attn(), self.t)
        self.mlp = MLPShards(self.hn, weights, self.t, "swiglu")

    def norm_attn(self, stream=None):
        tp.tp_rmsnorm("bf16", self.m, self.h, self.x, self.g_attn, self.case.eps, self.xn, stream)

    def norm_mlp(self, stream=None):
        tp.tp_rmsnorm("f32", self.m, self.h, self.attn.out, self.g_mlp, self.case.eps, self.hn, stream)

    def sum_norm_mlp(self, stream=None):
        """h1 = X + sum of the attention partials, and RMSNorm(h1), in one pass."""
        tp.tp_shard_sum_rmsnorm(self.t, self.m, self.h, list(self.attn.partials), self.x, "bf16",
                                self.attn.out, self.g_mlp, self.case.eps, self.hn, stream)

    def forward(self, stream=None, fused=True):
        self.norm_attn(stream)
        if fused:
            for r in range(self.t):
                self.attn.rank(r, stream=stream)
            self.sum_norm_mlp(stream)
        else:
            self.attn.forward(residual=self.x, residual_dt="bf16", stream=stream)
            self.norm_mlp(stream)
        self.mlp.forward(residual=self.attn.out, residual_dt="f32", stream=stream)
        return self.mlp.out

    def sp_runs(self) -> tuple[int, int, int]:
        """(nrun, run_rows, run_stride) of one rank's slice: positions
        [r S/t, (r+1) S/t) of each of the batch sequences (Shard(1) of
        (batch, seq, h)); rank r's runs start at row r S/t."""
        seq, t = self.case.seq, self.t
        if seq % t:
            raise ValueError(f"sequence parallelism needs t = {t} to divide the sequence length {seq}")
        return self.case.batch, seq // t, seq

    def sp_slices(self) -> list[list[tuple[int, int]]]:
        """Rank r's token rows as (first row, count) runs, one per sequence."""
        nrun, n, stride = self.sp_runs()
        return [[(b * stride + r * n, n) for b in range(nrun)] for r in range(self.t)]

    def forward_sp(self, stream=None):
        t, h, eps = self.t, self.h, self.case.eps
        runs = self.sp_runs()
        n = runs[1]
        ap, mp = self.attn.partials, self.mlp.partials
        # rank r: the norm of its slice of X, into the shared (gathered) input
        for r in range(t):
            o = r * n
            tp.tp_shard_sum_rmsnorm(0, 0, h, [], self.x[o:], "bf16", None, self.g_attn, eps, self.xn[o:],
                                    stream, runs=runs)
        for r in range(t):
            self.attn.rank(r, stream=stream)
        # rank r: reduce-scatter onto its slice, + X, and the MLP norm of the slice
        for r in range(t):
            o = r * n
            tp.tp_shard_sum_rmsnorm(t, 0, h, [ap[i][o:] for i in range(t)], self.x[o:], "bf16",
                                    self.attn.out[o:], self.g_mlp, eps, self.hn[o:], stream, runs=runs)
        for r in range(t):
            self.mlp.rank(r, stream=stream)
        # rank r: reduce-scatter onto its slice, + h1
        for r in range(t):
            o = r * n
            tp.tp_shard_sum_rmsnorm(t, 0, h, [mp[i][o:] for i in range(t)], self.attn.out[o:], "f32",
                                    self.mlp.out[o:], None, eps, None, stream, runs=runs)
        return self.mlp.out
