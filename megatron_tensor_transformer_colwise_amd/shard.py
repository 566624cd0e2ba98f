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

    def rank_save(self, r: int, x=None, stream=None) -> None:
        """Rank r's forward that also keeps its pre-activation for the backward
        (bf16 [m, f] for GeLU, [m, 2 f] = [gate | up] for SwiGLU)."""
        if getattr(self, "pre", None) is None:
            fin = 2 * self.f_shard if self.act == "swiglu" else self.f_shard
            self.pre = [torch.empty(self.m, fin, dtype=torch.bfloat16, device=self.x.device)
                        for _ in range(self.t)]
        tp.tp_colwise_save(self.act, self.m, self.h, self.f_shard, self.x if x is None else x, self.w_in[r],
                           self.act_ws, self.pre[r], stream)
        self.rowwise(r, stream)

    def forward(self, x=None, residual=None, residual_dt="f32", stream=None, grouped=False, save=False):
        """All ranks and the sum; ``save`` keeps every rank's pre-activation so
        the backward does not recompute it."""
        self.saved = save
        if save:
            for r in range(self.t):
                self.rank_save(r, x, stream)
        elif grouped:
            self.all_ranks_grouped(x, stream)
        else:
            for r in range(self.t):
                self.rank(r, x, stream)
        self.reduce(residual, residual_dt, stream)
        return self.out

    # ---- backward ("f and g": every rank gets the whole dZ; the dX partials are summed)

    def _bwd_buffers(self):
        if getattr(self, "bwd_ws", None) is None:
            dev, m, h, f = self.x.device, self.m, self.h, self.f_shard
            fin = 2 * f if self.act == "swiglu" else f
            self.bwd_ws_bytes = tp.tp_shard_mlp_backward_workspace_bytes(self.act, m, h, f)
            self.bwd_ws = torch.empty(self.bwd_ws_bytes, dtype=torch.uint8, device=dev)
            self.dx_partials = torch.empty(self.t, m, h, dtype=torch.float32, device=dev)
            self.dw_in = [torch.empty(fin, h, dtype=torch.float32, device=dev) for _ in range(self.t)]
            self.dw_out = [torch.empty(h, f, dtype=torch.float32, device=dev) for _ in range(self.t)]
            self.dx = torch.empty(m, h, dtype=torch.float32, device=dev)

    def backward_rank(self, r: int, dz, stream=None) -> None:
        """Rank r's gradients: its dX partial and its weight shards' gradients
        (from the saved pre-activation after a saving forward, else recomputing it)."""
        self._bwd_buffers()
        pre = self.pre[r] if getattr(self, "saved", False) else None
        tp.tp_shard_mlp_backward(self.act, self.m, self.h, self.f_shard, self.x, self.w_in[r], self.w_out[r], dz,
                                 None, None, self.bwd_ws, self.bwd_ws_bytes, self.dx_partials[r], self.dw_in[r],
                                 self.dw_out[r], stream, pre=pre)

    def backward(self, dz, stream=None):
        for r in range(self.t):
            self.backward_rank(r, dz, stream)
        tp.tp_shard_sum(self.t, self.m * self.h, list(self.dx_partials), None, "f32", self.dx, stream)
        return self.dx


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
        tp.tp_shard_attn("bf16", self.batch, self.seq, self.h, rk.hq, rk.hkv, self.d, self.case.rope_base,
                         self.causal, self.x if x is None else x, rk.w_qkv, rk.w_o, self.ws,
                         self.ws_bytes, self.partials[r], stream)

    def reduce(self, residual=None, residual_dt="f32", stream=None) -> None:
        m = self.batch * self.seq
        tp.tp_shard_sum(self.t, m * self.h, list(self.partials), residual, residual_dt, self.out, stream)

    def rank_parts(self, r: int, x=None, stream=None, mark=None) -> None:
        """Rank r's attention as its three component calls (the kernels
        tp_shard_attn launches, in the same order, on buffers of its own);
        ``mark(name)`` runs before and ``mark(None)`` after each, e.g. to
        bracket each kernel with events."""
        rk = self.ranks[r]
        if getattr(self, "part_bufs", None) is None:
            dev, m, d = self.x.device, self.batch * self.seq, self.d
            hq, hkv = self.ranks[0].hq, max(q.hkv for q in self.ranks)
            sp = (self.seq + 63) // 64 * 64
            bf = torch.bfloat16
            self.part_bufs = (torch.empty(m, hq * d, dtype=bf, device=dev),
                              torch.empty(m, hkv * d, dtype=bf, device=dev),
                              torch.empty(self.batch * hkv * d * sp, dtype=bf, device=dev),
                              torch.empty(m, hq * d, dtype=bf, device=dev))
        q, k, vt, o = self.part_bufs
        mark = mark or (lambda name: None)
        m = self.batch * self.seq
        mark("qkv_rope")
        tp.tp_qkv_rope(self.batch, self.seq, self.h, rk.hq, rk.hkv, self.d, self.case.rope_base,
                       self.x if x is None else x, rk.w_qkv, q, k, vt, stream)
        mark(None)
        mark("flash_attn")
        tp.tp_flash_attn(self.batch, self.seq, rk.hq, rk.hkv, self.d, self.causal, q, k, vt, o, stream)
        mark(None)
        mark("o_proj")
        tp.tp_rowwise("bf16", m, rk.hq * self.d, self.h, o, rk.w_o, self.partials[r], stream)
        mark(None)

    def rank_save(self, r: int, x=None, stream=None) -> None:
        """Rank r's forward keeping Q, K, V^T, O and the log-sum-exp for the backward."""
        rk = self.ranks[r]
        if getattr(self, "saved_acts", None) is None:
            dev, m, d = self.x.device, self.batch * self.seq, self.d
            sp = (self.seq + 63) // 64 * 64
            self.saved_acts = [(torch.empty(m, q.hq * d, dtype=torch.bfloat16, device=dev),
                                torch.empty(m, q.hkv * d, dtype=torch.bfloat16, device=dev),
                                torch.empty(self.batch, q.hkv, d, sp, dtype=torch.bfloat16, device=dev),
                                torch.empty(m, q.hq * d, dtype=torch.bfloat16, device=dev),
                                torch.empty(self.batch, q.hq, sp, dtype=torch.float32, device=dev))
                               for q in self.ranks]
        q, k, vt, o, lse = self.saved_acts[r]
        tp.tp_shard_attn_save(self.batch, self.seq, self.h, rk.hq, rk.hkv, self.d, self.case.rope_base, self.causal,
                              self.x if x is None else x, rk.w_qkv, rk.w_o, q, k, vt, o, lse, self.partials[r], stream)

    def forward(self, x=None, residual=None, residual_dt="f32", stream=None, save=False):
        """All ranks and the sum; ``save`` keeps every rank's activations so the
        backward does not recompute the forward."""
        self.saved = save
        for r in range(self.t):
            if save:
                self.rank_save(r, x, stream)
            else:
                self.rank(r, x, stream)
        self.reduce(residual, residual_dt, stream)
        return self.out

    # ---- backward ("Self-attention" + "f and g": each rank differentiates its
    # own heads from the whole dZ; the dX partials are summed)

    def _bwd_buffers(self):
        if getattr(self, "bwd_ws", None) is None:
            dev, m, h, d = self.x.device, self.batch * self.seq, self.h, self.d
            hq, hkv = self.ranks[0].hq, max(rk.hkv for rk in self.ranks)
            self.bwd_ws_bytes = tp.tp_shard_attn_backward_workspace_bytes(self.batch, self.seq, h, hq, hkv, d)
            self.bwd_ws = torch.empty(self.bwd_ws_bytes, dtype=torch.uint8, device=dev)
            self.dx_partials = torch.empty(self.t, m, h, dtype=torch.float32, device=dev)
            self.dw_qkv = [torch.empty((rk.hq + 2 * rk.hkv) * d, h, dtype=torch.float32, device=dev)
                           for rk in self.ranks]
            self.dw_o = [torch.empty(h, rk.hq * d, dtype=torch.float32, device=dev) for rk in self.ranks]
            self.dx = torch.empty(m, h, dtype=torch.float32, device=dev)

    def backward_rank(self, r: int, dz, x=None, stream=None) -> None:
        """Rank r's gradients: its dX partial and the gradients of its W_qkv
        rows and W_o columns."""
        self._bwd_buffers()
        rk = self.ranks[r]
        saved = self.saved_acts[r] if getattr(self, "saved", False) else None
        tp.tp_shard_attn_backward(self.batch, self.seq, self.h, rk.hq, rk.hkv, self.d, self.case.rope_base,
                                  self.causal, self.x if x is None else x, rk.w_qkv, rk.w_o, dz, None, None,
                                  self.bwd_ws, self.bwd_ws_bytes, self.dx_partials[r], self.dw_qkv[r],
                                  self.dw_o[r], stream, saved=saved)

    def backward(self, dz, x=None, stream=None):
        for r in range(self.t):
            self.backward_rank(r, dz, x, stream)
        m = self.batch * self.seq
        tp.tp_shard_sum(self.t, m * self.h, list(self.dx_partials), None, "f32", self.dx, stream)
        return self.dx


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

    # ---- backward ("f and g": each sublayer's dX partials are summed, then the
    # replicated norm's gradient is taken and the residual's gradient added)

    def _bwd_buffers(self):
        if getattr(self, "d_x", None) is None:
            dev, m, h = self.x.device, self.m, self.h
            self.dh1 = torch.empty(m, h, dtype=torch.float32, device=dev)
            self.dh1_bf16 = torch.empty(m, h, dtype=torch.bfloat16, device=dev)
            self.d_x = torch.empty(m, h, dtype=torch.float32, device=dev)
            self.dg_attn = torch.empty(h, dtype=torch.float32, device=dev)
            self.dg_mlp = torch.empty(h, dtype=torch.float32, device=dev)
            self.norm_ws_bytes = tp.tp_shard_sum_rmsnorm_backward_workspace_bytes(m, h)
            self.norm_ws = torch.empty(max(self.norm_ws_bytes, 256), dtype=torch.uint8, device=dev)

    def backward(self, dz, stream=None):
        """Gradients of the block for the bf16 output gradient dZ, after
        ``forward`` (its normed inputs and h1 are the saved activations):
        every MLP rank's backward, their dX partials summed through the MLP
        norm's backward plus dZ (dh1); every attention rank's backward for
        dh1, their partials summed through the first norm's backward plus dh1
        (dX).  Weight gradients stay in the sublayers' per-rank buffers."""
        self._bwd_buffers()
        m, h, eps = self.m, self.h, self.case.eps
        for r in range(self.t):
            self.mlp.backward_rank(r, dz, stream)
        tp.tp_shard_sum_rmsnorm_backward(self.t, m, h, list(self.mlp.dx_partials), self.attn.out, "f32", self.g_mlp,
                                         eps, dz, "bf16", self.dh1, self.dh1_bf16, self.dg_mlp, self.norm_ws,
                                         self.norm_ws_bytes, stream)
        for r in range(self.t):
            self.attn.backward_rank(r, self.dh1_bf16, stream=stream)
        tp.tp_shard_sum_rmsnorm_backward(self.t, m, h, list(self.attn.dx_partials), self.x, "bf16", self.g_attn,
                                         eps, self.dh1, "f32", self.d_x, None, self.dg_attn, self.norm_ws,
                                         self.norm_ws_bytes, stream)
        return self.d_x

    def forward(self, stream=None, fused=True, save=False):
        """``save`` keeps every rank's activations for ``backward`` (no
        recomputation there)."""
        self.norm_attn(stream)
        if fused:
            self.attn.saved = save
            for r in range(self.t):
                if save:
                    self.attn.rank_save(r, stream=stream)
                else:
                    self.attn.rank(r, stream=stream)
            self.sum_norm_mlp(stream)
        else:
            self.attn.forward(residual=self.x, residual_dt="bf16", stream=stream, save=save)
            self.norm_mlp(stream)
        self.mlp.forward(residual=self.attn.out, residual_dt="f32", stream=stream, save=save)
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

    def backward_sp(self, dz, stream=None):
        """The sequence-parallel form's backward ("Sequence parallelism": the
        backward of the all-gather before the colwise GEMMs is a reduce-scatter
        onto the slices, that of the reduce-scatter after the rowwise GEMMs an
        all-gather).  Every rank reads the whole dZ (the gathered slices; one
        shared buffer on one device); per rank, one launch sums the MLP ranks'
        dX partials over its slice, takes the MLP norm's gradient there and
        adds dZ (its slice of dh1, written into the shared, gathered dh1); the
        attention ranks' backward for dh1; one launch per rank for its slice of
        dX.  dX and dh1 are bitwise those of ``backward`` (row-local steps);
        each gain's gradient is the sum over the ranks' slices (an all-reduce
        in ascending rank order)."""
        self._bwd_buffers()
        t, h, eps = self.t, self.h, self.case.eps
        runs = self.sp_runs()
        n = runs[1]
        ms = runs[0] * n
        if getattr(self, "dg_sp", None) is None:
            self.dg_sp = torch.empty(2, t, h, dtype=torch.float32, device=self.x.device)
        for r in range(t):
            self.mlp.backward_rank(r, dz, stream)
        mp, ap = self.mlp.dx_partials, self.attn.dx_partials
        for r in range(t):
            o = r * n
            tp.tp_shard_sum_rmsnorm_backward(t, ms, h, [mp[i][o:] for i in range(t)], self.attn.out[o:], "f32",
                                             self.g_mlp, eps, dz[o:], "bf16", self.dh1[o:], self.dh1_bf16[o:],
                                             self.dg_sp[0, r], self.norm_ws, self.norm_ws_bytes, stream, runs=runs)
        for r in range(t):
            self.attn.backward_rank(r, self.dh1_bf16, stream=stream)
        for r in range(t):
            o = r * n
            tp.tp_shard_sum_rmsnorm_backward(t, ms, h, [ap[i][o:] for i in range(t)], self.x[o:], "bf16",
                                             self.g_attn, eps, self.dh1[o:], "f32", self.d_x[o:], None,
                                             self.dg_sp[1, r], self.norm_ws, self.norm_ws_bytes, stream, runs=runs)
        tp.tp_shard_sum(t, h, list(self.dg_sp[0]), None, "f32", self.dg_mlp, stream)
        tp.tp_shard_sum(t, h, list(self.dg_sp[1]), None, "f32", self.dg_attn, stream)
        return self.d_x


# ---------------------------------------------------------------- packed (fused) projections


def _packed_ranges(n: int, blocks, t: int, rank: int) -> list[tuple[int, int]]:
    """(start, stop) of rank ``rank``'s 1/t of every packed block of a
    dimension of n; blocks are proportions whose sum divides n, and each block
    must be divisible by t on its own (diffusers guide, "Fused projections",
    "Constraints and validation")."""
    total = sum(blocks)
    if n % total:
        raise ValueError(f"packed dimension {n} is not divisible by sum(blocks) = {total}")
    unit, out, start = n // total, [], 0
    for b in blocks:
        size = b * unit
        if size % t:
            raise ValueError(f"packed block of {size} is not divisible by t = {t}")
        out.append((start + rank * (size // t), start + (rank + 1) * (size // t)))
        start += size
    return out


def packed_colwise_weight(w: torch.Tensor, blocks, t: int, rank: int) -> torch.Tensor:
    """Rank's rows of an nn.Linear weight [out, in] whose output features pack
    several tensors: its 1/t of every block, in packed order (contiguous)."""
    return torch.cat([w[a:b] for a, b in _packed_ranges(w.shape[0], blocks, t, rank)]).contiguous()


def packed_rowwise_weights(w: torch.Tensor, blocks, t: int, rank: int) -> list[torch.Tensor]:
    """Rank's columns of an nn.Linear weight [out, in] whose input features pack
    several tensors, one contiguous [out, in_block / t] weight per block."""
    return [w[:, a:b].contiguous() for a, b in _packed_ranges(w.shape[1], blocks, t, rank)]


class SingleStreamShards:
    """A packed single-stream block, every rank on one device: one Linear
    projects X to [Q | K | V | gate | up] (output blocks [1, 1, 1, 3, 3], the
    guide's mlp_ratio = 3 example), attention runs on Q, K, V per head (no
    mask by default), SiLU(gate) * up is the MLP, and one Linear projects
    [attention | MLP] back (input blocks [1, 3]).  Rank r holds one buffer
    with its rows of every in-projection block; its Q|K|V rows feed the
    Q/K/V + RoPE GEMM and its gate|up rows the SwiGLU GEMM, in place.  Its
    out-projection share is two row-parallel partials, one per input block,
    and the sum runs over all 2t of them."""

    def __init__(self, x, w_in: torch.Tensor, w_out: torch.Tensor, heads: int, head_dim: int, batch: int,
                 seq: int, t: int, rope_base: float, causal: bool = False):
        self.x, self.t, self.d = x, t, head_dim
        self.m, self.h = x.shape
        if heads % t:
            raise ValueError(f"t = {t} does not divide the {heads} heads")
        if 2 * t > tp.TP_MAX_SHARDS:
            raise ValueError(f"t = {t}: the sum takes 2 t <= {tp.TP_MAX_SHARDS} partials")
        self.batch, self.seq, self.base, self.causal = batch, seq, rope_base, causal
        self.nh = heads // t
        self.hr, self.mr = self.h // t, 3 * self.h // t
        if self.hr != self.nh * head_dim:
            raise ValueError("hidden size must be heads x head_dim")
        self.w_in = [packed_colwise_weight(w_in, [1, 1, 1, 3, 3], t, r) for r in range(t)]
        self.w_out = [packed_rowwise_weights(w_out, [1, 3], t, r) for r in range(t)]
        dev, m = x.device, self.m
        seq_pad = (seq + 63) // 64 * 64
        bf = torch.bfloat16
        self.q = torch.empty(m, self.hr, dtype=bf, device=dev)
        self.k = torch.empty(m, self.hr, dtype=bf, device=dev)
        self.vt = torch.empty(batch, self.nh, head_dim, seq_pad, dtype=bf, device=dev)
        self.o = torch.empty(m, self.hr, dtype=bf, device=dev)
        self.y = torch.empty(m, self.mr, dtype=bf, device=dev)
        self.partials = torch.empty(2 * t, m, self.h, dtype=torch.float32, device=dev)
        self.out = torch.empty(m, self.h, dtype=torch.float32, device=dev)

    def rank(self, r: int, stream=None) -> None:
        w, (wo_a, wo_m) = self.w_in[r], self.w_out[r]
        hr, mr, nh, d = self.hr, self.mr, self.nh, self.d
        tp.tp_qkv_rope(self.batch, self.seq, self.h, nh, nh, d, self.base, self.x, w[:3 * hr], self.q, self.k,
                       self.vt, stream)
        tp.tp_flash_attn(self.batch, self.seq, nh, nh, d, self.causal, self.q, self.k, self.vt, self.o, stream)
        tp.tp_colwise("swiglu", "bf16", self.m, self.h, mr, self.x, w[3 * hr:], self.y, stream)
        tp.tp_rowwise("bf16", self.m, hr, self.h, self.o, wo_a, self.partials[2 * r], stream)
        tp.tp_rowwise("bf16", self.m, mr, self.h, self.y, wo_m, self.partials[2 * r + 1], stream)

    def forward(self, stream=None):
        for r in range(self.t):
            self.rank(r, stream)
        tp.tp_shard_sum(2 * self.t, self.m * self.h, list(self.partials), None, "f32", self.out, stream)
        return self.out


# ---------------------------------------------------------------- vocabulary-parallel embedding and loss


def embedding_rowwise(ids, table: torch.Tensor, t: int, partials=None, out=None, stream=None):
    """Vocabulary-sharded lookup, every rank on one device: rank r holds rows
    [r v/t, (r+1) v/t) of the [v, h] table, looks up the ids it holds (zeros
    for the others), and the ranks' partials are summed."""
    v, h = table.shape
    if v % t:
        raise ValueError(f"vocabulary {v} is not divisible by t = {t}")
    n, m = v // t, ids.shape[0]
    partials = torch.empty(t, m, h, dtype=torch.float32, device=table.device) if partials is None else partials
    out = torch.empty(m, h, dtype=torch.float32, device=table.device) if out is None else out
    for r in range(t):
        tp.tp_embedding(m, h, r * n, n, ids, table[r * n:(r + 1) * n], partials[r], h, stream)
    tp.tp_shard_sum(t, m * h, list(partials), None, "f32", out, stream)
    return out


def embedding_colwise(ids, table: torch.Tensor, t: int, out=None, stream=None):
    """Hidden-sharded lookup: rank r holds columns [r h/t, (r+1) h/t) of every
    row and writes its slice into the gathered [m, h] output."""
    v, h = table.shape
    if h % t or (h // t) % 8:
        raise ValueError(f"hidden {h} is not a multiple of 8 t (t = {t})")
    hs, m = h // t, ids.shape[0]
    out = torch.empty(m, h, dtype=torch.float32, device=table.device) if out is None else out
    for r in range(t):
        tp.tp_embedding(m, hs, 0, v, ids, table[:, r * hs:(r + 1) * hs].contiguous(), out[:, r * hs:], h, stream)
    return out


class VocabParallelCE:
    """Output layer and cross-entropy with the vocabulary split over t ranks,
    every rank on one device: rank r computes its [m, v/t] logits and, from
    them, per token the max, the sum of exponentials and the label's logit
    (if it holds the label); combining the ranks' statistics gives the loss
    without ever gathering the [m, v] logits."""

    def __init__(self, x, w: torch.Tensor, t: int):
        v, h = w.shape                                  # nn.Linear layout [vocab, hidden]
        if v % t or (v // t) % 8:
            raise ValueError(f"vocabulary {v} must split into t = {t} slices of a multiple of 8")
        self.x, self.t, self.v, self.h = x, t, v, h
        self.n = v // t
        self.m = x.shape[0]
        self.w = [w[r * self.n:(r + 1) * self.n] for r in range(t)]
        dev = x.device
        self.logits = torch.empty(self.m, self.n, dtype=torch.float32, device=dev)
        self.stats = torch.empty(t, self.m, 4, dtype=torch.float32, device=dev)
        self.loss = torch.empty(self.m, dtype=torch.float32, device=dev)
        self.mean = torch.empty(1, dtype=torch.float32, device=dev)

    def rank(self, r: int, labels, stream=None) -> None:
        tp.tp_vocab_logits(self.m, self.h, self.n, self.x, self.w[r], self.logits, stream)
        tp.tp_ce_stats(self.m, self.n, r * self.n, self.logits, labels, self.stats[r], stream)

    def forward(self, labels, stream=None):
        for r in range(self.t):
            self.rank(r, labels, stream)
        tp.tp_ce_combine(self.t, self.m, self.v, list(self.stats), labels, self.loss, self.mean, stream)
        return self.loss, self.mean

