"""CPU oracle for one rank of a Megatron-style tensor-parallel transformer block.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; the two meet only in the seeded inputs of
``megatron_tensor_transformer_colwise_amd/inputs.py``.

Everything here is plain numpy in float64 on the exact input values (bf16
inputs are widened exactly).  Intermediates are not rounded to bf16.  Where a
step has a plain definition it is that definition written out; sharding is
done here from the unsharded tensors, on its own.

Sources (the "Tensor parallelism" page of itwiki, by section):

* "Matmul split": a column-parallel linear splits ``A = [A_1 ... A_t]`` by
  columns and rank i computes ``X A_i`` from the full input; a row-parallel
  linear splits ``A`` by rows, rank i computes ``X_i A_i`` and the result is the
  sum over ranks.
* "MLP": ``Z = GeLU(X A) B``; with A split by columns and B by rows,
  ``Z = sum_i GeLU(X A_i) B_i``; splitting A by rows instead would need a sync
  before the GeLU.  The same split holds for the SwiGLU form
  ``W2 (SiLU(X W1) * X W3)`` with W1, W3 by columns and W2 by rows.
* "Self-attention": heads are independent; Q, K, V projections are split by
  columns so each rank holds a/t heads, o_proj is split by rows and summed.  a
  must be divisible by t.  With grouped-query attention, KV heads are
  replicated across ranks when there are fewer KV heads than t.
* "f and g": norms and residual connections are replicated on every rank; a
  block has one sum after attention and one after the MLP.
* transformers "Tensor parallelism" page (partitioning table, DTensor
  example): a column-parallel layer shards its bias with its output features;
  a row-parallel layer's bias is replicated and added once, after the sum.
* diffusers tensor-parallel guide (style table), "rowwise_split_input": a
  row-parallel layer over a replicated input, each rank taking its own slice
  of the input features.
* diffusers tensor-parallel guide, "Fused projections" and "Constraints and
  validation": a Linear that packs several logical tensors along the sharded
  dimension is sharded block by block (blocks given as proportions whose sum
  divides the packed dimension, each block divisible by t on its own), since
  a plain slice would cut across the packed parts.
* "Embedding and output layer": the embedding matrix is split along the
  vocabulary; instead of gathering the b x s x v logits, each rank computes
  from its own slice the maximum and the sum the cross-entropy needs, so only
  b x s values are exchanged.  transformers "Tensor parallelism" page,
  EmbeddingParallel: a vocabulary-sharded lookup sums the ranks' partial
  lookups; a hidden-sharded one gathers their column slices.
* "f and g" (backward): g's backward is the identity (every rank gets the whole
  output gradient), f's backward is the all-reduce of the ranks' input-gradient
  partials; each rank's weight gradients are the gradients of its own shards.
* "Self-attention" with "f and g" (backward): a rank's attention gradients
  are those of its own heads; its dX partial sums over them, and a KV head
  replicated on several ranks gets one weight-gradient share per rank.  The
  softmax and rotation gradients are their plain definitions (the Jacobian
  of the row softmax; the transpose of the RoPE rotation).
* "Sequence parallelism": the norms act on every token alone, so each rank
  can hold and normalise only its slice of the sequence; the sequence is
  gathered (all-gather) on entering the tensor-parallel region and, on
  leaving it, the sum over ranks is taken as a reduce-scatter that leaves
  each rank the sum for its own slice.  "Writing it in PyTorch": the slice is
  Shard(1) of a (batch, sequence, hidden) activation, the sequence dimension.

Readings where the pages say nothing (each stated where it is used):
erf GeLU (the page's example uses PyTorch's default GeLU, which is the erf
form); softmax scale 1/sqrt(d); query j uses KV head floor(j / (a/kv)); RoPE in
the rotate-half form with positions restarting in every sequence; RMSNorm
``x / sqrt(mean(x^2) + eps) * gain``; pre-norm residual structure; the
shard-sum adds partials in ascending rank order.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

# --------------------------------------------------------------------------
# scalar nonlinearities
# --------------------------------------------------------------------------


def gelu(x):
    """GeLU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)).

    The page's MLP example calls PyTorch's default GeLU, which is this exact
    erf form (not the tanh approximation)."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def silu(x):
    """SiLU(x) = x * sigmoid(x), the gate of the SwiGLU MLP ("MLP" section)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


# --------------------------------------------------------------------------
# sharding ("Matmul split")
# --------------------------------------------------------------------------


def split_columns(a: np.ndarray, t: int) -> list[np.ndarray]:
    """Column-parallel shards A_1..A_t: equal contiguous column blocks."""
    n = a.shape[1]
    if n % t:
        raise ValueError(f"{n} columns do not split {t} ways")
    w = n // t
    return [a[:, i * w:(i + 1) * w] for i in range(t)]


def split_rows(b: np.ndarray, t: int) -> list[np.ndarray]:
    """Row-parallel shards B_1..B_t: equal contiguous row blocks."""
    n = b.shape[0]
    if n % t:
        raise ValueError(f"{n} rows do not split {t} ways")
    w = n // t
    return [b[i * w:(i + 1) * w, :] for i in range(t)]


def shard_sum(partials) -> np.ndarray:
    """The sum over ranks that the all-reduce produces, in ascending rank order."""
    out = np.array(partials[0], dtype=np.float64, copy=True)
    for p in partials[1:]:
        out = out + p
    return out


def shard_sum_f32(partials, residual=None) -> np.ndarray:
    """The same sum carried out in float32 with one rounding per add, ascending
    rank order, then the residual added last.  This is the precision and order
    the GPU shard-sum uses, so integer-free inputs can be compared bit for bit."""
    out = np.array(partials[0], dtype=np.float32, copy=True)
    for p in partials[1:]:
        out = (out + np.asarray(p, dtype=np.float32)).astype(np.float32)
    if residual is not None:
        out = (out + np.asarray(residual, dtype=np.float32)).astype(np.float32)
    return out


# --------------------------------------------------------------------------
# MLP ("MLP" section)
# --------------------------------------------------------------------------


def mlp_gelu(x, a, b) -> np.ndarray:
    """Z = GeLU(X A) B.  With the full A and B this is the unsharded layer; with
    A_i and B_i it is rank i's partial."""
    return gelu(x @ a) @ b


def mlp_gelu_partials(x, a, b, t: int) -> list[np.ndarray]:
    """partial_i = GeLU(X A_i) B_i for the column shards of A and row shards of B."""
    return [mlp_gelu(x, ai, bi) for ai, bi in zip(split_columns(a, t), split_rows(b, t))]


def mlp_gelu_row_split(x, a, t: int) -> tuple[np.ndarray, np.ndarray]:
    """The split the page rules out: A by rows, X by columns.  Returns
    (GeLU(sum_i X_i A_i), sum_i GeLU(X_i A_i)), which differ in general."""
    xs = split_columns(x, t)
    aps = split_rows(a, t)
    pre = [xi @ ai for xi, ai in zip(xs, aps)]
    return gelu(shard_sum(pre)), shard_sum([gelu(p) for p in pre])


def linear(x, a, bias=None) -> np.ndarray:
    """X A (+ bias on every row)."""
    y = x @ a
    return y if bias is None else y + np.asarray(bias, dtype=np.float64)


def colwise_act(x, w_in, act: str, w_gate_up=None, bias=None, bias_gate_up=None) -> np.ndarray:
    """Rank-local colwise output Y_i: GeLU(X A_i + b_i), or
    SiLU(X W1_i + b1_i) * (X W3_i + b3_i); biases optional."""
    if act == "gelu":
        return gelu(linear(x, w_in, bias))
    if act == "swiglu":
        w1, w3 = w_gate_up
        b1, b3 = bias_gate_up if bias_gate_up is not None else (None, None)
        return silu(linear(x, w1, b1)) * linear(x, w3, b3)
    if act == "none":
        return linear(x, w_in, bias)
    raise ValueError(act)


# Biases (transformers "Tensor parallelism" page, partitioning table and its
# DTensor example): a column-parallel layer shards its bias with its output
# features, so rank i adds b_i before its nonlinearity; a row-parallel layer
# replicates its bias and it is added once, after the sum over ranks.


def split_vector(b, t: int) -> list[np.ndarray]:
    """Rank i's contiguous 1/t of a bias over output features."""
    b = np.asarray(b)
    if b.shape[0] % t:
        raise ValueError(f"{b.shape[0]} features are not divisible by t = {t}")
    n = b.shape[0] // t
    return [b[i * n:(i + 1) * n] for i in range(t)]


def mlp_gelu_bias(x, a, ba, b, bb) -> np.ndarray:
    """Z = GeLU(X A + ba) B + bb, the unsharded layer with biases."""
    return linear(gelu(linear(x, a, ba)), b, bb)


def mlp_gelu_bias_partials(x, a, ba, b, t: int) -> list[np.ndarray]:
    """partial_i = GeLU(X A_i + ba_i) B_i; the layer output is their sum plus bb once."""
    return [gelu(linear(x, ai, bai)) @ bi
            for ai, bai, bi in zip(split_columns(a, t), split_vector(ba, t), split_rows(b, t))]


def mlp_swiglu_bias(x, w1, b1, w3, b3, w2, b2) -> np.ndarray:
    """Z = (SiLU(X W1 + b1) * (X W3 + b3)) W2 + b2."""
    return linear(silu(linear(x, w1, b1)) * linear(x, w3, b3), w2, b2)


def mlp_swiglu_bias_partials(x, w1, b1, w3, b3, w2, t: int) -> list[np.ndarray]:
    """partial_i = (SiLU(X W1_i + b1_i) * (X W3_i + b3_i)) W2_i."""
    return [(silu(linear(x, a, ba)) * linear(x, c, bc)) @ bw
            for a, ba, c, bc, bw in zip(split_columns(w1, t), split_vector(b1, t), split_columns(w3, t),
                                        split_vector(b3, t), split_rows(w2, t))]


# "rowwise_split_input" (diffusers tensor-parallel guide, style table): a
# row-parallel layer whose input is replicated; each rank multiplies its own
# slice of the input features by its rows of the weight.


def rowwise_split_input_partials(x, w, t: int) -> list[np.ndarray]:
    """partial_r = X[:, cols_r] W[cols_r, :] with cols_r the r-th 1/t of the input
    features; their sum is X W."""
    return [xr @ wr for xr, wr in zip(split_columns(x, t), split_rows(w, t))]


def mlp_swiglu(x, w1, w3, w2) -> np.ndarray:
    """Z = (SiLU(X W1) * (X W3)) W2; full weights give the unsharded layer."""
    return (silu(x @ w1) * (x @ w3)) @ w2


def mlp_swiglu_partials(x, w1, w3, w2, t: int) -> list[np.ndarray]:
    """partial_i with W1, W3 split by columns and W2 by rows."""
    return [
        mlp_swiglu(x, a, c, b)
        for a, c, b in zip(split_columns(w1, t), split_columns(w3, t), split_rows(w2, t))
    ]


# --------------------------------------------------------------------------
# attention ("Self-attention" section)
# --------------------------------------------------------------------------


def kv_head_of(j: int, heads: int, kv_heads: int) -> int:
    """KV head used by query head j: consecutive groups of heads/kv_heads query
    heads share one KV head (reading; the page only says KV heads must be
    taken into account and replicated when fewer than t)."""
    return j // (heads // kv_heads)


def rank_query_heads(rank: int, heads: int, t: int) -> list[int]:
    """Query heads of a rank: a/t consecutive heads; t must divide a."""
    if heads % t:
        raise ValueError(f"t={t} does not divide {heads} heads")
    hq = heads // t
    return list(range(rank * hq, (rank + 1) * hq))


def rank_kv_heads(rank: int, heads: int, kv_heads: int, t: int) -> list[int]:
    """KV heads a rank must hold: those its query heads use.  With fewer KV
    heads than t the same KV head appears on several ranks (replication)."""
    return sorted({kv_head_of(j, heads, kv_heads) for j in rank_query_heads(rank, heads, t)})


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotary position embedding, rotate-half form (reading: the pages do not
    name RoPE's convention).  x [..., n, d], pos [n]; the pair (k, k + d/2) is
    rotated by the angle pos * base^(-2k/d)."""
    d = x.shape[-1]
    half = d // 2
    k = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * k / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def causal_attention(q, k, v, q_pos=None) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v with key p' visible to query p iff p' <= p.

    q [nq, d] at positions q_pos (default 0..nq-1); k, v [n, d] at 0..n-1."""
    d = q.shape[-1]
    nq = q.shape[0]
    if q_pos is None:
        q_pos = np.arange(nq)
    s = (q @ k.T) / math.sqrt(d)
    mask = np.arange(k.shape[0])[None, :] > np.asarray(q_pos)[:, None]
    s = np.where(mask, -np.inf, s)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def attn_heads_output(x, wq, wk, wv, heads: int, kv_heads: int, head_dim: int,
                      batch: int, seq: int, rope_base: float, q_heads: list[int],
                      rows=None, bq=None, bk=None, bv=None) -> np.ndarray:
    """Concatenated outputs of the given query heads, [len(rows), len(q_heads)*d].

    x [batch*seq, h]; wq [h, heads*d]; wk, wv [h, kv_heads*d] (math convention);
    optional biases bq [heads*d], bk, bv [kv_heads*d], added before RoPE.
    ``rows`` selects output token rows (default: all); K and V are still
    computed for every token, since a row sees its whole causal prefix."""
    d = head_dim

    def proj(xx, w, b, j):
        return linear(xx, w[:, j * d:(j + 1) * d], None if b is None else b[j * d:(j + 1) * d])

    m = batch * seq
    rows = np.arange(m) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows), len(q_heads) * d))
    pos_all = np.arange(seq)
    kv_needed = sorted({kv_head_of(j, heads, kv_heads) for j in q_heads})
    for b in range(batch):
        sel = np.nonzero((rows >= b * seq) & (rows < (b + 1) * seq))[0]
        if len(sel) == 0:
            continue
        xb = x[b * seq:(b + 1) * seq]
        qpos = rows[sel] - b * seq
        kv = {}
        for g in kv_needed:
            kh = rope(proj(xb, wk, bk, g), pos_all, rope_base)
            vh = proj(xb, wv, bv, g)
            kv[g] = (kh, vh)
        xq = xb[qpos]
        for c, j in enumerate(q_heads):
            qh = rope(proj(xq, wq, bq, j), qpos, rope_base)
            kh, vh = kv[kv_head_of(j, heads, kv_heads)]
            out[sel, c * d:(c + 1) * d] = causal_attention(qh, kh, vh, qpos)
    return out


def attn_partial(x, w: dict, case, rank: int, t: int | None = None, rows=None) -> np.ndarray:
    """Rank ``rank``'s o_proj partial: the outputs of its a/t heads times the
    rows of Wo that belong to those heads.  ``t = 1`` gives the unsharded layer."""
    t = case.t if t is None else t
    q_heads = rank_query_heads(rank, case.heads, t)
    o = attn_heads_output(x, w["Wq"], w["Wk"], w["Wv"], case.heads, case.kv_heads,
                          case.head_dim, case.batch, case.seq, case.rope_base, q_heads, rows,
                          w.get("bq"), w.get("bk"), w.get("bv"))
    d = case.head_dim
    wo_rows = w["Wo"][q_heads[0] * d:(q_heads[-1] + 1) * d]
    return o @ wo_rows


# --------------------------------------------------------------------------
# norm and block ("f and g": norms and residuals are replicated)
# --------------------------------------------------------------------------


def rmsnorm(x, gain=None, eps: float = 1e-5) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain, per row (reading: eps and the gain are
    not given by the pages)."""
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x * r
    if gain is not None:
        y = y * np.asarray(gain, dtype=np.float64)
    return y


def block(x, w: dict, case, t: int | None = None, rows=None) -> dict:
    """One pre-norm block computed rank by rank and summed:

    h1 = X + sum_i Attn_i(RMSNorm(X)),  Z = h1 + sum_i MLP_i(RMSNorm(h1)).

    Returns the sampled rows of h1 and Z (all rows by default); ``t = 1`` is
    the unsharded block."""
    t = case.t if t is None else t
    m = case.tokens
    rows = np.arange(m) if rows is None else np.asarray(rows)
    xn = rmsnorm(x, w.get("g_attn"), case.eps)
    attn_parts = [attn_partial(xn, w, case, r, t, rows) for r in range(t)]
    h1 = x[rows] + shard_sum(attn_parts)
    hn = rmsnorm(h1, w.get("g_mlp"), case.eps)
    mlp_parts = mlp_swiglu_partials(hn, w["W1"], w["W3"], w["W2"], t)
    z = h1 + shard_sum(mlp_parts)
    return {"h1": h1, "z": z, "attn_partials": attn_parts, "mlp_partials": mlp_parts}


# --------------------------------------------------------------------------
# sequence-parallel form ("Sequence parallelism"; "Writing it in PyTorch")
# --------------------------------------------------------------------------


def seq_slices(batch: int, seq: int, t: int) -> list[np.ndarray]:
    """Token rows (row = b * seq + p) that rank r holds: positions
    [r seq/t, (r+1) seq/t) of every sequence, the Shard(1) split of a
    (batch, sequence, hidden) tensor.  Reading: t divides seq, so the slices
    are equal (the pages give no rule for a remainder)."""
    if seq % t:
        raise ValueError(f"sequence length {seq} is not divisible by t = {t}")
    n = seq // t
    return [np.concatenate([b * seq + np.arange(r * n, (r + 1) * n) for b in range(batch)])
            for r in range(t)]


def reduce_scatter(partials, slices) -> list[np.ndarray]:
    """Rank r receives the sum over ranks (ascending) of every partial's rows
    in its slice."""
    return [shard_sum([np.asarray(p)[rows] for p in partials]) for rows in slices]


def all_gather(pieces, slices, m: int) -> np.ndarray:
    """Every rank receives the full activation: the ranks' slices put back at
    their rows."""
    first = np.asarray(pieces[0])
    out = np.empty((m,) + first.shape[1:], dtype=np.float64)
    for rows, piece in zip(slices, pieces):
        out[rows] = piece
    return out


def sp_block(x, w: dict, case, t: int | None = None) -> dict:
    """The block with sequence parallelism, rank by rank:

    xn_r = RMSNorm(X[slice_r]);  xn = all-gather(xn_r)
    h1_r = X[slice_r] + reduce-scatter_r(Attn_i(xn))
    hn_r = RMSNorm(h1_r);        hn = all-gather(hn_r)
    Z_r  = h1_r + reduce-scatter_r(MLP_i(hn))

    Returns each rank's slices and the gathered h1 and Z."""
    t = case.t if t is None else t
    m = case.tokens
    x = np.asarray(x, dtype=np.float64)
    slices = seq_slices(case.batch, case.seq, t)
    xn = all_gather([rmsnorm(x[rows], w.get("g_attn"), case.eps) for rows in slices], slices, m)
    attn_parts = [attn_partial(xn, w, case, r, t) for r in range(t)]
    h1_r = [x[rows] + red for rows, red in zip(slices, reduce_scatter(attn_parts, slices))]
    hn = all_gather([rmsnorm(h, w.get("g_mlp"), case.eps) for h in h1_r], slices, m)
    mlp_parts = mlp_swiglu_partials(hn, w["W1"], w["W3"], w["W2"], t)
    z_r = [h + red for h, red in zip(h1_r, reduce_scatter(mlp_parts, slices))]
    return {"slices": slices, "h1_slices": h1_r, "z_slices": z_r,
            "h1": all_gather(h1_r, slices, m), "z": all_gather(z_r, slices, m)}


# --------------------------------------------------------------------------
# packed (fused) projections (diffusers guide, "Fused projections")
# --------------------------------------------------------------------------


def packed_blocks(dim: int, blocks, t: int) -> list[tuple[int, int]]:
    """(start, size) of each packed block of a dimension of ``dim``, from the
    proportions ``blocks``; each block must be divisible by t on its own."""
    total = sum(blocks)
    if dim % total:
        raise ValueError(f"packed dimension {dim} is not divisible by sum(blocks) = {total}")
    unit = dim // total
    out, start = [], 0
    for b in blocks:
        size = b * unit
        if size % t:
            raise ValueError(f"packed block of {size} is not divisible by t = {t}")
        out.append((start, size))
        start += size
    return out


def packed_rank_index(dim: int, blocks, t: int, rank: int) -> np.ndarray:
    """Indices of the packed dimension rank ``rank`` holds: its 1/t of every
    block, blocks in their packed order."""
    return np.concatenate([np.arange(s + rank * (n // t), s + (rank + 1) * (n // t))
                           for s, n in packed_blocks(dim, blocks, t)])


def full_attention(q, k, v) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v over every key (no mask)."""
    s = (q @ k.T) / math.sqrt(q.shape[-1])
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p / p.sum(axis=1, keepdims=True)) @ v


def single_stream_partial(x, w_in, w_out, heads: int, head_dim: int, batch: int, seq: int,
                          rope_base: float, t: int = 1, rank: int = 0, causal: bool = False,
                          naive: bool = False) -> np.ndarray:
    """Rank ``rank``'s partial of a packed single-stream block (t = 1: the
    whole layer):

    [Q | K | V | G | U] = X W_in   (W_in [h, 9h] in math convention, blocks
                                    [1, 1, 1, 3, 3]: the guide's mlp_ratio = 3)
    A = attention(RoPE(Q), RoPE(K), V) per head (every head its own K, V)
    M = SiLU(G) * U
    out = [A | M] W_out           (W_out [4h, h], input blocks [1, 3])

    The rank takes its 1/t of every block of W_in's columns (its heads and
    its slice of the MLP) and the matching rows of each block of W_out.
    ``naive`` instead slices both packed dimensions as plain contiguous
    ranges, the cut the guide warns against."""
    h = x.shape[1]
    d = head_dim
    if naive:
        n_in, n_out = w_in.shape[1] // t, w_out.shape[0] // t
        cols = np.arange(rank * n_in, (rank + 1) * n_in)
        rows = np.arange(rank * n_out, (rank + 1) * n_out)
    else:
        cols = packed_rank_index(w_in.shape[1], [1, 1, 1, 3, 3], t, rank)
        rows = packed_rank_index(w_out.shape[0], [1, 3], t, rank)
    w = w_in[:, cols]
    hr, mr = h // t, 3 * h // t
    wq, wk, wv = w[:, :hr], w[:, hr:2 * hr], w[:, 2 * hr:3 * hr]
    wg, wu = w[:, 3 * hr:3 * hr + mr], w[:, 3 * hr + mr:]
    nh = hr // d
    attn = np.zeros((x.shape[0], hr))
    pos = np.arange(seq)
    for b in range(batch):
        xb = x[b * seq:(b + 1) * seq]
        for j in range(nh):
            sl = slice(j * d, (j + 1) * d)
            q = rope(xb @ wq[:, sl], pos, rope_base)
            k = rope(xb @ wk[:, sl], pos, rope_base)
            v = xb @ wv[:, sl]
            attn[b * seq:(b + 1) * seq, sl] = causal_attention(q, k, v) if causal else full_attention(q, k, v)
    mlp = silu(x @ wg) * (x @ wu)
    return np.concatenate([attn, mlp], axis=1) @ w_out[rows]


# --------------------------------------------------------------------------
# vocabulary-parallel embedding and cross-entropy ("Embedding and output layer")
# --------------------------------------------------------------------------


def embedding_lookup(table, ids) -> np.ndarray:
    """Row ids[i] of the [v, h] table for every token (nn.Embedding layout;
    the page writes E in R^{h x v}, the same matrix transposed)."""
    return np.asarray(table, dtype=np.float64)[np.asarray(ids)]


def embedding_rowwise_partials(table, ids, t: int) -> list[np.ndarray]:
    """Rank r holds vocabulary rows [r v/t, (r+1) v/t): its partial is the row
    for the ids it holds and zero for the others; the sum is the lookup."""
    table = np.asarray(table, dtype=np.float64)
    ids = np.asarray(ids)
    v = table.shape[0]
    if v % t:
        raise ValueError(f"vocabulary {v} is not divisible by t = {t}")
    n = v // t
    out = []
    for r in range(t):
        mine = (ids >= r * n) & (ids < (r + 1) * n)
        p = np.zeros((len(ids), table.shape[1]))
        p[mine] = table[ids[mine]]
        out.append(p)
    return out


def embedding_colwise_slices(table, ids, t: int) -> list[np.ndarray]:
    """Rank r holds hidden columns [r h/t, (r+1) h/t) of every row; gathering
    the slices side by side gives the lookup."""
    return [embedding_lookup(c, ids) for c in split_columns(np.asarray(table, dtype=np.float64), t)]


def cross_entropy(logits, labels, v: int | None = None) -> tuple[np.ndarray, float]:
    """Per-token loss log(sum_j exp x_j) - x_label and the mean over tokens
    whose label lies in [0, v) (others are ignored: loss 0)."""
    x = np.asarray(logits, dtype=np.float64)
    labels = np.asarray(labels)
    v = x.shape[1] if v is None else v
    ok = (labels >= 0) & (labels < v)
    mx = x.max(axis=1)
    lse = np.log(np.exp(x - mx[:, None]).sum(axis=1)) + mx
    loss = np.where(ok, lse - x[np.arange(len(labels)), np.where(ok, labels, 0)], 0.0)
    return loss, (float(loss[ok].mean()) if ok.any() else 0.0)


def vocab_ce_stats(logits_r, labels, v_start: int) -> np.ndarray:
    """One rank's statistics per token from its slice of the logits (its
    vocabulary [v_start, v_start + n)): max, sum of exp(x - max), the label's
    logit if the rank holds the label (else 0), and 1 if it does (else 0)."""
    x = np.asarray(logits_r, dtype=np.float64)
    labels = np.asarray(labels)
    n = x.shape[1]
    mx = x.max(axis=1)
    s = np.exp(x - mx[:, None]).sum(axis=1)
    mine = (labels >= v_start) & (labels < v_start + n)
    z = np.where(mine, x[np.arange(len(labels)), np.clip(labels - v_start, 0, n - 1)], 0.0)
    return np.stack([mx, s, z, mine.astype(np.float64)], axis=1)


def vocab_ce_combine(stats) -> np.ndarray:
    """Per-token loss from every rank's statistics (the b x s exchange):
    M = max_r max_r, S = sum_r sum_r exp(max_r - M), loss = log S + M - x_label;
    a token no rank holds the label of is ignored (loss 0)."""
    st = np.stack([np.asarray(s, dtype=np.float64) for s in stats])   # [t, m, 4]
    mx = st[:, :, 0].max(axis=0)
    s = (st[:, :, 1] * np.exp(st[:, :, 0] - mx[None, :])).sum(axis=0)
    z = st[:, :, 2].sum(axis=0)
    owners = st[:, :, 3].sum(axis=0)
    return np.where(owners == 1, np.log(s) + mx - z, 0.0)


def vocab_parallel_ce(x, w_out, labels, t: int) -> np.ndarray:
    """Per-token loss of the output layer X W_out (W_out [h, v]) with the
    vocabulary split over t ranks: each rank's logits, its statistics, then
    the combination."""
    v = w_out.shape[1]
    if v % t:
        raise ValueError(f"vocabulary {v} is not divisible by t = {t}")
    n = v // t
    return vocab_ce_combine([vocab_ce_stats(x @ w_out[:, r * n:(r + 1) * n], labels, r * n) for r in range(t)])


# --------------------------------------------------------------------------
# backward of the MLP shard ("f and g": g's backward is the identity, f's is
# the all-reduce of the input-gradient partials)
# --------------------------------------------------------------------------


def gelu_grad(x):
    """d/dx [x Phi(x)] = Phi(x) + x phi(x)."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + _erf(x / math.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def silu_grad(x):
    """d/dx [x sigma(x)] = sigma(x) (1 + x (1 - sigma(x)))."""
    x = np.asarray(x, dtype=np.float64)
    sg = 1.0 / (1.0 + np.exp(-x))
    return sg * (1.0 + x * (1.0 - sg))


def mlp_gelu_backward(x, a, b, dz) -> dict:
    """Gradients of Z = GeLU(X A) B for the output gradient dZ (full A, B: the
    unsharded layer; A_i, B_i: rank i's share, whose dX is its partial)."""
    pre = x @ a
    dy = dz @ b.T
    dpre = dy * gelu_grad(pre)
    return {"dx": dpre @ a.T, "da": x.T @ dpre, "db": gelu(pre).T @ dz}


def mlp_gelu_backward_partials(x, a, b, dz, t: int) -> list[dict]:
    """Rank i's gradients from its column shard of A and row shard of B; the
    sum of the dX partials is dX (f's backward), the weight gradients are the
    shards of the full ones."""
    return [mlp_gelu_backward(x, ai, bi, dz) for ai, bi in zip(split_columns(a, t), split_rows(b, t))]


def mlp_swiglu_backward(x, w1, w3, w2, dz) -> dict:
    """Gradients of Z = (SiLU(X W1) * (X W3)) W2 for dZ."""
    g, u = x @ w1, x @ w3
    dy = dz @ w2.T
    dg = dy * u * silu_grad(g)
    du = dy * silu(g)
    return {"dx": dg @ w1.T + du @ w3.T, "dw1": x.T @ dg, "dw3": x.T @ du, "dw2": (silu(g) * u).T @ dz}


def mlp_swiglu_backward_partials(x, w1, w3, w2, dz, t: int) -> list[dict]:
    return [mlp_swiglu_backward(x, a, c, b, dz)
            for a, c, b in zip(split_columns(w1, t), split_columns(w3, t), split_rows(w2, t))]



# --------------------------------------------------------------------------
# backward of the attention shard ("f and g": the same rule as the MLP; the
# "Self-attention" split makes each rank's gradients those of its own heads)
# --------------------------------------------------------------------------


def rope_backward(g: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Gradient through ``rope``: each pair (k, k + d/2) is rotated by the
    angle's negative (the transpose of the rotation)."""
    d = g.shape[-1]
    half = d // 2
    k = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * k / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    g1, g2 = g[..., :half], g[..., half:]
    return np.concatenate([g1 * c + g2 * s, g2 * c - g1 * s], axis=-1)


def attention_lse(q, k, causal: bool = True) -> np.ndarray:
    """Per query row, log(sum_j exp(q k_j / sqrt(d))) over the visible keys
    (the softmax's normaliser in log form), natural log."""
    d = q.shape[-1]
    s = (q @ k.T) / math.sqrt(d)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > np.arange(q.shape[0])[:, None], -np.inf, s)
    mx = s.max(axis=1, keepdims=True)
    return (mx + np.log(np.exp(s - mx).sum(axis=1, keepdims=True)))[:, 0]


def causal_attention_backward(q, k, v, do, causal: bool = True):
    """Gradients (dq, dk, dv) of O = softmax(q k^T / sqrt(d), causal) v for dO
    (``causal=False``: every key visible).

    With P the probabilities: dV = P^T dO, dP = dO V^T, and the softmax
    Jacobian gives dS = P * (dP - rowsum(dP * P)); the scale carries through to
    dq = dS k / sqrt(d) and dk = dS^T q / sqrt(d)."""
    d = q.shape[-1]
    n = q.shape[0]
    s = (q @ k.T) / math.sqrt(d)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > np.arange(n)[:, None], -np.inf, s)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - np.sum(dp * p, axis=1, keepdims=True))
    return ds @ k / math.sqrt(d), ds.T @ q / math.sqrt(d), dv


def attn_backward(x, wq, wk, wv, wo, dz, heads: int, kv_heads: int, head_dim: int, batch: int,
                  seq: int, rope_base: float, q_heads: list[int] | None = None) -> dict:
    """Gradients of the attention sublayer Z = concat_j(attn_j) Wo restricted to
    the query heads ``q_heads`` (default all) and the KV heads they read, for
    the output gradient dZ.  Weights in math convention: wq [h, heads*d],
    wk, wv [h, kv_heads*d], wo [heads*d, h_out].

    Returns dx [m, h] (a rank's input-gradient partial), dwq [h, nq*d],
    dwk, dwv [h, nkv*d] (a KV head shared with other ranks gets only this
    rank's share), dwo [nq*d, h_out] and dqkv [m, (nq + 2 nkv) d], the
    gradient of the projections before RoPE packed as Q heads, K heads, V
    heads (what a rank feeds its weight-gradient products)."""
    d = head_dim
    q_heads = list(range(heads)) if q_heads is None else list(q_heads)
    kv_list = sorted({kv_head_of(j, heads, kv_heads) for j in q_heads})
    nq, nkv = len(q_heads), len(kv_list)
    m = batch * seq
    pos = np.arange(seq)
    wo_rows = np.concatenate([wo[j * d:(j + 1) * d] for j in q_heads], axis=0)
    do_all = dz @ wo_rows.T
    o_all = np.zeros((m, nq * d))
    dqkv = np.zeros((m, (nq + 2 * nkv) * d))
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        xb = x[rows]
        kv = {}
        for g in kv_list:
            kv[g] = (rope(xb @ wk[:, g * d:(g + 1) * d], pos, rope_base), xb @ wv[:, g * d:(g + 1) * d])
        dk = {g: np.zeros((seq, d)) for g in kv_list}
        dv = {g: np.zeros((seq, d)) for g in kv_list}
        for c, j in enumerate(q_heads):
            g = kv_head_of(j, heads, kv_heads)
            qh = rope(xb @ wq[:, j * d:(j + 1) * d], pos, rope_base)
            kh, vh = kv[g]
            o_all[rows, c * d:(c + 1) * d] = causal_attention(qh, kh, vh)
            dq_h, dk_h, dv_h = causal_attention_backward(qh, kh, vh, do_all[rows, c * d:(c + 1) * d])
            dqkv[rows, c * d:(c + 1) * d] = rope_backward(dq_h, pos, rope_base)
            dk[g] += dk_h
            dv[g] += dv_h
        for e, g in enumerate(kv_list):
            dqkv[rows, (nq + e) * d:(nq + e + 1) * d] = rope_backward(dk[g], pos, rope_base)
            dqkv[rows, (nq + nkv + e) * d:(nq + nkv + e + 1) * d] = dv[g]
    wq_r = np.concatenate([wq[:, j * d:(j + 1) * d] for j in q_heads], axis=1)
    wk_r = np.concatenate([wk[:, g * d:(g + 1) * d] for g in kv_list], axis=1)
    wv_r = np.concatenate([wv[:, g * d:(g + 1) * d] for g in kv_list], axis=1)
    w_r = np.concatenate([wq_r, wk_r, wv_r], axis=1)
    dw = x.T @ dqkv
    return {"dx": dqkv @ w_r.T, "dwq": dw[:, :nq * d], "dwk": dw[:, nq * d:(nq + nkv) * d],
            "dwv": dw[:, (nq + nkv) * d:], "dwo": o_all.T @ dz, "dqkv": dqkv, "o": o_all}


def attn_backward_partials(x, w: dict, dz, case, t: int | None = None) -> list[dict]:
    """Every rank's ``attn_backward`` over its a/t query heads."""
    t = case.t if t is None else t
    return [attn_backward(x, w["Wq"], w["Wk"], w["Wv"], w["Wo"], dz, case.heads, case.kv_heads,
                          case.head_dim, case.batch, case.seq, case.rope_base,
                          rank_query_heads(r, case.heads, t)) for r in range(t)]


# --------------------------------------------------------------------------
# backward of the block ("f and g": a block's backward has the two sums of
# the sublayers' dX partials; norms and residuals are replicated, so their
# gradients are taken on every rank after the sum)
# --------------------------------------------------------------------------


def rmsnorm_backward(x, gain, dy, eps: float = 1e-5) -> tuple[np.ndarray, np.ndarray]:
    """Gradients (dx, dgain) of y = x r gain, r = 1 / sqrt(mean(x^2) + eps), per
    row, for dy.  With g = gain * dy and x_hat = x r, differentiating r gives
    dx = r (g - x_hat mean(g x_hat)); dgain sums dy x_hat over the rows."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    gn = np.ones(x.shape[-1]) if gain is None else np.asarray(gain, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    xh = x * r
    g = dy * gn
    dx = r * (g - xh * np.mean(g * xh, axis=-1, keepdims=True))
    return dx, np.sum(dy * xh, axis=0)


def block_backward(x, w: dict, case, dz, t: int | None = None) -> dict:
    """Gradients of the pre-norm block of ``block`` for the output gradient dZ,
    rank by rank: the MLP ranks' dX partials are summed (f's backward) into the
    gradient of the MLP's normed input, taken through the norm and added to dZ
    (the residual) to give dh1; the attention ranks' dX partials for dh1 are
    summed and taken through the first norm, plus dh1, to give dX.  Returns
    dx, dh1, the gains' gradients and every rank's weight gradients."""
    t = case.t if t is None else t
    xn = rmsnorm(x, w.get("g_attn"), case.eps)
    h1 = x + shard_sum([attn_partial(xn, w, case, r, t) for r in range(t)])
    hn = rmsnorm(h1, w.get("g_mlp"), case.eps)
    mlp = mlp_swiglu_backward_partials(hn, w["W1"], w["W3"], w["W2"], dz, t)
    d_hn = shard_sum([p["dx"] for p in mlp])
    d1, dg_mlp = rmsnorm_backward(h1, w.get("g_mlp"), d_hn, case.eps)
    dh1 = dz + d1
    attn = attn_backward_partials(xn, w, dh1, case, t)
    d_xn = shard_sum([p["dx"] for p in attn])
    d0, dg_attn = rmsnorm_backward(x, w.get("g_attn"), d_xn, case.eps)
    return {"dx": dh1 + d0, "dh1": dh1, "dg_attn": dg_attn, "dg_mlp": dg_mlp, "mlp": mlp, "attn": attn}

