"""Seeded synthetic workloads: the five model shapes and their input tensors.

This module only draws numbers and names shapes; it holds none of the
tensor-parallel method's arithmetic.  The GPU path and the CPU oracle both take
their inputs from here, and from nowhere else.

Every tensor is drawn *unsharded* and in the math convention of the
"Tensor parallelism" (itwiki) page, section "Matmul split": a linear layer
computes ``Y = X @ A`` with ``A`` of shape ``[in, out]``.  Sharding is done by
each consumer on its own.

Two draws exist:

* ``"torch"`` -- the worked example of the same page (section "MLP"): the
  global CPU generator seeded with ``torch.manual_seed(seed)`` and
  ``torch.randn`` calls in the order X, A, B.  Used for the tiny fp32 case, so
  its inputs are exactly the page's.
* ``"counter"`` -- a counter-based generator in C (``synth/synth.c``:
  SplitMix64 + Box-Muller).  Element ``i`` of stream ``s`` depends only on
  ``(seed, s, i)``, so the multi-GB shapes draw in seconds on all host cores.
  Streams are numbered in the order the tensors are listed for each shape.

bf16 tensors are drawn in float32 and rounded once to nearest-even; they are
held as raw ``uint16`` bit patterns (numpy has no bfloat16).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from pathlib import Path

import numpy as np

_SYNTH = Path(__file__).resolve().parent / "synth" / "_synth.so"
_lib = None


def _synth():
    global _lib
    if _lib is None:
        if not _SYNTH.exists():
            from . import build

            build.build_synth()
        lib = ctypes.CDLL(str(_SYNTH))
        u64, i64, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32
        vp = ctypes.c_void_p
        lib.synth_normal_f32.argtypes = [u64, u64, i64, i64, ctypes.c_double, vp]
        lib.synth_normal_bf16.argtypes = [u64, u64, i64, i64, ctypes.c_double, vp]
        lib.synth_int_f32.argtypes = [u64, u64, i64, i64, i32, i32, vp]
        for f in (lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_int_f32):
            f.restype = None
        _lib = lib
    return _lib


# --------------------------------------------------------------------------
# host tensors
# --------------------------------------------------------------------------


@dataclass
class HostTensor:
    """A host array in the dtype the GPU path computes in.

    ``data`` is float32 for ``dtype == "f32"`` and the uint16 bit pattern for
    ``dtype == "bf16"``.
    """

    data: np.ndarray
    dtype: str

    @property
    def shape(self):
        return self.data.shape

    def f32(self) -> np.ndarray:
        if self.dtype == "f32":
            return self.data
        return bf16_bits_to_f32(self.data)

    def f64(self) -> np.ndarray:
        """Exact float64 copy (widened with torch's multithreaded conversion)."""
        return self.torch().to(dtype=_torch().float64).numpy()

    def torch(self):
        import torch

        if self.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(self.data))
        return torch.from_numpy(np.ascontiguousarray(self.data).view(np.int16)).view(torch.bfloat16)


def _torch():
    import torch

    return torch


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def normal(seed: int, stream: int, shape, std: float = 1.0, dtype: str = "bf16") -> HostTensor:
    n = int(np.prod(shape))
    lib = _synth()
    if dtype == "bf16":
        out = np.empty(n, np.uint16)
        lib.synth_normal_bf16(seed, stream, 0, n, std, out.ctypes.data)
    elif dtype == "f32":
        out = np.empty(n, np.float32)
        lib.synth_normal_f32(seed, stream, 0, n, std, out.ctypes.data)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    return HostTensor(out.reshape(shape), dtype)


def integers(seed: int, stream: int, shape, lo: int, hi: int, dtype: str = "bf16") -> HostTensor:
    """Integers uniform on [lo, hi]; exact in bf16 for |v| <= 256."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    _synth().synth_int_f32(seed, stream, 0, n, lo, hi, out.ctypes.data)
    out = out.reshape(shape)
    if dtype == "f32":
        return HostTensor(out, "f32")
    return HostTensor((out.view(np.uint32) >> 16).astype(np.uint16), "bf16")


def from_f32(values: np.ndarray, dtype: str) -> HostTensor:
    """Wraps float32 values; for bf16 they are rounded to nearest-even."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    if dtype == "f32":
        return HostTensor(v, "f32")
    u = v.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return HostTensor(u.astype(np.uint16), "bf16")


def torch_seeded(seed: int, shapes) -> list[HostTensor]:
    """``torch.manual_seed(seed)`` then one ``torch.randn`` per shape, in order."""
    import torch

    g = torch.Generator().manual_seed(seed)
    return [HostTensor(torch.randn(*s, generator=g).numpy(), "f32") for s in shapes]


# --------------------------------------------------------------------------
# workload shapes
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class MLPCase:
    """``Z = act(X @ A) @ B`` sharded ``t`` ways (A colwise, B rowwise)."""

    name: str
    tokens: int
    hidden: int
    inter: int
    t: int
    act: str  # "gelu" | "swiglu"
    dtype: str  # "f32" | "bf16"
    seed: int
    draw: str = "counter"
    x_std: float = 1.0
    w_std: float = 0.02

    @property
    def f_shard(self) -> int:
        return self.inter // self.t


@dataclass(frozen=True)
class AttnCase:
    """Causal self-attention, heads split ``t`` ways, o_proj rowwise."""

    name: str
    batch: int
    seq: int
    hidden: int
    heads: int
    kv_heads: int
    head_dim: int
    t: int
    rope_base: float
    seed: int
    dtype: str = "bf16"
    x_std: float = 1.0
    w_std: float = 0.02

    @property
    def tokens(self) -> int:
        return self.batch * self.seq


@dataclass(frozen=True)
class BlockCase:
    """Pre-norm block: ``h1 = X + Attn(RMSNorm(X))``, ``Z = h1 + MLP(RMSNorm(h1))``."""

    name: str
    batch: int
    seq: int
    hidden: int
    heads: int
    kv_heads: int
    head_dim: int
    inter: int
    t: int
    rope_base: float
    seed: int
    eps: float = 1e-5
    gain_std: float = 0.0  # gain = 1 + gain_std * N(0,1); 0 means gain == 1
    dtype: str = "bf16"
    x_std: float = 1.0
    w_std: float = 0.02

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    def attn(self) -> AttnCase:
        return AttnCase(self.name + "/attn", self.batch, self.seq, self.hidden, self.heads,
                        self.kv_heads, self.head_dim, self.t, self.rope_base, self.seed)


CONFIGS = {
    # The worked example of the "Tensor parallelism" page, section "MLP".
    "tiny_mlp_f32": MLPCase("tiny_mlp_f32", tokens=4, hidden=16, inter=64, t=4, act="gelu",
                            dtype="f32", seed=0, draw="torch", w_std=1.0),
    "gpt_gelu_mlp": MLPCase("gpt_gelu_mlp", tokens=2048, hidden=1024, inter=4096, t=4,
                            act="gelu", dtype="bf16", seed=2),
    "llama8b_swiglu_mlp": MLPCase("llama8b_swiglu_mlp", tokens=4096, hidden=4096, inter=14336,
                                  t=4, act="swiglu", dtype="bf16", seed=3),
    "llama8b_attn": AttnCase("llama8b_attn", batch=2, seq=2048, hidden=4096, heads=32,
                             kv_heads=8, head_dim=128, t=4, rope_base=500000.0, seed=4),
    "llama70b_block_t8": BlockCase("llama70b_block_t8", batch=4, seq=2048, hidden=8192,
                                   heads=64, kv_heads=8, head_dim=128, inter=28672, t=8,
                                   rope_base=500000.0, seed=5),
    "llama70b_block_t16": BlockCase("llama70b_block_t16", batch=4, seq=2048, hidden=8192,
                                    heads=64, kv_heads=8, head_dim=128, inter=28672, t=16,
                                    rope_base=500000.0, seed=5),
}


def gen_mlp(case: MLPCase) -> dict[str, HostTensor]:
    """Unsharded MLP tensors in math convention.

    gelu: X [m,h], A [h,f], B [f,h]; swiglu: X [m,h], W1 [h,f], W3 [h,f], W2 [f,h].
    """
    m, h, f = case.tokens, case.hidden, case.inter
    if case.draw == "torch":
        if case.act != "gelu":
            raise ValueError("the torch draw reproduces the GeLU example only")
        x, a, b = torch_seeded(case.seed, [(m, h), (h, f), (f, h)])
        return {"X": x, "A": a, "B": b}
    d = case.dtype
    if case.act == "gelu":
        return {
            "X": normal(case.seed, 0, (m, h), case.x_std, d),
            "A": normal(case.seed, 1, (h, f), case.w_std, d),
            "B": normal(case.seed, 2, (f, h), case.w_std, d),
        }
    if case.act == "swiglu":
        return {
            "X": normal(case.seed, 0, (m, h), case.x_std, d),
            "W1": normal(case.seed, 1, (h, f), case.w_std, d),
            "W3": normal(case.seed, 2, (h, f), case.w_std, d),
            "W2": normal(case.seed, 3, (f, h), case.w_std, d),
        }
    raise ValueError(f"unknown activation {case.act!r}")


def gen_attn(case, stream0: int = 0) -> dict[str, HostTensor]:
    """X [m,h], Wq [h,a*d], Wk [h,kv*d], Wv [h,kv*d], Wo [a*d,h] (math convention)."""
    m, h, d = case.tokens, case.hidden, case.head_dim
    qd, kd = case.heads * d, case.kv_heads * d
    s, dt = case.seed, case.dtype
    return {
        "X": normal(s, stream0 + 0, (m, h), case.x_std, dt),
        "Wq": normal(s, stream0 + 1, (h, qd), case.w_std, dt),
        "Wk": normal(s, stream0 + 2, (h, kd), case.w_std, dt),
        "Wv": normal(s, stream0 + 3, (h, kd), case.w_std, dt),
        "Wo": normal(s, stream0 + 4, (qd, h), case.w_std, dt),
    }


def gen_block(case: BlockCase) -> dict[str, HostTensor]:
    """Attention tensors (streams 0-4), W1/W3/W2 (5-7), norm gains (8, 9) in float32."""
    out = gen_attn(case)
    h, f, s, dt = case.hidden, case.inter, case.seed, case.dtype
    out["W1"] = normal(s, 5, (h, f), case.w_std, dt)
    out["W3"] = normal(s, 6, (h, f), case.w_std, dt)
    out["W2"] = normal(s, 7, (f, h), case.w_std, dt)
    for k, stream in (("g_attn", 8), ("g_mlp", 9)):
        if case.gain_std:
            g = normal(s, stream, (h,), case.gain_std, "f32").data + np.float32(1.0)
        else:
            g = np.ones(h, np.float32)
        out[k] = HostTensor(g.astype(np.float32), "f32")
    return out


def sample_rows(batch: int, seq: int, per_seq: int, seed: int) -> np.ndarray:
    """Token rows for sampled parity checks: positions {0, 1, seq-1} of every
    sequence plus ``per_seq`` seeded positions, as sorted global row indices."""
    rows = []
    for b in range(batch):
        base = b * seq
        picks = {0, min(1, seq - 1), seq - 1}
        if per_seq:
            u = np.empty(per_seq, np.float32)
            _synth().synth_int_f32(seed, 1000 + b, 0, per_seq, 0, seq - 1, u.ctypes.data)
            picks.update(int(v) for v in u)
        rows.extend(base + p for p in sorted(picks))
    return np.asarray(rows, dtype=np.int64)
