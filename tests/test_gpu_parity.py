"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every comparison uses the same seeded inputs on both sides.  Bars:
* float32 cases: max |gpu - oracle| <= 1e-4 (the worked example's atol);
* bf16 cases: max |gpu - oracle| / max |oracle| <= 2e-2 per compared tensor;
* integer-valued GEMMs and the shard-sum: bit-exact.
Small cases are compared element by element; the full-size workloads on
sampled token rows (every op but attention is row-local, and attention rows
need only K and V, which the oracle computes for every token).
"""
import time

import math

import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_colwise_amd import inputs, shard, tpshard as tp

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_ATOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not tp.LIB_PATH.exists():
        raise RuntimeError("libtpshard.so is not built")
    torch.cuda.set_device(0)
    tp.tp_device_check()
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    e = float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))
    say(f"  max|gpu-oracle|/max|oracle| = {e:.3e}")
    return e


def to_dev(ht, dev):
    return ht.torch().to(dev)


def host(t, rows=None):
    if rows is not None:
        t = t[torch.from_numpy(np.asarray(rows)).to(t.device)]
    return t.detach().float().cpu().double().numpy()


# ---------------------------------------------------------------- worked example (float32)


def test_tiny_mlp_f32_worked_example(device):
    """Seed-0 example of the "MLP" section, float32: every partial and the sum
    within atol 1e-4 of the oracle, and the page's allclose predicate holds."""
    case = inputs.CONFIGS["tiny_mlp_f32"]
    say(f"case {case.name}")
    w = inputs.gen_mlp(case)
    dw = {k: to_dev(v, device) for k, v in w.items()}
    mlp = shard.MLPShards(dw["X"], dw, case.t, "gelu", "f32")
    out = mlp.forward()
    torch.cuda.synchronize()
    x, a, b = w["X"].f64(), w["A"].f64(), w["B"].f64()
    ref = oracle.mlp_gelu(x, a, b)
    parts = oracle.mlp_gelu_partials(x, a, b, case.t)
    for r in range(case.t):
        assert np.max(np.abs(host(mlp.partials[r]) - parts[r])) <= F32_ATOL
    got = host(out)
    say(f"  max|gpu-oracle| = {np.max(np.abs(got - ref)):.3e}")
    assert np.max(np.abs(got - ref)) <= F32_ATOL
    assert np.allclose(got, ref, atol=1e-4, rtol=1e-5)


# ---------------------------------------------------------------- exact GEMMs


@pytest.mark.parametrize("m,k,n", [(300, 520, 264), (520, 1032, 520), (1, 8, 8), (257, 64, 256)])
def test_rowwise_gemm_integer_bit_exact(device, m, k, n):
    """Integer inputs in [-2, 2]: every product and sum is exact in float32, so
    the partial must equal the oracle's float64 product bit for bit.  Shapes
    cover one and several 256 x 256 tiles, ragged m/n and a k tail."""
    say(f"case rowwise int m={m} k={k} n={n}")
    y = inputs.integers(7, 0, (m, k), -2, 2)
    w = inputs.integers(7, 1, (n, k), -2, 2)
    out = torch.empty(m, n, dtype=torch.float32, device=device)
    tp.tp_rowwise("bf16", m, k, n, to_dev(y, device), to_dev(w, device), out)
    torch.cuda.synchronize()
    ref = y.f64() @ w.f64().T
    assert np.array_equal(host(out), ref)


@pytest.mark.parametrize("m,k,n,plan", [
    (4096, 64, 4096, (256, 16, 256)),     # 256-row tiles
    (8192, 72, 1280, (192, 5, 192)),      # 192-row tiles, k tail of 8
    (8192, 64, 7168, (256, 24, 128)),     # main range at 256, tail columns at 128
    (4000, 136, 776, (128, 4, 128)),      # 128-row tiles, ragged m and n
    (1000, 136, 776, (64, 7, 64)),        # small tiles (64 x 128): ragged m and n, k tail of 8
    (2048, 1024, 1024, (64, 8, 64)),      # small tiles, the GPT MLP shape: whole k-steps only
    (130, 128, 200, (64, 2, 64)),         # small tiles, two k-steps (the ring never wraps)
    (130, 192, 200, (64, 2, 64)),         # small tiles, three k-steps (each ring slot once)
    (300, 4104, 264, (64, 3, 64)),        # small tiles, deep k with a tail
    (7777, 72, 1280, (192, 5, 192)),      # 192-row tiles (96-row waves), ragged m
    (5000, 64, 3584, (192, 8, 128)),      # 192-row main range, 128-row tail, ragged m
    (4000, 2056, 4000, (256, 16, 256)),   # four-wave 256-row tiles: ragged m and n, k tail of 8
    (4096, 2048, 4096, (256, 16, 256)),   # four-wave 256-row tiles, whole k-steps only
    (4000, 2056, 776, (128, 4, 128)),     # four-wave 128-row tiles, ragged m and n, k tail
    (4000, 4104, 776, (128, 4, 128)),     # 16x16-MFMA 128-row tiles, deep k
    (4000, 2056, 2560, (192, 10, 192)),   # four-wave 192-row tiles, ragged m, k tail
    (5000, 2056, 3584, (192, 8, 128)),    # four-wave 192/128 split launch, ragged m, k tail
    (4000, 4104, 4000, (256, 16, 256)),   # 16x16-MFMA 256-row tiles: ragged m and n, k tail of 8
    (4096, 4096, 4096, (256, 16, 256)),   # 16x16-MFMA 256-row tiles, whole k-steps only
    (4000, 4168, 2560, (192, 10, 192)),   # 16x16-MFMA 192-row tiles, ragged m, k tail of 8
    (5000, 4104, 3584, (192, 8, 128)),    # 16x16-MFMA 192/128 split launch, ragged m, k tail
])
def test_rowwise_gemm_plans_bit_exact(device, m, k, n, plan):
    """Every tile height and the split launch, bit-exact on integer inputs."""
    say(f"case rowwise plan m={m} k={k} n={n} plan={plan}")
    assert tp.tp_gemm_plan(m, n, k) == (*plan, 0)
    y = inputs.integers(9, 0, (m, k), -2, 2)
    w = inputs.integers(9, 1, (n, k), -2, 2)
    out = torch.empty(m, n, dtype=torch.float32, device=device)
    tp.tp_rowwise("bf16", m, k, n, to_dev(y, device), to_dev(w, device), out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), y.f64() @ w.f64().T)


@pytest.mark.parametrize("m,k,n,plan", [
    (6100, 1096, 5904, (192, 24, 192)),   # eight-wave tiles, k tail of 8
    (6100, 2120, 5904, (192, 24, 192)),   # four-wave tiles, k tail of 8
    (8000, 2048, 4400, (192, 18, 192)),   # four-wave tiles, whole k-steps only
    (6100, 4104, 5904, (192, 24, 192)),   # 16x16-MFMA tiles, k tail of 8
])
def test_rowwise_gemm_many_tiles_bit_exact(device, m, k, n, plan):
    """Several rounds of tiles per launch (more tiles than compute units),
    ragged m and n, with and without a k tail: bit-exact on integer inputs."""
    say(f"case rowwise many tiles m={m} k={k} n={n} plan={plan}")
    assert tp.tp_gemm_plan(m, n, k) == (*plan, 0)
    y = inputs.integers(10, 0, (m, k), -2, 2)
    w = inputs.integers(10, 1, (n, k), -2, 2)
    out = torch.full((m, n), float("nan"), dtype=torch.float32, device=device)
    tp.tp_rowwise("bf16", m, k, n, to_dev(y, device), to_dev(w, device), out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), y.f64() @ w.f64().T)


@pytest.mark.parametrize("out,xk,m,n,k", [
    ("f32", True, 4000, 4000, 520),     # x and w k-major, ragged m and n, k tail
    ("f32", True, 4000, 2560, 136),     # 192-row tiles (three block groups per k group)
    ("f32", True, 4000, 776, 1032),     # 128-row tiles, ragged n
    ("f32", False, 4000, 4000, 520),    # k-contiguous x beside k-major w
    ("f32", False, 4000, 2560, 4104),   # the same, deep k with a tail
    ("bf16", False, 4000, 776, 4104),   # bf16 output
    ("bf16", True, 1000, 4000, 64),     # one k step, ragged m
])
def test_gemm_kmajor_bit_exact(device, out, xk, m, n, k):
    """tp_gemm_kmajor (the backward's products of a transposed operand) on
    integer inputs in [-2, 2], strided operands: float32 outputs equal the
    exact sums, bf16 outputs their rounding.  Its launches use 192- and
    128-row tiles (the shapes here take both, main ranges and tails)."""
    say(f"case gemm k-major out={out} x_kmajor={xk} m={m} n={n} k={k}")
    xl = inputs.integers(17, 0, (m, k), -2, 2)             # the logical x'
    wl = inputs.integers(17, 1, (k, n), -2, 2)             # w' = w, [k, n]
    ldx = (m if xk else k) + 8
    ldw = n + 16
    xs = torch.zeros((k, ldx) if xk else (m, ldx), dtype=torch.bfloat16)
    if xk:
        xs[:, :m] = xl.torch().T
    else:
        xs[:, :k] = xl.torch()
    ws = torch.zeros((k, ldw), dtype=torch.bfloat16)
    ws[:, :n] = wl.torch()
    dt = torch.float32 if out == "f32" else torch.bfloat16
    o = torch.full((m, n), float("nan"), dtype=dt, device=device)
    tp.tp_gemm_kmajor(out, xk, m, n, k, xs.to(device), ldx, ws.to(device), ldw, o)
    torch.cuda.synchronize()
    ref = xl.f64() @ wl.f64()
    assert np.array_equal(host(o), ref if out == "f32" else _bf16_rne(ref))


def _bf16_rne(v: np.ndarray) -> np.ndarray:
    """float64 values that float32 holds exactly, rounded to bfloat16 (nearest,
    ties to even) and widened back: the rounding of a bf16 store."""
    bits = v.astype(np.float32).view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16 << 16
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("m,k,n", [(6100, 128, 5904), (6100, 2048, 5904), (6100, 4104, 5904)])
def test_colwise_none_many_tiles_bit_exact(device, m, k, n):
    """bf16 outputs of a launch with more tiles than compute units (eight-wave,
    four-wave and 16x16-MFMA tiles).  Inputs in {-1, 0, 1}: every sum is an
    integer held exactly in float32, so the output is its bf16 rounding."""
    say(f"case colwise many tiles m={m} k={k} n={n}")
    x = inputs.integers(11, 0, (m, k), -1, 1)
    w = inputs.integers(11, 1, (n, k), -1, 1)
    ref = x.f64() @ w.f64().T
    out = torch.empty(m, n, dtype=torch.bfloat16, device=device)
    tp.tp_colwise("none", "bf16", m, k, n, to_dev(x, device), to_dev(w, device), out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), _bf16_rne(ref))


@pytest.mark.parametrize("m,k,n,plan", [
    (2048, 4104, 12288, (256, 32, 256, 2)),   # a round of whole tiles, then 128 tiles as split-k pairs, k tail
    (2000, 4096, 12288, (256, 32, 256, 2)),   # ragged m, whole k-steps
    (520, 4104, 768, (256, 0, 256, 2)),       # split-k pairs only
])
def test_colwise_split_k_bit_exact(device, m, k, n, plan):
    """Tiles summed by two workgroups (half of k each, the partial handed over
    through the split workspace): bf16 outputs of integer inputs in {-1, 0, 1}
    equal the rounding of the exact sums, twice in a row on one stream (the
    flags' epoch advances) and once on a second stream (its own workspace)."""
    say(f"case colwise split-k m={m} k={k} n={n} plan={plan}")
    assert tp.tp_gemm_plan(m, n, k, "colwise") == plan
    x = inputs.integers(12, 0, (m, k), -1, 1)
    w = inputs.integers(12, 1, (n, k), -1, 1)
    ref = _bf16_rne(x.f64() @ w.f64().T)
    dx, dw = to_dev(x, device), to_dev(w, device)
    outs = []
    side = torch.cuda.Stream(device)
    for stream in (None, None, side):
        out = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=device)
        if stream is None:
            tp.tp_colwise("none", "bf16", m, k, n, dx, dw, out)
        else:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                tp.tp_colwise("none", "bf16", m, k, n, dx, dw, out, stream=side)
            torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        outs.append(host(out))
    for o in outs:
        assert np.array_equal(o, ref)


@pytest.mark.parametrize("m,k,n", [(300, 40, 264), (64, 48, 512)])
def test_colwise_none_integer_bit_exact(device, m, k, n):
    """Plain colwise projection, integers small enough (|sum| <= 2*2*48 < 256)
    that the bf16 output is exact."""
    say(f"case colwise int m={m} k={k} n={n}")
    x = inputs.integers(8, 0, (m, k), -2, 2)
    w = inputs.integers(8, 1, (n, k), -2, 2)
    out = torch.empty(m, n, dtype=torch.bfloat16, device=device)
    tp.tp_colwise("none", "bf16", m, k, n, to_dev(x, device), to_dev(w, device), out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), x.f64() @ w.f64().T)


# ---------------------------------------------------------------- projection variants


@pytest.mark.parametrize("m,k,n", [(300, 40, 264), (6100, 128, 5904), (777, 2056, 520)])
def test_colwise_bias_integer_bit_exact(device, m, k, n):
    """A column-parallel bias added in the epilogue: integer inputs and bias keep
    every sum within +-256, so the bf16 output is exact (eight- and four-wave
    tiles, several rounds of tiles, ragged m and n)."""
    say(f"case colwise bias int m={m} k={k} n={n}")
    x = inputs.integers(12, 0, (m, k), -1, 1)
    w = inputs.integers(12, 1, (n, k), -1, 1)
    b = inputs.integers(12, 2, (n,), -4, 4, "f32").data
    ref = x.f64() @ w.f64().T + b.astype(np.float64)
    assert np.max(np.abs(ref)) <= 256
    out = torch.empty(m, n, dtype=torch.bfloat16, device=device)
    tp.tp_colwise("none", "bf16", m, k, n, to_dev(x, device), to_dev(w, device), out,
                  bias=torch.from_numpy(b).to(device))
    torch.cuda.synchronize()
    assert np.array_equal(host(out), ref)


@pytest.mark.parametrize("act,dt,m,k,f", [("gelu", "bf16", 333, 256, 264), ("swiglu", "bf16", 333, 256, 264),
                                          ("swiglu", "bf16", 5000, 2056, 1792), ("gelu", "f32", 37, 64, 72),
                                          ("swiglu", "f32", 37, 64, 72), ("swiglu", "bf16", 1000, 4104, 1792),
                                          ("gelu", "bf16", 1000, 4104, 1000)])
def test_colwise_bias_activations(device, act, dt, m, k, f):
    """GeLU(X A_i + b_i) and SiLU(X W1_i + b1_i) * (X W3_i + b3_i) against the oracle."""
    say(f"case colwise bias {act} {dt} m={m} k={k} f={f}")
    x = inputs.normal(13, 0, (m, k), 1.0, dt)
    rows = 2 * f if act == "swiglu" else f
    w = inputs.normal(13, 1, (rows, k), 0.05, dt)
    b = inputs.normal(13, 2, (rows,), 0.5, "f32").data
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = torch.empty(m, f, dtype=tdt, device=device)
    tp.tp_colwise(act, dt, m, k, f, to_dev(x, device), to_dev(w, device), out, bias=torch.from_numpy(b).to(device))
    torch.cuda.synchronize()
    X, W, B = x.f64(), w.f64(), b.astype(np.float64)
    if act == "gelu":
        ref = oracle.colwise_act(X, W.T, "gelu", bias=B)
    else:
        ref = oracle.colwise_act(X, None, "swiglu", (W[:f].T, W[f:].T), bias_gate_up=(B[:f], B[f:]))
    if dt == "f32":
        assert np.max(np.abs(host(out) - ref)) <= F32_ATOL
    else:
        assert rel_err(host(out), ref) <= BF16_TOL


def test_qkv_rope_bias(device):
    """Q/K/V biases added before RoPE (Q, K) and before the transposed store (V),
    against the oracle's projections; sequence 100 leaves a ragged last key tile."""
    batch, seq, h, hq, hkv, d = 2, 100, 256, 4, 2, 128
    say(f"case qkv_rope bias batch={batch} seq={seq}")
    m, n = batch * seq, (hq + 2 * hkv) * d
    x = inputs.normal(14, 0, (m, h), 1.0, "bf16")
    w = inputs.normal(14, 1, (n, h), 0.05, "bf16")
    b = inputs.normal(14, 2, (n,), 0.5, "f32").data
    seq_pad = (seq + 63) // 64 * 64
    q = torch.empty(m, hq * d, dtype=torch.bfloat16, device=device)
    k = torch.empty(m, hkv * d, dtype=torch.bfloat16, device=device)
    vt = torch.empty(batch, hkv, d, seq_pad, dtype=torch.bfloat16, device=device)
    tp.tp_qkv_rope(batch, seq, h, hq, hkv, d, 500000.0, to_dev(x, device), to_dev(w, device), q, k, vt,
                   bias=torch.from_numpy(b).to(device))
    torch.cuda.synchronize()
    X, W, B = x.f64(), w.f64(), b.astype(np.float64)
    pos = np.tile(np.arange(seq), batch)
    for j in range(hq):
        ref = oracle.rope(oracle.linear(X, W[j * d:(j + 1) * d].T, B[j * d:(j + 1) * d]), pos, 500000.0)
        assert rel_err(host(q[:, j * d:(j + 1) * d]), ref) <= BF16_TOL
    for g in range(hkv):
        r0 = (hq + g) * d
        ref = oracle.rope(oracle.linear(X, W[r0:r0 + d].T, B[r0:r0 + d]), pos, 500000.0)
        assert rel_err(host(k[:, g * d:(g + 1) * d]), ref) <= BF16_TOL
        r0 = (hq + hkv + g) * d
        refv = oracle.linear(X, W[r0:r0 + d].T, B[r0:r0 + d])
        got = vt[:, g, :, :seq].permute(0, 2, 1).reshape(m, d)
        assert rel_err(host(got), refv) <= BF16_TOL
        assert not vt[:, g, :, seq:].any()


@pytest.mark.parametrize("batch,seq,h,hq,hkv,bm", [
    (2, 100, 4104, 4, 2, 128),     # seq a multiple of 4, not 8: V in 4-row stores; k tail of 8
    (3, 203, 4104, 8, 2, 128),     # odd seq: 4-row groups straddle sequences; ragged m
    (2, 1000, 4096, 8, 1, 128),    # V staged through LDS in one pass; ragged last tile
    (4, 2048, 4096, 8, 1, 192),    # the 70B t=8 rank's layout (192-row tiles) at k = 4096
    (2, 2048, 4096, 24, 4, 256),   # 256-row tiles: V staged in two passes
])
def test_qkv_rope_16x16(device, batch, seq, h, hq, hkv, bm):
    """Q/K/V + RoPE on the 16x16-MFMA kernel (depth >= 4096) at every tile
    height, with biases, against the oracle on sampled rows (every row of a
    tile's first and last 16-row block, plus random ones)."""
    d = 128
    say(f"case qkv_rope 16x16 batch={batch} seq={seq} h={h} hq={hq} hkv={hkv}")
    m, n = batch * seq, (hq + 2 * hkv) * d
    assert tp.tp_gemm_plan(m, n, h, "qkv")[0] == bm
    x = inputs.normal(16, 0, (m, h), 1.0, "bf16")
    w = inputs.normal(16, 1, (n, h), 0.02, "bf16")
    b = inputs.normal(16, 2, (n,), 0.5, "f32").data
    seq_pad = (seq + 63) // 64 * 64
    q = torch.empty(m, hq * d, dtype=torch.bfloat16, device=device)
    k = torch.empty(m, hkv * d, dtype=torch.bfloat16, device=device)
    vt = torch.full((batch, hkv, d, seq_pad), float("nan"), dtype=torch.bfloat16, device=device)
    tp.tp_qkv_rope(batch, seq, h, hq, hkv, d, 500000.0, to_dev(x, device), to_dev(w, device), q, k, vt,
                   bias=torch.from_numpy(b).to(device))
    torch.cuda.synchronize()
    rng = np.random.default_rng(16)
    rows = np.unique(np.concatenate([
        np.arange(m)[(np.arange(m) % bm < 16) | (np.arange(m) % bm >= bm - 16)][:512],
        np.arange(max(0, m - 40), m), rng.integers(0, m, 256)]))
    X, W, B = x.f64()[rows], w.f64(), b.astype(np.float64)
    pos = rows % seq
    qh, kh = host(q)[rows], host(k)[rows]
    vtok = host(vt[:, :, :, :seq].permute(0, 3, 1, 2).reshape(m, hkv * d))[rows]
    for j in range(hq):
        ref = oracle.rope(oracle.linear(X, W[j * d:(j + 1) * d].T, B[j * d:(j + 1) * d]), pos, 500000.0)
        assert rel_err(qh[:, j * d:(j + 1) * d], ref) <= BF16_TOL, ("q", j)
    for g in range(hkv):
        r0 = (hq + g) * d
        ref = oracle.rope(oracle.linear(X, W[r0:r0 + d].T, B[r0:r0 + d]), pos, 500000.0)
        assert rel_err(kh[:, g * d:(g + 1) * d], ref) <= BF16_TOL, ("k", g)
        r0 = (hq + hkv + g) * d
        refv = oracle.linear(X, W[r0:r0 + d].T, B[r0:r0 + d])
        assert rel_err(vtok[:, g * d:(g + 1) * d], refv) <= BF16_TOL, ("v", g)
    assert not torch.isnan(vt[:, :, :, :seq]).any()      # every V element written
    assert not vt[:, :, :, seq:].any()                   # the padding zeroed


@pytest.mark.parametrize("dt,m,k,n,t", [("bf16", 300, 4096, 264, 4), ("bf16", 6100, 1024, 5904, 2),
                                        ("f32", 37, 64, 40, 2)])
def test_rowwise_split_input_bit_exact(device, dt, m, k, n, t):
    """Each rank reads its own columns of the replicated input in place; the
    partials are bit-exact on integer inputs and sum to X W."""
    say(f"case rowwise split input {dt} m={m} k={k} n={n} t={t}")
    x = inputs.integers(15, 0, (m, k), -2, 2, dt)
    w_lin = inputs.integers(15, 1, (n, k), -2, 2, dt)          # nn.Linear layout [out, in]
    X, WL = x.f64(), w_lin.f64()
    parts = oracle.rowwise_split_input_partials(X, WL.T, t)
    dx = to_dev(x, device)
    dwl = to_dev(w_lin, device)
    ks = k // t
    total = np.zeros((m, n))
    for r in range(t):
        wr = dwl[:, r * ks:(r + 1) * ks].contiguous()
        out = torch.empty(m, n, dtype=torch.float32, device=device)
        tp.tp_rowwise_split_input(dt, m, k, n, t, r, dx, wr, out)
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()
        assert np.array_equal(got, parts[r])
        total += got
    assert np.array_equal(total, X @ WL.T)


def test_mlp_with_biases(device):
    """A biased GeLU MLP sharded over 4 ranks: column biases in the colwise
    epilogue, the row bias added once after the sum (bit-exact to a float32
    sum of the GPU partials, then the bias), against the unsharded oracle."""
    m, h, f, t = 512, 512, 2048, 4
    say(f"case biased mlp m={m} h={h} f={f} t={t}")
    x = inputs.normal(16, 0, (m, h), 1.0, "bf16")
    a = inputs.normal(16, 1, (h, f), 0.02, "bf16")     # math convention [in, out]
    b = inputs.normal(16, 2, (f, h), 0.02, "bf16")
    ba = inputs.normal(16, 3, (f,), 0.5, "f32").data
    bb = inputs.normal(16, 4, (h,), 0.5, "f32").data
    A, Bm = a.torch(), b.torch()
    dx = to_dev(x, device)
    fs = f // t
    act = torch.empty(m, fs, dtype=torch.bfloat16, device=device)
    parts = torch.empty(t, m, h, dtype=torch.float32, device=device)
    for r in range(t):
        w_in = A[:, r * fs:(r + 1) * fs].T.contiguous().to(device)
        w_out = Bm[r * fs:(r + 1) * fs, :].T.contiguous().to(device)
        tp.tp_colwise("gelu", "bf16", m, h, fs, dx, w_in, act, bias=torch.from_numpy(ba[r * fs:(r + 1) * fs].copy()).to(device))
        tp.tp_rowwise("bf16", m, fs, h, act, w_out, parts[r])
    z = torch.empty(m, h, dtype=torch.float32, device=device)
    y = torch.empty(m, h, dtype=torch.bfloat16, device=device)
    tp.tp_shard_sum_rmsnorm(t, m, h, list(parts), None, "f32", z, None, 1e-5, y, bias=torch.from_numpy(bb).to(device))
    torch.cuda.synchronize()
    p_host = [p.cpu().numpy() for p in parts]
    acc = p_host[0].copy()
    for p in p_host[1:]:
        acc = (acc + p).astype(np.float32)
    acc = (acc + bb).astype(np.float32)
    assert np.array_equal(z.cpu().numpy(), acc)
    ref = oracle.mlp_gelu_bias(x.f64(), a.f64(), ba.astype(np.float64), b.f64(), bb.astype(np.float64))
    assert rel_err(host(z), ref) <= BF16_TOL
    refn = oracle.rmsnorm(acc.astype(np.float64), None, 1e-5)
    assert np.all(np.abs(host(y) - refn) <= 2.0 ** -8 * np.abs(refn) + 1e-6)


@pytest.mark.parametrize("t,causal", [(2, False), (4, True)])
def test_packed_single_stream(device, t, causal):
    """Packed single-stream block: one [1, 1, 1, 3, 3] in-projection buffer per
    rank feeding the Q/K/V + RoPE and SwiGLU GEMMs in place, attention, and
    the [1, 3] out-projection as two partials per rank; each rank's share and
    the sum over ranks against the oracle."""
    h, heads, d, batch, seq = 512, 4, 128, 2, 96
    say(f"case packed single stream t={t} causal={causal}")
    m = batch * seq
    x = inputs.normal(17, 0, (m, h), 1.0, "bf16")
    w_in = inputs.normal(17, 1, (9 * h, h), 0.02, "bf16")      # nn.Linear [out, in]
    w_out = inputs.normal(17, 2, (h, 4 * h), 0.02, "bf16")
    blk = shard.SingleStreamShards(to_dev(x, device), to_dev(w_in, device), to_dev(w_out, device), heads, d,
                                   batch, seq, t, 500000.0, causal)
    z = blk.forward()
    torch.cuda.synchronize()
    X, WI, WO = x.f64(), w_in.f64().T, w_out.f64().T              # math convention
    for r in range(t):
        ref_r = oracle.single_stream_partial(X, WI, WO, heads, d, batch, seq, 500000.0, t, r, causal)
        got_r = host(blk.partials[2 * r]) + host(blk.partials[2 * r + 1])
        assert rel_err(got_r, ref_r) <= BF16_TOL
    ref = oracle.single_stream_partial(X, WI, WO, heads, d, batch, seq, 500000.0, 1, 0, causal)
    assert rel_err(host(z), ref) <= BF16_TOL


# ---------------------------------------------------------------- backward


def test_transpose_exact(device):
    say("case transpose")
    for rows, cols in [(1, 8), (65, 130), (1000, 264), (4096, 1024)]:
        a = inputs.normal(71, rows, (rows, cols), 1.0, "bf16")
        src = to_dev(a, device)
        dst = torch.empty(cols, rows, dtype=torch.bfloat16, device=device)
        tp.tp_transpose(rows, cols, src, dst)
        torch.cuda.synchronize()
        assert torch.equal(dst, src.T.contiguous())


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_mlp_act_backward(device, act):
    """dPre and the recomputed activation against the oracle's derivatives."""
    m, n = 300, 264
    say(f"case act backward {act}")
    pw = 2 * n if act == "swiglu" else n
    pre = inputs.normal(72, 0, (m, pw), 2.0, "bf16")
    dy = inputs.normal(72, 1, (m, n), 1.0, "bf16")
    dpre = torch.empty(m, pw, dtype=torch.bfloat16, device=device)
    y = torch.empty(m, n, dtype=torch.bfloat16, device=device)
    tp.tp_mlp_act_backward(act, m, n, to_dev(pre, device), to_dev(dy, device), dpre, y)
    torch.cuda.synchronize()
    P, D = pre.f64(), dy.f64()
    if act == "gelu":
        ref_d, ref_y = D * oracle.gelu_grad(P), oracle.gelu(P)
    else:
        g, u = P[:, :n], P[:, n:]
        ref_d = np.concatenate([D * u * oracle.silu_grad(g), D * oracle.silu(g)], axis=1)
        ref_y = oracle.silu(g) * u
    # one bf16 rounding of each output plus float32 arithmetic
    assert np.all(np.abs(host(dpre) - ref_d) <= 2.0 ** -8 * np.abs(ref_d) + 1e-5 * np.max(np.abs(ref_d)))
    assert np.all(np.abs(host(y) - ref_y) <= 2.0 ** -8 * np.abs(ref_y) + 1e-5 * np.max(np.abs(ref_y)))


@pytest.mark.parametrize("act,m,h,f,t", [("gelu", 256, 256, 1024, 2), ("swiglu", 264, 512, 1024, 4),
                                         ("swiglu", 2048, 1024, 4096, 4)])
def test_mlp_backward(device, act, m, h, f, t):
    """Each rank's dX partial and weight gradients against the oracle's, and
    the summed dX (f's backward) against the unsharded layer's."""
    say(f"case mlp backward {act} m={m} h={h} f={f} t={t}")
    case = inputs.MLPCase("bwd", m, h, f, t, act, "bf16", seed=73)
    w = inputs.gen_mlp(case)
    dz = inputs.normal(73, 9, (m, h), 1.0, "bf16")
    dw = {k: to_dev(v, device) for k, v in w.items()}
    mlp = shard.MLPShards(dw["X"], dw, t, act)
    dx = mlp.backward(to_dev(dz, device))
    torch.cuda.synchronize()
    W = {k: v.f64() for k, v in w.items()}
    DZ = dz.f64()
    fs = f // t
    if act == "gelu":
        parts = oracle.mlp_gelu_backward_partials(W["X"], W["A"], W["B"], DZ, t)
        full = oracle.mlp_gelu_backward(W["X"], W["A"], W["B"], DZ)
        for r in range(t):
            assert rel_err(host(mlp.dx_partials[r]), parts[r]["dx"]) <= BF16_TOL
            assert rel_err(host(mlp.dw_in[r]), parts[r]["da"].T) <= BF16_TOL       # [f_shard, h]
            assert rel_err(host(mlp.dw_out[r]), parts[r]["db"].T) <= BF16_TOL      # [h, f_shard]
    else:
        parts = oracle.mlp_swiglu_backward_partials(W["X"], W["W1"], W["W3"], W["W2"], DZ, t)
        full = oracle.mlp_swiglu_backward(W["X"], W["W1"], W["W3"], W["W2"], DZ)
        for r in range(t):
            assert rel_err(host(mlp.dx_partials[r]), parts[r]["dx"]) <= BF16_TOL
            g = host(mlp.dw_in[r])                                                 # [2 f_shard, h]
            assert rel_err(g[:fs], parts[r]["dw1"].T) <= BF16_TOL
            assert rel_err(g[fs:], parts[r]["dw3"].T) <= BF16_TOL
            assert rel_err(host(mlp.dw_out[r]), parts[r]["dw2"].T) <= BF16_TOL
    assert rel_err(host(dx), full["dx"]) <= BF16_TOL


def _attn_core_inputs(device, batch, seq, hq, hkv, seed, d=128):
    """Seeded bf16 q, k, v, dO (token-major) and the per-head transposed V the
    forward reads (zero past seq)."""
    m = batch * seq
    q = inputs.normal(seed, 1, (m, hq * d), 1.0, "bf16").torch()
    k = inputs.normal(seed, 2, (m, hkv * d), 1.0, "bf16").torch()
    v = inputs.normal(seed, 3, (m, hkv * d), 1.0, "bf16").torch()
    do = inputs.normal(seed, 4, (m, hq * d), 1.0, "bf16").torch()
    seq_pad = (seq + 63) // 64 * 64
    vt = torch.zeros(batch, hkv, d, seq_pad, dtype=torch.bfloat16)
    vt[..., :seq] = v.view(batch, seq, hkv, d).permute(0, 2, 3, 1)
    return {"q": q, "k": k, "v": v, "do": do, "vt": vt, "seq_pad": seq_pad}


def _attn_core_backward(device, batch, seq, hq, hkv, causal, rope_base, t_in):
    """Forward with LSE, then the core backward, through the C ABI."""
    d = 128
    m = batch * seq
    dev = {k: v.to(device) for k, v in t_in.items() if torch.is_tensor(v)}
    o = torch.empty(m, hq * d, dtype=torch.bfloat16, device=device)
    lse = torch.full((batch, hq, t_in["seq_pad"]), float("nan"), dtype=torch.float32, device=device)
    tp.tp_flash_attn_lse(batch, seq, hq, hkv, d, causal, dev["q"], dev["k"], dev["vt"], o, lse)
    n = (hq + 2 * hkv) * d
    ws_bytes = tp.tp_flash_attn_backward_workspace_bytes(batch, seq, hq, hkv, d)
    # NaN-filled workspace: any read of a padding entry that is not masked shows up
    ws = torch.full((ws_bytes // 4,), float("nan"), dtype=torch.float32, device=device)
    dqkv = torch.full((m, n + 8), float("nan"), dtype=torch.bfloat16, device=device)
    tp.tp_flash_attn_backward(batch, seq, hq, hkv, d, rope_base, causal, dev["q"], dev["k"], dev["vt"], o, lse,
                              dev["do"], ws, ws_bytes, dqkv, n + 8)
    torch.cuda.synchronize()
    return o, lse, dqkv


@pytest.mark.parametrize("batch,seq,hq,hkv,causal", [(2, 130, 4, 2, True), (1, 300, 4, 1, True),
                                                     (2, 64, 2, 2, True), (1, 200, 4, 2, False),
                                                     (1, 1, 2, 1, True)])
def test_flash_attn_lse(device, batch, seq, hq, hkv, causal):
    """The forward's log-sum-exp (log2 units) against the oracle's natural-log
    normaliser times log2(e); the output is the forward's own."""
    say(f"case flash lse b={batch} s={seq} hq={hq} hkv={hkv} causal={causal}")
    d = 128
    t_in = _attn_core_inputs(device, batch, seq, hq, hkv, 81)
    m = batch * seq
    o = torch.empty(m, hq * d, dtype=torch.bfloat16, device=device)
    lse = torch.full((batch, hq, t_in["seq_pad"]), -7.0, dtype=torch.float32, device=device)
    tp.tp_flash_attn_lse(batch, seq, hq, hkv, d, causal, t_in["q"].to(device), t_in["k"].to(device),
                         t_in["vt"].to(device), o, lse)
    o2 = torch.empty_like(o)
    tp.tp_flash_attn(batch, seq, hq, hkv, d, causal, t_in["q"].to(device), t_in["k"].to(device),
                     t_in["vt"].to(device), o2)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    got = lse.cpu().double().numpy()
    assert np.all(got[:, :, seq:] == -7.0)  # padding untouched
    qh, kh = t_in["q"].double().numpy(), t_in["k"].double().numpy()
    worst = 0.0
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        for j in range(hq):
            g = j // (hq // hkv)
            ref = oracle.attention_lse(qh[rows, j * d:(j + 1) * d], kh[rows, g * d:(g + 1) * d], causal)
            worst = max(worst, float(np.max(np.abs(got[b, j, :seq] - ref / math.log(2.0)))))
    say(f"  max|lse gpu - oracle| = {worst:.3e} (log2 units)")
    # the scores are float32 sums of bf16 products; |s| / sqrt(d) stays below ~6 here
    assert worst <= 1e-3


@pytest.mark.parametrize("batch,seq,hq,hkv,causal,pieces", [
    (1, 700, 2, 1, True, 3), (1, 1000, 1, 1, True, 4), (1, 900, 2, 2, False, 7),
    (2, 333, 4, 2, True, 2), (1, 2048, 1, 1, True, 8)])
def test_flash_attn_split_pieces(device, batch, seq, hq, hkv, causal, pieces):
    """Few heads, so each pair of query blocks is cut into several pieces and
    blocks are completed from other workgroups' float32 partials: output and
    log-sum-exp against the oracle, bitwise equal on a second run.  Ragged
    sequences, an odd number of query blocks (the middle block cut on its
    own), GQA and attention over all keys."""
    say(f"case flash split b={batch} s={seq} hq={hq} hkv={hkv} causal={causal}")
    assert tp.tp_flash_attn_plan(batch, seq, hq, causal) == pieces
    d = 128
    t_in = _attn_core_inputs(device, batch, seq, hq, hkv, 83)
    m = batch * seq
    dev = {k: v.to(device) for k, v in t_in.items() if torch.is_tensor(v)}
    outs = []
    for _ in range(2):
        o = torch.full((m, hq * d), float("nan"), dtype=torch.bfloat16, device=device)
        lse = torch.full((batch, hq, t_in["seq_pad"]), -7.0, dtype=torch.float32, device=device)
        tp.tp_flash_attn_lse(batch, seq, hq, hkv, d, causal, dev["q"], dev["k"], dev["vt"], o, lse)
        torch.cuda.synchronize()
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    got, got_lse = host(outs[0][0]), outs[0][1].cpu().double().numpy()
    assert np.all(got_lse[:, :, seq:] == -7.0)
    qh, kh, vh = (t_in[n].double().numpy() for n in ("q", "k", "v"))
    worst = worst_lse = 0.0
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        for j in range(hq):
            g = j // (hq // hkv)
            qq, kk, vv = qh[rows, j * d:(j + 1) * d], kh[rows, g * d:(g + 1) * d], vh[rows, g * d:(g + 1) * d]
            ref = oracle.causal_attention(qq, kk, vv) if causal else oracle.full_attention(qq, kk, vv)
            worst = max(worst, rel_err(got[rows, j * d:(j + 1) * d], ref))
            ref_lse = oracle.attention_lse(qq, kk, causal) / math.log(2.0)
            worst_lse = max(worst_lse, float(np.max(np.abs(got_lse[b, j, :seq] - ref_lse))))
    say(f"  max rel err {worst:.3e}, max|lse gpu - oracle| {worst_lse:.3e}")
    assert worst <= BF16_TOL and worst_lse <= 1e-3


@pytest.mark.parametrize("batch,seq,hq,hkv,causal,rope", [
    (2, 130, 4, 2, True, 0.0), (1, 300, 4, 1, True, 500000.0), (2, 64, 2, 2, True, 10000.0),
    (1, 200, 4, 2, False, 0.0), (1, 1, 2, 1, True, 500000.0), (1, 257, 8, 1, True, 500000.0)])
def test_flash_attn_backward_core(device, batch, seq, hq, hkv, causal, rope):
    """dQ, dK, dV of the attention core (GQA groups summed, RoPE rotated back
    when rope > 0) against the oracle's, from the same bf16 q, k, v, dO;
    ragged sequences, a single token, several query tiles per key block and a
    head group split over workgroups; bitwise equal on a second run."""
    say(f"case flash backward b={batch} s={seq} hq={hq} hkv={hkv} causal={causal} rope={rope}")
    d = 128
    t_in = _attn_core_inputs(device, batch, seq, hq, hkv, 82)
    o, lse, dqkv = _attn_core_backward(device, batch, seq, hq, hkv, causal, rope, t_in)
    _, _, dqkv2 = _attn_core_backward(device, batch, seq, hq, hkv, causal, rope, t_in)
    n = (hq + 2 * hkv) * d
    assert torch.equal(dqkv[:, :n].view(torch.int16), dqkv2[:, :n].view(torch.int16))
    got = host(dqkv)
    assert np.all(np.isnan(got[:, n:]))  # the row padding is not written
    got = got[:, :n]
    qh, kh, vh, doh = (t_in[x].double().numpy() for x in ("q", "k", "v", "do"))
    ref = np.zeros_like(got)
    pos = np.arange(seq)
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        for j in range(hq):
            g = j // (hq // hkv)
            dq, dk, dv = oracle.causal_attention_backward(
                qh[rows, j * d:(j + 1) * d], kh[rows, g * d:(g + 1) * d], vh[rows, g * d:(g + 1) * d],
                doh[rows, j * d:(j + 1) * d], causal)
            ref[rows, j * d:(j + 1) * d] = dq
            ref[rows, (hq + g) * d:(hq + g + 1) * d] += dk
            ref[rows, (hq + hkv + g) * d:(hq + hkv + g + 1) * d] += dv
        if rope > 0:
            for c in range(hq + hkv):
                ref[rows, c * d:(c + 1) * d] = oracle.rope_backward(ref[rows, c * d:(c + 1) * d], pos, rope)
    for name, cols in (("dq", slice(0, hq * d)), ("dk", slice(hq * d, (hq + hkv) * d)),
                       ("dv", slice((hq + hkv) * d, n))):
        say(f"  {name}")
        if np.max(np.abs(ref[:, cols])) == 0.0:
            # one token: the softmax is constant, dq = dk = 0 exactly; the GPU
            # keeps only the rounding of dP - D (float32 sums in two orders)
            assert np.max(np.abs(got[:, cols])) <= 1e-5 * np.max(np.abs(ref)), name
        else:
            assert rel_err(got[:, cols], ref[:, cols]) <= BF16_TOL, name


@pytest.mark.parametrize("batch,seq,h,heads,kv,t", [(2, 72, 256, 8, 2, 2), (1, 136, 384, 8, 2, 4),
                                                    (2, 64, 256, 4, 4, 1)])
def test_attention_backward(device, batch, seq, h, heads, kv, t):
    """Each rank's dX partial and weight gradients (W_qkv rows, W_o columns)
    against the oracle's; the summed dX (f's backward) against the unsharded
    layer's; t = 4 > kv = 2 replicates a KV head on two ranks."""
    say(f"case attn backward b={batch} s={seq} h={h} heads={heads} kv={kv} t={t}")
    case = inputs.AttnCase("bwd", batch, seq, h, heads, kv, 128, t, 500000.0, seed=75)
    w = inputs.gen_attn(case)
    m = batch * seq
    dz = inputs.normal(75, 9, (m, h), 1.0, "bf16")
    dw = {k: to_dev(v, device) for k, v in w.items()}
    at = shard.AttnShards(dw["X"], dw, case)
    dx = at.backward(to_dev(dz, device))
    torch.cuda.synchronize()
    W = {k: v.f64() for k, v in w.items()}
    DZ = dz.f64()
    parts = oracle.attn_backward_partials(W["X"], W, DZ, case, t)
    for r in range(t):
        say(f"  rank {r}")
        p = parts[r]
        assert rel_err(host(at.dx_partials[r]), p["dx"]) <= BF16_TOL
        ref_qkv = np.concatenate([p["dwq"].T, p["dwk"].T, p["dwv"].T], axis=0)
        assert rel_err(host(at.dw_qkv[r]), ref_qkv) <= BF16_TOL
        assert rel_err(host(at.dw_o[r]), p["dwo"].T) <= BF16_TOL
    full = oracle.attn_backward(W["X"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], DZ, heads, kv, 128, batch, seq,
                                case.rope_base)
    assert rel_err(host(dx), full["dx"]) <= BF16_TOL


def test_saved_activation_backward_matches_recompute(device):
    """The block backward after a forward that keeps every rank's activations
    (the MLP's pre-activation from the GEMM epilogue, attention's Q, K, V^T, O
    and log-sum-exp) is bitwise the backward that recomputes them; the saved
    pre-activation is bitwise the recomputed one."""
    case = inputs.BlockCase("saved", 2, 72, 256, 4, 2, 128, 512, 2, 500000.0, seed=94, gain_std=0.1)
    say("case saved-activation block backward t=2")
    w = inputs.gen_block(case)
    dz = to_dev(inputs.normal(94, 20, (case.tokens, case.hidden), 1.0, "bf16"), device)
    dw = {k: to_dev(v, device) for k, v in w.items()}
    blk = shard.BlockShards(dw["X"], dw, case)
    blk.forward()
    z_plain = blk.mlp.out.clone()
    blk.backward(dz)
    ref = {"dx": blk.d_x.clone(), "dh1": blk.dh1.clone(), "dgm": blk.dg_mlp.clone(), "dga": blk.dg_attn.clone(),
           "dwi": [t.clone() for t in blk.mlp.dw_in], "dwq": [t.clone() for t in blk.attn.dw_qkv],
           "dwo": [t.clone() for t in blk.attn.dw_o]}
    blk.forward(save=True)
    assert torch.equal(blk.mlp.out, z_plain)  # the saving forward computes the same block
    recomputed = torch.empty_like(blk.mlp.pre[1])
    tp.tp_colwise("none", "bf16", case.tokens, case.hidden, 2 * blk.mlp.f_shard, blk.hn, blk.mlp.w_in[1], recomputed)
    blk.backward(dz)
    torch.cuda.synchronize()
    assert torch.equal(blk.mlp.pre[1].view(torch.int16), recomputed.view(torch.int16))
    for name, got, want in (("dx", blk.d_x, ref["dx"]), ("dh1", blk.dh1, ref["dh1"]), ("dg_mlp", blk.dg_mlp, ref["dgm"]),
                            ("dg_attn", blk.dg_attn, ref["dga"])):
        assert torch.equal(got, want), name
    for r in range(case.t):
        assert torch.equal(blk.mlp.dw_in[r], ref["dwi"][r])
        assert torch.equal(blk.attn.dw_qkv[r], ref["dwq"][r])
        assert torch.equal(blk.attn.dw_o[r], ref["dwo"][r])


@pytest.mark.parametrize("act,m,h,f", [("gelu", 1000, 256, 1024), ("swiglu", 520, 384, 768),
                                      ("swiglu", 520, 4104, 768), ("gelu", 600, 4104, 1024)])
def test_colwise_save_and_mlp_backward_from_it(device, act, m, h, f):
    """tp_colwise_save's output equals tp_colwise's and its pre-activation the
    plain GEMM's, bitwise, with and without a bias (ragged m, two rounds of
    tiles); the MLP backward from the saved pre-activation equals the
    recomputing backward bitwise."""
    say(f"case colwise save {act} m={m} h={h} f={f}")
    t = 2
    case = inputs.MLPCase("save", m, h, f, t, act, "bf16", seed=95)
    w = inputs.gen_mlp(case)
    dw = {k: to_dev(v, device) for k, v in w.items()}
    mlp = shard.MLPShards(dw["X"], dw, t, act)
    fs = mlp.f_shard
    fin = 2 * fs if act == "swiglu" else fs
    for bias in (None, (0.1 * inputs.normal(95, 30, (fin,), 1.0, "f32").torch()).to(device)):
        y0 = torch.empty(m, fs, dtype=torch.bfloat16, device=device)
        y1 = torch.empty_like(y0)
        pre = torch.empty(m, fin, dtype=torch.bfloat16, device=device)
        tp.tp_colwise(act, "bf16", m, h, fs, dw["X"], mlp.w_in[0], y0, bias=bias)
        tp.tp_colwise_save(act, m, h, fs, dw["X"], mlp.w_in[0], y1, pre, bias=bias)
        plain = torch.empty(m, fin, dtype=torch.bfloat16, device=device)
        tp.tp_colwise("none", "bf16", m, h, fin, dw["X"], mlp.w_in[0], plain,
                      bias=None if bias is None else bias)
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
        assert torch.equal(pre.view(torch.int16), plain.view(torch.int16))
    dz = to_dev(inputs.normal(95, 9, (m, h), 1.0, "bf16"), device)
    mlp.forward()
    mlp.backward(dz)
    ref = (mlp.dx.clone(), [a.clone() for a in mlp.dw_in], [a.clone() for a in mlp.dw_out])
    mlp.forward(save=True)
    mlp.backward(dz)
    torch.cuda.synchronize()
    assert torch.equal(mlp.dx, ref[0])
    for r in range(t):
        assert torch.equal(mlp.dw_in[r], ref[1][r]) and torch.equal(mlp.dw_out[r], ref[2][r])


@pytest.mark.parametrize("t", [2, 4])
def test_sequence_parallel_backward(device, t):
    """The sequence-parallel backward (per-rank norm backwards over each rank's
    slice of every sequence) gives dX and dh1 bitwise equal to the replicated
    backward, and the gains' gradients (summed over the ranks' slices) within
    float32 rounding of it."""
    case = inputs.BlockCase("spbwd", 2, 128, 256, 4, 2, 128, 512, t, 500000.0, seed=96, gain_std=0.1)
    say(f"case sequence-parallel backward t={t}")
    w = inputs.gen_block(case)
    dz = to_dev(inputs.normal(96, 20, (case.tokens, case.hidden), 1.0, "bf16"), device)
    dw = {k: to_dev(v, device) for k, v in w.items()}
    blk = shard.BlockShards(dw["X"], dw, case)
    blk.forward()
    blk.backward(dz)
    ref = (blk.d_x.clone(), blk.dh1.clone(), blk.dh1_bf16.clone(), blk.dg_mlp.clone(), blk.dg_attn.clone())
    blk.d_x.fill_(float("nan"))
    blk.dh1.fill_(float("nan"))
    blk.backward_sp(dz)
    torch.cuda.synchronize()
    assert torch.equal(blk.d_x, ref[0]) and torch.equal(blk.dh1, ref[1]) and torch.equal(blk.dh1_bf16, ref[2])
    assert rel_err(host(blk.dg_mlp), host(ref[3])) <= 1e-5
    assert rel_err(host(blk.dg_attn), host(ref[4])) <= 1e-5


def test_flash_attn_backward_one_tile_after_nan_lds(device):
    """Regression: workgroups that walk a single tile also run a fully masked
    second tile on their second LDS stage.  A GEMM over NaN inputs first
    leaves non-finite bits in every CU's LDS; a 64-token backward (one tile
    per workgroup, one head per KV group) must still match the oracle."""
    say("case flash backward after NaN-laden LDS")
    m, k, n = 4096, 2048, 4096
    xn = torch.full((m, k), float("nan"), dtype=torch.bfloat16, device=device)
    wn = torch.full((n, k), float("nan"), dtype=torch.bfloat16, device=device)
    yn = torch.empty(m, n, dtype=torch.bfloat16, device=device)
    batch, seq, hq, hkv, d = 8, 64, 4, 4, 128
    t_in = _attn_core_inputs(device, batch, seq, hq, hkv, 97)
    tp.tp_colwise("none", "bf16", m, k, n, xn, wn, yn)
    _, _, dqkv = _attn_core_backward(device, batch, seq, hq, hkv, True, 0.0, t_in)
    got = host(dqkv)[:, :(hq + 2 * hkv) * d]
    assert np.all(np.isfinite(got))
    qh, kh, vh, doh = (t_in[x].double().numpy() for x in ("q", "k", "v", "do"))
    ref = np.zeros_like(got)
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        for j in range(hq):
            dq, dk, dv = oracle.causal_attention_backward(qh[rows, j * d:(j + 1) * d], kh[rows, j * d:(j + 1) * d],
                                                          vh[rows, j * d:(j + 1) * d], doh[rows, j * d:(j + 1) * d])
            ref[rows, j * d:(j + 1) * d] = dq
            ref[rows, (hq + j) * d:(hq + j + 1) * d] = dk
            ref[rows, (2 * hq + j) * d:(2 * hq + j + 1) * d] = dv
    assert rel_err(got, ref) <= BF16_TOL


def test_flash_attn_backward_full_size_sampled(device):
    """The core backward at the 70B t = 8 rank's shape (4 sequences of 2048,
    8 query heads, 1 KV head, RoPE base 500000) in the configuration the
    benchmark times: for the last sequence, dQ of 64 sampled rows per head and
    dK, dV of 64 sampled rows (summed over the 8 heads) against the oracle."""
    batch, seq, hq, hkv, d, rope = 4, 2048, 8, 1, 128, 500000.0
    say(f"case flash backward full size b={batch} s={seq} hq={hq} hkv={hkv}")
    t_in = _attn_core_inputs(device, batch, seq, hq, hkv, 83)
    _, _, dqkv = _attn_core_backward(device, batch, seq, hq, hkv, True, rope, t_in)
    b = batch - 1
    rows = slice(b * seq, (b + 1) * seq)
    got = host(dqkv[b * seq:(b + 1) * seq])
    sample = np.sort(np.random.default_rng(7).choice(seq, 64, replace=False))
    sample[0], sample[-1] = 0, seq - 1
    qh, kh, vh, doh = (t_in[x][rows].double().numpy() for x in ("q", "k", "v", "do"))
    dk_sum = np.zeros((seq, d))
    dv_sum = np.zeros((seq, d))
    pos = np.arange(seq)
    for j in range(hq):
        dq, dk, dv = oracle.causal_attention_backward(qh[:, j * d:(j + 1) * d], kh, vh, doh[:, j * d:(j + 1) * d])
        dk_sum += dk
        dv_sum += dv
        ref = oracle.rope_backward(dq, pos, rope)[sample]
        assert rel_err(got[sample, j * d:(j + 1) * d], ref) <= BF16_TOL, j
    say("  dk, dv")
    assert rel_err(got[sample, hq * d:(hq + 1) * d], oracle.rope_backward(dk_sum, pos, rope)[sample]) <= BF16_TOL
    assert rel_err(got[sample, (hq + 1) * d:(hq + 2) * d], dv_sum[sample]) <= BF16_TOL


@pytest.mark.parametrize("t,m,h,xdt,res,gain", [(1, 7, 64, "f32", None, False), (4, 1000, 1024, "bf16", "f32", True),
                                               (8, 3001, 8192, "f32", "bf16", True), (16, 130, 264, "bf16", "f32", True),
                                               (3, 2048, 4096, "f32", "inplace", True)])
def test_shard_sum_rmsnorm_backward(device, t, m, h, xdt, res, gain):
    """f's backward sum (ascending), the RMSNorm gradient and the residual
    gradient, and dgain summed over row runs, against the oracle's
    rmsnorm_backward on the same partials and x; float32 arithmetic, so within
    1e-5 of the float64 result (relative to its largest value); in place over
    a float32 residual gradient; ragged row runs and column groups."""
    say(f"case norm backward t={t} m={m} h={h} x={xdt} res={res} gain={gain}")
    parts = [inputs.normal(91, s, (m, h), 1.0, "f32").torch() for s in range(t)]
    x = inputs.normal(91, 40, (m, h), 1.0, xdt).torch()
    g = (1.0 + 0.2 * inputs.normal(91, 41, (h,), 1.0, "f32").torch()) if gain else None
    rgrad = None
    if res is not None:
        rgrad = inputs.normal(91, 42, (m, h), 1.0, "bf16" if res == "bf16" else "f32").torch()
    dparts = [p.to(device) for p in parts]
    dres = None if rgrad is None else rgrad.to(device)
    dx = dres if res == "inplace" else torch.full((m, h), float("nan"), dtype=torch.float32, device=device)
    dxb = torch.empty(m, h, dtype=torch.bfloat16, device=device)
    dgn = torch.full((h,), float("nan"), dtype=torch.float32, device=device)
    wsb = tp.tp_shard_sum_rmsnorm_backward_workspace_bytes(m, h)
    ws = torch.empty(wsb, dtype=torch.uint8, device=device)
    tp.tp_shard_sum_rmsnorm_backward(t, m, h, dparts, x.to(device), xdt, None if g is None else g.to(device), 1e-5,
                                     dres, "bf16" if res == "bf16" else "f32", dx, dxb, dgn, ws, wsb)
    torch.cuda.synchronize()
    dy = sum(p.double().numpy() for p in parts)
    ref_dx, ref_dg = oracle.rmsnorm_backward(x.double().numpy(), None if g is None else g.double().numpy(), dy, 1e-5)
    if rgrad is not None:
        ref_dx = ref_dx + rgrad.double().numpy()
    assert rel_err(host(dx), ref_dx) <= 1e-5
    assert rel_err(host(dgn), ref_dg) <= 1e-5
    assert torch.equal(dxb, dx.to(torch.bfloat16))


@pytest.mark.parametrize("t", [1, 2])
def test_block_backward(device, t):
    """The whole pre-norm block's backward (after its forward): dX, dh1, both
    gains' gradients and every rank's weight gradients against the oracle's
    block_backward from the same bf16 inputs."""
    case = inputs.BlockCase("bwd", 2, 64, 256, 4, 2, 128, 512, t, 500000.0, seed=92, gain_std=0.1)
    say(f"case block backward t={t}")
    w = inputs.gen_block(case)
    dz = inputs.normal(92, 20, (case.tokens, case.hidden), 1.0, "bf16")
    dw = {k: to_dev(v, device) for k, v in w.items()}
    blk = shard.BlockShards(dw["X"], dw, case)
    blk.forward()
    dx = blk.backward(to_dev(dz, device))
    torch.cuda.synchronize()
    W = {k: v.f64() for k, v in w.items()}
    ref = oracle.block_backward(W["X"], W, case, dz.f64(), t)
    for name, got, want in (("dh1", blk.dh1, ref["dh1"]), ("dx", dx, ref["dx"]), ("dg_mlp", blk.dg_mlp, ref["dg_mlp"]),
                            ("dg_attn", blk.dg_attn, ref["dg_attn"])):
        say(f"  {name}")
        assert rel_err(host(got), want) <= BF16_TOL, name
    fs = case.inter // t
    for r in range(t):
        say(f"  rank {r} weights")
        p = ref["mlp"][r]
        gw = host(blk.mlp.dw_in[r])
        assert rel_err(gw[:fs], p["dw1"].T) <= BF16_TOL
        assert rel_err(gw[fs:], p["dw3"].T) <= BF16_TOL
        assert rel_err(host(blk.mlp.dw_out[r]), p["dw2"].T) <= BF16_TOL
        a = ref["attn"][r]
        assert rel_err(host(blk.attn.dw_qkv[r]), np.concatenate([a["dwq"].T, a["dwk"].T, a["dwv"].T])) <= BF16_TOL
        assert rel_err(host(blk.attn.dw_o[r]), a["dwo"].T) <= BF16_TOL


# ---------------------------------------------------------------- vocabulary parallel


@pytest.mark.parametrize("t", [1, 4])
def test_vocab_parallel_embedding(device, t):
    """Vocabulary-sharded lookup (partials summed) and hidden-sharded lookup
    (slices gathered): exactly the table's rows, ids on every shard boundary."""
    v, h, m = 1000, 264, 333
    say(f"case embedding t={t}")
    table = inputs.normal(61, 0, (v, h), 1.0, "bf16")
    n = v // t
    ids = np.concatenate([np.array([0, v - 1] + [r * n for r in range(t)] + [r * n - 1 for r in range(1, t)]),
                          np.random.default_rng(5).integers(0, v, m)]).astype(np.int32)[:m]
    d_ids = torch.from_numpy(ids).to(device)
    dt = to_dev(table, device)
    ref = oracle.embedding_lookup(table.f64(), ids)
    got = shard.embedding_rowwise(d_ids, dt, t)
    torch.cuda.synchronize()
    assert np.array_equal(host(got), ref)
    if h % (8 * t) == 0:
        got = shard.embedding_colwise(d_ids, dt, t)
        torch.cuda.synchronize()
        assert np.array_equal(host(got), ref)


@pytest.mark.parametrize("t,m,h,v", [(1, 300, 512, 1000), (4, 300, 512, 4096), (8, 1000, 256, 32768)])
def test_vocab_parallel_cross_entropy(device, t, m, h, v):
    """Per-token loss and mean from the ranks' statistics, against the oracle
    (float64, same bf16 inputs); the statistics themselves against the
    oracle's on the GPU's own logits; ignored labels give 0."""
    say(f"case vocab-parallel CE t={t} m={m} h={h} v={v}")
    x = inputs.normal(62, 0, (m, h), 1.0, "bf16")
    w = inputs.normal(62, 1, (v, h), 0.05, "bf16")            # nn.Linear [vocab, hidden]
    labels = np.random.default_rng(6).integers(0, v, m).astype(np.int32)
    labels[[3, 17]] = -100
    d_lab = torch.from_numpy(labels).to(device)
    ce = shard.VocabParallelCE(to_dev(x, device), to_dev(w, device), t)
    loss, mean = ce.forward(d_lab)
    torch.cuda.synchronize()
    X, W = x.f64(), w.f64()
    ref = oracle.vocab_parallel_ce(X, W.T, labels, t)
    got = host(loss)
    assert got[3] == 0 and got[17] == 0
    assert np.max(np.abs(got - ref)) <= 1e-3 * max(1.0, np.max(np.abs(ref)))
    ok = labels >= 0
    assert abs(float(mean.item()) - ref[ok].mean()) <= 1e-3 * max(1.0, abs(ref[ok].mean()))
    # the last rank's statistics against the oracle's on the same float32 logits
    n = v // t
    st = oracle.vocab_ce_stats(host(ce.logits), labels, (t - 1) * n)
    gs = host(ce.stats[t - 1])
    assert np.array_equal(gs[:, 0], st[:, 0]) and np.array_equal(gs[:, 2:], st[:, 2:])
    assert np.max(np.abs(gs[:, 1] / st[:, 1] - 1)) <= 1e-5


# ---------------------------------------------------------------- MLP, small


@pytest.mark.parametrize("act,m,h,inter,t", [("gelu", 300, 264, 400, 2), ("swiglu", 333, 256, 544, 2),
                                             ("gelu", 64, 128, 1024, 4), ("swiglu", 512, 512, 2048, 4)])
def test_mlp_small(device, act, m, h, inter, t):
    say(f"case mlp {act} m={m} h={h} inter={inter} t={t}")
    case = inputs.MLPCase("small", m, h, inter, t, act, "bf16", seed=21)
    w = inputs.gen_mlp(case)
    dw = {k: to_dev(v, device) for k, v in w.items()}
    mlp = shard.MLPShards(dw["X"], dw, t, act)
    out = mlp.forward()
    torch.cuda.synchronize()
    W = {k: v.f64() for k, v in w.items()}
    if act == "gelu":
        parts = oracle.mlp_gelu_partials(W["X"], W["A"], W["B"], t)
        full = oracle.mlp_gelu(W["X"], W["A"], W["B"])
    else:
        parts = oracle.mlp_swiglu_partials(W["X"], W["W1"], W["W3"], W["W2"], t)
        full = oracle.mlp_swiglu(W["X"], W["W1"], W["W3"], W["W2"])
    for r in range(t):
        e = rel_err(host(mlp.partials[r]), parts[r])
        assert e <= BF16_TOL, (r, e)
    assert rel_err(host(out), full) <= BF16_TOL


@pytest.mark.parametrize("act,dt,m,h,inter,t", [("gelu", "bf16", 2048, 1024, 4096, 4),
                                                ("swiglu", "bf16", 300, 256, 1024, 8),
                                                ("gelu", "f32", 4, 16, 64, 4)])
def test_mlp_group_bitwise_equals_single_calls(device, act, dt, m, h, inter, t):
    """tp_shard_mlp_group: every partial bitwise equal to the per-rank call."""
    say(f"case mlp group {act} {dt} m={m} h={h} inter={inter} t={t}")
    case = inputs.MLPCase("group", m, h, inter, t, act, dt, seed=23,
                          draw="torch" if dt == "f32" else "counter", w_std=1.0 if dt == "f32" else 0.02)
    w = inputs.gen_mlp(case)
    dw = {k: to_dev(v, device) for k, v in w.items()}
    mlp = shard.MLPShards(dw["X"], dw, t, act, dt)
    single = []
    for r in range(t):
        mlp.rank(r)
        single.append(mlp.partials[r].clone())
    mlp.partials.zero_()
    mlp.all_ranks_grouped()
    torch.cuda.synchronize()
    for r in range(t):
        assert torch.equal(mlp.partials[r], single[r]), r
    if act == "gelu" and dt == "bf16":
        W = {k: v.f64() for k, v in w.items()}
        parts = oracle.mlp_gelu_partials(W["X"], W["A"], W["B"], t)
        for r in range(t):
            assert rel_err(host(mlp.partials[r]), parts[r]) <= BF16_TOL


def test_colwise_activation_slices(device):
    """The colwise output Y_i itself (bf16) against the oracle's activation."""
    say("case colwise slices")
    m, h, f, t = 200, 128, 512, 2
    for act in ("gelu", "swiglu"):
        case = inputs.MLPCase("slices", m, h, f, t, act, "bf16", seed=22)
        w = inputs.gen_mlp(case)
        dw = {k: to_dev(v, device) for k, v in w.items()}
        mlp = shard.MLPShards(dw["X"], dw, t, act)
        W = {k: v.f64() for k, v in w.items()}
        for r in range(t):
            mlp.colwise(r)
            torch.cuda.synchronize()
            if act == "gelu":
                ref = oracle.colwise_act(W["X"], oracle.split_columns(W["A"], t)[r], "gelu")
            else:
                ref = oracle.colwise_act(W["X"], None, "swiglu",
                                         (oracle.split_columns(W["W1"], t)[r], oracle.split_columns(W["W3"], t)[r]))
            assert rel_err(host(mlp.act_ws), ref) <= BF16_TOL


@pytest.mark.parametrize("m,k,plan", [(64, 256, 64), (4096, 1024, 128), (1024, 4096, 256)])
def test_gelu_epilogue_elementwise(device, m, k, plan):
    """The bf16 GEMM's GeLU epilogue (erfc from a Chebyshev fit) element by
    element over [-14, 14], signed zeros and the tails, through an identity
    weight so each output is GeLU of one bf16 input exactly: within a bf16
    rounding step of the oracle's erf form (plus the oracle's own float64
    error in the far negative tail), on small tiles, the eight-wave 32x32 kernel and
    the 16x16 kernel (k = 4096, as split-k pairs)."""
    say(f"case gelu epilogue m={m} k={k}")
    assert tp.tp_gemm_plan(m, k, k, "colwise")[0] == plan
    vals = np.linspace(-14.0, 14.0, m * k).reshape(m, k)
    vals[0, :4] = [0.0, -0.0, 1e-6, -1e-6]
    xb = inputs.from_f32(vals.astype(np.float32), "bf16")
    w = inputs.from_f32(np.eye(k, dtype=np.float32), "bf16")
    y = torch.empty(m, k, dtype=torch.bfloat16, device=device)
    tp.tp_colwise("gelu", "bf16", m, k, k, to_dev(xb, device), to_dev(w, device), y)
    torch.cuda.synchronize()
    got = host(y)
    ref = oracle.gelu(xb.f64())
    err = np.abs(got - ref)
    # the oracle's float64 1 + erf(x / sqrt 2) cancels below x ~ -8 (its
    # absolute error there is ~1e-16 while GeLU falls below it), hence the
    # absolute term; elsewhere a bf16 rounding step of the value
    bound = 2.0 ** -8 * np.abs(ref) + 1e-15
    worst = float(np.max(err / bound))
    say(f"  max |err| / (2^-8 |ref| + 1e-15) = {worst:.3f}")
    assert worst <= 1.0


@pytest.mark.parametrize("act,m,h,f,plan", [
    ("swiglu", 3000, 64, 1536, (192, 12, 192)),
    ("swiglu", 1000, 136, 520, (64, 9, 64)),        # small tiles: 64 outputs each, ragged m and f
    ("gelu", 1000, 1032, 776, (64, 7, 64)),         # small tiles, ragged m and f, k tail
    ("swiglu", 5000, 64, 1792, (192, 8, 128)),
    ("swiglu", 4000, 2056, 2048, (256, 16, 256)),   # four-wave tiles, ragged m, k tail
    ("gelu", 4000, 2056, 4000, (256, 16, 256)),     # four-wave tiles, ragged m and n
    ("swiglu", 5000, 2056, 1792, (192, 8, 128)),    # four-wave 192/128 split, ragged m, k tail
    ("swiglu", 4000, 4104, 2048, (256, 16, 256)),   # 16x16-MFMA tiles, ragged m, k tail
    ("gelu", 4000, 4104, 4000, (256, 16, 256)),     # 16x16-MFMA tiles, ragged m and n
    ("swiglu", 5000, 4104, 1792, (192, 8, 128)),    # 16x16-MFMA 192/128 split, ragged m, k tail
    ("swiglu", 2048, 4104, 6144, (256, 32, 256, 2)),   # one round, then split-k pairs (k tail in the upper half)
    ("gelu", 2000, 4104, 12288, (256, 32, 256, 2)),    # the same with GeLU, ragged m
])
def test_colwise_activation_tile_heights(device, act, m, h, f, plan):
    """GeLU and SwiGLU epilogues (gate/up pairing, 4-column stores) at every
    tile layout, ragged m, against the oracle's activation."""
    say(f"case {act} colwise m={m} h={h} f={f} plan={plan}")
    assert tp.tp_gemm_plan(m, f, h, "swiglu" if act == "swiglu" else "colwise") == (plan + (0,))[:4]
    case = inputs.MLPCase("heights", m, h, f, 1, act, "bf16", seed=24)
    w = inputs.gen_mlp(case)
    dw = {k: to_dev(v, device) for k, v in w.items()}
    mlp = shard.MLPShards(dw["X"], dw, 1, act)
    mlp.colwise(0)
    torch.cuda.synchronize()
    W = {k: v.f64() for k, v in w.items()}
    if act == "swiglu":
        ref = oracle.colwise_act(W["X"], None, "swiglu", (W["W1"], W["W3"]))
    else:
        ref = oracle.colwise_act(W["X"], W["A"], "gelu")
    assert rel_err(host(mlp.act_ws), ref) <= BF16_TOL


# ---------------------------------------------------------------- attention, small


@pytest.mark.parametrize("batch,seq,h,heads,kv,t,causal", [
    (2, 200, 256, 8, 2, 2, True),     # ragged seq (not a multiple of 64 or 128)
    (3, 203, 256, 8, 2, 2, True),     # seq not a multiple of 4: row groups straddle sequences
    (1, 128, 128, 4, 1, 4, True),     # one head per rank
    (2, 96, 256, 8, 2, 8, True),      # kv < t: each KV head replicated on 4 ranks
    (3, 64, 256, 4, 4, 1, True),      # MHA, one rank
    (1, 1, 128, 2, 1, 1, True),       # a single token
    (5, 1400, 128, 8, 2, 1, True),    # Q/K/V projection on 192-row tiles, ragged m and seq
    (2, 2000, 2056, 20, 4, 1, True),  # Q/K/V projection on four-wave 256-row tiles, k tail
])
def test_attention_small(device, batch, seq, h, heads, kv, t, causal):
    say(f"case attn b={batch} s={seq} h={h} heads={heads} kv={kv} t={t} causal={causal}")
    case = inputs.AttnCase("small", batch, seq, h, heads, kv, 128, t, 500000.0, seed=31)
    w = inputs.gen_attn(case)
    dw = {k: to_dev(v, device) for k, v in w.items()}
    at = shard.AttnShards(dw["X"], dw, case, causal=causal)
    out = at.forward()
    torch.cuda.synchronize()
    W = {k: v.f64() for k, v in w.items()}
    full = oracle.attn_partial(W["X"], W, case, 0, t=1)
    for r in range(t):
        ref = oracle.attn_partial(W["X"], W, case, r, t=t)
        e = rel_err(host(at.partials[r]), ref)
        assert e <= BF16_TOL, (r, e)
    assert rel_err(host(out), full) <= BF16_TOL


def test_attention_core_non_causal(device):
    """Non-causal core on its own: Q/K/V written by tp_qkv_rope, compared with
    softmax(q k^T / sqrt d) v over the whole sequence in float64."""
    say("case attn core non-causal")
    batch, seq, hq, hkv, d = 2, 130, 4, 2, 128
    m = batch * seq
    g = torch.Generator().manual_seed(5)
    q = torch.randn(m, hq * d, generator=g).to(torch.bfloat16)
    k = torch.randn(m, hkv * d, generator=g).to(torch.bfloat16)
    v = torch.randn(m, hkv * d, generator=g).to(torch.bfloat16)
    seq_pad = (seq + 63) // 64 * 64
    vt = torch.zeros(batch, hkv, d, seq_pad, dtype=torch.bfloat16)
    vt[..., :seq] = v.view(batch, seq, hkv, d).permute(0, 2, 3, 1)
    o = torch.empty(m, hq * d, dtype=torch.bfloat16, device=device)
    tp.tp_flash_attn(batch, seq, hq, hkv, d, 0, q.to(device), k.to(device), vt.to(device), o)
    torch.cuda.synchronize()
    qh, kh, vh = (a.double().numpy() for a in (q, k, v))
    got = host(o)
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        for j in range(hq):
            gk = j // (hq // hkv)
            qq, kk, vv = qh[rows, j * d:(j + 1) * d], kh[rows, gk * d:(gk + 1) * d], vh[rows, gk * d:(gk + 1) * d]
            s = qq @ kk.T / np.sqrt(d)
            p = np.exp(s - s.max(1, keepdims=True))
            ref = (p / p.sum(1, keepdims=True)) @ vv
            assert rel_err(got[rows, j * d:(j + 1) * d], ref) <= BF16_TOL


# ---------------------------------------------------------------- shard-sum and norm


@pytest.mark.parametrize("t,n,res", [(1, 7, None), (2, 1000003, "f32"), (5, 4099, "bf16"),
                                     (16, 262147, "f32"), (8, 4, None), (3, 1 << 20, "bf16")])
def test_shard_sum_bit_exact(device, t, n, res):
    """Ascending-rank float32 sum (+ residual last) is bit-exact to the
    oracle's float32 mode; n covers ragged tails."""
    say(f"case shard_sum t={t} n={n} res={res}")
    parts = [inputs.normal(41, s, (n,), 1.0, "f32").data for s in range(t)]
    # one allocation per partial: the ABI requires 16-byte aligned pointers
    dparts = [torch.from_numpy(p).to(device) for p in parts]
    out = torch.empty(n, dtype=torch.float32, device=device)
    r_host = None
    r_dev = None
    if res is not None:
        rt = inputs.normal(41, 99, (n,), 1.0, res)
        r_host = rt.f32()
        r_dev = to_dev(rt, device)
    tp.tp_shard_sum(t, n, dparts, r_dev, res or "f32", out)
    torch.cuda.synchronize()
    ref = oracle.shard_sum_f32(parts, r_host)
    assert np.array_equal(out.cpu().numpy(), ref)


def test_shard_sum_in_place_residual(device):
    say("case shard_sum in place")
    n, t = 10000, 4
    parts = [inputs.normal(42, s, (n,), 1.0, "f32").data for s in range(t)]
    res = inputs.normal(42, 50, (n,), 1.0, "f32").data
    dparts = torch.stack([torch.from_numpy(p) for p in parts]).to(device)
    acc = torch.from_numpy(res.copy()).to(device)
    tp.tp_shard_sum(t, n, list(dparts), acc, "f32", acc)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), oracle.shard_sum_f32(parts, res))


@pytest.mark.parametrize("in_dt,m,h,gain", [("bf16", 37, 8192, True), ("f32", 5, 136, False),
                                            ("f32", 300, 4096, True), ("bf16", 1, 16392, True)])
def test_rmsnorm(device, in_dt, m, h, gain):
    say(f"case rmsnorm {in_dt} m={m} h={h} gain={gain}")
    x = inputs.normal(51, 0, (m, h), 3.0, in_dt)
    gv = (inputs.normal(51, 1, (h,), 0.1, "f32").data + np.float32(1)) if gain else None
    y = torch.empty(m, h, dtype=torch.bfloat16, device=device)
    tp.tp_rmsnorm(in_dt, m, h, to_dev(x, device), None if gv is None else torch.from_numpy(gv).to(device),
                  1e-5, y)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(x.f64(), None if gv is None else gv.astype(np.float64), 1e-5)
    got = host(y)
    # bf16 output: one rounding (2^-9 relative) plus float32 arithmetic
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


@pytest.mark.parametrize("t,m,h,res,gain", [(8, 37, 8192, "bf16", True), (1, 5, 136, None, False),
                                             (3, 300, 4096, "f32", True), (16, 3, 16392, "f32", False),
                                             (2, 1, 24, "bf16", False)])
def test_shard_sum_rmsnorm(device, t, m, h, res, gain):
    """The fused sum + norm: the sum is bit-exact to the oracle's float32
    shard-sum, the normed rows bitwise those of tp_shard_sum then tp_rmsnorm
    (and within one bf16 rounding of the float64 norm of that sum); h beyond
    8192 reads back the stored sums."""
    say(f"case shard_sum_rmsnorm t={t} m={m} h={h} res={res} gain={gain}")
    parts = [inputs.normal(53, s, (m, h), 1.0, "f32").data for s in range(t)]
    dparts = [torch.from_numpy(p).to(device) for p in parts]
    r_host = r_dev = None
    if res is not None:
        rt = inputs.normal(53, 99, (m, h), 1.0, res)
        r_host, r_dev = rt.f32(), to_dev(rt, device)
    gv = (inputs.normal(53, 100, (h,), 0.1, "f32").data + np.float32(1)) if gain else None
    g_dev = None if gv is None else torch.from_numpy(gv).to(device)
    out = torch.empty(m, h, dtype=torch.float32, device=device)
    y = torch.empty(m, h, dtype=torch.bfloat16, device=device)
    tp.tp_shard_sum_rmsnorm(t, m, h, dparts, r_dev, res or "f32", out, g_dev, 1e-5, y)
    out2 = torch.empty_like(out)
    y2 = torch.empty_like(y)
    tp.tp_shard_sum(t, m * h, dparts, r_dev, res or "f32", out2)
    tp.tp_rmsnorm("f32", m, h, out2, g_dev, 1e-5, y2)
    torch.cuda.synchronize()
    ref_sum = oracle.shard_sum_f32(parts, r_host)
    assert np.array_equal(out.cpu().numpy(), ref_sum)
    assert torch.equal(y, y2)
    ref = oracle.rmsnorm(ref_sum.astype(np.float64), None if gv is None else gv.astype(np.float64), 1e-5)
    assert np.all(np.abs(host(y) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


def test_shard_sum_rmsnorm_in_place_residual(device):
    """out may be the float32 residual itself (the residual stream updated in place)."""
    say("case shard_sum_rmsnorm in place")
    t, m, h = 4, 64, 1024
    parts = [inputs.normal(54, s, (m, h), 1.0, "f32").data for s in range(t)]
    dparts = [torch.from_numpy(p).to(device) for p in parts]
    r = inputs.normal(54, 99, (m, h), 1.0, "f32").data
    acc = torch.from_numpy(r.copy()).to(device)
    y = torch.empty(m, h, dtype=torch.bfloat16, device=device)
    tp.tp_shard_sum_rmsnorm(t, m, h, dparts, acc, "f32", acc, None, 1e-5, y)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), oracle.shard_sum_f32(parts, r))


@pytest.mark.parametrize("t", [4, 12])
def test_shard_sum_rmsnorm_runs(device, t):
    """Rank slices as runs (positions [r S/t, (r+1) S/t) of every sequence): the
    norm alone (t = 0), the reduce-scatter with norm, and the reduce-scatter
    alone each write exactly their rows, bitwise equal to the whole-matrix
    calls, and leave every other row alone."""
    say(f"case shard_sum_rmsnorm runs t={t}")
    batch, seq, h = 3, 48, 264
    m, n = batch * seq, seq // t
    parts = torch.stack([torch.from_numpy(inputs.normal(55, s, (m, h), 1.0, "f32").data) for s in range(t)]).to(device)
    x = to_dev(inputs.normal(55, 99, (m, h), 1.0, "bf16"), device)
    g = torch.from_numpy(inputs.normal(55, 100, (h,), 0.1, "f32").data + np.float32(1)).to(device)
    # whole-matrix references
    xn_ref = torch.empty(m, h, dtype=torch.bfloat16, device=device)
    tp.tp_rmsnorm("bf16", m, h, x, g, 1e-5, xn_ref)
    h1_ref = torch.empty(m, h, device=device)
    hn_ref = torch.empty(m, h, dtype=torch.bfloat16, device=device)
    tp.tp_shard_sum_rmsnorm(t, m, h, list(parts), x, "bf16", h1_ref, g, 1e-5, hn_ref)
    z_ref = torch.empty(m, h, device=device)
    tp.tp_shard_sum(t, m * h, list(parts), h1_ref, "f32", z_ref)
    # per-rank runs, into buffers prefilled with a sentinel
    sent = float("nan")
    xn = torch.full((m, h), sent, dtype=torch.bfloat16, device=device)
    h1 = torch.full((m, h), sent, device=device)
    hn = torch.full((m, h), sent, dtype=torch.bfloat16, device=device)
    z = torch.full((m, h), sent, device=device)
    runs = (batch, n, seq)
    for r in range(t):
        o = r * n
        tp.tp_shard_sum_rmsnorm(0, 0, h, [], x[o:], "bf16", None, g, 1e-5, xn[o:], runs=runs)
        tp.tp_shard_sum_rmsnorm(t, 0, h, [parts[i][o:] for i in range(t)], x[o:], "bf16", h1[o:], g, 1e-5,
                                hn[o:], runs=runs)
        tp.tp_shard_sum_rmsnorm(t, 0, h, [parts[i][o:] for i in range(t)], h1[o:], "f32", z[o:], None, 1e-5,
                                None, runs=runs)
        if r == 0:  # after rank 0 alone, only its rows are written
            torch.cuda.synchronize()
            rows0 = np.concatenate([b * seq + np.arange(n) for b in range(batch)])
            others = np.setdiff1d(np.arange(m), rows0)
            assert torch.isnan(xn[others].float()).all() and torch.isnan(z[others]).all()
            assert not torch.isnan(xn[rows0].float()).any() and not torch.isnan(z[rows0]).any()
    torch.cuda.synchronize()
    assert torch.equal(xn, xn_ref) and torch.equal(h1, h1_ref) and torch.equal(hn, hn_ref)
    assert torch.equal(z, z_ref)
    assert np.array_equal(h1.cpu().numpy(), oracle.shard_sum_f32([p.cpu().numpy() for p in parts],
                                                                 inputs.normal(55, 99, (m, h), 1.0, "bf16").f32()))


def test_sequence_parallel_block(device):
    """The sequence-parallel block (norms on each rank's Shard(1) slices,
    reduce-scatter + norm per slice, shared gathered inputs) against the
    oracle's sequence-parallel block, and bitwise equal to the replicated
    forms (fused and two-pass)."""
    case = inputs.BlockCase("sp_block", batch=2, seq=192, hidden=512, heads=8, kv_heads=2,
                            head_dim=128, inter=1024, t=4, rope_base=500000.0, seed=71, gain_std=0.1)
    say(f"case sequence-parallel block {case}")
    w = inputs.gen_block(case)
    dw = {k: to_dev(v, device) for k, v in w.items()}
    blk = shard.BlockShards(dw["X"], dw, case)
    z_sp = blk.forward_sp().clone()
    h1_sp = blk.attn.out.clone()
    z_rep = blk.forward().clone()
    z_two = blk.forward(fused=False).clone()
    torch.cuda.synchronize()
    assert torch.equal(z_sp, z_rep) and torch.equal(z_rep, z_two)
    W = {k: v.f64() for k, v in w.items()}
    ref = oracle.sp_block(W["X"], W, case)
    assert rel_err(host(h1_sp), ref["h1"]) <= BF16_TOL
    assert rel_err(host(z_sp), ref["z"]) <= BF16_TOL


# ---------------------------------------------------------------- determinism


def test_bitwise_deterministic(device):
    say("case determinism")
    case = inputs.AttnCase("det", 2, 256, 512, 8, 2, 128, 2, 500000.0, seed=61)
    w = inputs.gen_attn(case)
    dw = {k: to_dev(v, device) for k, v in w.items()}
    at = shard.AttnShards(dw["X"], dw, case)
    a = at.forward().clone()
    b = at.forward().clone()
    assert torch.equal(a, b)
    mc = inputs.MLPCase("det", 512, 512, 2048, 2, "swiglu", "bf16", seed=62)
    mw = {k: to_dev(v, device) for k, v in inputs.gen_mlp(mc).items()}
    mlp = shard.MLPShards(mw["X"], mw, 2, "swiglu")
    a = mlp.forward().clone()
    b = mlp.forward().clone()
    assert torch.equal(a, b)


# ---------------------------------------------------------------- full-size workloads


def test_config_gpt_gelu_mlp(device):
    """GPT-style GeLU MLP, 2048 tokens, h=1024, inter 4096, t=4: all partials
    and the shard-sum against the full float64 oracle."""
    case = inputs.CONFIGS["gpt_gelu_mlp"]
    say(f"case {case.name}")
    t0 = time.time()
    w = inputs.gen_mlp(case)
    dw = {k: to_dev(v, device) for k, v in w.items()}
    mlp = shard.MLPShards(dw["X"], dw, case.t, "gelu")
    out = mlp.forward()
    torch.cuda.synchronize()
    W = {k: v.f64() for k, v in w.items()}
    parts = oracle.mlp_gelu_partials(W["X"], W["A"], W["B"], case.t)
    for r in range(case.t):
        assert rel_err(host(mlp.partials[r]), parts[r]) <= BF16_TOL
    assert rel_err(host(out), oracle.mlp_gelu(W["X"], W["A"], W["B"])) <= BF16_TOL
    say(f"  done in {time.time() - t0:.1f}s")


def test_config_llama8b_swiglu_mlp(device):
    """Llama-3-8B-shaped SwiGLU MLP, 4096 tokens, t=4, on 64 sampled rows."""
    case = inputs.CONFIGS["llama8b_swiglu_mlp"]
    say(f"case {case.name}")
    t0 = time.time()
    w = inputs.gen_mlp(case)
    dw = {k: to_dev(v, device) for k, v in w.items()}
    mlp = shard.MLPShards(dw["X"], dw, case.t, "swiglu")
    out = mlp.forward()
    torch.cuda.synchronize()
    rows = inputs.sample_rows(1, case.tokens, 61, seed=3)
    X = w["X"].f64()[rows]
    W1, W3, W2 = w["W1"].f64(), w["W3"].f64(), w["W2"].f64()
    parts = oracle.mlp_swiglu_partials(X, W1, W3, W2, case.t)
    for r in range(case.t):
        assert rel_err(host(mlp.partials[r], rows), parts[r]) <= BF16_TOL
    assert rel_err(host(out, rows), oracle.shard_sum(parts)) <= BF16_TOL
    say(f"  done in {time.time() - t0:.1f}s")


def test_config_llama8b_attn(device):
    """Llama-3-8B-shaped attention, batch 2 x 2048, 32/8 heads, t=4, sampled rows."""
    case = inputs.CONFIGS["llama8b_attn"]
    say(f"case {case.name}")
    t0 = time.time()
    w = inputs.gen_attn(case)
    dw = {k: to_dev(v, device) for k, v in w.items()}
    at = shard.AttnShards(dw["X"], dw, case)
    out = at.forward()
    torch.cuda.synchronize()
    rows = inputs.sample_rows(case.batch, case.seq, 29, seed=4)
    W = {k: v.f64() for k, v in w.items()}
    parts = [oracle.attn_partial(W["X"], W, case, r, rows=rows) for r in range(case.t)]
    for r in range(case.t):
        assert rel_err(host(at.partials[r], rows), parts[r]) <= BF16_TOL
    assert rel_err(host(out, rows), oracle.shard_sum(parts)) <= BF16_TOL
    say(f"  done in {time.time() - t0:.1f}s")


@pytest.fixture(scope="module")
def block70b():
    case = inputs.CONFIGS["llama70b_block_t8"]
    w = inputs.gen_block(case)
    rows = inputs.sample_rows(case.batch, case.seq, 13, seed=5)
    W = {k: v.f64() for k, v in w.items()}
    ref = oracle.block(W["X"], W, case, t=1, rows=rows)
    return case, w, rows, ref


@pytest.mark.parametrize("t", [8, 16])
def test_config_70b_block(device, block70b, t):
    """70B-shaped block (attention + SwiGLU MLP, RMSNorm replicated), batch
    4 x 2048, at t=8 and t=16 (a KV head on 2 ranks): sampled rows of h1 and Z
    against the unsharded float64 block, and the same rows at t=8 and t=16."""
    case, w, rows, ref = block70b
    say(f"case llama70b block t={t}")
    t0 = time.time()
    dw = {k: to_dev(v, device) for k, v in w.items()}
    blk = shard.BlockShards(dw["X"], dw, case, t=t)
    z = blk.forward().clone()
    torch.cuda.synchronize()
    assert rel_err(host(blk.attn.out, rows), ref["h1"]) <= BF16_TOL
    assert rel_err(host(z, rows), ref["z"]) <= BF16_TOL
    # the sequence-parallel form of the same block: bitwise the same result
    assert torch.equal(blk.forward_sp(), z)
    say(f"  done in {time.time() - t0:.1f}s")


# Error of each sublayer alone at the 70B t=8 block (max|gpu-ref|/max|ref| on
# the sampled rows, the oracle fed with the GPU's own bf16 normed input;
# measured 3.5e-3 and 1.6e-3 when the block test's error budget was
# analysed): bars at about 1.5 times those, so a regression in one sublayer
# fails here, by name, long before the block's 2e-2 bar.
ATTN_SUBLAYER_TOL = 5e-3
MLP_SUBLAYER_TOL = 2.5e-3


def test_config_70b_sublayers(device, block70b):
    """The 70B t=8 block's two sublayers, each against the float64 oracle fed
    with the GPU's own normalised input (RMSNorm(X) for attention,
    RMSNorm(h1) for the MLP), on the sampled rows of the first and last
    sequences; the ranks' partials are summed in float64, so only the
    sublayer's own arithmetic is measured."""
    case, w, rows, _ = block70b
    say("case llama70b sublayers t=8")
    t0 = time.time()
    dw = {k: to_dev(v, device) for k, v in w.items()}
    blk = shard.BlockShards(dw["X"], dw, case, t=8)
    blk.forward()
    torch.cuda.synchronize()
    W = {k: v.f64() for k, v in w.items()}
    m = case.batch * case.seq
    sel = rows[(rows < case.seq) | (rows >= m - case.seq)]
    # attention on the GPU's normed X (every token: K and V need the whole prefix)
    xn = host(blk.xn)
    ref_a = oracle.attn_partial(xn, W, case.attn(), 0, t=1, rows=sel)
    got_a = sum(host(blk.attn.partials[r], sel) for r in range(8))
    e_a = rel_err(got_a, ref_a)
    # MLP on the GPU's normed h1 (row-local)
    hn = host(blk.hn, sel)
    ref_m = oracle.mlp_swiglu(hn, W["W1"], W["W3"], W["W2"])
    got_m = sum(host(blk.mlp.partials[r], sel) for r in range(8))
    e_m = rel_err(got_m, ref_m)
    say(f"  attention {e_a:.2e} (bar {ATTN_SUBLAYER_TOL}), MLP {e_m:.2e} (bar {MLP_SUBLAYER_TOL}),"
        f" {time.time() - t0:.1f}s")
    assert e_a <= ATTN_SUBLAYER_TOL
    assert e_m <= MLP_SUBLAYER_TOL


def test_smoke_entry(device):
    import __graft_entry__

    __graft_entry__.smoke()
