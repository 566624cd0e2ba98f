"""tp_shard_attn_noalloc (the attention sublayer with its workspace in the
library's static device array) against tp_shard_attn (caller workspace),
both through the C ABI.

The two run the same kernels on the same inputs, so their partials must be
bitwise equal -- stricter than the bf16 bar of the parity tests.  Two calls
in a row, the second on a smaller shape, show that what the first left in
the shared array does not leak into the second.  The second shape is also
checked against the oracle at the bf16 bar.
"""
import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_colwise_amd import inputs, shard, tpshard as tp

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not tp.LIB_PATH.exists():
        raise RuntimeError("libtpshard.so is not built")
    torch.cuda.set_device(0)
    tp.tp_device_check()
    return torch.device("cuda:0")


def _compare(device, batch, seq, h, heads, kv, t, causal, seed, check_oracle=False):
    print(f"case noalloc b={batch} s={seq} h={h} heads={heads} kv={kv} t={t} causal={causal}", flush=True)
    case = inputs.AttnCase("noalloc", batch, seq, h, heads, kv, 128, t, 500000.0, seed=seed)
    w = inputs.gen_attn(case)
    dw = {k: v.torch().to(device) for k, v in w.items()}
    at = shard.AttnShards(dw["X"], dw, case, causal=causal)
    m = batch * seq
    W = {k: v.f64() for k, v in w.items()} if check_oracle else None
    for r, rk in enumerate(at.ranks):
        ref = torch.full((m, h), float("nan"), dtype=torch.float32, device=device)
        got = torch.full((m, h), float("nan"), dtype=torch.float32, device=device)
        tp.tp_shard_attn("bf16", batch, seq, h, rk.hq, rk.hkv, 128, case.rope_base, causal, dw["X"], rk.w_qkv,
                         rk.w_o, at.ws, at.ws_bytes, ref)
        tp.tp_shard_attn_noalloc("bf16", batch, seq, h, rk.hq, rk.hkv, 128, case.rope_base, causal, dw["X"],
                                 rk.w_qkv, rk.w_o, got)
        torch.cuda.synchronize()
        assert torch.isfinite(got).all()
        assert torch.equal(got, ref), f"rank {r}: max |diff| {float((got - ref).abs().max())}"
        if check_oracle:
            want = oracle.attn_partial(W["X"], W, case, r, t=t)
            g = got.double().cpu().numpy()
            e = float(np.max(np.abs(g - want)) / np.max(np.abs(want)))
            print(f"  rank {r}: max|gpu-oracle|/max|oracle| = {e:.3e}", flush=True)
            assert e <= BF16_TOL


def test_noalloc_attention_matches_workspace_call(device):
    # a larger call first (two ranks, GQA, a ragged sequence, no mask), then a
    # smaller causal one, also against the oracle (whose attention is causal)
    _compare(device, batch=2, seq=700, h=1024, heads=8, kv=2, t=2, causal=False, seed=61)
    _compare(device, batch=1, seq=130, h=256, heads=4, kv=2, t=1, causal=True, seed=62, check_oracle=True)


def test_noalloc_attention_rejects_shapes_beyond_the_scratch(device):
    # 4 x 8192 tokens with 16 query heads needs more than the 64 MiB array
    need = tp.tp_shard_attn_workspace_bytes(4, 8192, 16, 1, 128)
    assert need > (64 << 20)
    dummy = torch.empty(16, dtype=torch.float32, device=device)
    with pytest.raises(tp.TpError) as ei:
        tp.tp_shard_attn_noalloc("bf16", 4, 8192, 2048, 16, 1, 128, 500000.0, 1, dummy, dummy, dummy, dummy)
    assert ei.value.status == tp.TP_ERR_WORKSPACE and "static scratch" in ei.value.message
