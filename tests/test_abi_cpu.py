"""C-ABI contract checks that need no GPU.

The library must load, export every function ``include/tpshard.h`` declares,
and reject bad arguments with the documented status before touching a device
(argument checks run on the host first, so these calls never reach HIP).
"""
import ctypes

import pytest
import torch

from megatron_tensor_transformer_colwise_amd import shard, tpshard as tp


@pytest.fixture(scope="module")
def L():
    if not tp.LIB_PATH.exists():
        import __graft_entry__

        __graft_entry__.build()
    return tp.lib()


def test_exports_match_header(L):
    names = tp.header_exports()
    assert "tp_shard_mlp" in names and "tp_shard_attn" in names and "tp_shard_sum" in names
    for n in names:
        assert hasattr(L, n), f"{n} declared in the header but not exported"
    assert set(names) == set(tp._SIGS)


A16 = 1 << 20        # a fake, 16-byte aligned "device address" (never dereferenced)
MIS = A16 + 4        # misaligned


def status(fn, *args):
    return getattr(tp.lib(), fn)(*args)


def test_colwise_rowwise_validation(L):
    # k not a multiple of 8
    assert status("tp_colwise", 1, 1, 4, 12, 16, A16, A16, None, A16, None) == tp.TP_ERR_SHAPE
    assert "k = 12" in tp.tp_last_error()
    # n not positive
    assert status("tp_colwise", 1, 1, 4, 16, 0, A16, A16, None, A16, None) == tp.TP_ERR_SHAPE
    # negative m
    assert status("tp_rowwise", 1, -1, 16, 16, A16, A16, A16, None) == tp.TP_ERR_SHAPE
    # unknown dtype / activation
    assert status("tp_colwise", 1, 7, 4, 16, 16, A16, A16, None, A16, None) == tp.TP_ERR_INVALID_ARG
    assert status("tp_colwise", 9, 1, 4, 16, 16, A16, A16, None, A16, None) == tp.TP_ERR_INVALID_ARG
    # null and misaligned pointers
    assert status("tp_colwise", 1, 1, 4, 16, 16, None, A16, None, A16, None) == tp.TP_ERR_INVALID_ARG
    assert "x is NULL" in tp.tp_last_error()
    assert status("tp_rowwise", 1, 4, 16, 16, A16, MIS, A16, None) == tp.TP_ERR_INVALID_ARG
    assert "w is not 16-byte aligned" in tp.tp_last_error()
    # weight over the 2 GiB operand limit
    assert status("tp_colwise", 2, 1, 4, 65536, 65536, A16, A16, None, A16, None) == tp.TP_ERR_SHAPE


def test_m_zero_is_a_noop(L):
    # nothing to do: OK without touching pointers or the device
    assert status("tp_colwise", 1, 1, 0, 16, 16, None, None, None, None, None) == tp.TP_OK
    assert status("tp_rowwise", 1, 0, 16, 16, None, None, None, None) == tp.TP_OK
    assert status("tp_shard_mlp", 2, 1, 0, 16, 16, None, None, None, None, None, None) == tp.TP_OK
    arr = (ctypes.c_void_p * 1)(None)
    assert status("tp_shard_sum", 1, 0, arr, None, 0, None, None) == tp.TP_OK
    assert status("tp_rmsnorm", 1, 0, 16, None, None, 1e-5, None, None) == tp.TP_OK


def test_shard_mlp_needs_an_activation(L):
    assert status("tp_shard_mlp", 0, 1, 4, 16, 16, A16, A16, A16, A16, A16, None) == tp.TP_ERR_INVALID_ARG


def test_attention_validation(L):
    args = dict(batch=2, seq=64, h=256, hq=4, hkv=2, d=128)

    def attn(dt=tp.TP_BF16, **kw):
        a = {**args, **kw}
        return status("tp_shard_attn", dt, a["batch"], a["seq"], a["h"], a["hq"], a["hkv"], a["d"],
                      500000.0, 1, A16, A16, A16, A16, 1 << 30, A16, None)

    # the contract's dtype argument: only bf16 attention is built
    assert attn(dt=tp.TP_F32) == tp.TP_ERR_UNSUPPORTED
    assert "only bf16" in tp.tp_last_error()
    assert attn(dt=7) == tp.TP_ERR_INVALID_ARG
    assert attn(d=64) == tp.TP_ERR_UNSUPPORTED
    assert attn(hq=3, hkv=2) == tp.TP_ERR_SHAPE
    assert "multiple of hkv" in tp.tp_last_error()
    assert attn(hkv=0) == tp.TP_ERR_SHAPE
    assert attn(h=260) == tp.TP_ERR_SHAPE
    ws_need = tp.tp_shard_attn_workspace_bytes(2, 64, 4, 2, 128)
    m = 2 * 64
    expect = 4 * 128 * m * 2 + 2 * 128 * m * 2 + 2 * 2 * 128 * 64 * 2 + 4 * 128 * m * 2
    assert ws_need == expect
    st = status("tp_shard_attn", tp.TP_BF16, 2, 64, 256, 4, 2, 128, 500000.0, 1, A16, A16, A16, A16, ws_need - 1,
                A16, None)
    assert st == tp.TP_ERR_WORKSPACE
    assert status("tp_qkv_rope", 2, 64, 256, 4, 2, 128, 0.5, A16, A16, None, A16, A16, A16, None) == tp.TP_ERR_INVALID_ARG
    assert status("tp_flash_attn", 2, 64, 4, 2, 128, 1, A16, A16, None, A16, None) == tp.TP_ERR_INVALID_ARG
    # the variant on the library's static scratch: same checks, plus its size limit
    assert status("tp_shard_attn_noalloc", tp.TP_F32, 2, 64, 256, 4, 2, 128, 500000.0, 1, A16, A16, A16, A16,
                  None) == tp.TP_ERR_UNSUPPORTED
    assert status("tp_shard_attn_noalloc", tp.TP_BF16, 2, 64, 256, 3, 2, 128, 500000.0, 1, A16, A16, A16, A16,
                  None) == tp.TP_ERR_SHAPE
    assert tp.tp_shard_attn_workspace_bytes(4, 8192, 16, 1, 128) > (64 << 20)
    assert status("tp_shard_attn_noalloc", tp.TP_BF16, 4, 8192, 2048, 16, 1, 128, 500000.0, 1, A16, A16, A16,
                  A16, None) == tp.TP_ERR_WORKSPACE
    assert "static scratch" in tp.tp_last_error()
    assert status("tp_shard_attn_noalloc", tp.TP_BF16, 0, 64, 256, 4, 2, 128, 500000.0, 1, None, None, None,
                  None, None) == tp.TP_OK
    # seq padding to 64 in the transposed-V region
    assert tp.tp_shard_attn_workspace_bytes(1, 65, 1, 1, 128) >= 128 * 128 * 2


def test_shard_sum_validation(L):
    ptrs = (ctypes.c_void_p * 17)(*([A16 + 64 * i for i in range(17)]))
    assert status("tp_shard_sum", 0, 16, ptrs, None, 0, A16 + 4096, None) == tp.TP_ERR_SHAPE
    assert status("tp_shard_sum", 17, 16, ptrs, None, 0, A16 + 4096, None) == tp.TP_ERR_SHAPE
    assert status("tp_shard_sum", 2, 16, ptrs, None, 0, A16, None) == tp.TP_ERR_INVALID_ARG  # out aliases
    assert "aliases partials[0]" in tp.tp_last_error()
    bad = (ctypes.c_void_p * 2)(A16, MIS)
    assert status("tp_shard_sum", 2, 16, bad, None, 0, A16 + 4096, None) == tp.TP_ERR_INVALID_ARG
    assert "partials[1]" in tp.tp_last_error()
    # out may alias a float32 residual but not a bf16 one
    assert status("tp_shard_sum", 2, 16, ptrs, A16 + 4096, 1, A16 + 4096, None) == tp.TP_ERR_INVALID_ARG
    assert status("tp_shard_sum", 2, 16, ptrs, A16 + 4096, 5, A16 + 8192, None) == tp.TP_ERR_INVALID_ARG


def test_shard_sum_rmsnorm_validation(L):
    ptrs = (ctypes.c_void_p * 17)(*([A16 + 64 * i for i in range(17)]))
    out, y = A16 + 8192, A16 + 16384

    def call(t, h=16, res=None, rdt=0, o=out, g=None, eps=1e-5, yy=y, runs=(1, 4, 4), arr=ptrs, bias=None):
        return status("tp_shard_sum_rmsnorm", t, runs[0], runs[1], runs[2], h, arr, bias, res, rdt, o, g, eps, yy,
                      None)

    assert call(-1) == tp.TP_ERR_SHAPE
    assert call(17) == tp.TP_ERR_SHAPE
    assert call(2, runs=(-1, 4, 4)) == tp.TP_ERR_SHAPE
    assert call(2, runs=(2, 4, 3)) == tp.TP_ERR_SHAPE                # runs overlap
    assert "run_stride" in tp.tp_last_error()
    assert call(2, h=12) == tp.TP_ERR_SHAPE                          # h not a multiple of 8
    assert call(2, eps=-1.0) == tp.TP_ERR_INVALID_ARG
    assert call(2, o=A16) == tp.TP_ERR_INVALID_ARG                   # out aliases partials[0]
    assert "aliases partials[0]" in tp.tp_last_error()
    assert call(2, res=out, rdt=1) == tp.TP_ERR_INVALID_ARG          # bf16 residual aliased by out
    assert call(2, res=A16 + 4096, rdt=7) == tp.TP_ERR_INVALID_ARG    # unknown residual dtype
    assert call(2, g=MIS) == tp.TP_ERR_INVALID_ARG                   # misaligned gain
    assert call(0) == tp.TP_ERR_INVALID_ARG                          # no partials and no residual
    assert "needs a residual" in tp.tp_last_error()
    assert call(2, o=None, yy=None) == tp.TP_ERR_INVALID_ARG         # nothing to write
    assert call(2, arr=None) == tp.TP_ERR_INVALID_ARG
    assert call(2, bias=MIS) == tp.TP_ERR_INVALID_ARG                 # misaligned bias
    assert call(0, res=A16 + 4096, rdt=0, bias=A16 + 4096) == tp.TP_ERR_INVALID_ARG  # bias without partials
    # nothing to do: OK without touching pointers or the device
    assert call(2, runs=(0, 4, 4), o=None, yy=y, arr=None) == tp.TP_OK
    assert call(2, runs=(3, 0, 4), arr=None) == tp.TP_OK


def test_rmsnorm_validation(L):
    assert status("tp_rmsnorm", 1, 4, 12, A16, None, 1e-5, A16, None) == tp.TP_ERR_SHAPE
    assert status("tp_rmsnorm", 3, 4, 16, A16, None, 1e-5, A16, None) == tp.TP_ERR_INVALID_ARG
    assert status("tp_rmsnorm", 1, 4, 16, A16, None, -1.0, A16, None) == tp.TP_ERR_INVALID_ARG
    assert status("tp_rmsnorm", 1, 4, 16, A16, MIS, 1e-5, A16, None) == tp.TP_ERR_INVALID_ARG


def test_gemm_plans(L):
    """Tile plans of the workload shapes (host-only call)."""
    # SwiGLU, 70B t=8: 24 tile columns on 3 whole rounds, the last 4 as split-k pairs
    assert tp.tp_gemm_plan(8192, 3584, 8192, "swiglu") == (256, 24, 256, 2)
    assert tp.tp_gemm_plan(8192, 8192, 3584) == (256, 32, 256, 0)          # down proj
    assert tp.tp_gemm_plan(8192, 8192, 1024) == (256, 32, 256, 0)          # o_proj
    assert tp.tp_gemm_plan(8192, 1280, 8192, "qkv") == (192, 5, 192, 0)    # QKV, 70B t=8
    assert tp.tp_gemm_plan(8192, 768, 8192, "qkv") == (128, 3, 128, 0)     # QKV, 70B t=16
    assert tp.tp_gemm_plan(4096, 3584, 4096, "swiglu") == (256, 28, 256, 0)  # SwiGLU, Llama-8B
    # GPT MLP (2048 x 1024 x 1024): 256 small tiles of 64 x 128 instead of 64 of 128 x 256
    assert tp.tp_gemm_plan(2048, 1024, 1024, "colwise") == (64, 8, 64, 0)
    assert tp.tp_gemm_plan(2048, 1024, 1024) == (64, 8, 64, 0)
    assert tp.tp_gemm_plan(1000, 520, 136, "swiglu") == (64, 9, 64, 0)    # 64 outputs per small tile
    # small tiles only where they beat the large ones (a tie keeps the large tiles)
    assert tp.tp_gemm_plan(2048, 1024, 1024, "swiglu") == (128, 8, 128, 0)
    assert tp.tp_gemm_plan(4000, 776, 136) == (128, 4, 128, 0)
    assert tp.tp_gemm_plan(300, 264, 520, "qkv")[0] != 64               # Q/K/V: large tiles only
    # split-k only for bf16 outputs of depth >= 4096
    assert tp.tp_gemm_plan(520, 768, 4104, "colwise") == (256, 0, 256, 2)
    assert tp.tp_gemm_plan(520, 768, 4104, "rowwise")[3] == 0
    assert tp.tp_gemm_plan(520, 768, 4032, "colwise")[3] == 0
    assert tp.tp_gemm_plan(520, 1280, 8192, "qkv")[3] == 0
    with pytest.raises(tp.TpError):
        tp.tp_gemm_plan(0, 16)
    with pytest.raises(tp.TpError):
        tp.tp_gemm_plan(16, 16, 0)
    assert L.tp_gemm_plan(16, 16, 16, 7, *[ctypes.byref(ctypes.c_int32()) for _ in range(4)]) == tp.TP_ERR_INVALID_ARG


def test_flash_attn_plans(L):
    """Pieces per pair of query blocks (host-only call): one from 512 pair
    units, two from 32, below that toward two workgroups per CU; at least 4
    key tiles per piece."""
    assert tp.tp_flash_attn_plan(4, 2048, 8) == 2      # 70B t=8 rank: 8 pairs x 32 = 256 units
    assert tp.tp_flash_attn_plan(4, 2048, 4) == 2      # 70B t=16 rank: 128 units
    assert tp.tp_flash_attn_plan(2, 2048, 8) == 2      # Llama-8B rank: 128 units
    assert tp.tp_flash_attn_plan(1, 2048, 4) == 2      # 32 units
    assert tp.tp_flash_attn_plan(1, 2048, 2) == 8      # 16 units
    assert tp.tp_flash_attn_plan(4, 4096, 8) == 1      # 512 units
    assert tp.tp_flash_attn_plan(1, 2048, 1) == 8      # 34 tiles per pair: at most 8 pieces
    assert tp.tp_flash_attn_plan(1, 1000, 1) == 4      # 18 tiles per pair
    assert tp.tp_flash_attn_plan(1, 900, 2, False) == 7  # all keys: 30 tiles per pair
    assert tp.tp_flash_attn_plan(1, 130, 4) == 1       # 5 tiles: no split
    assert tp.tp_flash_attn_plan(64, 2048, 16) == 1    # enough pairs to fill the chip
    assert tp.tp_flash_attn_plan(0, 2048, 8) == 1
    with pytest.raises(tp.TpError):
        tp.tp_flash_attn_plan(1, -1, 8)
    assert L.tp_flash_attn_plan(1, 16, 1, 1, None) == tp.TP_ERR_INVALID_ARG


def test_binding_raises_with_message(L):
    with pytest.raises(tp.TpError) as e:
        tp.tp_colwise("gelu", "bf16", 4, 12, 16, A16, A16, A16, stream=0)
    assert e.value.status == tp.TP_ERR_SHAPE


# ---------------------------------------------------------------- sharding rules


def test_sharding_rules_raise_value_error():
    with pytest.raises(ValueError):
        shard.attn_heads(heads=32, kv_heads=8, t=3, rank=0)      # t does not divide heads
    with pytest.raises(ValueError):
        shard.attn_heads(heads=12, kv_heads=8, t=4, rank=0)      # kv does not divide heads
    with pytest.raises(ValueError):
        shard.attn_heads(heads=24, kv_heads=6, t=4, rank=0)      # neither split nor replicate
    with pytest.raises(ValueError):
        shard.colwise_weight(torch.zeros(4, 10), 4, 0)


def test_sharding_layouts():
    a = torch.arange(6 * 8, dtype=torch.float32).reshape(6, 8)
    w = shard.colwise_weight(a, 2, 1)
    assert w.shape == (4, 6) and torch.equal(w, a[:, 4:8].t())
    b = torch.arange(8 * 6, dtype=torch.float32).reshape(8, 6)
    assert torch.equal(shard.rowwise_weight(b, 4, 3), b[6:8].t())
    g = shard.packed_gate_up(a, a + 1000, 2, 0)
    assert torch.equal(g[:4], a[:, :4].t()) and torch.equal(g[4:], (a + 1000)[:, :4].t())
    # GQA: 64 query heads / 8 KV heads; t = 16 replicates each KV head on 2 ranks
    assert shard.attn_heads(64, 8, 16, 0) == ([0, 1, 2, 3], [0])
    assert shard.attn_heads(64, 8, 16, 1) == ([4, 5, 6, 7], [0])
    assert shard.attn_heads(64, 8, 16, 15)[1] == [7]
    assert shard.attn_heads(32, 8, 4, 1) == ([8, 9, 10, 11, 12, 13, 14, 15], [2, 3])
    d = 2
    wq = torch.arange(3 * 8 * d, dtype=torch.float32).reshape(3, 8 * d)
    wk = -torch.arange(3 * 2 * d, dtype=torch.float32).reshape(3, 2 * d)
    wv = wk - 100
    wo = torch.arange(8 * d * 3, dtype=torch.float32).reshape(8 * d, 3)
    r = shard.attn_rank(wq, wk, wv, wo, heads=8, kv_heads=2, head_dim=d, t=4, rank=3)
    assert (r.hq, r.hkv) == (2, 1)
    assert torch.equal(r.w_qkv[: 2 * d], wq[:, 6 * d:8 * d].t())
    assert torch.equal(r.w_qkv[2 * d:3 * d], wk[:, d:2 * d].t())
    assert torch.equal(r.w_qkv[3 * d:], wv[:, d:2 * d].t())
    assert torch.equal(r.w_o, wo[6 * d:8 * d].t())


def test_sequence_parallel_slices_host():
    """Rank r's runs are positions [r S/t, (r+1) S/t) of every sequence; a
    sequence length that t does not divide is refused (host-only)."""
    from megatron_tensor_transformer_colwise_amd import inputs

    case = inputs.BlockCase("sp_host", batch=3, seq=8, hidden=16, heads=4, kv_heads=2, head_dim=128,
                            inter=32, t=4, rope_base=500000.0, seed=1)
    w = {k: v.torch() for k, v in inputs.gen_block(case).items()}
    blk = shard.BlockShards(w["X"], w, case)
    assert blk.sp_slices()[1] == [(2, 2), (10, 2), (18, 2)]
    blk2 = shard.BlockShards(w["X"], w, inputs.BlockCase("sp_host2", batch=1, seq=6, hidden=16, heads=4,
                                                         kv_heads=2, head_dim=128, inter=32, t=4,
                                                         rope_base=500000.0, seed=1))
    with pytest.raises(ValueError):
        blk2.sp_slices()


def test_rowwise_split_input_validation(L):
    f = lambda t, r, k=64, n=16, x=A16, w=A16, o=A16 + 8192, dt=1: status(  # noqa: E731
        "tp_rowwise_split_input", dt, 4, k, n, t, r, x, w, o, None)
    assert f(0, 0) == tp.TP_ERR_SHAPE
    assert f(17, 0) == tp.TP_ERR_SHAPE
    assert f(4, 4) == tp.TP_ERR_SHAPE and "rank = 4" in tp.tp_last_error()
    assert f(4, -1) == tp.TP_ERR_SHAPE
    assert f(3, 0, k=64) == tp.TP_ERR_SHAPE      # 64 / 3 is not whole
    assert f(4, 0, k=48) == tp.TP_ERR_SHAPE      # 48 / 4 = 12: not a multiple of 8
    assert f(4, 0, x=MIS) == tp.TP_ERR_INVALID_ARG
    assert f(4, 0, dt=5) == tp.TP_ERR_INVALID_ARG
    assert status("tp_rowwise_split_input", 1, 0, 64, 16, 4, 0, None, None, None, None) == tp.TP_OK


def test_bias_pointer_checked(L):
    assert status("tp_colwise", 1, 1, 4, 16, 16, A16, A16, MIS, A16, None) == tp.TP_ERR_INVALID_ARG
    assert "bias" in tp.tp_last_error()


def test_packed_weight_slices_match_oracle_indices():
    """The packed-weight helpers take exactly the oracle's per-rank indices of
    every block (host-only), and refuse blocks t does not divide."""
    import numpy as np

    import oracle

    w = torch.arange(36 * 5, dtype=torch.float32).reshape(36, 5)
    for t in (1, 2, 4):
        for r in range(t):
            rows = shard.packed_colwise_weight(w, [1, 1, 1, 3, 3], t, r)
            idx = oracle.packed_rank_index(36, [1, 1, 1, 3, 3], t, r)
            assert torch.equal(rows, w[torch.from_numpy(idx)])
    wo = torch.arange(5 * 16, dtype=torch.float32).reshape(5, 16)
    a, b = shard.packed_rowwise_weights(wo, [1, 3], 2, 1)
    idx = oracle.packed_rank_index(16, [1, 3], 2, 1)
    assert torch.equal(torch.cat([a, b], dim=1), wo[:, torch.from_numpy(idx)])
    with pytest.raises(ValueError):
        shard.packed_colwise_weight(w, [1, 1, 1, 3, 3], 8, 0)   # blocks of 4 rows are not divisible by 8
    assert np.array_equal(oracle.packed_rank_index(36, [1, 1, 1, 3, 3], 2, 0)[:2], [0, 1])


def test_vocab_parallel_validation(L):
    assert status("tp_embedding", 4, 12, 0, 10, A16, A16, A16, 16, None) == tp.TP_ERR_SHAPE     # w not x8
    assert status("tp_embedding", 4, 16, 0, 10, A16, A16, A16, 8, None) == tp.TP_ERR_SHAPE      # ld < w
    assert status("tp_embedding", 4, 16, -1, 10, A16, A16, A16, 16, None) == tp.TP_ERR_SHAPE
    assert status("tp_embedding", 4, 16, 0, 10, MIS, A16, A16, 16, None) == tp.TP_ERR_INVALID_ARG
    assert status("tp_embedding", 0, 16, 0, 10, None, None, None, 16, None) == tp.TP_OK
    assert status("tp_vocab_logits", 4, 16, 12, A16, A16, A16, None) == tp.TP_ERR_SHAPE           # v_shard not x8
    assert status("tp_ce_stats", 4, 12, 0, A16, A16, A16, None) == tp.TP_ERR_SHAPE
    assert status("tp_ce_stats", 4, 16, 0, A16, None, A16, None) == tp.TP_ERR_INVALID_ARG
    arr = (ctypes.c_void_p * 2)(A16, MIS)
    assert status("tp_ce_combine", 0, 4, 16, arr, A16, A16, None, None) == tp.TP_ERR_SHAPE
    assert status("tp_ce_combine", 2, 4, 0, arr, A16, A16, None, None) == tp.TP_ERR_SHAPE
    assert status("tp_ce_combine", 2, 4, 16, arr, A16, A16, None, None) == tp.TP_ERR_INVALID_ARG
    assert "stats[1]" in tp.tp_last_error()


def test_mlp_backward_validation(L):
    ws = tp.tp_shard_mlp_backward_workspace_bytes("gelu", 16, 16, 32)
    assert ws > 0
    args = lambda act, m, wsb=ws, x=A16: status(  # noqa: E731
        "tp_shard_mlp_backward", act, m, 16, 32, x, A16, A16, A16, None, None, None, A16, wsb, A16, A16, A16, None)
    assert args(0, 16) == tp.TP_ERR_INVALID_ARG          # needs an activation
    assert args(1, 12) == tp.TP_ERR_SHAPE                # m not a multiple of 8
    assert args(1, 16, wsb=ws - 1) == tp.TP_ERR_WORKSPACE
    assert args(1, 16, x=MIS) == tp.TP_ERR_INVALID_ARG
    assert status("tp_shard_mlp_backward", 1, 16, 16, 32, A16, A16, A16, A16, None, None, MIS, A16, ws, A16, A16,
                  A16, None) == tp.TP_ERR_INVALID_ARG                                 # misaligned saved pre
    save = lambda act, n=16, pre=A16 + 8192, y=A16 + 4096: status(  # noqa: E731
        "tp_colwise_save", act, 4, 16, n, A16, A16 + 12288, None, y, pre, None)
    assert save(0) == tp.TP_ERR_INVALID_ARG                                           # needs a nonlinearity
    assert save(1, pre=None) == tp.TP_ERR_INVALID_ARG
    assert save(2, pre=A16 + 4096) == tp.TP_ERR_INVALID_ARG                          # pre aliases y
    assert save(1, n=12) == tp.TP_ERR_SHAPE
    assert status("tp_transpose", 4, 4, A16, A16, None) == tp.TP_ERR_INVALID_ARG    # in place
    # the k-major product: sizes, strides and dtype checked before any launch
    assert status("tp_gemm_kmajor", 9, 1, 16, 16, 16, A16, 16, A16, 16, A16, None) == tp.TP_ERR_INVALID_ARG
    assert status("tp_gemm_kmajor", tp.TP_F32, 1, 12, 16, 16, A16, 16, A16, 16, A16, None) == tp.TP_ERR_SHAPE
    assert status("tp_gemm_kmajor", tp.TP_F32, 1, 16, 16, 16, A16, 8, A16, 16, A16, None) == tp.TP_ERR_SHAPE  # ldx < m
    assert status("tp_gemm_kmajor", tp.TP_F32, 0, 16, 16, 24, A16, 16, A16, 16, A16, None) == tp.TP_ERR_SHAPE  # ldx < k
    assert status("tp_gemm_kmajor", tp.TP_F32, 0, 16, 16, 16, A16, 16, A16, 8, A16, None) == tp.TP_ERR_SHAPE   # ldw < n
    assert status("tp_gemm_kmajor", tp.TP_BF16, 1, 16, 16, 1 << 20, A16, 1 << 10, A16, 16, A16, None) == tp.TP_ERR_SHAPE
    assert status("tp_gemm_kmajor", tp.TP_F32, 1, 0, 16, 16, None, 16, None, 16, None, None) == tp.TP_OK
    assert status("tp_gemm_kmajor", tp.TP_F32, 1, 16, 16, 16, None, 16, A16, 16, A16, None) == tp.TP_ERR_INVALID_ARG
    assert status("tp_transpose", 0, 4, None, None, None) == tp.TP_OK
    assert status("tp_mlp_act_backward", 0, 4, 16, A16, A16, A16, None, None) == tp.TP_ERR_INVALID_ARG
    assert status("tp_mlp_act_backward", 1, 4, 12, A16, A16, A16, None, None) == tp.TP_ERR_SHAPE



def test_attention_backward_validation(L):
    ws = tp.tp_flash_attn_backward_workspace_bytes(2, 64, 4, 2, 128)
    assert ws > 0 and tp.tp_flash_attn_backward_workspace_bytes(2, 64, 4, 3, 128) == 0
    core = lambda d=128, rope=500000.0, ld=1024, wsb=ws, hq=4, hkv=2, q=A16: status(  # noqa: E731
        "tp_flash_attn_backward", 2, 64, hq, hkv, d, rope, 1, q, A16, A16, A16, A16, A16, A16, wsb, A16, ld, None)
    assert core(d=64) == tp.TP_ERR_UNSUPPORTED
    assert core(rope=0.5) == tp.TP_ERR_INVALID_ARG        # neither 0 nor > 1
    assert core(ld=1016) == tp.TP_ERR_SHAPE               # < (hq + 2 hkv) d
    assert core(ld=1028) == tp.TP_ERR_SHAPE               # not a multiple of 8
    assert core(hq=4, hkv=3) == tp.TP_ERR_SHAPE
    assert core(wsb=ws - 1) == tp.TP_ERR_WORKSPACE
    assert core(q=MIS) == tp.TP_ERR_INVALID_ARG
    assert status("tp_flash_attn_lse", 2, 64, 4, 2, 128, 1, A16, A16, A16, A16, None, None) == tp.TP_ERR_INVALID_ARG
    sws = tp.tp_shard_attn_backward_workspace_bytes(2, 64, 256, 4, 2, 128)
    assert sws > ws
    shard_bwd = lambda seq=64, wsb=sws, rope=500000.0, x=A16: status(  # noqa: E731
        "tp_shard_attn_backward", 2, seq, 256, 4, 2, 128, rope, 1, x, A16, A16, A16, None, None, None, None, None,
        None, None, A16, wsb, A16, A16, A16, None)
    assert shard_bwd(seq=63) == tp.TP_ERR_SHAPE           # batch * seq not a multiple of 8
    assert shard_bwd(rope=0.0) == tp.TP_ERR_INVALID_ARG
    assert shard_bwd(wsb=sws - 1) == tp.TP_ERR_WORKSPACE
    assert shard_bwd(x=MIS) == tp.TP_ERR_INVALID_ARG
    assert status("tp_shard_attn_backward", 2, 64, 256, 4, 2, 128, 500000.0, 1, A16, A16, A16, A16, None, None,
                  A16, A16, None, A16, A16, A16, sws, A16, A16, A16, None) == tp.TP_ERR_INVALID_ARG  # vt missing
    assert status("tp_shard_attn_save", 2, 64, 256, 4, 2, 64, 500000.0, 1, A16, A16, A16, A16, A16, A16, A16, A16,
                  A16, None) == tp.TP_ERR_UNSUPPORTED
    assert status("tp_flash_attn_backward", 0, 64, 4, 2, 128, 0.0, 1, None, None, None, None, None, None, None, 0,
                  None, 1024, None) == tp.TP_OK


def test_norm_backward_validation(L):
    ws = tp.tp_shard_sum_rmsnorm_backward_workspace_bytes(16, 64)
    assert ws >= 16 * 64 * 4 or ws >= 64 * 4
    arr = (ctypes.c_void_p * 2)(A16, A16 + 4096)
    f = lambda t=2, m=16, h=64, x=A16 + 8192, xdt=1, eps=1e-5, res=None, rdt=0, dx=A16 + 12288, dxb=None, \
        dg=None, w=None, wsb=0: status(  # noqa: E731
        "tp_shard_sum_rmsnorm_backward", t, 1, m, m, h, arr, x, xdt, None, eps, res, rdt, dx, dxb, dg, w, wsb, None)
    assert f(t=0) == tp.TP_ERR_SHAPE
    assert f(t=17) == tp.TP_ERR_SHAPE
    assert f(h=60) == tp.TP_ERR_SHAPE
    assert f(h=8200) == tp.TP_ERR_SHAPE                       # wider than the register-held row
    assert f(xdt=7) == tp.TP_ERR_INVALID_ARG
    assert f(eps=-1.0) == tp.TP_ERR_INVALID_ARG
    assert f(dx=None) == tp.TP_ERR_INVALID_ARG                 # no output
    assert f(dx=A16) == tp.TP_ERR_INVALID_ARG                  # aliases a partial
    assert f(x=A16 + 12288) == tp.TP_ERR_INVALID_ARG           # output aliases x
    assert f(res=A16 + 12288, rdt=1) == tp.TP_ERR_INVALID_ARG  # bf16 residual overwritten
    assert f(dg=A16 + 16384, w=A16 + 20480, wsb=ws - 1) == tp.TP_ERR_WORKSPACE
    assert f(x=MIS) == tp.TP_ERR_INVALID_ARG
    assert f(m=0, x=None, dx=None) == tp.TP_OK
    assert status("tp_shard_sum_rmsnorm_backward", 2, 4, 8, 4, 64, arr, A16 + 8192, 1, None, 1e-5, None, 0,
                  A16 + 12288, None, None, None, 0, None) == tp.TP_ERR_SHAPE  # run_stride < run_rows
