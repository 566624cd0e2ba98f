"""Python binding of ``libtpshard.so`` (declared in ``include/tpshard.h``).

Argument marshalling only: every function here forwards to the C function of
the same name.  Tensor arguments may be torch tensors (their ``data_ptr()`` is
passed) or raw integer device addresses; ``stream`` defaults to torch's current
stream.  A non-OK status raises :class:`TpError` with the library's message.
There is no fallback: if the library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libtpshard.so"
HEADER = Path(__file__).resolve().parent.parent / "include" / "tpshard.h"

TP_OK = 0
TP_ERR_INVALID_ARG = 1
TP_ERR_SHAPE = 2
TP_ERR_WORKSPACE = 3
TP_ERR_UNSUPPORTED = 4
TP_ERR_HIP = 5
STATUS_NAMES = {0: "TP_OK", 1: "TP_ERR_INVALID_ARG", 2: "TP_ERR_SHAPE", 3: "TP_ERR_WORKSPACE",
                4: "TP_ERR_UNSUPPORTED", 5: "TP_ERR_HIP"}

TP_F32, TP_BF16 = 0, 1
TP_ACT_NONE, TP_ACT_GELU, TP_ACT_SWIGLU = 0, 1, 2
DTYPES = {"f32": TP_F32, "bf16": TP_BF16}
ACTS = {"none": TP_ACT_NONE, "gelu": TP_ACT_GELU, "swiglu": TP_ACT_SWIGLU}
TP_MAX_SHARDS = 16


class TpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_lib = None

_i64, _i32, _f32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
_SIGS = {
    "tp_colwise": [_i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp],
    "tp_rowwise": [_i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp],
    "tp_rowwise_split_input": [_i32, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp],
    "tp_shard_mlp": [_i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp],
    "tp_shard_mlp_group": [_i32, _i32, _i32, _i64, _i64, _i64, _vp, ctypes.POINTER(_vp),
                           ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp],
    "tp_qkv_rope": [_i64, _i64, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "tp_flash_attn": [_i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp],
    "tp_shard_attn_workspace_bytes": [_i64, _i64, _i32, _i32, _i32],
    "tp_shard_attn": [_i32, _i64, _i64, _i64, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp,
                      ctypes.c_size_t, _vp, _vp],
    "tp_shard_attn_noalloc": [_i32, _i64, _i64, _i64, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _vp],
    "tp_shard_sum": [_i32, _i64, ctypes.POINTER(_vp), _vp, _i32, _vp, _vp],
    "tp_rmsnorm": [_i32, _i64, _i64, _vp, _vp, _f32, _vp, _vp],
    "tp_shard_sum_rmsnorm": [_i32, _i64, _i64, _i64, _i64, ctypes.POINTER(_vp), _vp, _vp, _i32, _vp, _vp,
                             _f32, _vp, _vp],
    "tp_gemm_plan": [_i64, _i64, _i64, _i32] + [ctypes.POINTER(_i32)] * 4,
    "tp_flash_attn_plan": [_i64, _i64, _i32, _i32, ctypes.POINTER(_i32)],
    "tp_embedding": [_i64, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp],
    "tp_shard_mlp_backward_workspace_bytes": [_i32, _i64, _i64, _i64],
    "tp_shard_mlp_backward": [_i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                              _vp, _vp, _vp, _vp],
    "tp_colwise_save": [_i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp],
    "tp_transpose": [_i64, _i64, _vp, _vp, _vp],
    "tp_gemm_kmajor": [_i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp],
    "tp_mlp_act_backward": [_i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp],
    "tp_shard_sum_rmsnorm_backward_workspace_bytes": [_i64, _i64],
    "tp_shard_sum_rmsnorm_backward": [_i32, _i64, _i64, _i64, _i64, ctypes.POINTER(_vp), _vp, _i32, _vp, _f32, _vp,
                                      _i32, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp],
    "tp_flash_attn_lse": [_i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp],
    "tp_flash_attn_backward_workspace_bytes": [_i64, _i64, _i32, _i32, _i32],
    "tp_flash_attn_backward": [_i64, _i64, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               ctypes.c_size_t, _vp, _i64, _vp],
    "tp_shard_attn_backward_workspace_bytes": [_i64, _i64, _i64, _i32, _i32, _i32],
    "tp_shard_attn_backward": [_i64, _i64, _i64, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp, _vp, _vp, _vp],
    "tp_shard_attn_save": [_i64, _i64, _i64, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           _vp, _vp],
    "tp_vocab_logits": [_i64, _i64, _i64, _vp, _vp, _vp, _vp],
    "tp_ce_stats": [_i64, _i64, _i64, _vp, _vp, _vp, _vp],
    "tp_ce_combine": [_i32, _i64, _i64, ctypes.POINTER(_vp), _vp, _vp, _vp, _vp],
    "tp_last_error": [],
    "tp_device_check": [],
}


def lib() -> ctypes.CDLL:
    """Loads ``libtpshard.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(str(LIB_PATH))
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.tp_last_error.restype = ctypes.c_char_p
        L.tp_shard_attn_workspace_bytes.restype = ctypes.c_size_t
        L.tp_shard_mlp_backward_workspace_bytes.restype = ctypes.c_size_t
        L.tp_flash_attn_backward_workspace_bytes.restype = ctypes.c_size_t
        L.tp_shard_sum_rmsnorm_backward_workspace_bytes.restype = ctypes.c_size_t
        L.tp_shard_attn_backward_workspace_bytes.restype = ctypes.c_size_t
        _lib = L
    return _lib


def header_exports() -> list[str]:
    """Function names declared in include/tpshard.h."""
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_0-9]+)\s*\(", text)))


def _p(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _s(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _e(v, table):
    return table[v] if isinstance(v, str) else int(v)


def _check(status: int) -> None:
    if status != TP_OK:
        raise TpError(status, lib().tp_last_error().decode())


def tp_last_error() -> str:
    return lib().tp_last_error().decode()


_PLAN_KIND = {"rowwise": 0, "colwise": 1, "swiglu": 2, "qkv": 3}


def tp_gemm_plan(m, n, k=64, kind="rowwise") -> tuple[int, int, int, int]:
    """(bm_main, split, bm_tail, split_k) of the bf16 GEMM for an m x n output
    over depth k; kind is "rowwise", "colwise", "swiglu" or "qkv"."""
    a, b, c, d = _i32(), _i32(), _i32(), _i32()
    _check(lib().tp_gemm_plan(m, n, k, _PLAN_KIND[kind], ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                              ctypes.byref(d)))
    return a.value, b.value, c.value, d.value


def tp_flash_attn_plan(batch, seq, hq, causal=True) -> int:
    """Pieces each pair of query blocks is cut into by the flash attention."""
    p = _i32()
    _check(lib().tp_flash_attn_plan(batch, seq, hq, 1 if causal else 0, ctypes.byref(p)))
    return p.value


def tp_device_check() -> None:
    _check(lib().tp_device_check())


def tp_colwise(act, dt, m, k, n, x, w, y, stream=None, bias=None) -> None:
    _check(lib().tp_colwise(_e(act, ACTS), _e(dt, DTYPES), m, k, n, _p(x), _p(w), _p(bias), _p(y),
                            _s(stream)))


def tp_rowwise(dt, m, k, n, y, w, partial, stream=None) -> None:
    _check(lib().tp_rowwise(_e(dt, DTYPES), m, k, n, _p(y), _p(w), _p(partial), _s(stream)))


def tp_rowwise_split_input(dt, m, k, n, t, rank, x, w, partial, stream=None) -> None:
    _check(lib().tp_rowwise_split_input(_e(dt, DTYPES), m, k, n, t, rank, _p(x), _p(w), _p(partial),
                                        _s(stream)))


def tp_shard_mlp(act, dt, m, h, f_shard, x, w_in, w_out, act_ws, partial, stream=None) -> None:
    _check(lib().tp_shard_mlp(_e(act, ACTS), _e(dt, DTYPES), m, h, f_shard, _p(x), _p(w_in),
                              _p(w_out), _p(act_ws), _p(partial), _s(stream)))


def _arr(ptrs):
    return (_vp * max(len(ptrs), 1))(*[_p(q) for q in ptrs])


def tp_shard_mlp_group(act, dt, t, m, h, f_shard, x, w_in, w_out, act_ws, partial, stream=None) -> None:
    _check(lib().tp_shard_mlp_group(_e(act, ACTS), _e(dt, DTYPES), t, m, h, f_shard, _p(x),
                                    _arr(w_in), _arr(w_out), _arr(act_ws), _arr(partial), _s(stream)))


def tp_qkv_rope(batch, seq, h, hq, hkv, head_dim, rope_base, x, w_qkv, q, k, vt, stream=None,
                bias=None) -> None:
    _check(lib().tp_qkv_rope(batch, seq, h, hq, hkv, head_dim, rope_base, _p(x), _p(w_qkv), _p(bias),
                             _p(q), _p(k), _p(vt), _s(stream)))


def tp_flash_attn(batch, seq, hq, hkv, head_dim, causal, q, k, vt, o, stream=None) -> None:
    _check(lib().tp_flash_attn(batch, seq, hq, hkv, head_dim, int(causal), _p(q), _p(k), _p(vt),
                               _p(o), _s(stream)))


def tp_shard_attn_workspace_bytes(batch, seq, hq, hkv, head_dim) -> int:
    return int(lib().tp_shard_attn_workspace_bytes(batch, seq, hq, hkv, head_dim))


def tp_shard_attn(dt, batch, seq, h, hq, hkv, head_dim, rope_base, causal, x, w_qkv, w_o, ws, ws_bytes,
                  partial, stream=None) -> None:
    _check(lib().tp_shard_attn(_e(dt, DTYPES), batch, seq, h, hq, hkv, head_dim, rope_base, int(causal), _p(x),
                               _p(w_qkv), _p(w_o), _p(ws), ws_bytes, _p(partial), _s(stream)))


def tp_shard_attn_noalloc(dt, batch, seq, h, hq, hkv, head_dim, rope_base, causal, x, w_qkv, w_o, partial,
                          stream=None) -> None:
    _check(lib().tp_shard_attn_noalloc(_e(dt, DTYPES), batch, seq, h, hq, hkv, head_dim, rope_base, int(causal),
                                       _p(x), _p(w_qkv), _p(w_o), _p(partial), _s(stream)))


def tp_shard_sum(t, n, partials, residual, residual_dt, out, stream=None) -> None:
    arr = (_vp * max(len(partials), 1))(*[_p(p) for p in partials])
    _check(lib().tp_shard_sum(t, n, arr, _p(residual), _e(residual_dt, DTYPES), _p(out), _s(stream)))


def tp_rmsnorm(in_dt, m, h, x, gain, eps, y, stream=None) -> None:
    _check(lib().tp_rmsnorm(_e(in_dt, DTYPES), m, h, _p(x), _p(gain), eps, _p(y), _s(stream)))


def tp_shard_sum_rmsnorm(t, m, h, partials, residual, residual_dt, out, gain, eps, y, stream=None,
                         runs=None, bias=None) -> None:
    """m rows (one run), or ``runs = (nrun, run_rows, run_stride)``."""
    nrun, run_rows, run_stride = runs if runs is not None else (1, m, m)
    arr = (_vp * max(len(partials), 1))(*[_p(p) for p in partials])
    _check(lib().tp_shard_sum_rmsnorm(t, nrun, run_rows, run_stride, h, arr, _p(bias), _p(residual),
                                      _e(residual_dt, DTYPES), _p(out), _p(gain), eps, _p(y), _s(stream)))


def tp_shard_sum_rmsnorm_backward_workspace_bytes(m, h) -> int:
    return int(lib().tp_shard_sum_rmsnorm_backward_workspace_bytes(m, h))


def tp_shard_sum_rmsnorm_backward(t, m, h, partials, x, x_dt, gain, eps, residual_grad, residual_dt, dx, dx_bf16,
                                  dgain, ws, ws_bytes, stream=None, runs=None) -> None:
    """m rows (one run), or ``runs = (nrun, run_rows, run_stride)``."""
    nrun, run_rows, run_stride = runs if runs is not None else (1, m, m)
    arr = (_vp * max(len(partials), 1))(*[_p(p) for p in partials])
    _check(lib().tp_shard_sum_rmsnorm_backward(t, nrun, run_rows, run_stride, h, arr, _p(x), _e(x_dt, DTYPES),
                                               _p(gain), eps, _p(residual_grad), _e(residual_dt, DTYPES), _p(dx),
                                               _p(dx_bf16), _p(dgain), _p(ws), ws_bytes, _s(stream)))


def tp_embedding(m, w, v_start, v_rows, ids, table, out, ld, stream=None) -> None:
    _check(lib().tp_embedding(m, w, v_start, v_rows, _p(ids), _p(table), _p(out), ld, _s(stream)))


def tp_vocab_logits(m, h, v_shard, x, w, logits, stream=None) -> None:
    _check(lib().tp_vocab_logits(m, h, v_shard, _p(x), _p(w), _p(logits), _s(stream)))


def tp_ce_stats(m, v_shard, v_start, logits, labels, stats, stream=None) -> None:
    _check(lib().tp_ce_stats(m, v_shard, v_start, _p(logits), _p(labels), _p(stats), _s(stream)))


def tp_ce_combine(t, m, v, stats, labels, loss, mean, stream=None) -> None:
    arr = (_vp * max(len(stats), 1))(*[_p(p) for p in stats])
    _check(lib().tp_ce_combine(t, m, v, arr, _p(labels), _p(loss), _p(mean), _s(stream)))


def tp_shard_mlp_backward_workspace_bytes(act, m, h, f_shard) -> int:
    return int(lib().tp_shard_mlp_backward_workspace_bytes(_e(act, ACTS), m, h, f_shard))


def tp_shard_mlp_backward(act, m, h, f_shard, x, w_in, w_out, dz, xt, dzt, ws, ws_bytes, dx_partial, dw_in,
                          dw_out, stream=None, pre=None) -> None:
    _check(lib().tp_shard_mlp_backward(_e(act, ACTS), m, h, f_shard, _p(x), _p(w_in), _p(w_out), _p(dz), _p(xt),
                                       _p(dzt), _p(pre), _p(ws), ws_bytes, _p(dx_partial), _p(dw_in), _p(dw_out),
                                       _s(stream)))


def tp_colwise_save(act, m, k, n, x, w, y, pre, stream=None, bias=None) -> None:
    _check(lib().tp_colwise_save(_e(act, ACTS), m, k, n, _p(x), _p(w), _p(bias), _p(y), _p(pre), _s(stream)))


def tp_flash_attn_lse(batch, seq, hq, hkv, head_dim, causal, q, k, vt, o, lse, stream=None) -> None:
    _check(lib().tp_flash_attn_lse(batch, seq, hq, hkv, head_dim, int(causal), _p(q), _p(k), _p(vt), _p(o),
                                   _p(lse), _s(stream)))


def tp_flash_attn_backward_workspace_bytes(batch, seq, hq, hkv, head_dim) -> int:
    return int(lib().tp_flash_attn_backward_workspace_bytes(batch, seq, hq, hkv, head_dim))


def tp_flash_attn_backward(batch, seq, hq, hkv, head_dim, rope_base, causal, q, k, vt, o, lse, dout, ws, ws_bytes,
                           dqkv, ld, stream=None) -> None:
    _check(lib().tp_flash_attn_backward(batch, seq, hq, hkv, head_dim, rope_base, int(causal), _p(q), _p(k), _p(vt),
                                        _p(o), _p(lse), _p(dout), _p(ws), ws_bytes, _p(dqkv), ld, _s(stream)))


def tp_shard_attn_backward_workspace_bytes(batch, seq, h, hq, hkv, head_dim) -> int:
    return int(lib().tp_shard_attn_backward_workspace_bytes(batch, seq, h, hq, hkv, head_dim))


def tp_shard_attn_backward(batch, seq, h, hq, hkv, head_dim, rope_base, causal, x, w_qkv, w_o, dz, xt, dzt, ws,
                           ws_bytes, dx_partial, dw_qkv, dw_o, stream=None, saved=None) -> None:
    """``saved``: (q, k, vt, o, lse) from tp_shard_attn_save, or None (recompute)."""
    sq, sk, svt, so, slse = saved if saved is not None else (None,) * 5
    _check(lib().tp_shard_attn_backward(batch, seq, h, hq, hkv, head_dim, rope_base, int(causal), _p(x), _p(w_qkv),
                                        _p(w_o), _p(dz), _p(xt), _p(dzt), _p(sq), _p(sk), _p(svt), _p(so),
                                        _p(slse), _p(ws), ws_bytes, _p(dx_partial), _p(dw_qkv), _p(dw_o),
                                        _s(stream)))


def tp_shard_attn_save(batch, seq, h, hq, hkv, head_dim, rope_base, causal, x, w_qkv, w_o, q, k, vt, o, lse,
                       partial, stream=None) -> None:
    _check(lib().tp_shard_attn_save(batch, seq, h, hq, hkv, head_dim, rope_base, int(causal), _p(x), _p(w_qkv),
                                    _p(w_o), _p(q), _p(k), _p(vt), _p(o), _p(lse), _p(partial), _s(stream)))


def tp_transpose(rows, cols, src, dst, stream=None) -> None:
    _check(lib().tp_transpose(rows, cols, _p(src), _p(dst), _s(stream)))


def tp_gemm_kmajor(out_dt, x_kmajor, m, n, k, x, ldx, w, ldw, out, stream=None) -> None:
    _check(lib().tp_gemm_kmajor(_e(out_dt, DTYPES), int(bool(x_kmajor)), m, n, k, _p(x), ldx, _p(w), ldw, _p(out),
                                _s(stream)))


def tp_mlp_act_backward(act, m, n, pre, dy, dpre, y, stream=None) -> None:
    _check(lib().tp_mlp_act_backward(_e(act, ACTS), m, n, _p(pre), _p(dy), _p(dpre), _p(y), _s(stream)))

