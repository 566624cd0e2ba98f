// C ABI of libtpshard: argument validation, then kernel launches on the
// caller's stream.  Every check runs on the host before anything is enqueued;
// failures return a status and leave a message for tp_last_error().
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kernels.h"
#include "tpshard.h"

static_assert(TP_STATIC_SCRATCH_BYTES == tpk::kStaticScratchBytes, "static scratch size differs from the header");

namespace {

thread_local char g_err[512] = "";

tp_status fail(tp_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

tp_status ok() {
  g_err[0] = '\0';
  return TP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

const int64_t kMaxOffset = (int64_t)1 << 31;  // buffer offsets are 32-bit, signed headroom

tp_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(TP_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(TP_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return TP_OK;
}

#define TRY(expr)                      \
  do {                                 \
    tp_status _s = (expr);             \
    if (_s != TP_OK) return _s;        \
  } while (0)

tp_status check_dim8(int64_t v, const char* name) {
  if (v <= 0 || (v & 7)) return fail(TP_ERR_SHAPE, "%s = %lld must be a positive multiple of 8", name, (long long)v);
  return TP_OK;
}

// Device check, cached per device id.
std::mutex g_dev_mu;
int g_dev_ok[64];  // 0 unknown, 1 gfx950, 2 other

tp_status device_check() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(TP_ERR_UNSUPPORTED, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(TP_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_dev_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    if (g_dev_ok[dev] == 2)
      return fail(TP_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev, prop.gcnArchName);
  }
  if (g_dev_ok[dev] != 1) return fail(TP_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return TP_OK;
}

tp_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TP_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int64_t seq_pad_of(int64_t seq) { return (seq + 63) / 64 * 64; }

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

struct AttnLayout {
  size_t q, k, vt, o, total;
};

AttnLayout attn_layout(int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t d) {
  const size_t m = (size_t)batch * (size_t)seq;
  AttnLayout L;
  L.q = 0;
  L.k = L.q + align256(m * hq * d * 2);
  L.vt = L.k + align256(m * hkv * d * 2);
  L.o = L.vt + align256((size_t)batch * hkv * d * (size_t)seq_pad_of(seq) * 2);
  L.total = L.o + align256(m * hq * d * 2);
  return L;
}

// Heads of a KV group one dK/dV workgroup of the attention backward walks:
// the whole group when that already gives the chip 512 workgroups, else the
// group is split (the smallest divisor of its size reaching 512, or all of
// them); each split adds a float32 partial of dK and dV summed afterwards.
int attn_bwd_nsplit(int64_t batch, int64_t seq, int32_t hq, int32_t hkv) {
  const int gs = hq / hkv;
  const int64_t base = batch * hkv * ((seq + 127) / 128);
  int n = 1;
  while (base * n < 512) {
    int m = n + 1;
    while (m <= gs && gs % m != 0) ++m;
    if (m > gs) break;
    n = m;
  }
  return n;
}

struct AttnBwdLayout {
  size_t dvec, kt, vtok, qt, dot, part, total;
};

AttnBwdLayout attn_bwd_layout(int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t d) {
  const size_t B = (size_t)batch, sp = (size_t)seq_pad_of(seq), D = (size_t)d;
  AttnBwdLayout L;
  L.dvec = 0;
  L.kt = L.dvec + align256(B * hq * sp * 4);
  L.vtok = L.kt + align256(B * hkv * D * sp * 2);
  L.qt = L.vtok + align256(B * hkv * sp * D * 2);
  L.dot = L.qt + align256(B * hq * D * sp * 2);
  L.part = L.dot + align256(B * hq * D * sp * 2);
  L.total = L.part + align256(B * hkv * (size_t)attn_bwd_nsplit(batch, seq, hq, hkv) * 2 * sp * D * 4);
  return L;
}

// Workspace of one rank's attention backward: the recomputed forward (Q, K,
// V^T, O and the log-sum-exp), dO and the packed dQKV, then the attention
// core's own.
struct AttnShardBwdLayout {
  size_t fwd, lse, dout, dqkv, core, total;
};

AttnShardBwdLayout attn_shard_bwd_layout(int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv,
                                         int32_t d) {
  const size_t M = (size_t)(batch * seq), QD = (size_t)hq * d, N = (size_t)(hq + 2 * hkv) * d;
  (void)h;
  AttnShardBwdLayout L;
  L.fwd = 0;
  L.lse = L.fwd + attn_layout(batch, seq, hq, hkv, d).total;
  L.dout = L.lse + align256((size_t)batch * hq * (size_t)seq_pad_of(seq) * 4);
  L.dqkv = L.dout + align256(M * QD * 2);
  L.core = L.dqkv + align256(M * N * 2);
  L.total = L.core + attn_bwd_layout(batch, seq, hq, hkv, d).total;
  return L;
}

// Workspace of one rank's MLP backward (F = f or 2 f rows of w_in).
struct MlpBwdLayout {
  size_t pre, wout_t, dy, dpre, y, win_t, y_t, dpre_t, xt, dzt, total;
};

MlpBwdLayout mlp_bwd_layout(tp_act act, int64_t m, int64_t h, int64_t f) {
  const size_t F = act == TP_ACT_SWIGLU ? 2 * (size_t)f : (size_t)f;
  const size_t M = (size_t)m, H = (size_t)h, Fs = (size_t)f;
  MlpBwdLayout L;
  L.pre = 0;
  L.wout_t = L.pre + align256(M * F * 2);
  L.dy = L.wout_t + align256(Fs * H * 2);
  L.dpre = L.dy + align256(M * Fs * 2);
  L.y = L.dpre + align256(M * F * 2);
  L.win_t = L.y + align256(M * Fs * 2);
  L.y_t = L.win_t + align256(H * F * 2);
  L.dpre_t = L.y_t + align256(Fs * M * 2);
  L.xt = L.dpre_t + align256(F * M * 2);
  L.dzt = L.xt + align256(H * M * 2);
  L.total = L.dzt + align256(H * M * 2);
  return L;
}

// Shared checks of one GEMM call: sizes, pointers, 32-bit offset ranges.
tp_status check_gemm(tp_act act, tp_dtype dt, int64_t m, int64_t k, int64_t n, const void* x,
                     const void* w, const void* out, const char* xn, const char* wn, const char* on) {
  if (dt != TP_F32 && dt != TP_BF16) return fail(TP_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (act != TP_ACT_NONE && act != TP_ACT_GELU && act != TP_ACT_SWIGLU)
    return fail(TP_ERR_INVALID_ARG, "unknown activation %d", (int)act);
  if (m < 0) return fail(TP_ERR_SHAPE, "m = %lld is negative", (long long)m);
  TRY(check_dim8(k, "k"));
  TRY(check_dim8(n, "n"));
  const int64_t esz = dt == TP_BF16 ? 2 : 4;
  const int64_t wrows = act == TP_ACT_SWIGLU ? 2 * n : n;
  if (dt == TP_BF16 && (wrows + 256) * k * esz >= kMaxOffset)
    return fail(TP_ERR_SHAPE, "weight of %lld x %lld exceeds the 2 GiB per-operand limit",
                (long long)wrows, (long long)k);
  if (dt == TP_BF16 && 256 * k * esz >= kMaxOffset) return fail(TP_ERR_SHAPE, "k = %lld too large", (long long)k);
  if (m == 0) return TP_OK;
  TRY(check_ptr(x, xn));
  TRY(check_ptr(w, wn));
  TRY(check_ptr(out, on));
  return TP_OK;
}

int epi_of(tp_act act) {
  switch (act) {
    case TP_ACT_GELU: return tpk::EPI_GELU;
    case TP_ACT_SWIGLU: return tpk::EPI_SWIGLU;
    default: return tpk::EPI_BF16;
  }
}

tp_status check_attn_shape(int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t d) {
  if (batch < 0 || seq < 0) return fail(TP_ERR_SHAPE, "batch and seq must be >= 0");
  if (d != 128) return fail(TP_ERR_UNSUPPORTED, "head_dim = %d; only 128 is built", d);
  if (hq <= 0 || hkv <= 0) return fail(TP_ERR_SHAPE, "hq = %d and hkv = %d must be positive", hq, hkv);
  if (hq % hkv) return fail(TP_ERR_SHAPE, "hq = %d is not a multiple of hkv = %d", hq, hkv);
  if (seq * (int64_t)hq * d * 2 >= kMaxOffset || seq * (int64_t)hkv * d * 2 >= kMaxOffset)
    return fail(TP_ERR_SHAPE, "one sequence of q or k exceeds 2 GiB");
  if ((int64_t)d * seq_pad_of(seq) * 2 >= kMaxOffset) return fail(TP_ERR_SHAPE, "seq too long");
  if (batch * seq * (int64_t)hq > ((int64_t)1 << 31)) return fail(TP_ERR_SHAPE, "too many query rows");
  return TP_OK;
}

}  // namespace

extern "C" {

const char* tp_last_error(void) { return g_err; }

tp_status tp_flash_attn_plan(int64_t batch, int64_t seq, int32_t hq, int32_t causal, int32_t* pieces) {
  if (batch < 0 || seq < 0 || hq < 1) return fail(TP_ERR_SHAPE, "batch and seq must be >= 0 and hq >= 1");
  if (!pieces) return fail(TP_ERR_INVALID_ARG, "NULL output pointer");
  *pieces = tpk::flash_attn_pieces(batch, seq, hq, causal ? 1 : 0);
  return ok();
}

tp_status tp_gemm_plan(int64_t m, int64_t n, int64_t k, int32_t kind, int32_t* bm_main, int32_t* split,
                       int32_t* bm_tail, int32_t* split_k) {
  if (m <= 0 || n <= 0 || k <= 0) return fail(TP_ERR_SHAPE, "m, n and k must be positive");
  if (kind < TP_PLAN_ROWWISE || kind > TP_PLAN_QKV) return fail(TP_ERR_INVALID_ARG, "unknown GEMM kind %d", (int)kind);
  if (!bm_main || !split || !bm_tail || !split_k) return fail(TP_ERR_INVALID_ARG, "NULL output pointer");
  int a, b, c, d;
  tpk::gemm_plan(m, n, k, kind, 1, &a, &b, &c, &d);
  *bm_main = a;
  *split = b;
  *bm_tail = c;
  *split_k = d;
  return ok();
}

tp_status tp_device_check(void) {
  TRY(device_check());
  return ok();
}

tp_status tp_colwise(tp_act act, tp_dtype dt, int64_t m, int64_t k, int64_t n, const void* x,
                     const void* w, const float* bias, void* y, void* stream) {
  TRY(check_gemm(act, dt, m, k, n, x, w, y, "x", "w", "y"));
  if (m == 0) return ok();
  if (bias) TRY(check_ptr(bias, "bias"));
  TRY(device_check());
  hipError_t e;
  if (dt == TP_BF16)
    e = tpk::launch_gemm_bf16(epi_of(act), m, n, k, x, w, y, nullptr, as_stream(stream), bias);
  else
    e = tpk::launch_gemm_f32(epi_of(act), m, n, k, static_cast<const float*>(x),
                             static_cast<const float*>(w), static_cast<float*>(y), as_stream(stream), bias);
  return launched(e, "tp_colwise");
}

tp_status tp_colwise_save(tp_act act, int64_t m, int64_t k, int64_t n, const void* x, const void* w,
                          const float* bias, void* y, void* pre, void* stream) {
  if (act != TP_ACT_GELU && act != TP_ACT_SWIGLU)
    return fail(TP_ERR_INVALID_ARG, "tp_colwise_save needs GELU or SWIGLU, got %d", (int)act);
  TRY(check_gemm(act, TP_BF16, m, k, n, x, w, y, "x", "w", "y"));
  if (m == 0) return ok();
  TRY(check_ptr(pre, "pre"));
  if (pre == y || pre == x) return fail(TP_ERR_INVALID_ARG, "pre aliases x or y");
  const int64_t pw = act == TP_ACT_SWIGLU ? 2 * n : n;
  if (m * pw * 2 >= ((int64_t)1 << 40)) return fail(TP_ERR_SHAPE, "pre too large");
  if (bias) TRY(check_ptr(bias, "bias"));
  TRY(device_check());
  return launched(tpk::launch_gemm_bf16(act == TP_ACT_SWIGLU ? tpk::EPI_SWIGLU_SAVE : tpk::EPI_GELU_SAVE, m, n, k,
                                        x, w, y, nullptr, as_stream(stream), bias, 0, pre),
                  "tp_colwise_save");
}

tp_status tp_rowwise(tp_dtype dt, int64_t m, int64_t k, int64_t n, const void* y, const void* w,
                     float* partial, void* stream) {
  TRY(check_gemm(TP_ACT_NONE, dt, m, k, n, y, w, partial, "y", "w", "partial"));
  if (m == 0) return ok();
  TRY(device_check());
  hipError_t e;
  if (dt == TP_BF16)
    e = tpk::launch_gemm_bf16(tpk::EPI_F32, m, n, k, y, w, partial, nullptr, as_stream(stream));
  else
    e = tpk::launch_gemm_f32(tpk::EPI_F32, m, n, k, static_cast<const float*>(y),
                             static_cast<const float*>(w), partial, as_stream(stream));
  return launched(e, "tp_rowwise");
}

tp_status tp_rowwise_split_input(tp_dtype dt, int64_t m, int64_t k, int64_t n, int32_t t, int32_t rank,
                                 const void* x, const void* w, float* partial, void* stream) {
  if (t < 1 || t > TP_MAX_SHARDS) return fail(TP_ERR_SHAPE, "t = %d outside 1..%d", t, TP_MAX_SHARDS);
  if (rank < 0 || rank >= t) return fail(TP_ERR_SHAPE, "rank = %d outside 0..%d", rank, t - 1);
  TRY(check_dim8(k, "k"));
  if (k % t != 0 || (k / t) % 8 != 0)
    return fail(TP_ERR_SHAPE, "k / t = %lld / %d must be a whole multiple of 8", (long long)k, t);
  const int64_t ks = k / t;
  TRY(check_gemm(TP_ACT_NONE, dt, m, ks, n, x, w, partial, "x", "w", "partial"));
  const int64_t esz = dt == TP_BF16 ? 2 : 4;
  if (dt == TP_BF16 && 256 * k * esz >= kMaxOffset) return fail(TP_ERR_SHAPE, "k = %lld too large", (long long)k);
  if (m == 0) return ok();
  TRY(device_check());
  const char* xs = static_cast<const char*>(x) + rank * ks * esz;  // the rank's input columns
  hipError_t e;
  if (dt == TP_BF16)
    e = tpk::launch_gemm_bf16(tpk::EPI_F32, m, n, ks, xs, w, partial, nullptr, as_stream(stream), nullptr, k);
  else
    e = tpk::launch_gemm_f32(tpk::EPI_F32, m, n, ks, reinterpret_cast<const float*>(xs),
                             static_cast<const float*>(w), partial, as_stream(stream), nullptr, k);
  return launched(e, "tp_rowwise_split_input");
}

tp_status tp_shard_mlp(tp_act act, tp_dtype dt, int64_t m, int64_t h, int64_t f_shard,
                       const void* x, const void* w_in, const void* w_out, void* act_ws,
                       float* partial, void* stream) {
  if (act != TP_ACT_GELU && act != TP_ACT_SWIGLU)
    return fail(TP_ERR_INVALID_ARG, "tp_shard_mlp needs GELU or SWIGLU, got %d", (int)act);
  TRY(check_gemm(act, dt, m, h, f_shard, x, w_in, act_ws, "x", "w_in", "act_ws"));
  TRY(check_gemm(TP_ACT_NONE, dt, m, f_shard, h, act_ws, w_out, partial, "act_ws", "w_out", "partial"));
  TRY(tp_colwise(act, dt, m, h, f_shard, x, w_in, nullptr, act_ws, stream));
  return tp_rowwise(dt, m, f_shard, h, act_ws, w_out, partial, stream);
}

tp_status tp_shard_mlp_group(tp_act act, tp_dtype dt, int32_t t, int64_t m, int64_t h,
                             int64_t f_shard, const void* x, const void* const* w_in,
                             const void* const* w_out, void* const* act_ws,
                             float* const* partial, void* stream) {
  if (act != TP_ACT_GELU && act != TP_ACT_SWIGLU)
    return fail(TP_ERR_INVALID_ARG, "tp_shard_mlp_group needs GELU or SWIGLU, got %d", (int)act);
  if (t < 1 || t > TP_MAX_SHARDS) return fail(TP_ERR_SHAPE, "t = %d outside 1..%d", t, TP_MAX_SHARDS);
  if (m > 0 && (!w_in || !w_out || !act_ws || !partial))
    return fail(TP_ERR_INVALID_ARG, "a pointer array is NULL");
  for (int i = 0; i < t && m > 0; ++i) {
    TRY(check_gemm(act, dt, m, h, f_shard, x, w_in[i], act_ws[i], "x", "w_in[i]", "act_ws[i]"));
    TRY(check_gemm(TP_ACT_NONE, dt, m, f_shard, h, act_ws[i], w_out[i], partial[i], "act_ws[i]",
                   "w_out[i]", "partial[i]"));
  }
  TRY(check_gemm(act, dt, m, h, f_shard, x, x, x, "x", "x", "x"));
  if (m == 0) return ok();
  if (dt == TP_F32) {
    for (int i = 0; i < t; ++i)
      TRY(tp_shard_mlp(act, dt, m, h, f_shard, x, w_in[i], w_out[i], act_ws[i], partial[i], stream));
    return ok();
  }
  TRY(device_check());
  const void* xs[TP_MAX_SHARDS];
  for (int i = 0; i < t; ++i) xs[i] = x;
  hipError_t e = tpk::launch_gemm_bf16_group(epi_of(act), t, m, f_shard, h, xs, w_in, act_ws, nullptr,
                                             as_stream(stream));
  if (e != hipSuccess) return launched(e, "tp_shard_mlp_group");
  e = tpk::launch_gemm_bf16_group(tpk::EPI_F32, t, m, h, f_shard, act_ws, w_out,
                                  reinterpret_cast<void* const*>(partial), nullptr, as_stream(stream));
  return launched(e, "tp_shard_mlp_group");
}

tp_status tp_qkv_rope(int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv,
                      int32_t head_dim, float rope_base, const void* x, const void* w_qkv,
                      const float* bias, void* q, void* k, void* vt, void* stream) {
  TRY(check_attn_shape(batch, seq, hq, hkv, head_dim));
  if (!(rope_base > 1.0f)) return fail(TP_ERR_INVALID_ARG, "rope_base must be > 1");
  const int64_t n = (int64_t)(hq + 2 * hkv) * head_dim;
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, batch * seq, h, n, x, w_qkv, q, "x", "w_qkv", "q"));
  const int64_t m = batch * seq;
  if (m == 0) return ok();
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(vt, "vt"));
  if (bias) TRY(check_ptr(bias, "bias"));
  TRY(device_check());
  tpk::QkvOut o;
  o.q = q;
  o.k = k;
  o.vt = vt;
  o.seq = seq;
  o.seq_pad = seq_pad_of(seq);
  o.hq = hq;
  o.hkv = hkv;
  o.log2_base = log2f(rope_base);
  return launched(tpk::launch_gemm_bf16(tpk::EPI_QKV, m, n, h, x, w_qkv, nullptr, &o, as_stream(stream), bias),
                  "tp_qkv_rope");
}

tp_status tp_flash_attn(int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim,
                        int32_t causal, const void* q, const void* k, const void* vt, void* o,
                        void* stream) {
  TRY(check_attn_shape(batch, seq, hq, hkv, head_dim));
  if (batch * seq == 0) return ok();
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(vt, "vt"));
  TRY(check_ptr(o, "o"));
  TRY(device_check());
  return launched(tpk::launch_flash_attn(batch, seq, seq_pad_of(seq), hq, hkv, causal, q, k, vt, o,
                                         as_stream(stream)),
                  "tp_flash_attn");
}

tp_status tp_flash_attn_lse(int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim,
                            int32_t causal, const void* q, const void* k, const void* vt, void* o, float* lse,
                            void* stream) {
  TRY(check_attn_shape(batch, seq, hq, hkv, head_dim));
  if (batch * seq == 0) return ok();
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(vt, "vt"));
  TRY(check_ptr(o, "o"));
  TRY(check_ptr(lse, "lse"));
  TRY(device_check());
  return launched(tpk::launch_flash_attn(batch, seq, seq_pad_of(seq), hq, hkv, causal, q, k, vt, o,
                                         as_stream(stream), lse),
                  "tp_flash_attn_lse");
}

size_t tp_flash_attn_backward_workspace_bytes(int64_t batch, int64_t seq, int32_t hq, int32_t hkv,
                                              int32_t head_dim) {
  if (batch < 0 || seq < 0 || hq <= 0 || hkv <= 0 || head_dim <= 0 || hq % hkv != 0) return 0;
  return attn_bwd_layout(batch, seq, hq, hkv, head_dim).total;
}

tp_status tp_flash_attn_backward(int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim,
                                 float rope_base, int32_t causal, const void* q, const void* k, const void* vt,
                                 const void* o, const float* lse, const void* dout, void* ws, size_t ws_bytes,
                                 void* dqkv, int64_t ld, void* stream) {
  TRY(check_attn_shape(batch, seq, hq, hkv, head_dim));
  if (!(rope_base == 0.0f || rope_base > 1.0f))
    return fail(TP_ERR_INVALID_ARG, "rope_base must be 0 (no rotation) or > 1");
  const int64_t n = (int64_t)(hq + 2 * hkv) * head_dim;
  if (ld < n || ld % 8 != 0)
    return fail(TP_ERR_SHAPE, "ld = %lld must be a multiple of 8 and >= (hq + 2 hkv) * head_dim = %lld",
                (long long)ld, (long long)n);
  if (seq * ld * 2 >= kMaxOffset) return fail(TP_ERR_SHAPE, "one sequence of dqkv exceeds 2 GiB");
  if (batch * (int64_t)hq > 65535) return fail(TP_ERR_SHAPE, "batch * hq must be at most 65535");
  if (batch * seq == 0) return ok();
  const void* ptrs[] = {q, k, vt, o, lse, dout, ws, dqkv};
  const char* names[] = {"q", "k", "vt", "o", "lse", "dout", "ws", "dqkv"};
  for (int i = 0; i < 8; ++i) TRY(check_ptr(ptrs[i], names[i]));
  const AttnBwdLayout L = attn_bwd_layout(batch, seq, hq, hkv, head_dim);
  if (ws_bytes < L.total) return fail(TP_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, L.total);
  TRY(device_check());
  hipStream_t s = as_stream(stream);
  char* w = static_cast<char*>(ws);
  const int64_t sp = seq_pad_of(seq), D = head_dim;
  hipError_t e;
#define TP_STEP(call, what) \
  if ((e = (call)) != hipSuccess) return launched(e, what);
  TP_STEP(tpk::launch_attn_dvec(batch, seq, sp, hq, o, dout, reinterpret_cast<float*>(w + L.dvec), s),
          "tp_flash_attn_backward (D)");
  // K^T and Q^T, dO^T per head, zero-padded to seq_pad; V token-major from V^T
  TP_STEP(tpk::launch_transpose_batched(batch, hkv, seq, sp, D, hkv * D, sp, seq * hkv * D, D, hkv * D * sp, D * sp,
                                        k, w + L.kt, s),
          "tp_flash_attn_backward (K^T)");
  TP_STEP(tpk::launch_transpose_batched(batch * hkv, 1, D, D, sp, sp, D, D * sp, 0, sp * D, 0, vt, w + L.vtok, s),
          "tp_flash_attn_backward (V)");
  TP_STEP(tpk::launch_transpose_batched(batch, hq, seq, sp, D, hq * D, sp, seq * hq * D, D, hq * D * sp, D * sp, q,
                                        w + L.qt, s),
          "tp_flash_attn_backward (Q^T)");
  TP_STEP(tpk::launch_transpose_batched(batch, hq, seq, sp, D, hq * D, sp, seq * hq * D, D, hq * D * sp, D * sp,
                                        dout, w + L.dot, s),
          "tp_flash_attn_backward (dO^T)");
  tpk::AttnBwdIn in;
  in.q = q;
  in.k = k;
  in.vtok = w + L.vtok;
  in.kt = w + L.kt;
  in.qt = w + L.qt;
  in.dout = dout;
  in.dot = w + L.dot;
  in.lse = lse;
  in.dvec = reinterpret_cast<const float*>(w + L.dvec);
  TP_STEP(tpk::launch_flash_attn_bwd(batch, seq, sp, hq, hkv, causal, rope_base > 0.0f ? log2((double)rope_base) : 0.0,
                                     in, reinterpret_cast<float*>(w + L.part), attn_bwd_nsplit(batch, seq, hq, hkv),
                                     dqkv, ld, s),
          "tp_flash_attn_backward");
#undef TP_STEP
  return ok();
}

size_t tp_shard_attn_backward_workspace_bytes(int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv,
                                              int32_t head_dim) {
  if (batch < 0 || seq < 0 || h <= 0 || hq <= 0 || hkv <= 0 || head_dim <= 0 || hq % hkv != 0) return 0;
  return attn_shard_bwd_layout(batch, seq, h, hq, hkv, head_dim).total;
}

tp_status tp_shard_attn_save(int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv, int32_t head_dim,
                             float rope_base, int32_t causal, const void* x, const void* w_qkv, const void* w_o,
                             void* q, void* k, void* vt, void* o, float* lse, float* partial, void* stream) {
  TRY(check_attn_shape(batch, seq, hq, hkv, head_dim));
  const int64_t m = batch * seq;
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, m, (int64_t)hq * head_dim, h, x, w_o, partial, "x", "w_o", "partial"));
  if (m == 0) return ok();
  TRY(tp_qkv_rope(batch, seq, h, hq, hkv, head_dim, rope_base, x, w_qkv, nullptr, q, k, vt, stream));
  TRY(tp_flash_attn_lse(batch, seq, hq, hkv, head_dim, causal, q, k, vt, o, lse, stream));
  return tp_rowwise(TP_BF16, m, (int64_t)hq * head_dim, h, o, w_o, partial, stream);
}

tp_status tp_shard_attn_backward(int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv, int32_t head_dim,
                                 float rope_base, int32_t causal, const void* x, const void* w_qkv, const void* w_o,
                                 const void* dz, const void* xt, const void* dzt, const void* saved_q,
                                 const void* saved_k, const void* saved_vt, const void* saved_o,
                                 const float* saved_lse, void* ws, size_t ws_bytes, float* dx_partial, float* dw_qkv,
                                 float* dw_o, void* stream) {
  TRY(check_attn_shape(batch, seq, hq, hkv, head_dim));
  if (!(rope_base > 1.0f)) return fail(TP_ERR_INVALID_ARG, "rope_base must be > 1");
  const int64_t m = batch * seq;
  if (m % 8 != 0)
    return fail(TP_ERR_SHAPE, "batch * seq = %lld must be a multiple of 8 (the weight gradients reduce over tokens)",
                (long long)m);
  const int64_t qd = (int64_t)hq * head_dim, n = (int64_t)(hq + 2 * hkv) * head_dim;
  // the forward's projection and the backward's five products, with their operand sizes
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, m, h, n, x, w_qkv, ws, "x", "w_qkv", "ws"));
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, m, h, qd, dz, ws, ws, "dz", "ws", "ws"));
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, m, n, h, ws, ws, dx_partial, "ws", "ws", "dx_partial"));
  if (m == 0) return ok();
  TRY(check_ptr(w_o, "w_o"));
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, h, m, qd, ws, ws, dw_o, "ws", "ws", "dw_o"));
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, n, m, h, ws, ws, dw_qkv, "ws", "ws", "dw_qkv"));
  (void)xt;  // the weight-gradient products read x and dz in place
  (void)dzt;
  if (m * std::max(h, n) * 2 >= kMaxOffset)
    return fail(TP_ERR_SHAPE, "batch * seq x %lld activations exceed 2 GiB", (long long)std::max(h, n));
  const void* sv[5] = {saved_q, saved_k, saved_vt, saved_o, saved_lse};
  const int nsaved = (saved_q != nullptr) + (saved_k != nullptr) + (saved_vt != nullptr) + (saved_o != nullptr) +
                     (saved_lse != nullptr);
  if (nsaved != 0 && nsaved != 5)
    return fail(TP_ERR_INVALID_ARG, "saved q, k, vt, o and lse come all together or not at all");
  for (int i = 0; i < nsaved; ++i) TRY(check_ptr(sv[i], "a saved activation"));
  const AttnShardBwdLayout L = attn_shard_bwd_layout(batch, seq, h, hq, hkv, head_dim);
  if (ws_bytes < L.total) return fail(TP_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, L.total);
  TRY(device_check());
  hipStream_t s = as_stream(stream);
  char* b = static_cast<char*>(ws);
  const AttnLayout F = attn_layout(batch, seq, hq, hkv, head_dim);
  char* f = b + L.fwd;
  auto km = [&](int epi, bool x_kmajor, int64_t M, int64_t N, int64_t K, const void* a, int64_t lda, const void* w,
                int64_t ldw, void* c) {
    return tpk::launch_gemm_bf16_km(epi, x_kmajor, M, N, K, a, lda, w, ldw, c, s);
  };
  hipError_t e;
#define TP_STEP(call, what) \
  if ((e = (call)) != hipSuccess) return launched(e, what);
  // the forward's saved Q, K, V^T (RoPE applied), O and log-sum-exp, or them recomputed
  const void* q = saved_q;
  const void* k = saved_k;
  const void* vt = saved_vt;
  const void* o = saved_o;
  const float* lse = saved_lse;
  if (!nsaved) {
    TRY(tp_qkv_rope(batch, seq, h, hq, hkv, head_dim, rope_base, x, w_qkv, nullptr, f + F.q, f + F.k, f + F.vt,
                    stream));
    TRY(tp_flash_attn_lse(batch, seq, hq, hkv, head_dim, causal, f + F.q, f + F.k, f + F.vt, f + F.o,
                          reinterpret_cast<float*>(b + L.lse), stream));
    q = f + F.q;
    k = f + F.k;
    vt = f + F.vt;
    o = f + F.o;
    lse = reinterpret_cast<const float*>(b + L.lse);
  }
  // dO = dZ W_o (W_o [h, hq d] read as the k-major operand)
  TP_STEP(km(tpk::EPI_BF16, false, m, qd, h, dz, h, w_o, qd, b + L.dout), "tp_shard_attn_backward (dO)");
  // the attention core: dQKV before RoPE, packed like the projection's output
  TRY(tp_flash_attn_backward(batch, seq, hq, hkv, head_dim, rope_base, causal, q, k, vt, o, lse, b + L.dout,
                             b + L.core, L.total - L.core, b + L.dqkv, n, stream));
  // dX partial = dQKV W_qkv (W_qkv [n, h] read k-major); f's backward sums these over ranks
  TP_STEP(km(tpk::EPI_F32, false, m, h, n, b + L.dqkv, n, w_qkv, h, dx_partial), "tp_shard_attn_backward (dX)");
  // dW_o = dZ^T O and dW_qkv = dQKV^T X, reducing over the tokens: both
  // operands read k-major (token rows) where they lie
  TP_STEP(km(tpk::EPI_F32, true, h, qd, m, dz, h, o, qd, dw_o), "tp_shard_attn_backward (dW_o)");
  TP_STEP(km(tpk::EPI_F32, true, n, h, m, b + L.dqkv, n, x, h, dw_qkv), "tp_shard_attn_backward (dW_qkv)");
#undef TP_STEP
  return ok();
}

size_t tp_shard_sum_rmsnorm_backward_workspace_bytes(int64_t m, int64_t h) {
  if (m <= 0 || h <= 0) return 0;
  return align256((size_t)tpk::norm_bwd_blocks(m) * (size_t)h * 4);
}

tp_status tp_shard_sum_rmsnorm_backward(int32_t t, int64_t nrun, int64_t run_rows, int64_t run_stride, int64_t h,
                                        const float* const* partials, const void* x, tp_dtype x_dt, const float* gain,
                                        float eps, const void* residual_grad, tp_dtype residual_dt, float* dx,
                                        void* dx_bf16, float* dgain, void* ws, size_t ws_bytes, void* stream) {
  if (t < 1 || t > TP_MAX_SHARDS) return fail(TP_ERR_SHAPE, "t = %d outside 1..%d", t, TP_MAX_SHARDS);
  if (nrun < 0 || run_rows < 0) return fail(TP_ERR_SHAPE, "nrun and run_rows must be >= 0");
  if (nrun > 1 && run_stride < run_rows)
    return fail(TP_ERR_SHAPE, "run_stride = %lld < run_rows = %lld", (long long)run_stride, (long long)run_rows);
  const int64_t m = nrun * run_rows;
  TRY(check_dim8(h, "h"));
  if (h > 8192) return fail(TP_ERR_SHAPE, "h = %lld: the norm backward keeps rows of at most 8192 in registers",
                            (long long)h);
  if (x_dt != TP_F32 && x_dt != TP_BF16) return fail(TP_ERR_INVALID_ARG, "unknown x dtype %d", (int)x_dt);
  if (residual_grad && residual_dt != TP_F32 && residual_dt != TP_BF16)
    return fail(TP_ERR_INVALID_ARG, "unknown residual dtype %d", (int)residual_dt);
  if (!(eps >= 0.0f) || eps > 1.0f) return fail(TP_ERR_INVALID_ARG, "eps must be in [0, 1]");
  if (m == 0) return ok();
  if (!partials) return fail(TP_ERR_INVALID_ARG, "partials is NULL");
  for (int i = 0; i < t; ++i) {
    char name[32];
    snprintf(name, sizeof name, "partials[%d]", i);
    TRY(check_ptr(partials[i], name));
    if (partials[i] == dx) return fail(TP_ERR_INVALID_ARG, "dx aliases %s", name);
  }
  TRY(check_ptr(x, "x"));
  if (!dx && !dx_bf16) return fail(TP_ERR_INVALID_ARG, "dx and dx_bf16 are both NULL");
  if (dx) TRY(check_ptr(dx, "dx"));
  if (dx_bf16) TRY(check_ptr(dx_bf16, "dx_bf16"));
  if (x == dx || x == dx_bf16) return fail(TP_ERR_INVALID_ARG, "an output aliases x");
  if (residual_grad) {
    TRY(check_ptr(residual_grad, "residual_grad"));
    if (residual_grad == dx_bf16 || (residual_grad == dx && residual_dt != TP_F32))
      return fail(TP_ERR_INVALID_ARG, "only a float32 residual_grad may be overwritten by dx");
  }
  if (gain) TRY(check_ptr(gain, "gain"));
  if (dgain) {
    TRY(check_ptr(dgain, "dgain"));
    TRY(check_ptr(ws, "ws"));
    const size_t need = tp_shard_sum_rmsnorm_backward_workspace_bytes(m, h);
    if (ws_bytes < need) return fail(TP_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  }
  TRY(device_check());
  return launched(tpk::launch_sum_rmsnorm_bwd(t, nrun, run_rows, run_stride, h, partials, x, x_dt == TP_BF16, gain,
                                              eps, residual_grad, residual_dt == TP_BF16, dx, dx_bf16, dgain,
                                              static_cast<float*>(ws), as_stream(stream)),
                  "tp_shard_sum_rmsnorm_backward");
}

size_t tp_shard_attn_workspace_bytes(int64_t batch, int64_t seq, int32_t hq, int32_t hkv,
                                     int32_t head_dim) {
  if (batch < 0 || seq < 0 || hq <= 0 || hkv <= 0 || head_dim <= 0) return 0;
  return attn_layout(batch, seq, hq, hkv, head_dim).total;
}

namespace {

// tp_shard_attn with the flash attention's split workspace given (NULL: the
// library's per-stream one).
tp_status shard_attn(int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv, int32_t head_dim,
                     float rope_base, int32_t causal, const void* x, const void* w_qkv, const void* w_o, void* ws,
                     size_t ws_bytes, float* partial, void* stream, const tpk::FaSplitWs* fws) {
  TRY(check_attn_shape(batch, seq, hq, hkv, head_dim));
  const int64_t m = batch * seq;
  const int64_t qd = (int64_t)hq * head_dim;
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, m, qd, h, x, w_o, partial, "x", "w_o", "partial"));
  const AttnLayout L = attn_layout(batch, seq, hq, hkv, head_dim);
  if (m == 0) return ok();
  TRY(check_ptr(ws, "ws"));
  if (ws_bytes < L.total)
    return fail(TP_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, L.total);
  char* base = static_cast<char*>(ws);
  TRY(tp_qkv_rope(batch, seq, h, hq, hkv, head_dim, rope_base, x, w_qkv, nullptr, base + L.q, base + L.k,
                  base + L.vt, stream));
  TRY(launched(tpk::launch_flash_attn(batch, seq, seq_pad_of(seq), hq, hkv, causal, base + L.q, base + L.k,
                                      base + L.vt, base + L.o, as_stream(stream), nullptr, fws),
               "tp_flash_attn"));
  return tp_rowwise(TP_BF16, m, qd, h, base + L.o, w_o, partial, stream);
}

}  // namespace

tp_status tp_shard_attn(tp_dtype dt, int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv,
                        int32_t head_dim, float rope_base, int32_t causal, const void* x,
                        const void* w_qkv, const void* w_o, void* ws, size_t ws_bytes,
                        float* partial, void* stream) {
  if (dt == TP_F32) return fail(TP_ERR_UNSUPPORTED, "tp_shard_attn: only bf16 attention is built");
  if (dt != TP_BF16) return fail(TP_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  return shard_attn(batch, seq, h, hq, hkv, head_dim, rope_base, causal, x, w_qkv, w_o, ws, ws_bytes, partial,
                    stream, nullptr);
}

tp_status tp_shard_attn_noalloc(tp_dtype dt, int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv,
                                int32_t head_dim, float rope_base, int32_t causal, const void* x,
                                const void* w_qkv, const void* w_o, float* partial, void* stream) {
  if (dt == TP_F32) return fail(TP_ERR_UNSUPPORTED, "tp_shard_attn_noalloc: only bf16 attention is built");
  if (dt != TP_BF16) return fail(TP_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  TRY(check_attn_shape(batch, seq, hq, hkv, head_dim));
  // the array: the split flags, then q, k, vt and o, then the split partials
  const size_t layout = attn_layout(batch, seq, hq, hkv, head_dim).total;
  const size_t split = tpk::flash_attn_split_bytes(batch, seq, hq, causal ? 1 : 0);
  const size_t need = tpk::kStaticFlagBytes + layout + split;
  if (need > tpk::kStaticScratchBytes)
    return fail(TP_ERR_WORKSPACE,
                "tp_shard_attn_noalloc: this shape needs %zu bytes of workspace, beyond the %zu-byte static "
                "scratch (use tp_shard_attn with a caller workspace)",
                need, tpk::kStaticScratchBytes);
  if (batch * seq == 0) return ok();
  TRY(device_check());
  void* base = nullptr;
  hipError_t e = tpk::static_scratch(&base);
  if (e != hipSuccess) return fail(TP_ERR_HIP, "static scratch address lookup failed: %s", hipGetErrorString(e));
  tpk::FaSplitWs fws;
  e = tpk::static_scratch_epoch(&fws.epoch);
  if (e != hipSuccess) return fail(TP_ERR_HIP, "static scratch epoch: %s", hipGetErrorString(e));
  char* const b = static_cast<char*>(base);
  fws.flag = reinterpret_cast<unsigned*>(b);
  char* const ws = b + tpk::kStaticFlagBytes;
  fws.part = reinterpret_cast<float*>(ws + layout);
  return shard_attn(batch, seq, h, hq, hkv, head_dim, rope_base, causal, x, w_qkv, w_o, ws, layout, partial,
                    stream, &fws);
}

tp_status tp_shard_sum(int32_t t, int64_t n, const float* const* partials, const void* residual,
                       tp_dtype residual_dt, float* out, void* stream) {
  if (t < 1 || t > TP_MAX_SHARDS) return fail(TP_ERR_SHAPE, "t = %d outside 1..%d", t, TP_MAX_SHARDS);
  if (n < 0) return fail(TP_ERR_SHAPE, "n = %lld is negative", (long long)n);
  if (residual && residual_dt != TP_F32 && residual_dt != TP_BF16)
    return fail(TP_ERR_INVALID_ARG, "unknown residual dtype %d", (int)residual_dt);
  if (n == 0) return ok();
  if (!partials) return fail(TP_ERR_INVALID_ARG, "partials is NULL");
  for (int i = 0; i < t; ++i) {
    char name[32];
    snprintf(name, sizeof(name), "partials[%d]", i);
    TRY(check_ptr(partials[i], name));
    if (partials[i] == out) return fail(TP_ERR_INVALID_ARG, "out aliases partials[%d]", i);
  }
  if (residual) {
    TRY(check_ptr(residual, "residual"));
    if (residual == out && residual_dt != TP_F32)
      return fail(TP_ERR_INVALID_ARG, "out may alias residual only for a float32 residual");
  }
  TRY(check_ptr(out, "out"));
  TRY(device_check());
  return launched(tpk::launch_shard_sum(t, n, partials, residual, residual_dt == TP_BF16, out,
                                        as_stream(stream)),
                  "tp_shard_sum");
}

tp_status tp_rmsnorm(tp_dtype in_dt, int64_t m, int64_t h, const void* x, const float* gain,
                     float eps, void* y, void* stream) {
  if (in_dt != TP_F32 && in_dt != TP_BF16) return fail(TP_ERR_INVALID_ARG, "unknown dtype %d", (int)in_dt);
  if (m < 0) return fail(TP_ERR_SHAPE, "m = %lld is negative", (long long)m);
  TRY(check_dim8(h, "h"));
  if (!(eps >= 0.0f)) return fail(TP_ERR_INVALID_ARG, "eps must be >= 0");
  if (m == 0) return ok();
  if (m > 0x7FFFFFFF) return fail(TP_ERR_SHAPE, "m too large");
  TRY(check_ptr(x, "x"));
  if (gain) TRY(check_ptr(gain, "gain"));
  TRY(check_ptr(y, "y"));
  TRY(device_check());
  return launched(tpk::launch_rmsnorm(in_dt == TP_BF16, m, h, x, gain, eps, y, as_stream(stream)),
                  "tp_rmsnorm");
}

tp_status tp_shard_sum_rmsnorm(int32_t t, int64_t nrun, int64_t run_rows, int64_t run_stride, int64_t h,
                               const float* const* partials, const float* bias, const void* residual,
                               tp_dtype residual_dt, float* out, const float* gain, float eps, void* y,
                               void* stream) {
  if (t < 0 || t > TP_MAX_SHARDS) return fail(TP_ERR_SHAPE, "t = %d outside 0..%d", t, TP_MAX_SHARDS);
  if (nrun < 0 || run_rows < 0)
    return fail(TP_ERR_SHAPE, "nrun = %lld, run_rows = %lld: negative", (long long)nrun, (long long)run_rows);
  if (nrun > 1 && run_stride < run_rows)
    return fail(TP_ERR_SHAPE, "run_stride = %lld is below run_rows = %lld", (long long)run_stride,
                (long long)run_rows);
  TRY(check_dim8(h, "h"));
  if (residual && residual_dt != TP_F32 && residual_dt != TP_BF16)
    return fail(TP_ERR_INVALID_ARG, "unknown residual dtype %d", (int)residual_dt);
  if (!(eps >= 0.0f)) return fail(TP_ERR_INVALID_ARG, "eps must be >= 0");
  if (t == 0 && !residual) return fail(TP_ERR_INVALID_ARG, "t = 0 needs a residual");
  if (t == 0 && bias) return fail(TP_ERR_INVALID_ARG, "a bias needs partials to follow");
  if (!out && !y) return fail(TP_ERR_INVALID_ARG, "out and y are both NULL");
  if (nrun == 0 || run_rows == 0) return ok();
  if (nrun > 0x7FFFFFFF / run_rows) return fail(TP_ERR_SHAPE, "nrun * run_rows too large");
  if (t > 0 && !partials) return fail(TP_ERR_INVALID_ARG, "partials is NULL");
  for (int i = 0; i < t; ++i) {
    char name[32];
    snprintf(name, sizeof(name), "partials[%d]", i);
    TRY(check_ptr(partials[i], name));
    if (out && partials[i] == out) return fail(TP_ERR_INVALID_ARG, "out aliases partials[%d]", i);
  }
  if (residual) {
    TRY(check_ptr(residual, "residual"));
    if (residual == out && residual_dt != TP_F32)
      return fail(TP_ERR_INVALID_ARG, "out may alias residual only for a float32 residual");
  }
  if (out) TRY(check_ptr(out, "out"));
  if (bias) TRY(check_ptr(bias, "bias"));
  if (gain) TRY(check_ptr(gain, "gain"));
  if (y) TRY(check_ptr(y, "y"));
  TRY(device_check());
  return launched(tpk::launch_sum_rmsnorm(t, nrun, run_rows, run_stride, h, partials, bias, residual,
                                          residual_dt == TP_BF16, out, gain, eps, y, as_stream(stream)),
                  "tp_shard_sum_rmsnorm");
}

tp_status tp_embedding(int64_t m, int64_t w, int64_t v_start, int64_t v_rows, const int32_t* ids,
                       const void* table, float* out, int64_t ld, void* stream) {
  if (m < 0) return fail(TP_ERR_SHAPE, "m = %lld is negative", (long long)m);
  TRY(check_dim8(w, "w"));
  if (v_start < 0 || v_rows < 0) return fail(TP_ERR_SHAPE, "v_start and v_rows must be >= 0");
  if (ld < w || ld % 8 != 0) return fail(TP_ERR_SHAPE, "ld = %lld must be >= w and a multiple of 8", (long long)ld);
  if (m == 0) return ok();
  if (m > 0x7FFFFFFF) return fail(TP_ERR_SHAPE, "m too large");
  TRY(check_ptr(ids, "ids"));
  if (v_rows > 0) TRY(check_ptr(table, "table"));
  TRY(check_ptr(out, "out"));
  TRY(device_check());
  return launched(tpk::launch_embedding(m, w, v_start, v_rows, ids, table, out, ld, as_stream(stream)),
                  "tp_embedding");
}

tp_status tp_vocab_logits(int64_t m, int64_t h, int64_t v_shard, const void* x, const void* w, float* logits,
                          void* stream) {
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, m, h, v_shard, x, w, logits, "x", "w", "logits"));
  if (m == 0) return ok();
  TRY(device_check());
  return launched(tpk::launch_gemm_bf16(tpk::EPI_F32, m, v_shard, h, x, w, logits, nullptr, as_stream(stream)),
                  "tp_vocab_logits");
}

tp_status tp_ce_stats(int64_t m, int64_t v_shard, int64_t v_start, const float* logits, const int32_t* labels,
                      float* stats, void* stream) {
  if (m < 0) return fail(TP_ERR_SHAPE, "m = %lld is negative", (long long)m);
  TRY(check_dim8(v_shard, "v_shard"));
  if (v_start < 0) return fail(TP_ERR_SHAPE, "v_start must be >= 0");
  if (m == 0) return ok();
  if (m > 0x7FFFFFFF) return fail(TP_ERR_SHAPE, "m too large");
  TRY(check_ptr(logits, "logits"));
  TRY(check_ptr(labels, "labels"));
  TRY(check_ptr(stats, "stats"));
  TRY(device_check());
  return launched(tpk::launch_ce_stats(m, v_shard, v_start, logits, labels, stats, as_stream(stream)),
                  "tp_ce_stats");
}

tp_status tp_ce_combine(int32_t t, int64_t m, int64_t v, const float* const* stats, const int32_t* labels,
                        float* loss, float* mean, void* stream) {
  if (t < 1 || t > TP_MAX_SHARDS) return fail(TP_ERR_SHAPE, "t = %d outside 1..%d", t, TP_MAX_SHARDS);
  if (m < 0) return fail(TP_ERR_SHAPE, "m = %lld is negative", (long long)m);
  if (v < 1) return fail(TP_ERR_SHAPE, "v = %lld must be >= 1", (long long)v);
  if (m == 0) return ok();
  if (!stats) return fail(TP_ERR_INVALID_ARG, "stats is NULL");
  for (int r = 0; r < t; ++r) {
    char name[32];
    snprintf(name, sizeof(name), "stats[%d]", r);
    TRY(check_ptr(stats[r], name));
  }
  TRY(check_ptr(labels, "labels"));
  TRY(check_ptr(loss, "loss"));
  if (mean) TRY(check_ptr(mean, "mean"));
  TRY(device_check());
  return launched(tpk::launch_ce_combine(t, m, stats, loss, labels, v, mean, as_stream(stream)), "tp_ce_combine");
}

tp_status tp_transpose(int64_t rows, int64_t cols, const void* src, void* dst, void* stream) {
  if (rows < 0 || cols < 0) return fail(TP_ERR_SHAPE, "rows and cols must be >= 0");
  if (rows == 0 || cols == 0) return ok();
  if (rows > (int64_t)65535 * 64 || cols > ((int64_t)1 << 31) * 64)
    return fail(TP_ERR_SHAPE, "rows = %lld too large", (long long)rows);
  TRY(check_ptr(src, "src"));
  TRY(check_ptr(dst, "dst"));
  if (src == dst) return fail(TP_ERR_INVALID_ARG, "dst aliases src");
  TRY(device_check());
  return launched(tpk::launch_transpose(rows, cols, src, dst, as_stream(stream)), "tp_transpose");
}

tp_status tp_gemm_kmajor(tp_dtype out_dt, int32_t x_kmajor, int64_t m, int64_t n, int64_t k, const void* x,
                         int64_t ldx, const void* w, int64_t ldw, void* out, void* stream) {
  if (out_dt != TP_F32 && out_dt != TP_BF16) return fail(TP_ERR_INVALID_ARG, "unknown output dtype %d", (int)out_dt);
  if (m < 0 || n < 0 || k < 0) return fail(TP_ERR_SHAPE, "m, n and k must be >= 0");
  if (m % 8 || n % 8 || k % 8) return fail(TP_ERR_SHAPE, "m, n and k must be multiples of 8");
  if (ldx < (x_kmajor ? m : k) || ldw < n || ldx % 8 || ldw % 8)
    return fail(TP_ERR_SHAPE, "ldx and ldw must be multiples of 8 covering a row of x and w");
  if (k * ldx * 2 >= kMaxOffset || k * ldw * 2 >= kMaxOffset || (!x_kmajor && 256 * ldx * 2 >= kMaxOffset))
    return fail(TP_ERR_SHAPE, "an operand exceeds the 2 GiB offset range");
  if (m == 0 || n == 0) return ok();
  TRY(check_ptr(x, "x"));
  TRY(check_ptr(w, "w"));
  TRY(check_ptr(out, "out"));
  TRY(device_check());
  return launched(tpk::launch_gemm_bf16_km(out_dt == TP_F32 ? tpk::EPI_F32 : tpk::EPI_BF16, x_kmajor != 0, m, n, k, x,
                                           ldx, w, ldw, out, as_stream(stream)),
                  "tp_gemm_kmajor");
}

tp_status tp_mlp_act_backward(tp_act act, int64_t m, int64_t n, const void* pre, const void* dy, void* dpre,
                              void* y, void* stream) {
  if (act != TP_ACT_GELU && act != TP_ACT_SWIGLU)
    return fail(TP_ERR_INVALID_ARG, "tp_mlp_act_backward needs GELU or SWIGLU, got %d", (int)act);
  if (m < 0) return fail(TP_ERR_SHAPE, "m = %lld is negative", (long long)m);
  TRY(check_dim8(n, "n"));
  if (m == 0) return ok();
  TRY(check_ptr(pre, "pre"));
  TRY(check_ptr(dy, "dy"));
  TRY(check_ptr(dpre, "dpre"));
  if (y) TRY(check_ptr(y, "y"));
  TRY(device_check());
  return launched(tpk::launch_act_backward(act == TP_ACT_SWIGLU, m, n, pre, dy, dpre, y, as_stream(stream)),
                  "tp_mlp_act_backward");
}

size_t tp_shard_mlp_backward_workspace_bytes(tp_act act, int64_t m, int64_t h, int64_t f_shard) {
  if (m < 0 || h <= 0 || f_shard <= 0) return 0;
  return mlp_bwd_layout(act, m, h, f_shard).total;
}

tp_status tp_shard_mlp_backward(tp_act act, int64_t m, int64_t h, int64_t f_shard, const void* x,
                                const void* w_in, const void* w_out, const void* dz, const void* xt,
                                const void* dzt, const void* pre, void* ws, size_t ws_bytes, float* dx_partial,
                                float* dw_in, float* dw_out, void* stream) {
  if (act != TP_ACT_GELU && act != TP_ACT_SWIGLU)
    return fail(TP_ERR_INVALID_ARG, "tp_shard_mlp_backward needs GELU or SWIGLU, got %d", (int)act);
  if (m % 8 != 0) return fail(TP_ERR_SHAPE, "m = %lld must be a multiple of 8 (the weight gradients reduce over tokens)",
                              (long long)m);
  const int64_t F = act == TP_ACT_SWIGLU ? 2 * f_shard : f_shard;
  // the forward's two GEMMs and the backward's six, with their operand sizes
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, m, h, F, x, w_in, ws, "x", "w_in", "ws"));
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, m, h, f_shard, dz, w_out, ws, "dz", "w_out", "ws"));
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, m, F, h, ws, ws, dx_partial, "ws", "ws", "dx_partial"));
  if (m == 0) return ok();
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, h, m, f_shard, ws, ws, dw_out, "ws", "ws", "dw_out"));
  TRY(check_gemm(TP_ACT_NONE, TP_BF16, F, m, h, ws, ws, dw_in, "ws", "ws", "dw_in"));
  if (xt) TRY(check_ptr(xt, "xt"));
  if (dzt) TRY(check_ptr(dzt, "dzt"));
  if (pre) TRY(check_ptr(pre, "pre"));
  TRY(check_ptr(ws, "ws"));
  const MlpBwdLayout L = mlp_bwd_layout(act, m, h, f_shard);
  if (ws_bytes < L.total) return fail(TP_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, L.total);
  TRY(device_check());
  hipStream_t s = as_stream(stream);
  char* b = static_cast<char*>(ws);
  auto gemm = [&](int epi, int64_t M, int64_t N, int64_t K, const void* a, const void* w, void* c) {
    return tpk::launch_gemm_bf16(epi, M, N, K, a, w, c, nullptr, s);
  };
  hipError_t e;
#define TP_BWD_STEP(call, what) \
  if ((e = (call)) != hipSuccess) return launched(e, what);
  // the forward's saved pre-activation, or it recomputed; dY = dZ W_out (W_out
  // transposed to [f, h])
  const void* pre_p = pre;
  if (!pre_p) {
    TP_BWD_STEP(gemm(tpk::EPI_BF16, m, F, h, x, w_in, b + L.pre), "tp_shard_mlp_backward (pre-activation)");
    pre_p = b + L.pre;
  }
  TP_BWD_STEP(tpk::launch_transpose(h, f_shard, w_out, b + L.wout_t, s), "tp_shard_mlp_backward (w_out^T)");
  TP_BWD_STEP(gemm(tpk::EPI_BF16, m, f_shard, h, dz, b + L.wout_t, b + L.dy), "tp_shard_mlp_backward (dY)");
  // dPre (and the activation Y again, for the output layer's weight gradient)
  TP_BWD_STEP(tpk::launch_act_backward(act == TP_ACT_SWIGLU, m, f_shard, pre_p, b + L.dy, b + L.dpre, b + L.y, s),
              "tp_shard_mlp_backward (activation)");
  // dX partial = dPre W_in (W_in transposed to [h, F]); f's backward sums these over ranks
  TP_BWD_STEP(tpk::launch_transpose(F, h, w_in, b + L.win_t, s), "tp_shard_mlp_backward (w_in^T)");
  TP_BWD_STEP(gemm(tpk::EPI_F32, m, h, F, b + L.dpre, b + L.win_t, dx_partial), "tp_shard_mlp_backward (dX)");
  // dW_out = dZ^T Y and dW_in = dPre^T X, reducing over the tokens
  const void* dzt_p = dzt;
  if (!dzt_p) {
    TP_BWD_STEP(tpk::launch_transpose(m, h, dz, b + L.dzt, s), "tp_shard_mlp_backward (dZ^T)");
    dzt_p = b + L.dzt;
  }
  const void* xt_p = xt;
  if (!xt_p) {
    TP_BWD_STEP(tpk::launch_transpose(m, h, x, b + L.xt, s), "tp_shard_mlp_backward (X^T)");
    xt_p = b + L.xt;
  }
  TP_BWD_STEP(tpk::launch_transpose(m, f_shard, b + L.y, b + L.y_t, s), "tp_shard_mlp_backward (Y^T)");
  TP_BWD_STEP(gemm(tpk::EPI_F32, h, f_shard, m, dzt_p, b + L.y_t, dw_out), "tp_shard_mlp_backward (dW_out)");
  TP_BWD_STEP(tpk::launch_transpose(m, F, b + L.dpre, b + L.dpre_t, s), "tp_shard_mlp_backward (dPre^T)");
  TP_BWD_STEP(gemm(tpk::EPI_F32, F, h, m, b + L.dpre_t, xt_p, dw_in), "tp_shard_mlp_backward (dW_in)");
#undef TP_BWD_STEP
  return ok();
}

}  // extern "C"
