// C ABI of the Llama decoder-block library (declared in include/llama_block.h).
//
// Host side only: argument validation (before anything is enqueued),
// workspace carve-up, RoPE frequency table (fp64), launch sequencing on the
// caller's stream and the optional per-kernel event timing.  No device
// memory is allocated and the stream is never synchronized.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/llama_block.h"
#include "kernels.hpp"

using lb::DType;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return LLAMA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(int t) { return t == LLAMA_F32 || t == LLAMA_BF16; }

size_t align_up(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

// Up to this many token rows the QKV epilogue evaluates the RoPE angles
// itself instead of reading a precomputed table.
constexpr int64_t kRopeInlineRows = 256;

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------
struct PendingTiming {
  std::string name;
  hipEvent_t start, stop;
};
struct TimingTotal {
  int64_t launches = 0;
  double ms = 0.0;
};
bool g_prof_on = false;
std::vector<PendingTiming> g_pending;
std::vector<hipEvent_t> g_event_pool;
std::map<std::string, TimingTotal> g_totals;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` (which enqueues exactly the kernels of one step of the path)
// and, when timing is on, brackets it with events on the same stream.  The
// record is keyed "step/kernel" (or just "step" when the launcher names no
// kernel variant, or names the step itself).
template <class F>
hipError_t timed(const char* step, hipStream_t s, F&& launch) {
  if (!g_prof_on) {
    const char* name = nullptr;
    return launch(&name);
  }
  hipEvent_t e0 = take_event(), e1 = take_event();
  if (e0) (void)hipEventRecord(e0, s);
  const char* name = nullptr;
  hipError_t err = launch(&name);
  if (e1) (void)hipEventRecord(e1, s);
  if (e0 && e1) {
    std::string key(step);
    if (name && key != name) key += std::string("/") + name;
    g_pending.push_back({key, e0, e1});
  }
  return err;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(LLAMA_ERR_HIP, "%s: HIP error %d (%s)", what, static_cast<int>(e), hipGetErrorString(e));
}

lb::RopeTable make_rope(int hd, double theta) {
  lb::RopeTable t{};
  for (int k = 0; k < hd / 2 && k < 128; ++k)
    t.inv_freq[k] = std::pow(theta, -2.0 * k / static_cast<double>(hd));
  return t;
}

// ---------------------------------------------------------------------------
// shared validation helpers
// ---------------------------------------------------------------------------
int check_heads(int32_t nq, int32_t nkv, int32_t hd) {
  if (nq <= 0 || nkv <= 0 || hd <= 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "head counts and head_dim must be positive (n_q=%d n_kv=%d hd=%d)", nq, nkv, hd);
  if (nq % nkv != 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", nq, nkv);
  if (hd % 2 != 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "head_dim (%d) must be even", hd);
  if (hd > 256) return fail(LLAMA_ERR_UNSUPPORTED, "head_dim (%d) > 256 is not supported", hd);
  return LLAMA_OK;
}

}  // namespace

extern "C" {

const char* llama_last_error(void) { return g_last_error.c_str(); }

const char* llama_status_string(int status) {
  switch (status) {
    case LLAMA_OK: return "ok";
    case LLAMA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LLAMA_ERR_UNSUPPORTED: return "unsupported";
    case LLAMA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case LLAMA_ERR_HIP: return "hip error";
    default: return "unknown status";
  }
}

int llama_version(void) { return LLAMA_BLOCK_VERSION; }

// ---------------------------------------------------------------------------
int llama_rmsnorm(const void* x, const void* residual, const void* gamma, void* out,
                  void* sum_out, int64_t n_rows, int32_t d_model, double eps, int wdtype,
                  int rdtype, void* stream) {
  if (!dtype_ok(wdtype) || !dtype_ok(rdtype))
    return fail(LLAMA_ERR_UNSUPPORTED, "unknown dtype code (wdtype=%d rdtype=%d)", wdtype, rdtype);
  if (n_rows < 0 || d_model <= 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "n_rows must be >= 0 and d_model > 0 (n_rows=%lld d_model=%d)",
                static_cast<long long>(n_rows), d_model);
  if (!(eps >= 0.0)) return fail(LLAMA_ERR_INVALID_ARGUMENT, "eps must be >= 0");
  if (n_rows > 0 && (!x || !gamma || !out))
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "x, gamma and out must be non-null");
  if (out && (out == x || (residual && out == residual)))
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "out must not alias x or residual");
  for (const void* p : std::initializer_list<const void*>{x, residual, gamma, static_cast<const void*>(out), static_cast<const void*>(sum_out)})
    if (p && !aligned16(p)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  if (n_rows > 0x7fffffff) return fail(LLAMA_ERR_UNSUPPORTED, "n_rows too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed("rmsnorm", s, [&](const char** name) {
    *name = "rmsnorm";
    return lb::launch_rmsnorm(x, residual, gamma, out, sum_out, n_rows, d_model,
                              static_cast<float>(eps), static_cast<DType>(wdtype),
                              static_cast<DType>(rdtype), s);
  });
  if (e != hipSuccess) return hip_fail(e, "llama_rmsnorm");
  return ok();
}

// ---------------------------------------------------------------------------
int llama_rope(void* q, void* k, const int32_t* positions, int64_t n_tokens, int32_t n_q_heads,
               int32_t n_kv_heads, int32_t head_dim, double rope_theta, int wdtype,
               void* stream) {
  if (!dtype_ok(wdtype)) return fail(LLAMA_ERR_UNSUPPORTED, "unknown dtype code %d", wdtype);
  if (n_tokens < 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "n_tokens must be >= 0");
  if (head_dim <= 0 || head_dim % 2 != 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "head_dim (%d) must be positive and even", head_dim);
  if (head_dim > 256) return fail(LLAMA_ERR_UNSUPPORTED, "head_dim (%d) > 256 is not supported", head_dim);
  if (q && n_q_heads <= 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "n_q_heads must be positive");
  if (k && n_kv_heads <= 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "n_kv_heads must be positive");
  if (!(rope_theta > 0.0)) return fail(LLAMA_ERR_INVALID_ARGUMENT, "rope_theta must be > 0");
  if (n_tokens > 0 && !positions) return fail(LLAMA_ERR_INVALID_ARGUMENT, "positions must be non-null");
  if (n_tokens > 0 && !q && !k) return fail(LLAMA_ERR_INVALID_ARGUMENT, "q and k are both null");
  for (const void* p : std::initializer_list<const void*>{static_cast<const void*>(q), static_cast<const void*>(k)})
    if (p && !aligned16(p)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const lb::RopeTable tab = make_rope(head_dim, rope_theta);
  hipError_t e = timed("rope", s, [&](const char** name) {
    *name = "rope";
    return lb::launch_rope(q, k, positions, n_tokens, n_q_heads, n_kv_heads, head_dim, tab,
                           static_cast<DType>(wdtype), s);
  });
  if (e != hipSuccess) return hip_fail(e, "llama_rope");
  return ok();
}

// ---------------------------------------------------------------------------
size_t llama_gqa_attention_workspace_bytes(int32_t batch, int32_t q_len, int32_t kv_len,
                                           int32_t n_q_heads, int32_t n_kv_heads,
                                           int32_t head_dim, int wdtype) {
  if (batch <= 0 || q_len <= 0 || kv_len <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
      !dtype_ok(wdtype))
    return 0;
  return lb::attention_workspace_bytes(static_cast<DType>(wdtype), batch, q_len, kv_len, n_q_heads,
                                       n_kv_heads, head_dim);
}

int llama_gqa_attention(const void* q, const void* k, const void* v, void* out,
                        const int32_t* positions, int32_t batch, int32_t q_len, int32_t kv_len,
                        int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int wdtype,
                        void* workspace, size_t ws_bytes, void* stream) {
  if (!dtype_ok(wdtype)) return fail(LLAMA_ERR_UNSUPPORTED, "unknown dtype code %d", wdtype);
  if (batch < 0 || q_len < 0 || kv_len <= 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "batch, q_len must be >= 0 and kv_len > 0");
  int st = check_heads(n_q_heads, n_kv_heads, head_dim);
  if (st != LLAMA_OK) return st;
  if (!positions && kv_len < q_len)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "without positions kv_len (%d) must be >= q_len (%d)", kv_len, q_len);
  if (batch > 0 && q_len > 0 && (!q || !k || !v || !out))
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "q, k, v and out must be non-null");
  if (out && (out == q || out == k || out == v))
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "out must not alias q, k or v");
  for (const void* p : std::initializer_list<const void*>{q, k, v, static_cast<const void*>(out), workspace})
    if (p && !aligned16(p)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  if (batch == 0 || q_len == 0) return ok();
  const size_t need = llama_gqa_attention_workspace_bytes(batch, q_len, kv_len, n_q_heads, n_kv_heads,
                                                          head_dim, wdtype);
  if (ws_bytes < need || (need > 0 && !workspace))
    return fail(LLAMA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  lb::AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out; a.positions = positions;
  a.B = batch; a.Tq = q_len; a.S = kv_len; a.nq = n_q_heads; a.nkv = n_kv_heads; a.hd = head_dim;
  a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(head_dim)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed("attention", s, [&](const char** name) {
    return lb::launch_attention(static_cast<DType>(wdtype), a, workspace, ws_bytes, s, name);
  });
  if (e != hipSuccess) return hip_fail(e, "llama_gqa_attention");
  return ok();
}

// ---------------------------------------------------------------------------
namespace {

struct FfnPlan {
  size_t mact, gemm_gu, gemm_down, total;
};

FfnPlan ffn_plan(int64_t n, int32_t d, int32_t dff, DType wdt) {
  FfnPlan p{};
  p.mact = align_up(static_cast<size_t>(n) * dff * lb::dtype_bytes(wdt));
  p.gemm_gu = align_up(lb::gemm_workspace_bytes(wdt, static_cast<int>(n), dff, d, true));
  p.gemm_down = align_up(lb::gemm_workspace_bytes(wdt, static_cast<int>(n), d, dff, false));
  p.total = p.mact + std::max(p.gemm_gu, p.gemm_down);
  return p;
}

// gate/up (+ SiLU product into mact) then down (+ residual) into out
hipError_t run_ffn(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                   const void* residual, void* out, int n, int d, int dff, DType wdt, DType rdt,
                   void* mact, void* gws, size_t gws_bytes, hipStream_t s) {
  lb::WSeg gu{};
  gu.ptr[0] = w_gate; gu.ptr[1] = w_up; gu.start[0] = 0; gu.start[1] = dff; gu.start[2] = 2 * dff; gu.nseg = 2;
  lb::GemmEpi e1{};
  e1.kind = lb::EpiKind::Silu; e1.out_dt = wdt; e1.out = mact; e1.ldo = dff;
  hipError_t e = timed("gate_up_silu", s, [&](const char** name) {
    return lb::launch_gemm(wdt, x, n, d, gu, dff, true, e1, gws, gws_bytes, s, name);
  });
  if (e != hipSuccess) return e;
  lb::WSeg dn{};
  dn.ptr[0] = w_down; dn.start[0] = 0; dn.start[1] = d; dn.nseg = 1;
  lb::GemmEpi e2{};
  if (residual) {
    e2.kind = lb::EpiKind::Resid; e2.out_dt = rdt; e2.out = out; e2.resid = residual; e2.ldo = d;
  } else {
    e2.kind = lb::EpiKind::Store; e2.out_dt = rdt; e2.out = out; e2.ldo = d;
  }
  return timed("down_resid", s, [&](const char** name) {
    return lb::launch_gemm(wdt, mact, n, dff, dn, d, false, e2, gws, gws_bytes, s, name);
  });
}

}  // namespace

size_t llama_swiglu_ffn_workspace_bytes(int64_t n_tokens, int32_t d_model, int32_t d_ff, int wdtype,
                                        int rdtype) {
  if (n_tokens <= 0 || d_model <= 0 || d_ff <= 0 || !dtype_ok(wdtype) || !dtype_ok(rdtype)) return 0;
  return ffn_plan(n_tokens, d_model, d_ff, static_cast<DType>(wdtype)).total;
}

int llama_swiglu_ffn(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                     const void* residual, void* out, int64_t n_tokens, int32_t d_model,
                     int32_t d_ff, int wdtype, int rdtype, void* workspace, size_t ws_bytes,
                     void* stream) {
  if (!dtype_ok(wdtype) || !dtype_ok(rdtype))
    return fail(LLAMA_ERR_UNSUPPORTED, "unknown dtype code (wdtype=%d rdtype=%d)", wdtype, rdtype);
  if (n_tokens < 0 || d_model <= 0 || d_ff <= 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "n_tokens must be >= 0, d_model and d_ff > 0");
  if (n_tokens > 0x7fffffff) return fail(LLAMA_ERR_UNSUPPORTED, "n_tokens too large");
  if (n_tokens > 0 && (!x || !w_gate || !w_up || !w_down || !out))
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "x, weights and out must be non-null");
  if (out && out == x) return fail(LLAMA_ERR_INVALID_ARGUMENT, "out must not alias x");
  for (const void* p : std::initializer_list<const void*>{x, w_gate, w_up, w_down, residual, static_cast<const void*>(out), workspace})
    if (p && !aligned16(p)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  if (n_tokens == 0) return ok();
  const DType wdt = static_cast<DType>(wdtype), rdt = static_cast<DType>(rdtype);
  const FfnPlan p = ffn_plan(n_tokens, d_model, d_ff, wdt);
  if (ws_bytes < p.total || !workspace)
    return fail(LLAMA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", p.total, ws_bytes);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipError_t e = run_ffn(x, w_gate, w_up, w_down, residual, out, static_cast<int>(n_tokens), d_model, d_ff,
                         wdt, rdt, ws, ws + p.mact, ws_bytes - p.mact, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "llama_swiglu_ffn");
  return ok();
}

// ---------------------------------------------------------------------------
namespace {

struct BlockPlan {
  size_t a, q, k, v, o, h, mact, attn, gemm, cs, total;
};

// fp8: the cache is 8-bit, so the new tokens' k and v go to workspace rows
// first and are quantized into the cache by a separate pass.
BlockPlan block_plan(int B, int T, int d, int nq, int nkv, int hd, int dff, int kv_cap, DType wdt,
                     DType rdt, bool fp8 = false) {
  const size_t M = static_cast<size_t>(B) * T;
  const size_t wb = lb::dtype_bytes(wdt), rb = lb::dtype_bytes(rdt);
  BlockPlan p{};
  p.a = align_up(M * d * wb);  // also holds f (the FFN pre-norm output)
  p.q = align_up(M * nq * hd * wb);
  p.k = kv_cap > 0 && !fp8 ? 0 : align_up(M * nkv * hd * wb);
  p.v = p.k;
  p.o = align_up(M * nq * hd * wb);
  p.h = align_up(M * d * rb);
  p.mact = align_up(M * dff * wb);
  const int S = kv_cap > 0 ? kv_cap : T;
  p.attn = align_up(fp8 ? lb::attention_fp8kv_workspace_bytes(B, S, nq, nkv)
                        : lb::attention_workspace_bytes(wdt, B, T, S, nq, nkv, hd));
  size_t g = lb::gemm_workspace_bytes(wdt, static_cast<int>(M), (nq + 2 * nkv) * hd, d, false);
  g = std::max(g, lb::gemm_workspace_bytes(wdt, static_cast<int>(M), d, nq * hd, false));
  g = std::max(g, lb::gemm_workspace_bytes(wdt, static_cast<int>(M), dff, d, true));
  g = std::max(g, lb::gemm_workspace_bytes(wdt, static_cast<int>(M), d, dff, false));
  p.gemm = align_up(g);
  p.cs = align_up(M * (hd / 2) * 2 * sizeof(float));
  p.total = p.a + p.q + p.k + p.v + p.o + p.h + p.mact + p.attn + p.gemm + p.cs;
  return p;
}

}  // namespace

size_t llama_block_forward_workspace_bytes(int32_t batch, int32_t seq_len, int32_t d_model,
                                           int32_t n_q_heads, int32_t n_kv_heads,
                                           int32_t head_dim, int32_t d_ff, int32_t kv_cap,
                                           int wdtype, int rdtype) {
  if (batch <= 0 || seq_len <= 0 || d_model <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
      d_ff <= 0 || kv_cap < 0 || !dtype_ok(wdtype) || !dtype_ok(rdtype))
    return 0;
  return block_plan(batch, seq_len, d_model, n_q_heads, n_kv_heads, head_dim, d_ff, kv_cap,
                    static_cast<DType>(wdtype), static_cast<DType>(rdtype))
      .total;
}

namespace {

// 8-bit cache of llama_block_forward_fp8kv
struct Fp8Cache {
  void* k8;
  void* v8;
  float* k_scale;
  float* v_scale;
};

// Validation shared by llama_block_forward and llama_block_forward_fp8kv.
int check_block_args(const void* x, void* y, const llama_block_weights* w, const int32_t* positions,
                     int32_t batch, int32_t seq_len, int32_t d_model, int32_t n_q_heads, int32_t n_kv_heads,
                     int32_t head_dim, int32_t d_ff, double rope_theta, double eps, int32_t kv_cap) {
  if (batch < 0 || seq_len < 0 || d_model <= 0 || d_ff <= 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "batch, seq_len must be >= 0; d_model, d_ff > 0");
  int st = check_heads(n_q_heads, n_kv_heads, head_dim);
  if (st != LLAMA_OK) return st;
  if (!(rope_theta > 0.0)) return fail(LLAMA_ERR_INVALID_ARGUMENT, "rope_theta must be > 0");
  if (!(eps >= 0.0)) return fail(LLAMA_ERR_INVALID_ARGUMENT, "eps must be >= 0");
  if (kv_cap < 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "kv_cap must be >= 0");
  if (static_cast<int64_t>(batch) * seq_len > 0x7fffffff)
    return fail(LLAMA_ERR_UNSUPPORTED, "batch*seq_len too large");
  if (batch == 0 || seq_len == 0) return LLAMA_OK;
  if (!x || !y || !w || !positions)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "x, y, weights and positions must be non-null");
  if (!w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo || !w->ffn_norm || !w->w_gate || !w->w_up ||
      !w->w_down)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "every weight pointer must be non-null");
  if (y == x) return fail(LLAMA_ERR_INVALID_ARGUMENT, "y must not alias x");
  for (const void* p : std::initializer_list<const void*>{x, static_cast<const void*>(y), w->attn_norm, w->wq, w->wk,
                                                          w->wv, w->wo, w->ffn_norm, w->w_gate, w->w_up, w->w_down})
    if (!aligned16(p)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  return LLAMA_OK;
}

// The block's launch sequence (arguments already validated).  With c8 the
// cache is 8-bit: the Q/K/V epilogue stores this call's k and v rows in the
// workspace, kv_append_fp8 quantizes them into the cache and the decode
// attention reads the codes and scales.
int run_block(const void* x, void* y, const llama_block_weights* w, const int32_t* positions, void* k_cache,
              void* v_cache, int32_t kv_cap, int B, int T, int d, int nq, int nkv, int hd, int d_ff,
              double rope_theta, double eps, DType wdt, DType rdt, void* workspace, size_t ws_bytes,
              hipStream_t s, const Fp8Cache* c8) {
  const bool has_cache = kv_cap > 0;
  const int M = B * T;
  const BlockPlan p = block_plan(B, T, d, nq, nkv, hd, d_ff, kv_cap, wdt, rdt, c8 != nullptr);
  if (ws_bytes < p.total || !workspace)
    return fail(LLAMA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", p.total, ws_bytes);

  uint8_t* cur = static_cast<uint8_t*>(workspace);
  auto carve = [&](size_t n) { uint8_t* r = cur; cur += n; return r; };
  void* a_buf = carve(p.a);
  void* q_buf = carve(p.q);
  void* k_buf = has_cache && !c8 ? k_cache : carve(p.k);
  void* v_buf = has_cache && !c8 ? v_cache : carve(p.v);
  void* o_buf = carve(p.o);
  void* h_buf = carve(p.h);
  void* mact = carve(p.mact);
  void* attn_ws = carve(p.attn);
  void* gemm_ws = carve(p.gemm);
  float* rope_cs = reinterpret_cast<float*>(carve(p.cs));
  const lb::RopeTable rope = make_rope(hd, rope_theta);
  const float feps = static_cast<float>(eps);
  hipError_t e;

  // a1: attention pre-norm
  e = timed("attn_norm", s, [&](const char** name) {
    *name = "rmsnorm";
    return lb::launch_rmsnorm(x, nullptr, w->attn_norm, a_buf, nullptr, M, d, feps, wdt, rdt, s);
  });
  if (e != hipSuccess) return hip_fail(e, "block forward: attention norm");

  // a2-a4: fused Q/K/V projection with RoPE and (cache) stores
  {
    lb::WSeg wqkv{};
    wqkv.ptr[0] = w->wq; wqkv.ptr[1] = w->wk; wqkv.ptr[2] = w->wv;
    wqkv.start[0] = 0; wqkv.start[1] = nq * hd; wqkv.start[2] = (nq + nkv) * hd;
    wqkv.start[3] = (nq + 2 * nkv) * hd; wqkv.nseg = 3;
    lb::GemmEpi ep{};
    ep.kind = lb::EpiKind::Qkv; ep.out_dt = wdt;
    ep.q = q_buf; ep.k = k_buf; ep.v = v_buf; ep.positions = positions;
    ep.nq_hd = nq * hd; ep.nkv_hd = nkv * hd; ep.hd = hd; ep.seq_len = T; ep.kv_cap = c8 ? 0 : kv_cap;
    // Many tokens: the rotation angles' (cos, sin) are tabulated once per
    // token and pair, then read by every GEMM tile; few tokens (decode): the
    // epilogue evaluates them itself and the extra launch is skipped.
    const bool table = M > kRopeInlineRows;
    ep.rope_cs = table ? rope_cs : nullptr;
    ep.rope_base = std::pow(rope_theta, -2.0 / static_cast<double>(hd));
    e = timed("qkv_rope", s, [&](const char** name) {
      if (table) {
        hipError_t er = lb::launch_rope_table(positions, M, hd, rope, wdt, rope_cs, s);
        if (er != hipSuccess) return er;
      }
      return lb::launch_gemm(wdt, a_buf, M, d, wqkv, (nq + 2 * nkv) * hd, false, ep, gemm_ws, p.gemm, s, name);
    });
    if (e != hipSuccess) return hip_fail(e, "block forward: qkv projection");
  }
  if (c8) {
    e = timed("kv_append_fp8", s, [&](const char** name) {
      *name = "kv_append_fp8";
      return lb::launch_kv_append_fp8(k_buf, v_buf, positions, M, T, nkv, hd, wdt, c8->k8, c8->v8, c8->k_scale,
                                      c8->v_scale, kv_cap, s);
    });
    if (e != hipSuccess) return hip_fail(e, "block forward: 8-bit cache append");
  }

  // a5/a6: attention
  {
    lb::AttnArgs aa{};
    aa.q = q_buf; aa.k = c8 ? c8->k8 : k_buf; aa.v = c8 ? c8->v8 : v_buf; aa.out = o_buf;
    aa.positions = has_cache ? positions : nullptr;
    aa.B = B; aa.Tq = T; aa.S = has_cache ? kv_cap : T; aa.nq = nq; aa.nkv = nkv; aa.hd = hd;
    aa.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(hd)));
    if (c8) {
      aa.k_scale = c8->k_scale;
      aa.v_scale = c8->v_scale;
    }
    e = timed("attention", s, [&](const char** name) {
      return c8 ? lb::launch_attention_fp8kv(aa, attn_ws, p.attn, s, name)
                : lb::launch_attention(wdt, aa, attn_ws, p.attn, s, name);
    });
    if (e != hipSuccess) return hip_fail(e, "block forward: attention");
  }

  // a7: O projection + residual into h
  {
    lb::WSeg wo{};
    wo.ptr[0] = w->wo; wo.start[0] = 0; wo.start[1] = d; wo.nseg = 1;
    lb::GemmEpi ep{};
    ep.kind = lb::EpiKind::Resid; ep.out_dt = rdt; ep.out = h_buf; ep.resid = x; ep.ldo = d;
    // few rows: the residual add joins the FFN pre-norm in one pass over
    // the split-K partials (this leg then leaves only the partials)
    const bool fused = lb::resid_norm_fused(wdt, rdt, M, nq * hd, wo, d);
    e = timed("o_resid", s, [&](const char** name) {
      return fused ? lb::launch_gemm_partials(wdt, o_buf, M, nq * hd, wo, d, gemm_ws, p.gemm, s, name)
                   : lb::launch_gemm(wdt, o_buf, M, nq * hd, wo, d, false, ep, gemm_ws, p.gemm, s, name);
    });
    if (e != hipSuccess) return hip_fail(e, "block forward: o projection");

    // a8: FFN pre-norm (f reuses the a buffer)
    e = timed("ffn_norm", s, [&](const char** name) {
      if (fused) return lb::launch_resid_norm(M, nq * hd, d, gemm_ws, x, h_buf, w->ffn_norm, a_buf, feps, s, name);
      *name = "rmsnorm";
      return lb::launch_rmsnorm(h_buf, nullptr, w->ffn_norm, a_buf, nullptr, M, d, feps, wdt, rdt, s);
    });
    if (e != hipSuccess) return hip_fail(e, "block forward: ffn norm");
  }

  // a9/a10: SwiGLU FFN + residual into y
  e = run_ffn(a_buf, w->w_gate, w->w_up, w->w_down, h_buf, y, M, d, d_ff, wdt, rdt, mact, gemm_ws, p.gemm, s);
  if (e != hipSuccess) return hip_fail(e, "block forward: ffn");
  return ok();
}

}  // namespace

namespace {

// Validation of llama_block_forward and llama_block_forward_noalloc (all but
// the workspace): LLAMA_OK to go on, or the status to return.
int check_block_call(const void* x, void* y, const llama_block_weights* w, const int32_t* positions,
                     void* k_cache, void* v_cache, int32_t kv_cap, int32_t batch, int32_t seq_len,
                     int32_t d_model, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t d_ff,
                     double rope_theta, double eps, int wdtype, int rdtype) {
  if (!dtype_ok(wdtype) || !dtype_ok(rdtype))
    return fail(LLAMA_ERR_UNSUPPORTED, "unknown dtype code (wdtype=%d rdtype=%d)", wdtype, rdtype);
  int st = check_block_args(x, y, w, positions, batch, seq_len, d_model, n_q_heads, n_kv_heads, head_dim, d_ff,
                            rope_theta, eps, kv_cap);
  if (st != LLAMA_OK) return st;
  const bool has_cache = kv_cap > 0;
  if (has_cache != (k_cache != nullptr) || has_cache != (v_cache != nullptr))
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "k_cache and v_cache must both be given exactly when kv_cap > 0");
  return LLAMA_OK;
}

// Alignment of the caches and the workspace (checked once the call is known
// to do work, as for every entry point).
int check_block_buffers(const void* k_cache, const void* v_cache, const void* workspace) {
  for (const void* p : std::initializer_list<const void*>{k_cache, v_cache, workspace})
    if (p && !aligned16(p)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  return LLAMA_OK;
}

}  // namespace

int llama_block_forward(const void* x, void* y, const llama_block_weights* w,
                        const int32_t* positions, void* k_cache, void* v_cache, int32_t kv_cap,
                        int32_t batch, int32_t seq_len, int32_t d_model, int32_t n_q_heads,
                        int32_t n_kv_heads, int32_t head_dim, int32_t d_ff, double rope_theta,
                        double eps, int wdtype, int rdtype, void* workspace, size_t ws_bytes,
                        void* stream) {
  int st = check_block_call(x, y, w, positions, k_cache, v_cache, kv_cap, batch, seq_len, d_model, n_q_heads,
                            n_kv_heads, head_dim, d_ff, rope_theta, eps, wdtype, rdtype);
  if (st != LLAMA_OK) return st;
  if (batch == 0 || seq_len == 0) return ok();
  st = check_block_buffers(k_cache, v_cache, workspace);
  if (st != LLAMA_OK) return st;
  return run_block(x, y, w, positions, k_cache, v_cache, kv_cap, batch, seq_len, d_model, n_q_heads, n_kv_heads,
                   head_dim, d_ff, rope_theta, eps, static_cast<DType>(wdtype), static_cast<DType>(rdtype),
                   workspace, ws_bytes, static_cast<hipStream_t>(stream), nullptr);
}

// ---------------------------------------------------------------------------
// llama_block_forward_noalloc: the block forward on a fixed device scratch
// ---------------------------------------------------------------------------
namespace {

// The scratch of llama_block_forward_noalloc (what llama_block_forward takes
// as its workspace): a fixed array in the library's code object.  Every GPU
// the library runs on holds its own copy, at its own address, until the
// process ends.  In host code the array's name is not a device address: the
// address of each GPU's copy comes from hipGetSymbolAddress, looked up once
// per device with that device current and kept in g_scratch_ptr.
__device__ __align__(256) uint8_t scratch[LLAMA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` and the device's index.
hipError_t current_scratch(void** ptr, int* dev) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return e;
  if (*dev < 0 || *dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[*dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[*dev] = p;
  }
  *ptr = g_scratch_ptr[*dev];
  return hipSuccess;
}

}  // namespace

int llama_block_forward_noalloc(const void* x, void* y, const llama_block_weights* w,
                                const int32_t* positions, void* k_cache, void* v_cache, int32_t kv_cap,
                                int32_t batch, int32_t seq_len, int32_t d_model, int32_t n_q_heads,
                                int32_t n_kv_heads, int32_t head_dim, int32_t d_ff, double rope_theta,
                                double eps, int wdtype, int rdtype, void* stream) {
  int st = check_block_call(x, y, w, positions, k_cache, v_cache, kv_cap, batch, seq_len, d_model, n_q_heads,
                            n_kv_heads, head_dim, d_ff, rope_theta, eps, wdtype, rdtype);
  if (st != LLAMA_OK) return st;
  if (batch == 0 || seq_len == 0) return ok();
  st = check_block_buffers(k_cache, v_cache, nullptr);
  if (st != LLAMA_OK) return st;
  const size_t need = block_plan(batch, seq_len, d_model, n_q_heads, n_kv_heads, head_dim, d_ff, kv_cap,
                                 static_cast<DType>(wdtype), static_cast<DType>(rdtype))
                          .total;
  if (need > LLAMA_NOALLOC_SCRATCH_BYTES)
    return fail(LLAMA_ERR_WORKSPACE_TOO_SMALL,
                "this call needs %zu bytes of scratch; the fixed scratch holds %zu "
                "(llama_block_forward with a caller workspace takes any size)",
                need, static_cast<size_t>(LLAMA_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  int dev = -1;
  hipError_t e = current_scratch(&ws, &dev);
  if (e != hipSuccess) return hip_fail(e, "llama_block_forward_noalloc: scratch address");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (s) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return hip_fail(e, "llama_block_forward_noalloc: stream device");
    if (sdev != dev)
      return fail(LLAMA_ERR_INVALID_ARGUMENT, "the stream belongs to device %d but device %d is current",
                  static_cast<int>(sdev), dev);
  }
  return run_block(x, y, w, positions, k_cache, v_cache, kv_cap, batch, seq_len, d_model, n_q_heads, n_kv_heads,
                   head_dim, d_ff, rope_theta, eps, static_cast<DType>(wdtype), static_cast<DType>(rdtype), ws,
                   LLAMA_NOALLOC_SCRATCH_BYTES, s, nullptr);
}

// ---------------------------------------------------------------------------
// 8-bit KV cache
// ---------------------------------------------------------------------------
namespace {

int check_fp8_cache(const void* k8, const void* v8, const float* ks, const float* vs, int32_t kv_cap) {
  if (kv_cap <= 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "kv_cap must be > 0");
  if (!k8 || !v8 || !ks || !vs)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "the 8-bit caches and their scales must be non-null");
  for (const void* p : std::initializer_list<const void*>{k8, v8, static_cast<const void*>(ks),
                                                          static_cast<const void*>(vs)})
    if (!aligned16(p)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  return LLAMA_OK;
}

}  // namespace

int llama_kv_append_fp8(const void* k, const void* v, const int32_t* positions, int32_t batch,
                        int32_t seq_len, int32_t n_kv_heads, int32_t head_dim, int wdtype, void* k_cache,
                        void* v_cache, float* k_scale, float* v_scale, int32_t kv_cap, void* stream) {
  if (!dtype_ok(wdtype)) return fail(LLAMA_ERR_UNSUPPORTED, "unknown dtype code %d", wdtype);
  if (batch < 0 || seq_len < 0 || n_kv_heads <= 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "batch, seq_len must be >= 0 and n_kv_heads > 0");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(LLAMA_ERR_UNSUPPORTED, "the 8-bit cache needs head_dim 64, 128 or 256 (got %d)", head_dim);
  int st = check_fp8_cache(k_cache, v_cache, k_scale, v_scale, kv_cap);
  if (st != LLAMA_OK) return st;
  const int64_t n = static_cast<int64_t>(batch) * seq_len;
  if (n == 0) return ok();
  if (!k || !v || !positions) return fail(LLAMA_ERR_INVALID_ARGUMENT, "k, v and positions must be non-null");
  if (!aligned16(k) || !aligned16(v)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  if (n * n_kv_heads * 2 > 0x7fffffffLL * 4) return fail(LLAMA_ERR_UNSUPPORTED, "too many rows");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed("kv_append_fp8", s, [&](const char** name) {
    *name = "kv_append_fp8";
    return lb::launch_kv_append_fp8(k, v, positions, n, seq_len, n_kv_heads, head_dim, static_cast<DType>(wdtype),
                                    k_cache, v_cache, k_scale, v_scale, kv_cap, s);
  });
  if (e != hipSuccess) return hip_fail(e, "llama_kv_append_fp8");
  return ok();
}

size_t llama_gqa_attention_fp8kv_workspace_bytes(int32_t batch, int32_t kv_cap, int32_t n_q_heads,
                                                 int32_t n_kv_heads, int32_t head_dim) {
  if (batch <= 0 || kv_cap <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim != 128) return 0;
  return lb::attention_fp8kv_workspace_bytes(batch, kv_cap, n_q_heads, n_kv_heads);
}

namespace {

int check_fp8_attention_shape(int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim) {
  int st = check_heads(n_q_heads, n_kv_heads, head_dim);
  if (st != LLAMA_OK) return st;
  const int r = n_q_heads / n_kv_heads;
  if (head_dim != 128 || (r != 1 && r != 2 && r != 4 && r != 8))
    return fail(LLAMA_ERR_UNSUPPORTED, "this decode attention needs head_dim 128 and n_q/n_kv in {1,2,4,8}");
  return LLAMA_OK;
}

}  // namespace

int llama_gqa_attention_fp8kv(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                              const float* v_scale, void* out, const int32_t* positions, int32_t batch,
                              int32_t kv_cap, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                              void* workspace, size_t ws_bytes, void* stream) {
  if (batch < 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "batch must be >= 0");
  int st = check_fp8_attention_shape(n_q_heads, n_kv_heads, head_dim);
  if (st != LLAMA_OK) return st;
  st = check_fp8_cache(k_cache, v_cache, k_scale, v_scale, kv_cap);
  if (st != LLAMA_OK) return st;
  if (batch == 0) return ok();
  if (!q || !out || !positions) return fail(LLAMA_ERR_INVALID_ARGUMENT, "q, out and positions must be non-null");
  if (out == q) return fail(LLAMA_ERR_INVALID_ARGUMENT, "out must not alias q");
  for (const void* p : std::initializer_list<const void*>{q, static_cast<const void*>(out), workspace})
    if (p && !aligned16(p)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  const size_t need = llama_gqa_attention_fp8kv_workspace_bytes(batch, kv_cap, n_q_heads, n_kv_heads, head_dim);
  if (ws_bytes < need || !workspace)
    return fail(LLAMA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  lb::AttnArgs a{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.out = out; a.positions = positions;
  a.B = batch; a.Tq = 1; a.S = kv_cap; a.nq = n_q_heads; a.nkv = n_kv_heads; a.hd = head_dim;
  a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(head_dim)));
  a.k_scale = k_scale; a.v_scale = v_scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed("attention", s, [&](const char** name) {
    return lb::launch_attention_fp8kv(a, workspace, ws_bytes, s, name);
  });
  if (e != hipSuccess) return hip_fail(e, "llama_gqa_attention_fp8kv");
  return ok();
}

size_t llama_block_forward_fp8kv_workspace_bytes(int32_t batch, int32_t d_model, int32_t n_q_heads,
                                                 int32_t n_kv_heads, int32_t head_dim, int32_t d_ff,
                                                 int32_t kv_cap, int rdtype) {
  if (batch <= 0 || d_model <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 || d_ff <= 0 ||
      kv_cap <= 0 || !dtype_ok(rdtype))
    return 0;
  return block_plan(batch, 1, d_model, n_q_heads, n_kv_heads, head_dim, d_ff, kv_cap, DType::BF16,
                    static_cast<DType>(rdtype), true)
      .total;
}

int llama_block_forward_fp8kv(const void* x, void* y, const llama_block_weights* w, const int32_t* positions,
                              void* k_cache, void* v_cache, float* k_scale, float* v_scale, int32_t kv_cap,
                              int32_t batch, int32_t d_model, int32_t n_q_heads, int32_t n_kv_heads,
                              int32_t head_dim, int32_t d_ff, double rope_theta, double eps, int rdtype,
                              void* workspace, size_t ws_bytes, void* stream) {
  if (!dtype_ok(rdtype)) return fail(LLAMA_ERR_UNSUPPORTED, "unknown dtype code (rdtype=%d)", rdtype);
  int st = check_block_args(x, y, w, positions, batch, 1, d_model, n_q_heads, n_kv_heads, head_dim, d_ff,
                            rope_theta, eps, kv_cap);
  if (st != LLAMA_OK) return st;
  st = check_fp8_attention_shape(n_q_heads, n_kv_heads, head_dim);
  if (st != LLAMA_OK) return st;
  st = check_fp8_cache(k_cache, v_cache, k_scale, v_scale, kv_cap);
  if (st != LLAMA_OK) return st;
  if (batch == 0) return ok();
  if (workspace && !aligned16(workspace)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  const Fp8Cache c8{k_cache, v_cache, k_scale, v_scale};
  return run_block(x, y, w, positions, nullptr, nullptr, kv_cap, batch, 1, d_model, n_q_heads, n_kv_heads,
                   head_dim, d_ff, rope_theta, eps, DType::BF16, static_cast<DType>(rdtype), workspace, ws_bytes,
                   static_cast<hipStream_t>(stream), &c8);
}

// ---------------------------------------------------------------------------
// paged KV cache
// ---------------------------------------------------------------------------
namespace {

int check_paged(const void* kp, const void* vp, const int32_t* table, int32_t max_pages, int32_t page_size,
                int64_t n_pages) {
  if (!kp || !vp || !table) return fail(LLAMA_ERR_INVALID_ARGUMENT, "page pools and block table must be non-null");
  if (max_pages <= 0 || page_size <= 0 || n_pages <= 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "max_pages, page_size and n_pages must be > 0");
  if (page_size % 32 != 0)
    return fail(LLAMA_ERR_UNSUPPORTED, "page_size (%d) must be a multiple of 32", page_size);
  if (static_cast<int64_t>(max_pages) * page_size > 0x7fffffff)
    return fail(LLAMA_ERR_UNSUPPORTED, "max_pages * page_size too large");
  for (const void* p : std::initializer_list<const void*>{kp, vp, static_cast<const void*>(table)})
    if (!aligned16(p)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  return LLAMA_OK;
}

}  // namespace

int llama_kv_append_paged(const void* k, const void* v, const int32_t* positions, const int32_t* block_table,
                          int32_t max_pages, int32_t page_size, int32_t batch, int32_t seq_len, int32_t n_kv_heads,
                          int32_t head_dim, void* k_pages, void* v_pages, int64_t n_pages, void* stream) {
  if (batch < 0 || seq_len < 0 || n_kv_heads <= 0 || head_dim <= 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "batch, seq_len must be >= 0; n_kv_heads, head_dim > 0");
  if (head_dim % 8 != 0 || head_dim > 256)
    return fail(LLAMA_ERR_UNSUPPORTED, "head_dim (%d) must be a multiple of 8 and at most 256", head_dim);
  int st = check_paged(k_pages, v_pages, block_table, max_pages, page_size, n_pages);
  if (st != LLAMA_OK) return st;
  const int64_t n = static_cast<int64_t>(batch) * seq_len;
  if (n == 0) return ok();
  if (!k || !v || !positions) return fail(LLAMA_ERR_INVALID_ARGUMENT, "k, v and positions must be non-null");
  if (!aligned16(k) || !aligned16(v)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed("kv_append_paged", s, [&](const char** name) {
    *name = "kv_append_paged";
    return lb::launch_kv_append_paged(k, v, positions, n, seq_len, n_kv_heads, head_dim, block_table, max_pages,
                                      page_size, n_pages, k_pages, v_pages, s);
  });
  if (e != hipSuccess) return hip_fail(e, "llama_kv_append_paged");
  return ok();
}

size_t llama_gqa_attention_paged_workspace_bytes(int32_t batch, int32_t max_pages, int32_t page_size,
                                                 int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim) {
  if (batch <= 0 || max_pages <= 0 || page_size <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim != 128)
    return 0;
  const int64_t S = static_cast<int64_t>(max_pages) * page_size;
  if (S > 0x7fffffff) return 0;
  return lb::attention_paged_workspace_bytes(batch, static_cast<int>(S), n_q_heads);
}

int llama_gqa_attention_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                              int32_t max_pages, int32_t page_size, int64_t n_pages, void* out,
                              const int32_t* positions, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                              int32_t head_dim, void* workspace, size_t ws_bytes, void* stream) {
  if (batch < 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "batch must be >= 0");
  int st = check_fp8_attention_shape(n_q_heads, n_kv_heads, head_dim);
  if (st != LLAMA_OK) return st;
  st = check_paged(k_pages, v_pages, block_table, max_pages, page_size, n_pages);
  if (st != LLAMA_OK) return st;
  if (batch == 0) return ok();
  if (!q || !out || !positions) return fail(LLAMA_ERR_INVALID_ARGUMENT, "q, out and positions must be non-null");
  if (out == q) return fail(LLAMA_ERR_INVALID_ARGUMENT, "out must not alias q");
  for (const void* p : std::initializer_list<const void*>{q, static_cast<const void*>(out), workspace})
    if (p && !aligned16(p)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  const size_t need = llama_gqa_attention_paged_workspace_bytes(batch, max_pages, page_size, n_q_heads, n_kv_heads,
                                                                head_dim);
  if (ws_bytes < need || !workspace)
    return fail(LLAMA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  lb::AttnArgs a{};
  a.q = q; a.k = k_pages; a.v = v_pages; a.out = out; a.positions = positions;
  a.B = batch; a.Tq = 1; a.S = max_pages * page_size; a.nq = n_q_heads; a.nkv = n_kv_heads; a.hd = head_dim;
  a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(head_dim)));
  a.block_table = block_table; a.max_pages = max_pages; a.page_size = page_size; a.n_pages = n_pages;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed("attention", s, [&](const char** name) {
    return lb::launch_attention_paged(a, workspace, ws_bytes, s, name);
  });
  if (e != hipSuccess) return hip_fail(e, "llama_gqa_attention_paged");
  return ok();
}

// ---------------------------------------------------------------------------
// output layer: final RMSNorm, linear head, argmax
// ---------------------------------------------------------------------------
namespace {

struct HeadPlan {
  size_t f, logits, gemm, arg, total;
};

HeadPlan head_plan(int64_t n, int32_t d, int32_t vocab, DType wdt) {
  HeadPlan p{};
  p.f = align_up(static_cast<size_t>(n) * d * lb::dtype_bytes(wdt));
  p.logits = align_up(static_cast<size_t>(n) * vocab * sizeof(float));
  p.gemm = align_up(lb::gemm_workspace_bytes(wdt, static_cast<int>(n), vocab, d, false));
  p.arg = align_up(lb::argmax_workspace_bytes(n, vocab));
  p.total = p.f + p.logits + p.gemm + p.arg;
  return p;
}

}  // namespace

size_t llama_lm_head_argmax_workspace_bytes(int64_t n_rows, int32_t d_model, int32_t vocab, int wdtype,
                                            int rdtype) {
  if (n_rows <= 0 || n_rows > 0x7fffffff || d_model <= 0 || vocab <= 0 || !dtype_ok(wdtype) || !dtype_ok(rdtype))
    return 0;
  return head_plan(n_rows, d_model, vocab, static_cast<DType>(wdtype)).total;
}

int llama_lm_head_argmax(const void* h, const void* gamma, const void* w_head, int32_t* token, float* logits,
                         float* best, int64_t n_rows, int32_t d_model, int32_t vocab, double eps, int wdtype,
                         int rdtype, void* workspace, size_t ws_bytes, void* stream) {
  if (!dtype_ok(wdtype) || !dtype_ok(rdtype))
    return fail(LLAMA_ERR_UNSUPPORTED, "unknown dtype code (wdtype=%d rdtype=%d)", wdtype, rdtype);
  if (n_rows < 0 || d_model <= 0 || vocab <= 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "n_rows must be >= 0; d_model, vocab > 0");
  if (!(eps >= 0.0)) return fail(LLAMA_ERR_INVALID_ARGUMENT, "eps must be >= 0");
  if (n_rows > 0x7fffffff) return fail(LLAMA_ERR_UNSUPPORTED, "n_rows too large");
  if (n_rows == 0) return ok();
  if (!h || !gamma || !w_head || !token)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "h, gamma, w_head and token must be non-null");
  for (const void* p : std::initializer_list<const void*>{h, gamma, w_head, static_cast<const void*>(token),
                                                          static_cast<const void*>(logits),
                                                          static_cast<const void*>(best), workspace})
    if (p && !aligned16(p)) return fail(LLAMA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  const DType wdt = static_cast<DType>(wdtype), rdt = static_cast<DType>(rdtype);
  const HeadPlan p = head_plan(n_rows, d_model, vocab, wdt);
  if (ws_bytes < p.total || !workspace)
    return fail(LLAMA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", p.total, ws_bytes);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  void* f = ws;
  float* lg = logits ? logits : reinterpret_cast<float*>(ws + p.f);
  void* gws = ws + p.f + p.logits;
  void* aws = ws + p.f + p.logits + p.gemm;
  const int M = static_cast<int>(n_rows);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed("final_norm", s, [&](const char** name) {
    *name = "rmsnorm";
    return lb::launch_rmsnorm(h, nullptr, gamma, f, nullptr, M, d_model, static_cast<float>(eps), wdt, rdt, s);
  });
  if (e != hipSuccess) return hip_fail(e, "llama_lm_head_argmax: final norm");
  lb::WSeg wh{};
  wh.ptr[0] = w_head; wh.start[0] = 0; wh.start[1] = vocab; wh.nseg = 1;
  lb::GemmEpi ep{};
  ep.kind = lb::EpiKind::Store; ep.out_dt = DType::F32; ep.out = lg; ep.ldo = vocab;
  e = timed("lm_head", s, [&](const char** name) {
    return lb::launch_gemm(wdt, f, M, d_model, wh, vocab, false, ep, gws, p.gemm, s, name);
  });
  if (e != hipSuccess) return hip_fail(e, "llama_lm_head_argmax: head projection");
  e = timed("argmax", s, [&](const char** name) {
    *name = "argmax";
    return lb::launch_argmax_rows(lg, M, vocab, vocab, token, best, aws, s);
  });
  if (e != hipSuccess) return hip_fail(e, "llama_lm_head_argmax: argmax");
  return ok();
}

// ---------------------------------------------------------------------------
int llama_profile_enable(int on) {
  g_prof_on = on != 0;
  return ok();
}

int llama_profile_reset(void) {
  for (auto& pt : g_pending) {
    g_event_pool.push_back(pt.start);
    g_event_pool.push_back(pt.stop);
  }
  g_pending.clear();
  g_totals.clear();
  return ok();
}

int llama_profile_collect(void) {
  for (auto& pt : g_pending) {
    hipError_t e = hipEventSynchronize(pt.stop);
    if (e != hipSuccess) return hip_fail(e, "llama_profile_collect");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, pt.start, pt.stop);
    if (e != hipSuccess) return hip_fail(e, "llama_profile_collect");
    TimingTotal& t = g_totals[pt.name];
    t.launches += 1;
    t.ms += ms;
    g_event_pool.push_back(pt.start);
    g_event_pool.push_back(pt.stop);
  }
  g_pending.clear();
  return ok();
}

int llama_profile_query(const char* kernel_name, int64_t* launches, double* total_ms) {
  if (!kernel_name) return fail(LLAMA_ERR_INVALID_ARGUMENT, "kernel_name is null");
  auto it = g_totals.find(kernel_name);
  if (it == g_totals.end()) return fail(LLAMA_ERR_INVALID_ARGUMENT, "no timing recorded for '%s'", kernel_name);
  if (launches) *launches = it->second.launches;
  if (total_ms) *total_ms = it->second.ms;
  return ok();
}

int llama_profile_names(char* buf, size_t cap) {
  std::string all;
  for (auto& kv : g_totals) {
    all += kv.first;
    all += '\n';
  }
  if (!buf || cap == 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "buffer is null or empty");
  std::strncpy(buf, all.c_str(), cap - 1);
  buf[cap - 1] = '\0';
  return ok();
}

}  // extern "C"
