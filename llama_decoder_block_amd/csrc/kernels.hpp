// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace lb {

enum class DType : int { F32 = 0, BF16 = 1 };

inline size_t dtype_bytes(DType t) { return t == DType::F32 ? 4 : 2; }

// ---------------------------------------------------------------------------
// GEMM operand description.  The weight operand is a logical [N, K] matrix
// (row-major, K contiguous) assembled from up to three row segments stored
// in separate buffers: logical row n in [start[i], start[i+1]) lives at
// ptr[i] + (n - start[i]) * K.  Q/K/V projections use three segments; the
// fused gate/up projection uses two (gate rows then up rows).
// ---------------------------------------------------------------------------
struct WSeg {
  const void* ptr[3];
  int start[4];  // start[nseg] == N
  int nseg;
};

// ---------------------------------------------------------------------------
// Epilogues.  A GEMM computes acc[m][n] = sum_k X[m][k] * W[n][k] in fp32 and
// hands each output row m four consecutive columns n..n+3 (n % 4 == 0,
// `cnt` of them valid) to the epilogue.  For the fused gate/up product the
// epilogue receives the gate and up accumulators of the same column c.
//
// The single-operand epilogues also offer a split form for whole groups of
// four columns (when vec_ok()): col(n) resolves what depends on the column
// group only, row_from(m, row_key(m)) what depends on the row only,
// pre(row, col) issues the group's loads (or computes its factors), and
// put(row, col, pre, v) finishes and stores.  A tile epilogue resolves its
// lane's column once, computes row_key() once per row in the lane that owns
// the row and shares it between lanes, and issues pre() for many groups
// before the first put(), so their loads are in flight together instead of
// one load-use-store round trip per group.  pre() and put() are kept free of
// branches but for the store itself: a branch between a load and its use
// makes the compiler wait for every outstanding memory operation there.
// ---------------------------------------------------------------------------

// out[m, n] = acc (stored in TO)
template <typename TO>
struct EpiStore {
  TO* out;
  int ldo;
  using Row = int64_t;
  using Col = int;
  using Key = int;
  static constexpr bool kRowKey = false;
  __device__ __forceinline__ bool vec_ok() const { return (ldo & 3) == 0; }
  __device__ __forceinline__ Row row(int m) const { return static_cast<int64_t>(m) * ldo; }
  __device__ __forceinline__ Col col(int n) const { return n; }
  __device__ __forceinline__ int row_key(int) const { return 0; }
  __device__ __forceinline__ Row row_from(int m, int) const { return row(m); }
  __device__ __forceinline__ f32x4 pre(Row, int) const { return f32x4{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void put(Row r, int n, f32x4, const float v[4]) const {
    Vec4<TO>::store(out + r + n, v);
  }
  __device__ __forceinline__ void operator()(int m, int n, const float v[4], int cnt) const {
    TO* p = out + static_cast<int64_t>(m) * ldo + n;
    if (cnt == 4 && (ldo & 3) == 0) {
      Vec4<TO>::store(p, v);
    } else {
      for (int i = 0; i < cnt; ++i) st(p + i, v[i]);
    }
  }
};

// out[m, n] = resid[m, n] + acc   (residual stream in TR; out may alias resid)
template <typename TR>
struct EpiResid {
  TR* out;
  const TR* resid;
  int ldo;
  using Row = int64_t;
  using Col = int;
  using Key = int;
  static constexpr bool kRowKey = false;
  __device__ __forceinline__ bool vec_ok() const { return (ldo & 3) == 0; }
  __device__ __forceinline__ Row row(int m) const { return static_cast<int64_t>(m) * ldo; }
  __device__ __forceinline__ Col col(int n) const { return n; }
  __device__ __forceinline__ int row_key(int) const { return 0; }
  __device__ __forceinline__ Row row_from(int m, int) const { return row(m); }
  __device__ __forceinline__ f32x4 pre(Row r, int n) const {
    float t[4];
    Vec4<TR>::load(resid + r + n, t);
    return f32x4{t[0], t[1], t[2], t[3]};
  }
  __device__ __forceinline__ void put(Row r, int n, f32x4 res, const float v[4]) const {
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = res[i] + v[i];
    Vec4<TR>::store(out + r + n, o);
  }
  __device__ __forceinline__ void operator()(int m, int n, const float v[4], int cnt) const {
    const int64_t off = static_cast<int64_t>(m) * ldo + n;
    if (cnt == 4 && (ldo & 3) == 0) {
      float r[4], o[4];
      Vec4<TR>::load(resid + off, r);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = r[i] + v[i];
      Vec4<TR>::store(out + off, o);
    } else {
      for (int i = 0; i < cnt; ++i) st(out + off + i, ld(resid + off + i) + v[i]);
    }
  }
};

// Q/K/V projection epilogue: RoPE on the Q and K columns (adjacent pairs
// (2k, 2k+1) of each head rotated by pos * theta^(-2k/hd)), then the stores:
// Q to q[m, :]; K and V either to k/v[m, :] (no cache) or to the caches at
// slot positions[m] of sequence m / seq_len.  A token whose position lies
// outside [0, kv_cap) has no cache slot: its K and V are not stored (its Q
// still is), as the 8-bit and paged cache writers skip such rows.
template <typename T>
struct EpiQkv {
  T* q;
  T* k;            // [M, nkv_hd] when kv_cap == 0, else cache [B, kv_cap, nkv_hd]
  T* v;
  const int32_t* positions;
  int nq_hd, nkv_hd, hd, seq_len, kv_cap;
  const float* cs;  // [M, hd/2] (cos, sin) of each row's rotation angles (launch_rope_table),
                    // or null: angles evaluated here (few rows) with theta_k = rope_base^k
  double rope_base;  // theta_base^(-2/hd)

  // a K/V store of a cached token with no slot in [0, kv_cap)
  __device__ __forceinline__ bool no_slot(int n, int pos) const {
    return n >= nq_hd && kv_cap > 0 && (pos < 0 || pos >= kv_cap);
  }
  __device__ __forceinline__ T* dest(int m, int n, int pos) const {
    if (n < nq_hd) return q + static_cast<int64_t>(m) * nq_hd + n;
    const bool is_k = n < nq_hd + nkv_hd;
    const int nn = is_k ? n - nq_hd : n - nq_hd - nkv_hd;
    int64_t row = m;
    if (kv_cap > 0) row = static_cast<int64_t>(m / seq_len) * kv_cap + pos;
    return (is_k ? k : v) + row * nkv_hd + nn;
  }
  __device__ __forceinline__ const float* angle(int m, int n) const {
    return cs + (static_cast<int64_t>(m) * (hd >> 1) + ((n % hd) >> 1)) * 2;
  }

  // split form (whole groups of four columns inside one head of one segment,
  // angles from the table).  Everything that depends on the column group is
  // resolved once in col(), everything that depends on the row once per row
  // in row_key(), so that pre() and put() are straight-line code: one table
  // load, the rotation, one store (skipped only for a K/V row with no slot).
  struct Col {
    T* base;     // the group's first column in row 0 of its output (q, k or v)
    int stride;  // elements per output row
    bool is_q;   // Q: token rows; K / V: the row_key() rows
    bool rot;    // Q or K: rotate the pairs
    int pair;    // first rotation pair of the group within its head
  };
  struct Row {
    int64_t m;   // token row
    int64_t kv;  // row of k / v (cache slot row when kv_cap > 0); -1: no slot
  };
  using Key = int64_t;
  static constexpr bool kRowKey = true;
  __device__ __forceinline__ bool vec_ok() const {
    return cs != nullptr && (hd & 3) == 0 && (nq_hd & 3) == 0 && (nkv_hd & 3) == 0;
  }
  __device__ __forceinline__ Col col(int n) const {
    Col c;
    c.is_q = n < nq_hd;
    const bool is_k = !c.is_q && n < nq_hd + nkv_hd;
    c.rot = c.is_q || is_k;
    const int nn = c.is_q ? n : is_k ? n - nq_hd : n - nq_hd - nkv_hd;
    c.base = (c.is_q ? q : is_k ? k : v) + nn;
    c.stride = c.is_q ? nq_hd : nkv_hd;
    c.pair = (n % hd) >> 1;
    return c;
  }
  // the k / v row of token m
  __device__ __forceinline__ Key row_key(int m) const {
    if (kv_cap <= 0) return m;
    const int pos = positions[m];
    return pos < 0 || pos >= kv_cap ? int64_t{-1} : static_cast<int64_t>(m / seq_len) * kv_cap + pos;
  }
  __device__ __forceinline__ Row row_from(int m, Key kv) const { return Row{m, kv}; }
  // (cos, sin) of the group's two pairs; identity for V
  __device__ __forceinline__ f32x4 pre(const Row& r, const Col& c) const {
    const f32x4 t = *reinterpret_cast<const f32x4*>(cs + (r.m * (hd >> 1) + c.pair) * 2);
    return c.rot ? t : f32x4{1.f, 0.f, 1.f, 0.f};
  }
  __device__ __forceinline__ void put(const Row& r, const Col& c, f32x4 t, const float a[4]) const {
    float o[4];
    o[0] = c.rot ? a[0] * t[0] - a[1] * t[1] : a[0];
    o[1] = c.rot ? a[0] * t[1] + a[1] * t[0] : a[1];
    o[2] = c.rot ? a[2] * t[2] - a[3] * t[3] : a[2];
    o[3] = c.rot ? a[2] * t[3] + a[3] * t[2] : a[3];
    const int64_t row = c.is_q ? r.m : r.kv;
    if (row >= 0) Vec4<T>::store(c.base + row * c.stride, o);
  }
  __device__ __forceinline__ void operator()(int m, int n, const float v4[4], int cnt) const {
    const int pos = kv_cap > 0 ? positions[m] : 0;
    if (no_slot(n, pos)) return;
    float v[4] = {v4[0], v4[1], v4[2], v4[3]};
    const bool rot = n < nq_hd + nkv_hd;  // Q or K: rotate the pairs; V is stored as is
    if (cnt == 4 && (hd & 3) == 0) {
      // four columns (two pairs) in one head of one segment: one 4-wide store
      if (rot) {
        f32x4 t;
        if (cs) {
          t = *reinterpret_cast<const f32x4*>(angle(m, n));
        } else {
          const int k = (n % hd) >> 1;
          float s0, c0, s1, c1;
          rope_sincos_t<T>(positions[m], rope_inv_freq_pow(rope_base, k), &s0, &c0);
          rope_sincos_t<T>(positions[m], rope_inv_freq_pow(rope_base, k + 1), &s1, &c1);
          t = f32x4{c0, s0, c1, s1};
        }
        const float a0 = v[0] * t[0] - v[1] * t[1], b0 = v[0] * t[1] + v[1] * t[0];
        const float a1 = v[2] * t[2] - v[3] * t[3], b1 = v[2] * t[3] + v[3] * t[2];
        v[0] = a0; v[1] = b0; v[2] = a1; v[3] = b1;
      }
      Vec4<T>::store(dest(m, n, pos), v);
      return;
    }
    for (int pr = 0; pr + 1 < cnt; pr += 2) {
      float a = v[pr], b = v[pr + 1];
      // per pair: a group of four columns may straddle Q and K or K and V
      if (n + pr < nq_hd + nkv_hd) {
        f32x2 t;
        if (cs)
          t = *reinterpret_cast<const f32x2*>(angle(m, n + pr));
        else {
          float s0, c0;
          rope_sincos_t<T>(positions[m], rope_inv_freq_pow(rope_base, ((n + pr) % hd) >> 1), &s0, &c0);
          t = f32x2{c0, s0};
        }
        const float ra = a * t[0] - b * t[1];
        b = a * t[1] + b * t[0];
        a = ra;
      }
      if (!no_slot(n + pr, pos)) {
        T* d = dest(m, n + pr, pos);
        st(d, a);
        st(d + 1, b);
      }
    }
  }
};

// SwiGLU product: out[m, c] = SiLU(gate) * up with SiLU(z) = z / (1 + e^-z)
template <typename TO>
struct EpiSilu {
  TO* out;
  int ldo;
  __device__ __forceinline__ void operator()(int m, int c, const float g[4], const float u[4],
                                             int cnt) const {
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = silu_t<TO>(g[i]) * u[i];
    TO* p = out + static_cast<int64_t>(m) * ldo + c;
    if (cnt == 4 && (ldo & 3) == 0) {
      Vec4<TO>::store(p, o);
    } else {
      for (int i = 0; i < cnt; ++i) st(p + i, o[i]);
    }
  }
};

// Raw fp32 partial sums of one K-split: part[z][m][n]
// (split z = blockIdx.z).  For the fused gate/up product the partial rows are
// the logical rows: gate column c at c, up column c at half + c.
struct EpiPartial {
  float* part;
  int ldo;
  int64_t split_stride;  // elements between consecutive splits
  int half;              // gate/up product: offset of the up columns (= N)
  using Row = int64_t;
  using Col = int;
  using Key = int;
  static constexpr bool kRowKey = false;
  __device__ __forceinline__ bool vec_ok() const { return (ldo & 3) == 0; }
  __device__ __forceinline__ Row row(int m) const {
    return blockIdx.z * split_stride + static_cast<int64_t>(m) * ldo;
  }
  __device__ __forceinline__ Col col(int n) const { return n; }
  __device__ __forceinline__ int row_key(int) const { return 0; }
  __device__ __forceinline__ Row row_from(int m, int) const { return row(m); }
  __device__ __forceinline__ f32x4 pre(Row, int) const { return f32x4{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void put(Row r, int n, f32x4, const float v[4]) const {
    Vec4<float>::store(part + r + n, v);
  }
  __device__ __forceinline__ void operator()(int m, int n, const float v[4], int cnt) const {
    float* p = part + blockIdx.z * split_stride + static_cast<int64_t>(m) * ldo + n;
    if (cnt == 4 && (ldo & 3) == 0) {
      Vec4<float>::store(p, v);
    } else {
      for (int i = 0; i < cnt; ++i) p[i] = v[i];
    }
  }
  __device__ __forceinline__ void operator()(int m, int c, const float g[4], const float u[4], int cnt) const {
    (*this)(m, c, g, cnt);
    (*this)(m, half + c, u, cnt);
  }
};

// ---------------------------------------------------------------------------
// GEMM front end: chooses the MFMA kernel (bf16, K % 8 == 0), possibly with a
// K-split and a reduction pass for few rows, or the generic VALU kernel.
// ---------------------------------------------------------------------------
enum class EpiKind { Store, Resid, Qkv, Silu };

struct GemmEpi {
  EpiKind kind;
  DType out_dt;        // Store: dtype of out; Resid: residual dtype
  void* out;
  const void* resid;
  int ldo;
  // Qkv
  void* q; void* k; void* v;
  const int32_t* positions;
  int nq_hd, nkv_hd, hd, seq_len, kv_cap;
  const float* rope_cs;  // [M, hd/2] (cos, sin) table from launch_rope_table, or null
  double rope_base;       // theta_base^(-2/hd) (angles evaluated in the epilogue when rope_cs is null)
};

// Workspace bytes the GEMM needs for a given problem (split-K partials).
size_t gemm_workspace_bytes(DType dt, int M, int N, int K, bool dual);

hipError_t launch_gemm(DType dt, const void* X, int M, int K, const WSeg& W, int N, bool dual,
                       const GemmEpi& epi, void* ws, size_t ws_bytes, hipStream_t s,
                       const char** kernel_name);

// Few token rows (the skinny split-K path), a residual epilogue and an
// RMSNorm of its result, as in the decode step's O projection and FFN
// pre-norm: the GEMM leaves fp32 partials in ws (launch_gemm_partials), and
// launch_resid_norm sums them with the residual into h (fp32, the additions of
// launch_gemm's residual epilogue in the same order) and writes
// f = RMSNorm(h) * gamma (bf16).
// resid_norm_fused says whether a shape takes this path (bf16 operands, fp32
// residual, N a multiple of 1024 up to 8192, a K split); otherwise the caller
// runs launch_gemm and launch_rmsnorm.  ws needs gemm_workspace_bytes(dt, M,
// N, K, false) bytes and must not be touched between the two calls.
bool resid_norm_fused(DType dt, DType rdt, int M, int K, const WSeg& W, int N);
hipError_t launch_gemm_partials(DType dt, const void* X, int M, int K, const WSeg& W, int N, void* ws,
                                size_t ws_bytes, hipStream_t s, const char** kernel_name);
hipError_t launch_resid_norm(int M, int K, int N, const void* ws, const void* resid, void* h, const void* gamma,
                             void* f, float eps, hipStream_t s, const char** kernel_name);

// ---------------------------------------------------------------------------
// Other launchers
// ---------------------------------------------------------------------------
hipError_t launch_rmsnorm(const void* x, const void* res, const void* gamma, void* out,
                          void* sum_out, int64_t rows, int d, float eps, DType wdt, DType rdt,
                          hipStream_t s);

hipError_t launch_rope(void* q, void* k, const int32_t* positions, int64_t n_tokens, int nq,
                       int nkv, int hd, const RopeTable& rope, DType dt, hipStream_t s);

// cs[m][k] = (cos, sin) of positions[m] * inv_freq[k] for k < hd/2, fp32, the
// angle reduced in fp64; accurate sin/cos for fp32 outputs (dt F32), the
// hardware ones for bf16 outputs.  cs holds n_tokens * hd/2 float pairs.
hipError_t launch_rope_table(const int32_t* positions, int64_t n_tokens, int hd, const RopeTable& rope,
                             DType dt, float* cs, hipStream_t s);

struct AttnArgs {
  const void* q;       // [B, Tq, nq, hd]
  const void* k;       // [B, S, nkv, hd]
  const void* v;
  void* out;           // [B, Tq, nq, hd]
  const int32_t* positions;  // [B, Tq] or null (query t sees 0..t)
  int B, Tq, S, nq, nkv, hd;
  float scale;         // 1/sqrt(hd)
  const float* k_scale;  // 8-bit cache only: fp32 row scales [B, nkv, S] of k and v
  const float* v_scale;
  // paged cache only: k, v are page pools [n_pages, page_size, nkv, hd] and
  // slot j of sequence b is row j % page_size of page
  // block_table[b * max_pages + j / page_size]; S = max_pages * page_size
  const int32_t* block_table;
  int max_pages, page_size;
  int64_t n_pages;
};

size_t attention_workspace_bytes(DType dt, int B, int Tq, int S, int nq, int nkv, int hd);

hipError_t launch_attention(DType dt, const AttnArgs& a, void* ws, size_t ws_bytes,
                            hipStream_t s, const char** kernel_name);

// ---------------------------------------------------------------------------
// 8-bit KV cache: E4M3 codes [B, nkv, S, hd] (one byte per element; the slots
// of one KV head are contiguous) with one fp32 scale per (sequence, KV head,
// slot) in [B, nkv, S].
// ---------------------------------------------------------------------------
// Decode attention (Tq == 1, hd == 128, bf16 q and out) over the 8-bit cache
// a.k / a.v with scales a.k_scale / a.v_scale.
size_t attention_fp8kv_workspace_bytes(int B, int S, int nq, int nkv);
hipError_t launch_attention_fp8kv(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s,
                                  const char** kernel_name);

// Decode attention (Tq == 1, hd == 128, bf16) over a paged cache (the
// block_table / max_pages / page_size / n_pages fields; page_size % 32 == 0).
size_t attention_paged_workspace_bytes(int B, int S, int nq);
hipError_t launch_attention_paged(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s,
                                  const char** kernel_name);

// Copies rows k, v [n_tokens, nkv, hd] (bf16) to the paged pools at slot
// positions[n] of sequence n / seq_len (tokens whose slot or page is outside
// the table / pool are skipped).
hipError_t launch_kv_append_paged(const void* k, const void* v, const int32_t* positions, int64_t n_tokens,
                                  int seq_len, int nkv, int hd, const int32_t* block_table, int max_pages,
                                  int page_size, int64_t n_pages, void* k_pool, void* v_pool, hipStream_t s);

// token[r] = argmax over the n fp32 logits of row r (row stride ld; ties go to
// the smallest column); best_value (nullable) receives the maximum.
size_t argmax_workspace_bytes(int64_t rows, int n);
hipError_t launch_argmax_rows(const float* logits, int64_t rows, int64_t ld, int n, int32_t* token,
                              float* best_value, void* ws, hipStream_t s);

// Quantizes rows k, v [n_tokens, nkv, hd] (dtype dt) and stores them at slot
// positions[n] of sequence n / seq_len (tokens whose slot is outside
// [0, kv_cap) are skipped).  hd must be a multiple of 64, at most 256.
hipError_t launch_kv_append_fp8(const void* k, const void* v, const int32_t* positions, int64_t n_tokens,
                                int seq_len, int nkv, int hd, DType dt, void* k8, void* v8, float* k_scale,
                                float* v_scale, int kv_cap, hipStream_t s);

}  // namespace lb
