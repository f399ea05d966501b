/*
 * llama_block.h -- C ABI of the MI355X (gfx950) forward pass of one Llama
 * decoder block: pre-RMSNorm, Q/K/V projection, RoPE on Q and K, causal
 * grouped-query attention, O projection + residual, pre-RMSNorm, SwiGLU FFN
 * + residual; prefill and the one-token decode step against a KV cache.
 *
 * Pages cited by tag:
 *   [LA] "Llama Architecture: RMSNorm, SwiGLU, RoPE, GQA, and PyTorch
 *        Implementation" (ailinkdeeptech.com/research/llama)
 *   [RN] "RMSNorm: Root Mean Square Layer Normalization" study note
 *        (ai-engineer-exhaustive.pages.dev/research/llama/llama-rmsnorm)
 *   [L3] "LLaMA-3 8B 现代 LLM 架构、计算规模与能耗" (ienjoy.github.io/llama3-8b.html)
 *   [MA] "LLaMA Architecture > Model Architecture" (mbrenndoerfer.com)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership: the caller owns every buffer (inputs, weights, outputs, KV
 *   caches, workspace).  All tensor pointers are DEVICE pointers on the
 *   current HIP device.  The library allocates no device memory, keeps no
 *   state between calls (apart from the optional kernel-timing records and
 *   the thread-local error text) and never synchronizes the stream.
 * Stream: `stream` is a hipStream_t passed as void*; NULL means the default
 *   stream.  All work is enqueued on it in order.
 * Layout: row-major and contiguous.  Activations are token-major:
 *   x, y [B, T, d_model]; Q [B, T, n_q, hd]; K, V [B, T, n_kv, hd];
 *   caches [B, kv_cap, n_kv, hd].  Weights are [out, in] and a projection is
 *   y = x W^T (the nn.Linear modules of [LA] "Production PyTorch
 *   Implementation"): W_q [n_q*hd, d], W_k, W_v [n_kv*hd, d], W_o
 *   [d, n_q*hd], W_gate, W_up [d_ff, d], W_down [d, d_ff], gains [d].
 *   Feature index of head h, element i is h*hd + i.  Positions are int32.
 * Dtypes: `wdtype` (LLAMA_F32 or LLAMA_BF16) is the storage type of the
 *   weights, gains and every GEMM / attention operand (normed activations,
 *   Q, K, V, caches, attention output, SwiGLU product).  `rdtype` is the
 *   storage type of the residual stream (x, h, y).  Accumulation is always
 *   fp32; every fp32 -> bf16 conversion rounds to nearest even.
 * Alignment: every pointer must be 16-byte aligned.
 * Errors: every function returns LLAMA_OK (0) or a negative status.  All
 *   argument checks run on the host before anything is enqueued; on error
 *   nothing is enqueued and llama_last_error() holds a thread-local message.
 *   Faults inside a kernel surface at the caller's next synchronization.
 *   No C++ exception crosses this ABI.
 * Empty problems: a count of rows, tokens or sequences equal to 0 is a valid
 *   empty call; it returns LLAMA_OK, enqueues nothing and writes nothing.
 *   Negative counts and zero widths (d_model, head_dim, d_ff, head counts,
 *   vocab, cache capacity) are LLAMA_ERR_INVALID_ARGUMENT.
 */
#ifndef LLAMA_BLOCK_H
#define LLAMA_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LLAMA_BLOCK_VERSION 10100 /* major*10000 + minor*100 + patch */

enum llama_dtype { LLAMA_F32 = 0, LLAMA_BF16 = 1 };

enum llama_status {
  LLAMA_OK = 0,
  LLAMA_ERR_INVALID_ARGUMENT = -1,    /* null pointer, negative count, zero width, n_q % n_kv != 0, odd head_dim, ... */
  LLAMA_ERR_UNSUPPORTED = -2,         /* valid but not handled (dtype code, head_dim > 256, misaligned pointer) */
  LLAMA_ERR_WORKSPACE_TOO_SMALL = -3, /* ws_bytes below the matching *_workspace_bytes() */
  LLAMA_ERR_HIP = -4                  /* a HIP launch reported an error */
};

/* Device pointers to the nine parameter tensors of one block ([LA] "Step 2",
 * LlamaTransformerBlock; [L3] §六 parameter tables).  All in `wdtype`. */
typedef struct llama_block_weights {
  const void* attn_norm; /* gamma of the attention pre-norm  [d]          */
  const void* wq;        /* [n_q*hd, d]                                   */
  const void* wk;        /* [n_kv*hd, d]                                  */
  const void* wv;        /* [n_kv*hd, d]                                  */
  const void* wo;        /* [d, n_q*hd]                                   */
  const void* ffn_norm;  /* gamma of the FFN pre-norm  [d]                */
  const void* w_gate;    /* [d_ff, d]                                     */
  const void* w_up;      /* [d_ff, d]                                     */
  const void* w_down;    /* [d, d_ff]                                     */
} llama_block_weights;

/* RMSNorm, optionally fused with a residual add.
 * [LA] §1 and the RMSNorm module of "Step 1"; [RN] "How it works";
 * [MA] RMSNorm equation.  Per row r of n_rows rows of width d_model:
 *   s   = x[r] (+ residual[r] if residual != NULL)
 *   out = s * (mean(s^2) + eps)^(-1/2) * gamma   (sum of squares in fp32,
 *         eps inside the square root, reduction over d_model only)
 * If sum_out != NULL, s is also stored there (may alias x or residual).
 * x, residual, sum_out: rdtype [n_rows, d_model]; gamma, out: wdtype.
 * out must not alias x or residual. */
int llama_rmsnorm(const void* x, const void* residual, const void* gamma, void* out,
                  void* sum_out, int64_t n_rows, int32_t d_model, double eps, int wdtype,
                  int rdtype, void* stream);

/* RoPE in place on Q and K ([LA] §3 rotation matrix; [L3] §四.3).
 * For token n at position m = positions[n], head h and pair k < hd/2:
 *   phi = m * rope_theta^(-2k/hd);
 *   (x_2k, x_2k+1) <- (x_2k cos phi - x_2k+1 sin phi, x_2k sin phi + x_2k+1 cos phi)
 * q: [n_tokens, n_q_heads, hd]; k: [n_tokens, n_kv_heads, hd] (either may be
 * NULL to rotate only the other; its head count is then ignored).  Angles are
 * formed and reduced modulo 2*pi in fp64, then sin/cos evaluated in fp32.
 * positions: [n_tokens], each >= 0.  V is never rotated. */
int llama_rope(void* q, void* k, const int32_t* positions, int64_t n_tokens,
               int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, double rope_theta,
               int wdtype, void* stream);

/* Causal grouped-query attention ([LA] §4 GQA equation; [L3] §4.4-4.7).
 * Query head h reads KV head floor(h / (n_q/n_kv)); scores are q.k/sqrt(hd);
 * softmax over the visible slots; output = weighted sum of V; heads are
 * concatenated in order.  K/V are read shared by the n_q/n_kv query heads of a
 * group, never copied.
 *   q, out: [batch, q_len, n_q, hd];  k, v: [batch, kv_len, n_kv, hd]
 *   positions: [batch, q_len] or NULL.  Query (b, t) sees slots
 *     0..positions[b*q_len + t] (which must be < kv_len); with NULL it sees
 *     slots 0..t (plain causal self-attention; needs kv_len >= q_len).
 * q_len == 1 selects the split-K decode kernel, q_len > 1 the flash-style
 * prefill kernel.  workspace: device scratch of at least
 * llama_gqa_attention_workspace_bytes(...) bytes (may be NULL if that is 0).
 * out must not alias q, k or v. */
int llama_gqa_attention(const void* q, const void* k, const void* v, void* out,
                        const int32_t* positions, int32_t batch, int32_t q_len, int32_t kv_len,
                        int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int wdtype,
                        void* workspace, size_t ws_bytes, void* stream);
size_t llama_gqa_attention_workspace_bytes(int32_t batch, int32_t q_len, int32_t kv_len,
                                           int32_t n_q_heads, int32_t n_kv_heads,
                                           int32_t head_dim, int wdtype);

/* SwiGLU feed-forward network ([LA] §2 equation and the SwiGLUFFN module;
 * [L3] §五; [MA] FFN equation).  The pre-norm is not included:
 *   out = (residual +) W_down (SiLU(W_gate x) * (W_up x)),  SiLU(z) = z/(1+e^-z)
 * x: wdtype [n_tokens, d_model] (already normalised); residual (nullable) and
 * out: rdtype [n_tokens, d_model]; out may alias residual.  The product
 * SiLU(.)*(.) is stored in wdtype in the workspace of at least
 * llama_swiglu_ffn_workspace_bytes(...) bytes. */
int llama_swiglu_ffn(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                     const void* residual, void* out, int64_t n_tokens, int32_t d_model,
                     int32_t d_ff, int wdtype, int rdtype, void* workspace, size_t ws_bytes,
                     void* stream);
size_t llama_swiglu_ffn_workspace_bytes(int64_t n_tokens, int32_t d_model, int32_t d_ff,
                                        int wdtype, int rdtype);

/* One decoder block ([LA] "Step 2" block forward; [MA] block equations;
 * [L3] §二 data flow, §七 KV cache, §九 decode):
 *   h = x + W_o Attn(RoPE(W_q a), RoPE(W_k a), W_v a),  a = RMSNorm(x; attn_norm)
 *   y = h + W_down(SiLU(W_gate f) * W_up f),             f = RMSNorm(h; ffn_norm)
 * x, y: rdtype [batch, seq_len, d_model] (y must not alias x).
 * positions: [batch, seq_len] RoPE positions.
 * Without a cache (kv_cap == 0, k_cache == v_cache == NULL) the keys are this
 *   call's own tokens and token t attends tokens 0..t.
 * With a cache (kv_cap > 0, both cache pointers non-NULL, [batch, kv_cap,
 *   n_kv, hd] in wdtype): the rotated k and the v of token (b, t) are written
 *   at slot positions[b, t] (< kv_cap), and query (b, t) attends slots
 *   0..positions[b, t] of the updated cache.  seq_len == 1 is the decode step;
 *   seq_len > 1 fills the cache during prefill.  Slots above a query's
 *   position are never read.
 * workspace: at least llama_block_forward_workspace_bytes(...) bytes. */
int llama_block_forward(const void* x, void* y, const llama_block_weights* w,
                        const int32_t* positions, void* k_cache, void* v_cache, int32_t kv_cap,
                        int32_t batch, int32_t seq_len, int32_t d_model, int32_t n_q_heads,
                        int32_t n_kv_heads, int32_t head_dim, int32_t d_ff, double rope_theta,
                        double eps, int wdtype, int rdtype, void* workspace, size_t ws_bytes,
                        void* stream);
size_t llama_block_forward_workspace_bytes(int32_t batch, int32_t seq_len, int32_t d_model,
                                           int32_t n_q_heads, int32_t n_kv_heads,
                                           int32_t head_dim, int32_t d_ff, int32_t kv_cap,
                                           int wdtype, int rdtype);

/* llama_block_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same operation, arguments and kernels, minus the
 * workspace.  Its scratch is a fixed device array of
 * LLAMA_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held from
 * the first call on that GPU until the process ends; the call makes no
 * allocation of any kind (with the library's opt-in profiler off).
 * A call whose workspace (llama_block_forward_workspace_bytes of the same
 * shape) exceeds LLAMA_NOALLOC_SCRATCH_BYTES returns
 * LLAMA_ERR_WORKSPACE_TOO_SMALL before enqueueing anything.  Every call on a
 * GPU shares that GPU's scratch: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must be serialized by the caller.
 * The stream must belong to the current device (LLAMA_ERR_INVALID_ARGUMENT
 * otherwise).  At 64 MiB the scratch holds, for example, the Llama-3-8B
 * decode step of 64 sequences or a prefill of several hundred tokens. */
#define LLAMA_NOALLOC_SCRATCH_BYTES (64u << 20)
int llama_block_forward_noalloc(const void* x, void* y, const llama_block_weights* w,
                                const int32_t* positions, void* k_cache, void* v_cache, int32_t kv_cap,
                                int32_t batch, int32_t seq_len, int32_t d_model, int32_t n_q_heads,
                                int32_t n_kv_heads, int32_t head_dim, int32_t d_ff, double rope_theta,
                                double eps, int wdtype, int rdtype, void* stream);

/* 8-bit KV cache ([LA] "Troubleshooting Common Deployment Faults", item 3:
 * an 8-bit KV cache halves the bytes_per_elem factor of the KV-cache memory
 * formula in [LA] §4).  The pages fix no format or scale; this library uses
 * OCP FP8 E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities, largest finite 448, 0x7F/0xFF are NaN and never written) with
 * one fp32 scale per cached row of head_dim values:
 *   s = max_i |x_i| / 448 (fp32 division);
 *   code_i = x_i / s (fp32 division) rounded to the nearest E4M3 value, ties
 *            to the even mantissa, magnitudes beyond 448 clamped, sign kept;
 *   a row whose maximum is 0 stores s = 0 and all-zero codes;
 *   the cached value is s * E4M3(code_i).
 * Layouts: codes k_cache, v_cache [batch, n_kv, kv_cap, hd] (one byte each:
 * unlike the bf16 caches, the slots of one KV head are contiguous, so the
 * decode kernel streams each head's history as one block); scales k_scale,
 * v_scale [batch, n_kv, kv_cap] fp32.  Slots never written
 * hold arbitrary bytes and are never read (a query at position p reads slots
 * 0..p only). */

/* Quantizes the rows k, v [batch, seq_len, n_kv, hd] (wdtype; NaN inputs are
 * not supported) and stores codes and scales at slot positions[b, t] of
 * sequence b.  Tokens whose slot is outside [0, kv_cap) are skipped on the
 * device (no write).  head_dim must be 64, 128 or 256. */
int llama_kv_append_fp8(const void* k, const void* v, const int32_t* positions, int32_t batch,
                        int32_t seq_len, int32_t n_kv_heads, int32_t head_dim, int wdtype,
                        void* k_cache, void* v_cache, float* k_scale, float* v_scale, int32_t kv_cap,
                        void* stream);

/* Decode attention over an 8-bit cache: one query token per sequence,
 * otherwise the operation of llama_gqa_attention with q_len == 1.  Scores are
 * k_scale[slot] * (q . E4M3(codes)) / sqrt(hd); the weights multiply
 * v_scale[slot] * E4M3(codes).  q, out: bf16 [batch, n_q, hd]; positions:
 * [batch] (query b sees slots 0..positions[b], each < kv_cap).  head_dim must
 * be 128 and n_q/n_kv one of 1, 2, 4, 8.  workspace: at least
 * llama_gqa_attention_fp8kv_workspace_bytes(...) bytes. */
int llama_gqa_attention_fp8kv(const void* q, const void* k_cache, const void* v_cache,
                              const float* k_scale, const float* v_scale, void* out,
                              const int32_t* positions, int32_t batch, int32_t kv_cap,
                              int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                              void* workspace, size_t ws_bytes, void* stream);
size_t llama_gqa_attention_fp8kv_workspace_bytes(int32_t batch, int32_t kv_cap, int32_t n_q_heads,
                                                 int32_t n_kv_heads, int32_t head_dim);

/* The decode step of llama_block_forward (seq_len == 1, bf16 weights and
 * operands, residual stream in rdtype) against an 8-bit cache: the new
 * token's rotated k and its v are quantized into slot positions[b] (as
 * llama_kv_append_fp8 does), then query b attends slots 0..positions[b]
 * through llama_gqa_attention_fp8kv's kernel.  x, y: [batch, 1, d_model];
 * positions: [batch].  workspace: at least
 * llama_block_forward_fp8kv_workspace_bytes(...) bytes. */
int llama_block_forward_fp8kv(const void* x, void* y, const llama_block_weights* w,
                              const int32_t* positions, void* k_cache, void* v_cache,
                              float* k_scale, float* v_scale, int32_t kv_cap, int32_t batch,
                              int32_t d_model, int32_t n_q_heads, int32_t n_kv_heads,
                              int32_t head_dim, int32_t d_ff, double rope_theta, double eps,
                              int rdtype, void* workspace, size_t ws_bytes, void* stream);
size_t llama_block_forward_fp8kv_workspace_bytes(int32_t batch, int32_t d_model, int32_t n_q_heads,
                                                 int32_t n_kv_heads, int32_t head_dim, int32_t d_ff,
                                                 int32_t kv_cap, int rdtype);

/* Paged KV cache ([LA] "Troubleshooting Common Deployment Faults", item 3:
 * a paged cache allocates KV history in fixed-size pages of a shared pool
 * instead of one contiguous region per sequence).  Pools k_pages, v_pages:
 * bf16 [n_pages, page_size, n_kv, hd] (a page holds page_size consecutive
 * slots of one sequence, token-major like the contiguous cache);
 * block_table: int32 [batch, max_pages]; slot j of sequence b is row
 * j % page_size of page block_table[b*max_pages + j/page_size].  page_size
 * must be a multiple of 32.  Table entries for visible slots must lie in
 * [0, n_pages); the kernels clamp other entries into the pool (so a bad table
 * reads wrong rows but stays inside memory). */

/* Copies the bf16 rows k, v [batch, seq_len, n_kv, hd] into the pools at slot
 * positions[b, t] (tokens whose slot lies outside the table, or whose page
 * entry lies outside [0, n_pages), are skipped).  head_dim % 8 == 0, <= 256. */
int llama_kv_append_paged(const void* k, const void* v, const int32_t* positions,
                          const int32_t* block_table, int32_t max_pages, int32_t page_size,
                          int32_t batch, int32_t seq_len, int32_t n_kv_heads, int32_t head_dim,
                          void* k_pages, void* v_pages, int64_t n_pages, void* stream);

/* Decode attention (one bf16 query token per sequence, the operation of
 * llama_gqa_attention with q_len == 1) over a paged cache.  q, out: bf16
 * [batch, n_q, hd]; positions: [batch] (query b sees slots 0..positions[b],
 * each < max_pages * page_size).  head_dim must be 128 and n_q/n_kv one of
 * 1, 2, 4, 8.  workspace: at least
 * llama_gqa_attention_paged_workspace_bytes(...) bytes. */
int llama_gqa_attention_paged(const void* q, const void* k_pages, const void* v_pages,
                              const int32_t* block_table, int32_t max_pages, int32_t page_size,
                              int64_t n_pages, void* out, const int32_t* positions, int32_t batch,
                              int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                              void* workspace, size_t ws_bytes, void* stream);
size_t llama_gqa_attention_paged_workspace_bytes(int32_t batch, int32_t max_pages, int32_t page_size,
                                                 int32_t n_q_heads, int32_t n_kv_heads,
                                                 int32_t head_dim);

/* Output layer with the greedy choice ([L3] §十: after the last block a
 * final RMSNorm, the linear head to vocabulary logits, and argmax, the
 * deterministic one of the choices it lists; the head is applied to the last
 * position of each sequence, so the caller passes those rows):
 *   f = RMSNorm(h; gamma)   (as llama_rmsnorm: fp32 sum of squares, eps inside)
 *   logits = f W_head^T     (fp32 accumulation and result)
 *   token[r] = argmax_v logits[r, v]  (ties go to the smallest v; NaN is
 *              never chosen)
 * h: rdtype [n_rows, d_model]; gamma: wdtype [d_model]; w_head: wdtype
 * [vocab, d_model] ([out, in]); token: int32 [n_rows]; logits (nullable):
 * fp32 [n_rows, vocab] receives the logits (otherwise they stay in the
 * workspace); best (nullable): fp32 [n_rows] receives each chosen logit.
 * workspace: at least llama_lm_head_argmax_workspace_bytes(...) bytes. */
int llama_lm_head_argmax(const void* h, const void* gamma, const void* w_head, int32_t* token,
                         float* logits, float* best, int64_t n_rows, int32_t d_model, int32_t vocab,
                         double eps, int wdtype, int rdtype, void* workspace, size_t ws_bytes,
                         void* stream);
size_t llama_lm_head_argmax_workspace_bytes(int64_t n_rows, int32_t d_model, int32_t vocab,
                                            int wdtype, int rdtype);

/* Host-only helpers. */
const char* llama_last_error(void);    /* thread-local text of the last failure ("" if none) */
const char* llama_status_string(int status);
int llama_version(void);               /* LLAMA_BLOCK_VERSION of the built library */

/* Kernel timing for benchmarks.  While enabled, every kernel this library
 * enqueues is bracketed by a pair of HIP events recorded on the stream the
 * kernel is launched on.  llama_profile_collect() waits for the recorded
 * events, adds each pair's elapsed time to a per-kernel total and releases
 * the events; llama_profile_query() then reports launches and total
 * milliseconds for one kernel name (LLAMA_ERR_INVALID_ARGUMENT if never seen);
 * llama_profile_names() writes the known names, newline-separated, into buf.
 * Not thread-safe: profile from one host thread. */
int llama_profile_enable(int on);
int llama_profile_reset(void);
int llama_profile_collect(void);
int llama_profile_query(const char* kernel_name, int64_t* launches, double* total_ms);
int llama_profile_names(char* buf, size_t cap);

#ifdef __cplusplus
}
#endif

#endif /* LLAMA_BLOCK_H */
