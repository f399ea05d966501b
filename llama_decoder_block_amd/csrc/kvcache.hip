// 8-bit KV cache writer.  "Llama Architecture: RMSNorm, SwiGLU, RoPE, GQA, and
// PyTorch Implementation", "Troubleshooting Common Deployment Faults" item 3,
// names an 8-bit KV cache as the way to halve the bytes-per-element factor of
// the KV-cache memory formula of its §4; the pages fix no format or scale, so
// this library uses OCP FP8 E4M3 codes with one fp32 scale per cached row:
//   s = max_i |x_i| / 448 (fp32 division), code_i = E4M3 of x_i / s (fp32
//   division), rounded to nearest with ties to the even mantissa, magnitudes
//   beyond 448 clamped to 448, the sign kept; a row whose maximum is 0 stores
//   s = 0 and all-zero codes.  The stored value is s * E4M3(code).
//
// kv_append_fp8_kernel: one wavefront per (token, KV head, K or V) row of hd
// elements; the row maximum is a wavefront reduction and the encoding is done
// on the fp32 bit pattern (exponent and mantissa fields), not with a
// conversion instruction, so its rounding is exactly the rule above.
// kv_append_paged_kernel: the bf16 rows of new tokens into a paged cache
// (the same page's slots are consecutive; the block table maps a sequence's
// slot range to pages of a shared pool, the remedy the same troubleshooting
// item names for fragmented contiguous caches).
#include "common.hpp"
#include "kernels.hpp"

namespace lb {

namespace {

// E4M3 code of q: |q| >= 448 -> 0x7E; |q| < 2^-6 -> subnormal code
// rint(|q| * 2^9) (0..8, where 8 is the first normal code); otherwise with
// |q| in [2^e, 2^(e+1)) the mantissa rint(|q| * 2^(3-e)) in 8..16 (16 carries
// into the next binade's code).  rint rounds half to even.  NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  if (a != a) return 0x7Fu;
  uint32_t c;
  if (a >= 448.f) {
    c = 0x7Eu;
  } else if (a < 0.015625f) {
    c = static_cast<uint32_t>(__builtin_rintf(a * 512.f));
  } else {
    const int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xffu) - 127;
    const float m = __builtin_rintf(__builtin_ldexpf(a, 3 - e));
    c = static_cast<uint32_t>((e + 7) * 8) + static_cast<uint32_t>(m) - 8u;
    c = c > 0x7Eu ? 0x7Eu : c;
  }
  return c | sign;
}

template <typename T, int EPL>
__global__ void __launch_bounds__(256)
kv_append_fp8_kernel(const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ positions,
                     int64_t n_tokens, int seq_len, int nkv, uint8_t* __restrict__ k8, uint8_t* __restrict__ v8,
                     float* __restrict__ ks, float* __restrict__ vs, int kv_cap) {
  constexpr int HD = EPL * 64;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);  // (token, head, k|v)
  if (row >= n_tokens * nkv * 2) return;
  const bool is_v = row & 1;
  const int64_t th = row >> 1;
  const int g = static_cast<int>(th % nkv);
  const int64_t n = th / nkv;
  const int pos = positions[n];
  if (pos < 0 || pos >= kv_cap) return;
  const int64_t b = n / seq_len;
  const T* src = (is_v ? v : k) + th * HD + lane * EPL;
  float x[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) x[i] = Elem<T>::load(src + i);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = wave_max(amax);
  const float s = amax / 448.f;
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) packed |= (s == 0.f ? 0u : e4m3_code(x[i] / s)) << (8 * i);
  uint8_t* dst = (is_v ? v8 : k8) + ((b * nkv + g) * kv_cap + pos) * HD + lane * EPL;
  if constexpr (EPL == 1) *dst = static_cast<uint8_t>(packed);
  if constexpr (EPL == 2) *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(packed);
  if constexpr (EPL == 4) *reinterpret_cast<uint32_t*>(dst) = packed;
  if (lane == 0) (is_v ? vs : ks)[(b * nkv + g) * kv_cap + pos] = s;
}

template <typename T>
hipError_t launch_append_t(const void* k, const void* v, const int32_t* positions, int64_t n_tokens, int seq_len,
                           int nkv, int hd, void* k8, void* v8, float* k_scale, float* v_scale, int kv_cap,
                           hipStream_t s) {
  const int64_t rows = n_tokens * nkv * 2;
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  const T* kp = static_cast<const T*>(k);
  const T* vp = static_cast<const T*>(v);
  uint8_t* k8p = static_cast<uint8_t*>(k8);
  uint8_t* v8p = static_cast<uint8_t*>(v8);
  switch (hd) {
    case 64:
      hipLaunchKernelGGL((kv_append_fp8_kernel<T, 1>), grid, dim3(256), 0, s, kp, vp, positions, n_tokens, seq_len, nkv,
                         k8p, v8p, k_scale, v_scale, kv_cap);
      break;
    case 128:
      hipLaunchKernelGGL((kv_append_fp8_kernel<T, 2>), grid, dim3(256), 0, s, kp, vp, positions, n_tokens, seq_len, nkv,
                         k8p, v8p, k_scale, v_scale, kv_cap);
      break;
    case 256:
      hipLaunchKernelGGL((kv_append_fp8_kernel<T, 4>), grid, dim3(256), 0, s, kp, vp, positions, n_tokens, seq_len, nkv,
                         k8p, v8p, k_scale, v_scale, kv_cap);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Paged bf16 cache writer: one thread per 16 bytes of a (token, KV head) row.
__global__ void __launch_bounds__(256)
kv_append_paged_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v, const int32_t* __restrict__ positions,
                       int64_t n_tokens, int seq_len, int nkv, int chunks, const int32_t* __restrict__ table,
                       int max_pages, int page_size, int64_t n_pages, u32x4* __restrict__ kp, u32x4* __restrict__ vp) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;  // (token, head, chunk)
  const int64_t row_chunks = static_cast<int64_t>(nkv) * chunks;
  if (i >= n_tokens * row_chunks) return;
  const int64_t n = i / row_chunks;
  const int64_t within = i - n * row_chunks;  // head * chunks + chunk
  const int pos = positions[n];
  const int64_t b = n / seq_len;
  if (pos < 0 || pos >= max_pages * page_size) return;
  const int64_t pg = table[b * max_pages + pos / page_size];
  if (pg < 0 || pg >= n_pages) return;
  const int64_t dst = ((pg * page_size + pos % page_size) * nkv) * chunks + within;
  kp[dst] = k[i];
  vp[dst] = v[i];
}

}  // namespace

hipError_t launch_kv_append_paged(const void* k, const void* v, const int32_t* positions, int64_t n_tokens,
                                  int seq_len, int nkv, int hd, const int32_t* block_table, int max_pages,
                                  int page_size, int64_t n_pages, void* k_pool, void* v_pool, hipStream_t s) {
  if (n_tokens == 0) return hipSuccess;
  if (hd % 8 != 0) return hipErrorInvalidValue;
  const int chunks = hd / 8;  // 16-byte pieces of a bf16 row
  const int64_t threads = n_tokens * nkv * chunks;
  hipLaunchKernelGGL(kv_append_paged_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s,
                     static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), positions, n_tokens, seq_len, nkv,
                     chunks, block_table, max_pages, page_size, n_pages, static_cast<u32x4*>(k_pool),
                     static_cast<u32x4*>(v_pool));
  return hipGetLastError();
}

hipError_t launch_kv_append_fp8(const void* k, const void* v, const int32_t* positions, int64_t n_tokens,
                                int seq_len, int nkv, int hd, DType dt, void* k8, void* v8, float* k_scale,
                                float* v_scale, int kv_cap, hipStream_t s) {
  if (n_tokens == 0) return hipSuccess;
  if (dt == DType::BF16)
    return launch_append_t<bf16_t>(k, v, positions, n_tokens, seq_len, nkv, hd, k8, v8, k_scale, v_scale, kv_cap, s);
  return launch_append_t<float>(k, v, positions, n_tokens, seq_len, nkv, hd, k8, v8, k_scale, v_scale, kv_cap, s);
}

}  // namespace lb
