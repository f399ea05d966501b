// Standalone in-place RoPE on Q [n_tokens, n_q, hd] and K [n_tokens, n_kv, hd].
//
// Adjacent pairs (x_2k, x_2k+1) of each head at position m are rotated by
// m * theta^(-2k/hd) ("Llama Architecture: RMSNorm, SwiGLU, RoPE, GQA, and
// PyTorch Implementation" §3, rotation matrix; "LLaMA-3 8B 现代 LLM 架构、计算规模与能耗"
// §四.3).  HBM-bound: every element of Q and K is read once and written once.
//
// Main kernel (head_dim a multiple of one 16-byte vector): one launch covers Q
// and K.  A thread owns one 16-byte column vector of the head (8 bf16 or 4
// fp32 elements) at one token, forms that vector's angles once, and applies
// them to the same column of up to kHeadsPerThread heads (Q heads first, then
// K heads), whose loads are all issued before the first store.  Sixteen
// lanes cover one 256-byte head row of bf16, so every access is a whole
// 16-byte vector in a contiguous run.
#include "common.hpp"
#include "kernels.hpp"

namespace lb {

namespace {

template <typename T>
__global__ void __launch_bounds__(256)
rope_kernel(T* __restrict__ x, const int32_t* __restrict__ positions, int64_t n_tokens,
            int row_len, int hd, RopeTable rope) {
  // one thread per 4-element group (row_len % 4 == 0, hd % 2 == 0)
  const int groups_per_row = row_len >> 2;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= n_tokens * groups_per_row) return;
  const int64_t tok = gid / groups_per_row;
  const int col = static_cast<int>(gid - tok * groups_per_row) * 4;
  const int pos = positions[tok];
  T* p = x + tok * row_len + col;
  float v[4];
  Vec4<T>::load(p, v);
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    const int kidx = ((col + 2 * pr) % hd) >> 1;
    float s, c;
    rope_sincos_t<T>(pos, rope.inv_freq[kidx], &s, &c);
    const float a = v[2 * pr], b = v[2 * pr + 1];
    v[2 * pr] = a * c - b * s;
    v[2 * pr + 1] = a * s + b * c;
  }
  Vec4<T>::store(p, v);
}

constexpr int kHeadsPerThread = 8;

template <typename T>
__global__ void __launch_bounds__(256)
rope_heads_kernel(T* __restrict__ q, T* __restrict__ k, const int32_t* __restrict__ positions,
                  int64_t n_tokens, int nq, int nkv, int hd, int chunks, RopeTable rope) {
  constexpr int E = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte vector
  constexpr int P = E / 2;                              // pairs per vector
  const int vecs = hd / E;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= n_tokens * chunks * vecs) return;
  const int vi = static_cast<int>(gid % vecs);
  const int64_t rest = gid / vecs;
  const int chunk = static_cast<int>(rest % chunks);
  const int64_t tok = rest / chunks;
  const int pos = positions[tok];
  float sn[P], cs[P];
#pragma unroll
  for (int p = 0; p < P; ++p) rope_sincos_t<T>(pos, rope.inv_freq[vi * P + p], &sn[p], &cs[p]);

  const int h0 = chunk * kHeadsPerThread;
  const int nh = min(kHeadsPerThread, nq + nkv - h0);
  u32x4* ptr[kHeadsPerThread];
  u32x4 v[kHeadsPerThread];
#pragma unroll
  for (int j = 0; j < kHeadsPerThread; ++j) {
    const int h = h0 + j;
    T* row = h < nq ? q + (tok * nq + h) * static_cast<int64_t>(hd)
                    : k + (tok * nkv + (h - nq)) * static_cast<int64_t>(hd);
    ptr[j] = reinterpret_cast<u32x4*>(row + vi * E);
    if (j < nh) v[j] = *ptr[j];
  }
#pragma unroll
  for (int j = 0; j < kHeadsPerThread; ++j) {
    if (j >= nh) break;
    float x[E];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        x[2 * w] = __uint_as_float(v[j][w] << 16);
        x[2 * w + 1] = __uint_as_float(v[j][w] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) x[w] = __uint_as_float(v[j][w]);
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const float a = x[2 * p], b = x[2 * p + 1];
      x[2 * p] = a * cs[p] - b * sn[p];
      x[2 * p + 1] = a * sn[p] + b * cs[p];
    }
    u32x4 o;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = pack_bf16x2(x[2 * w], x[2 * w + 1]);
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = __float_as_uint(x[w]);
    }
    *ptr[j] = o;
  }
}

template <typename T>
hipError_t rope_heads(T* q, T* k, const int32_t* positions, int64_t n_tokens, int nq, int nkv, int hd,
                      const RopeTable& rope, hipStream_t s) {
  constexpr int E = 16 / static_cast<int>(sizeof(T));
  const int chunks = (nq + nkv + kHeadsPerThread - 1) / kHeadsPerThread;
  const int64_t n = n_tokens * chunks * (hd / E);
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  hipLaunchKernelGGL((rope_heads_kernel<T>), dim3(blocks), dim3(256), 0, s, q, k, positions, n_tokens, nq, nkv,
                     hd, chunks, rope);
  return hipGetLastError();
}

// Fallback for rows whose length is not a multiple of 4: one thread per pair.
template <typename T>
__global__ void __launch_bounds__(256)
rope_pair_kernel(T* __restrict__ x, const int32_t* __restrict__ positions, int64_t n_tokens,
                 int row_len, int hd, RopeTable rope) {
  const int pairs_per_row = row_len >> 1;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= n_tokens * pairs_per_row) return;
  const int64_t tok = gid / pairs_per_row;
  const int col = static_cast<int>(gid - tok * pairs_per_row) * 2;
  const int pos = positions[tok];
  T* p = x + tok * row_len + col;
  float s, c;
  rope_sincos_t<T>(pos, rope.inv_freq[(col % hd) >> 1], &s, &c);
  const float a = ld(p), b = ld(p + 1);
  st(p, a * c - b * s);
  st(p + 1, a * s + b * c);
}

template <typename T>
hipError_t rope_one(T* x, const int32_t* positions, int64_t n_tokens, int heads, int hd,
                    const RopeTable& rope, hipStream_t s) {
  const int row_len = heads * hd;
  if (row_len % 4 == 0) {
    const int64_t n = n_tokens * (row_len / 4);
    const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
    hipLaunchKernelGGL((rope_kernel<T>), dim3(blocks), dim3(256), 0, s, x, positions, n_tokens,
                       row_len, hd, rope);
  } else {
    const int64_t n = n_tokens * (row_len / 2);
    const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
    hipLaunchKernelGGL((rope_pair_kernel<T>), dim3(blocks), dim3(256), 0, s, x, positions,
                       n_tokens, row_len, hd, rope);
  }
  return hipGetLastError();
}

// One thread per (token row, pair): the rotation angle's (cos, sin).
template <typename T>
__global__ void __launch_bounds__(256)
rope_table_kernel(const int32_t* __restrict__ positions, int64_t n_tokens, int half, RopeTable rope,
                  f32x2* __restrict__ cs) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= n_tokens * half) return;
  const int64_t tok = gid / half;
  const int k = static_cast<int>(gid - tok * half);
  float s, c;
  rope_sincos_t<T>(positions[tok], rope.inv_freq[k], &s, &c);
  cs[gid] = f32x2{c, s};
}

}  // namespace

hipError_t launch_rope_table(const int32_t* positions, int64_t n_tokens, int hd, const RopeTable& rope,
                             DType dt, float* cs, hipStream_t s) {
  if (n_tokens == 0) return hipSuccess;
  const int half = hd / 2;
  const unsigned blocks = static_cast<unsigned>((n_tokens * half + 255) / 256);
  if (dt == DType::F32)
    hipLaunchKernelGGL((rope_table_kernel<float>), dim3(blocks), dim3(256), 0, s, positions, n_tokens, half, rope,
                       reinterpret_cast<f32x2*>(cs));
  else
    hipLaunchKernelGGL((rope_table_kernel<bf16_t>), dim3(blocks), dim3(256), 0, s, positions, n_tokens, half, rope,
                       reinterpret_cast<f32x2*>(cs));
  return hipGetLastError();
}

hipError_t launch_rope(void* q, void* k, const int32_t* positions, int64_t n_tokens, int nq,
                       int nkv, int hd, const RopeTable& rope, DType dt, hipStream_t s) {
  if (n_tokens == 0) return hipSuccess;
  const int nq_used = q ? nq : 0, nkv_used = k ? nkv : 0;
  if (hd % (dt == DType::F32 ? 4 : 8) == 0)
    return dt == DType::F32
               ? rope_heads(static_cast<float*>(q), static_cast<float*>(k), positions, n_tokens, nq_used,
                            nkv_used, hd, rope, s)
               : rope_heads(static_cast<bf16_t*>(q), static_cast<bf16_t*>(k), positions, n_tokens, nq_used,
                            nkv_used, hd, rope, s);
  hipError_t e = hipSuccess;
  if (q) {
    e = dt == DType::F32
            ? rope_one(static_cast<float*>(q), positions, n_tokens, nq, hd, rope, s)
            : rope_one(static_cast<bf16_t*>(q), positions, n_tokens, nq, hd, rope, s);
    if (e != hipSuccess) return e;
  }
  if (k) {
    e = dt == DType::F32
            ? rope_one(static_cast<float*>(k), positions, n_tokens, nkv, hd, rope, s)
            : rope_one(static_cast<bf16_t*>(k), positions, n_tokens, nkv, hd, rope, s);
  }
  return e;
}

}  // namespace lb
