// Standalone in-place RoPE on Q [n_tokens, n_q, hd] and K [n_tokens, n_kv, hd].
//
// Adjacent pairs (x_2k, x_2k+1) of each head at position m are rotated by
// m * theta^(-2k/hd) ("Llama Architecture: RMSNorm, SwiGLU, RoPE, GQA, and
// PyTorch Implementation" §3, rotation matrix; "LLaMA-3 8B 现代 LLM 架构、计算规模与能耗"
// §四.3).  Each thread handles four consecutive elements (two pairs) of one
// token row, so a wavefront reads and writes 64 x 4 contiguous elements.
// HBM-bound: every element of Q and K is read once and written once.
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
