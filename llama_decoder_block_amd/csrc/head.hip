// Greedy token choice from the output layer's logits ("LLaMA-3 8B 现代 LLM
// 架构、计算规模与能耗" §十: after the last block, a final RMSNorm, the linear
// head to vocabulary logits, and argmax as the deterministic choice among the
// sampling methods it lists; argmax of the softmax is argmax of the logits).
//
// argmax_chunk_kernel: one workgroup of 256 threads per (row, 4096-column
// chunk) of fp32 logits.  Each thread scans its columns with 16-byte loads
// (scalar loads when the row length is not a multiple of 4), keeping the
// largest value and, among equal values, the smallest column; the wavefronts
// reduce their (value, column) pairs with shuffles and meet in LDS.
// argmax_merge_kernel: one wavefront per row merges the chunks' candidates
// with the same rule.  NaN never compares greater, so a NaN logit is never
// chosen (a row of NaN only returns column 0).
#include "common.hpp"
#include "kernels.hpp"

namespace lb {

namespace {

__device__ __forceinline__ void better(float v, int i, float& bv, int& bi) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// (value, column) of the best element of columns [c0, c1) of one row, for the
// whole workgroup (thread 0 holds it)
__device__ __forceinline__ void block_best(const float* p, int c0, int c1, bool vec, float& bv, int& bi) {
  const int tid = threadIdx.x;
  bv = -INFINITY;
  bi = 0x7fffffff;
  if (vec) {
    for (int c = c0 / 4 + tid; c < c1 / 4; c += 256) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p + 4 * static_cast<int64_t>(c));
#pragma unroll
      for (int e = 0; e < 4; ++e) better(v[e], 4 * c + e, bv, bi);
    }
  } else {
    for (int c = c0 + tid; c < c1; c += 256) better(p[c], c, bv, bi);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off, kWave);
    const int oi = __shfl_xor(bi, off, kWave);
    better(ov, oi, bv, bi);
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  const int w = tid >> 6;
  if ((tid & 63) == 0) {
    sv[w] = bv;
    si[w] = bi;
  }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int k = 1; k < 4; ++k) better(sv[k], si[k], bv, bi);
  }
}

// pass 1: workgroup (chunk, row) reduces kArgChunk columns to one candidate
constexpr int kArgChunk = 4096;

__global__ void __launch_bounds__(256)
argmax_chunk_kernel(const float* __restrict__ logits, int64_t ld, int n, int chunks, float* __restrict__ cand_v,
                    int32_t* __restrict__ cand_i) {
  const int chunk = blockIdx.x;
  const int64_t row = blockIdx.y;
  const int c0 = chunk * kArgChunk, c1 = min(n, c0 + kArgChunk);
  float bv;
  int bi;
  block_best(logits + row * ld, c0, c1, (n & 3) == 0 && (ld & 3) == 0, bv, bi);
  if (threadIdx.x == 0) {
    cand_v[row * chunks + chunk] = bv;
    cand_i[row * chunks + chunk] = bi;
  }
}

// pass 2: one wavefront per row merges the row's candidates
__global__ void __launch_bounds__(256)
argmax_merge_kernel(const float* __restrict__ cand_v, const int32_t* __restrict__ cand_i, int64_t rows, int chunks,
                    int32_t* __restrict__ token, float* __restrict__ best_value) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int c = lane; c < chunks; c += 64) better(cand_v[row * chunks + c], cand_i[row * chunks + c], bv, bi);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off, kWave);
    const int oi = __shfl_xor(bi, off, kWave);
    better(ov, oi, bv, bi);
  }
  if (lane == 0) {
    token[row] = bi == 0x7fffffff ? 0 : bi;
    if (best_value) best_value[row] = bv;
  }
}

}  // namespace

size_t argmax_workspace_bytes(int64_t rows, int n) {
  const int64_t chunks = (n + kArgChunk - 1) / kArgChunk;
  return static_cast<size_t>(rows * chunks) * (sizeof(float) + sizeof(int32_t));
}

hipError_t launch_argmax_rows(const float* logits, int64_t rows, int64_t ld, int n, int32_t* token,
                              float* best_value, void* ws, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int chunks = (n + kArgChunk - 1) / kArgChunk;
  float* cand_v = static_cast<float*>(ws);
  int32_t* cand_i = reinterpret_cast<int32_t*>(cand_v + rows * chunks);
  hipLaunchKernelGGL(argmax_chunk_kernel, dim3(static_cast<unsigned>(chunks), static_cast<unsigned>(rows)),
                     dim3(256), 0, s, logits, ld, n, chunks, cand_v, cand_i);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(argmax_merge_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, s, cand_v,
                     cand_i, rows, chunks, token, best_value);
  return hipGetLastError();
}

}  // namespace lb
