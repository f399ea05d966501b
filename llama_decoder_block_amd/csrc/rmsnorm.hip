// RMSNorm with optional fused residual add, one workgroup per row.
//
// Computes, per row, s = x (+ residual), out = s * (mean(s^2) + eps)^-1/2 * gamma
// ("Llama Architecture: RMSNorm, SwiGLU, RoPE, GQA, and PyTorch Implementation"
// §1 and its RMSNorm module; the "RMSNorm" study note, multiply-rsqrt form with
// eps inside the root).  The sum of squares is accumulated in fp32 per lane,
// reduced across the wavefront with butterfly shuffles and across the four
// wavefronts through LDS.  HBM-bound: each element is read once and written
// once; the row stays in registers between the reduction and the scaling.
#include "common.hpp"
#include "kernels.hpp"

namespace lb {

namespace {

constexpr int kNormThreads = 256;

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kNormThreads / 64; ++i) t += red[i];
  return t;
}

// Vector path: d % 4 == 0, every row held in registers (d <= 4*256*CH).
template <typename TR, typename TO, int CH>
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_vec_kernel(const TR* __restrict__ x, const TR* __restrict__ res,
                   const TO* __restrict__ gamma, TO* __restrict__ out, TR* sum_out,
                   int d, float eps) {
  __shared__ float red[kNormThreads / 64];
  const int64_t row = blockIdx.x;
  const TR* xr = x + row * d;
  const int nchunk = d >> 2;
  float v[CH][4];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = threadIdx.x + c * kNormThreads;
    if (ch < nchunk) {
      Vec4<TR>::load(xr + 4 * ch, v[c]);
      if (res) {
        float r[4];
        Vec4<TR>::load(res + row * d + 4 * ch, r);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[c][e] += r[e];
      }
      if (sum_out) Vec4<TR>::store(sum_out + row * d + 4 * ch, v[c]);
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += v[c][e] * v[c][e];
    }
  }
  const float tot = block_sum(ss, red);
  const float inv = rsqrtf(tot / static_cast<float>(d) + eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = threadIdx.x + c * kNormThreads;
    if (ch < nchunk) {
      float g[4], o[4];
      Vec4<TO>::load(gamma + 4 * ch, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = v[c][e] * inv * g[e];
      Vec4<TO>::store(out + row * d + 4 * ch, o);
    }
  }
}

// Generic path: any d; the second pass re-reads the row (L2-resident).
template <typename TR, typename TO>
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_any_kernel(const TR* __restrict__ x, const TR* __restrict__ res,
                   const TO* __restrict__ gamma, TO* __restrict__ out, TR* sum_out,
                   int d, float eps) {
  __shared__ float red[kNormThreads / 64];
  const int64_t row = blockIdx.x;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += kNormThreads) {
    float s = ld(x + row * d + i);
    if (res) s += ld(res + row * d + i);
    ss += s * s;
  }
  const float tot = block_sum(ss, red);
  const float inv = rsqrtf(tot / static_cast<float>(d) + eps);
  for (int i = threadIdx.x; i < d; i += kNormThreads) {
    float s = ld(x + row * d + i);
    if (res) s += ld(res + row * d + i);
    if (sum_out) st(sum_out + row * d + i, s);
    st(out + row * d + i, s * inv * ld(gamma + i));
  }
}

template <typename TR, typename TO>
hipError_t launch_rmsnorm_t(const void* x, const void* res, const void* gamma, void* out,
                            void* sum_out, int64_t rows, int d, float eps, hipStream_t s) {
  const TR* xp = static_cast<const TR*>(x);
  const TR* rp = static_cast<const TR*>(res);
  const TO* gp = static_cast<const TO*>(gamma);
  TO* op = static_cast<TO*>(out);
  TR* sp = static_cast<TR*>(sum_out);
  dim3 grid(static_cast<unsigned>(rows)), block(kNormThreads);
  const bool vec = (d % 4 == 0);
  const int chunks_per_thread = (d / 4 + kNormThreads - 1) / kNormThreads;
  if (vec && chunks_per_thread <= 2)
    hipLaunchKernelGGL((rmsnorm_vec_kernel<TR, TO, 2>), grid, block, 0, s, xp, rp, gp, op, sp, d, eps);
  else if (vec && chunks_per_thread <= 4)
    hipLaunchKernelGGL((rmsnorm_vec_kernel<TR, TO, 4>), grid, block, 0, s, xp, rp, gp, op, sp, d, eps);
  else if (vec && chunks_per_thread <= 8)
    hipLaunchKernelGGL((rmsnorm_vec_kernel<TR, TO, 8>), grid, block, 0, s, xp, rp, gp, op, sp, d, eps);
  else
    hipLaunchKernelGGL((rmsnorm_any_kernel<TR, TO>), grid, block, 0, s, xp, rp, gp, op, sp, d, eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, const void* res, const void* gamma, void* out,
                          void* sum_out, int64_t rows, int d, float eps, DType wdt, DType rdt,
                          hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (rdt == DType::F32 && wdt == DType::F32)
    return launch_rmsnorm_t<float, float>(x, res, gamma, out, sum_out, rows, d, eps, s);
  if (rdt == DType::F32 && wdt == DType::BF16)
    return launch_rmsnorm_t<float, bf16_t>(x, res, gamma, out, sum_out, rows, d, eps, s);
  if (rdt == DType::BF16 && wdt == DType::BF16)
    return launch_rmsnorm_t<bf16_t, bf16_t>(x, res, gamma, out, sum_out, rows, d, eps, s);
  return launch_rmsnorm_t<bf16_t, float>(x, res, gamma, out, sum_out, rows, d, eps, s);
}

}  // namespace lb
