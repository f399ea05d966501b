// RMSNorm with optional fused residual add, one workgroup per row.
//
// Computes, per row, s = x (+ residual), out = s * (mean(s^2) + eps)^-1/2 * gamma
// ("Llama Architecture: RMSNorm, SwiGLU, RoPE, GQA, and PyTorch Implementation"
// §1 and its RMSNorm module; the "RMSNorm" study note, multiply-rsqrt form with
// eps inside the root).  The sum of squares is accumulated in fp32 per lane,
// reduced across the wavefront with butterfly shuffles and across the four
// wavefronts through LDS.  HBM-bound: each element is read once and written
// once; the row stays in registers between the reduction and the scaling.
#include <type_traits>

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

// Wavefront path (d = 256 * 2^k up to 8192): one wavefront per row,
// four rows per workgroup.  Each lane holds d/64 elements as V chunks of
// four (a wavefront load covers 256 contiguous elements), so every lane has V
// loads in flight at once and the sum of squares needs only the wavefront's
// own butterfly, no LDS and no barrier.
// EARLY_G: gamma is loaded with the row rather than after the reduction, one
// memory round trip per row instead of two (what sets the time of a few rows,
// as in decode), at the cost of the registers that hold it (occupancy, what
// sets the time of many rows).
template <typename TR, typename TO, int V, bool EARLY_G>
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_wave_kernel(const TR* __restrict__ x, const TR* __restrict__ res,
                    const TO* __restrict__ gamma, TO* __restrict__ out, TR* sum_out,
                    int64_t rows, int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kNormThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t base = row * d;
  float v[V][4];
  float gm[EARLY_G ? V : 1][4];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < V; ++c) Vec4<TR>::load(x + base + 4 * (lane + 64 * c), v[c]);
  if constexpr (EARLY_G) {
#pragma unroll
    for (int c = 0; c < V; ++c) Vec4<TO>::load(gamma + 4 * (lane + 64 * c), gm[c]);
  }
  if (res) {
#pragma unroll
    for (int c = 0; c < V; ++c) {
      float r[4];
      Vec4<TR>::load(res + base + 4 * (lane + 64 * c), r);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[c][e] += r[e];
    }
  }
#pragma unroll
  for (int c = 0; c < V; ++c) {
    if (sum_out) Vec4<TR>::store(sum_out + base + 4 * (lane + 64 * c), v[c]);
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += v[c][e] * v[c][e];
  }
  const float inv = rsqrtf(wave_sum(ss) / static_cast<float>(d) + eps);
#pragma unroll
  for (int c = 0; c < V; ++c) {
    float g[4], o[4];
    if constexpr (EARLY_G) {
#pragma unroll
      for (int e = 0; e < 4; ++e) g[e] = gm[c][e];
    } else {
      Vec4<TO>::load(gamma + 4 * (lane + 64 * c), g);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = v[c][e] * inv * g[e];
    Vec4<TO>::store(out + base + 4 * (lane + 64 * c), o);
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
  const int per_lane = d % 256 == 0 ? d / 256 : 0;  // 4-element chunks per lane on the wavefront path
  if (per_lane == 1 || per_lane == 2 || per_lane == 4 || per_lane == 8 || per_lane == 16 || per_lane == 32) {
    const dim3 wgrid(static_cast<unsigned>((rows + 3) / 4));
    // fewer row workgroups than CUs: latency-bound, gamma with the row
    const bool early = (rows + 3) / 4 < 256;
    auto go = [&](auto vc) {
      constexpr int V = decltype(vc)::value;
      if (early)
        hipLaunchKernelGGL((rmsnorm_wave_kernel<TR, TO, V, true>), wgrid, block, 0, s, xp, rp, gp, op, sp, rows, d, eps);
      else
        hipLaunchKernelGGL((rmsnorm_wave_kernel<TR, TO, V, false>), wgrid, block, 0, s, xp, rp, gp, op, sp, rows, d, eps);
    };
    switch (per_lane) {
      case 1: go(std::integral_constant<int, 1>{}); break;
      case 2: go(std::integral_constant<int, 2>{}); break;
      case 4: go(std::integral_constant<int, 4>{}); break;
      case 8: go(std::integral_constant<int, 8>{}); break;
      case 16: go(std::integral_constant<int, 16>{}); break;
      default: go(std::integral_constant<int, 32>{}); break;
    }
    return hipGetLastError();
  }
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
