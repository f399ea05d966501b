// Shared device helpers for the gfx950 (CDNA4) kernels: bf16 storage
// conversions, MFMA operand types, wavefront reductions and the RoPE angle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lb {

typedef uint16_t bf16_t;  // raw bfloat16 storage

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// scalar conversions (bf16 storage is the upper half of an IEEE binary32)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, b);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values to a packed bf16 pair (one v_cvt_pk_bf16_f32, RNE).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return Elem<T>::load(p); }
template <typename T>
__device__ __forceinline__ void st(T* p, float v) { Elem<T>::store(p, v); }

// Four consecutive elements (16-byte aligned for float, 8-byte for bf16).
template <typename T> struct Vec4;
template <> struct Vec4<float> {
  static __device__ __forceinline__ void load(const float* p, float v[4]) {
    f32x4 t = *reinterpret_cast<const f32x4*>(p);
    v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
  }
  static __device__ __forceinline__ void store(float* p, const float v[4]) {
    f32x4 t = {v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p) = t;
  }
};
template <> struct Vec4<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float v[4]) {
    u32x2 t = *reinterpret_cast<const u32x2*>(p);
    v[0] = __uint_as_float(t[0] << 16); v[1] = __uint_as_float(t[0] & 0xffff0000u);
    v[2] = __uint_as_float(t[1] << 16); v[3] = __uint_as_float(t[1] & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float v[4]) {
    u32x2 t = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2*>(p) = t;
  }
};

// ---------------------------------------------------------------------------
// buffer loads: a 128-bit resource (base, size in bytes) in SGPRs, a per-lane
// byte offset and a wave-uniform byte offset; reads past `bytes` return 0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// ---------------------------------------------------------------------------
// wavefront reductions (64 lanes)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// ---------------------------------------------------------------------------
// RoPE angle.  phi = pos * inv_freq with inv_freq = theta^(-2k/hd) precomputed
// in fp64 on the host; the product and its reduction modulo 2*pi are done in
// fp64 so the angle is accurate to ~1e-13 rad even at positions of 1e5+;
// sin/cos of the reduced angle are then evaluated in fp32.
// ---------------------------------------------------------------------------
struct RopeTable {
  double inv_freq[128];  // k = 0 .. hd/2-1 (hd <= 256)
};

// theta_base^(-2k/hd) as base^k with base = theta_base^(-2/hd), by binary
// powering in fp64 (k < 128: at most 7 squarings; relative error about
// k * 2^-53, so at any int32 position the angle moves by < 1e-9 rad).  Used
// where a per-pair table would have to travel by value with the kernel.
__device__ __forceinline__ double rope_inv_freq_pow(double base, int k) {
  double r = 1.0, b = base;
  while (k) {
    if (k & 1) r *= b;
    b *= b;
    k >>= 1;
  }
  return r;
}

// Angle reduction in fp64: phi = pos * inv_freq is formed and reduced to
// [-1/2, 1/2] revolutions exactly enough (~1e-16 relative) for any int32
// position; the reduced angle then has an fp32 error of ~2e-7 rad.
__device__ __forceinline__ float rope_revolutions(int pos, double inv_freq) {
  const double inv_two_pi = 0.15915494309189533576888376337251;
  const double rev = static_cast<double>(pos) * inv_freq * inv_two_pi;
  return static_cast<float>(rev - rint(rev));
}

// Accurate sin/cos (fp32 outputs).
__device__ __forceinline__ void rope_sincos(int pos, double inv_freq, float* s, float* c) {
  const float r = rope_revolutions(pos, inv_freq) * 6.2831853071795865f;
  sincosf(r, s, c);
}

// Hardware sin/cos of the reduced angle (v_sin_f32 / v_cos_f32 take
// revolutions); their error is far below half a bf16 ulp, so they serve
// every bf16 output.
__device__ __forceinline__ void rope_sincos_fast(int pos, double inv_freq, float* s, float* c) {
  const float r = rope_revolutions(pos, inv_freq);
  *s = __builtin_amdgcn_sinf(r);
  *c = __builtin_amdgcn_cosf(r);
}

template <typename T>
__device__ __forceinline__ void rope_sincos_t(int pos, double inv_freq, float* s, float* c) {
  if constexpr (sizeof(T) == 2)
    rope_sincos_fast(pos, inv_freq, s, c);
  else
    rope_sincos(pos, inv_freq, s, c);
}

// SiLU(z) = z / (1 + e^-z).  For bf16 outputs the hardware exp2 and
// reciprocal (about 1 fp32 ulp each) replace the IEEE-accurate sequence.
template <typename TO>
__device__ __forceinline__ float silu_t(float z) {
  if constexpr (sizeof(TO) == 2) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
  } else {
    return z / (1.0f + expf(-z));
  }
}

}  // namespace lb
