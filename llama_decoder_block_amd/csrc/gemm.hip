// GEMMs of the block: acc[m][n] = sum_k X[m][k] * W[n][k] (both operands K-
// contiguous, weights stored [out, in] as nn.Linear stores them in "Llama
// Architecture: RMSNorm, SwiGLU, RoPE, GQA, and PyTorch Implementation",
// "Production PyTorch Implementation"), followed by a fused epilogue:
// RoPE + Q/K/V (cache) stores, SiLU(gate) * up, residual add, or a plain store.
//
// gemm_mfma_kernel: bf16 operands on the CDNA4 matrix cores
//   (v_mfma_f32_32x32x16_bf16), fp32 accumulation.  Four wavefronts in a 2x2
//   arrangement; each owns a (BN/2) x (BM/2) block of the output as 32x32
//   MFMA tiles.  The weight tile is the MFMA "A" operand and the activation
//   tile the "B" operand, so each lane ends up with four consecutive output
//   columns (feature index) of one token row: RoPE pairs and 4-wide stores
//   stay inside a lane.  K is walked in steps of 64 through two LDS buffers;
//   the next step's global loads are in flight while the current step's
//   MFMAs run.  LDS rows are 128 B (64 bf16) with the 16-byte chunk index
//   XOR-swizzled by the row pair so that fragment reads do not collide in banks.
// gemm_valu_kernel: generic fp32-accumulating kernel for the fp32 path and
//   for shapes the MFMA kernel does not take (K % 8 != 0).
// split-K: for few token rows (decode) the MFMA kernel writes fp32 partial
//   sums per K-slice and splitk_reduce_kernel sums them and applies the
//   epilogue, so enough workgroups stream the weights.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lb {

namespace {

// ---------------------------------------------------------------------------
// weight row resolution over up to three segments
// ---------------------------------------------------------------------------
template <typename T>
struct WRows {
  const T* p[3];
  int s1, s2;  // segment starts 1 and 2 (INT_MAX if absent)
  int64_t ld;
  __device__ __forceinline__ const T* row(int n) const {
    if (n < s1) return p[0] + static_cast<int64_t>(n) * ld;
    if (n < s2) return p[1] + static_cast<int64_t>(n - s1) * ld;
    return p[2] + static_cast<int64_t>(n - s2) * ld;
  }
};

template <typename T>
WRows<T> make_rows(const WSeg& w, int K) {
  WRows<T> r;
  for (int i = 0; i < 3; ++i) r.p[i] = static_cast<const T*>(w.ptr[i < w.nseg ? i : 0]);
  r.s1 = w.nseg > 1 ? w.start[1] : 0x7fffffff;
  r.s2 = w.nseg > 2 ? w.start[2] : 0x7fffffff;
  r.ld = K;
  return r;
}

// XCD-aware tile order.  Consecutive workgroup ids are dealt round-robin to
// the 8 XCDs; remapping gives each XCD a contiguous range of the logical
// order, and the logical order walks GROUP_M row tiles before moving along
// N so that tiles resident on one XCD share operand panels in its L2.
__device__ __forceinline__ void tile_coords(int bid, int nblk, int tiles_m, int tiles_n,
                                            int* tm, int* tn) {
  int logical = bid;
  if ((nblk & 7) == 0) logical = (bid & 7) * (nblk >> 3) + (bid >> 3);
  constexpr int GROUP_M = 8;
  const int group_size = GROUP_M * tiles_n;
  const int group = logical / group_size;
  const int first_m = group * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in_group = logical - group * group_size;
  *tm = first_m + in_group % gm;
  *tn = in_group / gm;
}

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------
constexpr int kBK = 64;

// LDS tile rows are 128 B (64 bf16 of K).  gfx950 serves a 16-byte-per-lane
// LDS read 16 lanes (256 B, all 64 banks) at a time; a fragment read has 16
// consecutive lanes on 16 consecutive rows at the same K chunk, and each pair
// of rows shares one 256-B bank line.  XOR-ing the chunk index with
// (row / 2) % 8 gives the 8 row pairs 8 distinct chunks, so the 16 lanes hit
// 16 distinct 16-byte bank groups.  The row-major tile stores (8 lanes per
// row) stay conflict-free under the same map.
__device__ __forceinline__ int lds_idx(int row, int chunk) {  // in 16-byte units
  return row * 8 + (chunk ^ ((row >> 1) & 7));
}

template <int BN, int BM, bool DUAL, class Epi>
__global__ void __launch_bounds__(256, 1)
gemm_mfma_kernel(const bf16_t* __restrict__ X, WRows<bf16_t> W, int M, int N, int K,
                 int k_per_split, int tiles_m, int tiles_n, Epi epi) {
  constexpr int WN = BN / 2, WM = BM / 2;
  constexpr int TN = WN / 32, TM = WM / 32;
  constexpr int W_IT = BN / 32, X_IT = BM / 32;
  static_assert(!DUAL || TN % 2 == 0, "dual needs an even number of N subtiles per wave");
  __shared__ u32x4 lds[2][(BN + BM) * 8];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, &tm, &tn);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wave_n = wid & 1, wave_m = wid >> 1;
  const int out_n0 = tn * (DUAL ? BN / 2 : BN);
  const int m0 = tm * BM;
  const int kbeg = blockIdx.z * k_per_split;
  const int kend = min(K, kbeg + k_per_split);
  const int KT = (kend - kbeg + kBK - 1) / kBK;

  const int chunk = tid & 7, rbase = tid >> 3;
  const bf16_t* wsrc[W_IT];
  const bf16_t* xsrc[X_IT];
#pragma unroll
  for (int i = 0; i < W_IT; ++i) {
    const int r = rbase + 32 * i;
    const bf16_t* p;
    if constexpr (DUAL) {
      const int wv = r / WN, rr = r % WN;
      const bool up = rr >= WN / 2;
      int c = out_n0 + wv * (WN / 2) + (rr % (WN / 2));
      c = min(c, N - 1);
      p = (up ? W.p[1] : W.p[0]) + static_cast<int64_t>(c) * W.ld;
    } else {
      p = W.row(min(out_n0 + r, N - 1));
    }
    wsrc[i] = p + kbeg + chunk * 8;
  }
#pragma unroll
  for (int i = 0; i < X_IT; ++i) {
    const int r = min(m0 + rbase + 32 * i, M - 1);
    xsrc[i] = X + static_cast<int64_t>(r) * K + kbeg + chunk * 8;
  }

  u32x4 wreg[W_IT], xreg[X_IT];
  auto gload = [&](int kt) {
    const bool ok = kbeg + kt * kBK + chunk * 8 < kend;
#pragma unroll
    for (int i = 0; i < W_IT; ++i)
      wreg[i] = ok ? *reinterpret_cast<const u32x4*>(wsrc[i] + kt * kBK) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < X_IT; ++i)
      xreg[i] = ok ? *reinterpret_cast<const u32x4*>(xsrc[i] + kt * kBK) : u32x4{0, 0, 0, 0};
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < W_IT; ++i) lds[buf][lds_idx(rbase + 32 * i, chunk)] = wreg[i];
#pragma unroll
    for (int i = 0; i < X_IT; ++i) lds[buf][BN * 8 + lds_idx(rbase + 32 * i, chunk)] = xreg[i];
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  const int frag_row = lane & 31, frag_half = lane >> 5;
  if (KT > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int ch = kk * 2 + frag_half;
      bf16x8 af[TN], bf[TM];
#pragma unroll
      for (int a = 0; a < TN; ++a) {
        const int row = wave_n * WN + a * 32 + frag_row;
        af[a] = __builtin_bit_cast(bf16x8, lds[buf][lds_idx(row, ch)]);
      }
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        const int row = wave_m * WM + b * 32 + frag_row;
        bf[b] = __builtin_bit_cast(bf16x8, lds[buf][BN * 8 + lds_idx(row, ch)]);
      }
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  Output register e of a 32x32 tile holds row (e/4)*8 + half*4 +
  // e%4 of the A operand (feature n) and column lane%32 (token m).
#pragma unroll
  for (int b = 0; b < TM; ++b) {
    const int m = m0 + wave_m * WM + b * 32 + frag_row;
    if (m >= M) continue;
    if constexpr (DUAL) {
#pragma unroll
      for (int a = 0; a < TN / 2; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = out_n0 + wave_n * (WN / 2) + a * 32 + j * 8 + frag_half * 4;
          if (c >= N) continue;
          float g[4], u[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            g[i] = acc[a][b][j * 4 + i];
            u[i] = acc[a + TN / 2][b][j * 4 + i];
          }
          epi(m, c, g, u, min(4, N - c));
        }
    } else {
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = out_n0 + wave_n * WN + a * 32 + j * 8 + frag_half * 4;
          if (n >= N) continue;
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[a][b][j * 4 + i];
          epi(m, n, v, min(4, N - n));
        }
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA kernel, large tiles: 256 x 256 output tile, eight wavefronts (two per
// SIMD, so one wavefront's LDS and memory waits overlap the other's MFMAs).
// Wave grid 2 (N) x 4 (M); each wavefront owns 128 (N) x 64 (M) as 4 x 2
// tiles of 32 x 32.  Requires K % 64 == 0 (no K tail) so that the global
// loads of the next K step are issued unconditionally; rows past M or N are
// clamped on load and dropped by the epilogue.  Fragments of the next
// 16-wide K slice are read from LDS while the current slice's MFMAs run.
// ---------------------------------------------------------------------------
template <bool DUAL, class Epi>
__global__ void __launch_bounds__(512, 2)
gemm_mfma8_kernel(const bf16_t* __restrict__ X, WRows<bf16_t> W, int M, int N, int K,
                  int tiles_m, int tiles_n, Epi epi) {
  constexpr int BN = 256, BM = 256;
  constexpr int WN = 128, WM = 64;
  constexpr int TN = 4, TM = 2;
  constexpr int LD_IT = 4;  // 16-byte loads per thread per operand per K step
  __shared__ u32x4 lds[2][(BN + BM) * 8];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, &tm, &tn);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wave_n = wid & 1, wave_m = wid >> 1;
  const int out_n0 = tn * (DUAL ? BN / 2 : BN);
  const int m0 = tm * BM;
  const int KT = K / kBK;

  const int chunk = tid & 7, rbase = tid >> 3;  // rows rbase + 64 i
  const bf16_t* wsrc[LD_IT];
  const bf16_t* xsrc[LD_IT];
#pragma unroll
  for (int i = 0; i < LD_IT; ++i) {
    const int r = rbase + 64 * i;
    const bf16_t* p;
    if constexpr (DUAL) {
      // LDS rows [0,128): wave_n 0 (gate 0..63, up 0..63); [128,256): wave_n 1
      const int wv = r / WN, rr = r % WN;
      const bool up = rr >= WN / 2;
      const int c = min(out_n0 + wv * (WN / 2) + (rr % (WN / 2)), N - 1);
      p = (up ? W.p[1] : W.p[0]) + static_cast<int64_t>(c) * W.ld;
    } else {
      p = W.row(min(out_n0 + r, N - 1));
    }
    wsrc[i] = p + chunk * 8;
    xsrc[i] = X + static_cast<int64_t>(min(m0 + r, M - 1)) * K + chunk * 8;
  }

  // two register staging sets: the loads of K steps kt+1 and kt+2 are in
  // flight while step kt computes (hides memory latency of ~2 K steps)
  u32x4 wreg[2][LD_IT], xreg[2][LD_IT];
  auto gload = [&](int kt, auto S) {
    constexpr int st = decltype(S)::value;
#pragma unroll
    for (int i = 0; i < LD_IT; ++i) wreg[st][i] = *reinterpret_cast<const u32x4*>(wsrc[i] + kt * kBK);
#pragma unroll
    for (int i = 0; i < LD_IT; ++i) xreg[st][i] = *reinterpret_cast<const u32x4*>(xsrc[i] + kt * kBK);
  };
  auto lstore = [&](int buf, auto S) {
    constexpr int st = decltype(S)::value;
#pragma unroll
    for (int i = 0; i < LD_IT; ++i) lds[buf][lds_idx(rbase + 64 * i, chunk)] = wreg[st][i];
#pragma unroll
    for (int i = 0; i < LD_IT; ++i) lds[buf][BN * 8 + lds_idx(rbase + 64 * i, chunk)] = xreg[st][i];
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  f32x16 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  const int frag_row = lane & 31, frag_half = lane >> 5;
  int arow[TN], brow[TM];
#pragma unroll
  for (int a = 0; a < TN; ++a) arow[a] = wave_n * WN + a * 32 + frag_row;
#pragma unroll
  for (int b = 0; b < TM; ++b) brow[b] = BN + wave_m * WM + b * 32 + frag_row;

  auto compute = [&](int buf) {
    bf16x8 af[2][TN], bf[2][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
      af[0][a] = __builtin_bit_cast(bf16x8, lds[buf][lds_idx(arow[a], frag_half)]);
#pragma unroll
    for (int b = 0; b < TM; ++b)
      bf[0][b] = __builtin_bit_cast(bf16x8, lds[buf][lds_idx(brow[b], frag_half)]);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < kBK / 16) {
        const int ch = (kk + 1) * 2 + frag_half;
#pragma unroll
        for (int a = 0; a < TN; ++a)
          af[cur ^ 1][a] = __builtin_bit_cast(bf16x8, lds[buf][lds_idx(arow[a], ch)]);
#pragma unroll
        for (int b = 0; b < TM; ++b)
          bf[cur ^ 1][b] = __builtin_bit_cast(bf16x8, lds[buf][lds_idx(brow[b], ch)]);
      }
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][a], bf[cur][b], acc[a][b], 0, 0, 0);
    }
  };

  // K steps in pairs so that staging set and LDS buffer indices are static:
  // even steps compute LDS buffer 0 / refill set 0, odd steps buffer 1 / set 1.
  gload(0, S0{});
  if (KT > 1) gload(1, S1{});
  lstore(0, S0{});
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    if (kt + 2 < KT) gload(kt + 2, S0{});
    compute(0);
    lstore(1, S1{});
    __syncthreads();
    if (kt + 3 < KT) gload(kt + 3, S1{});
    compute(1);
    if (kt + 2 < KT) lstore(0, S0{});
    __syncthreads();
  }
  if (kt < KT) compute(0);

#pragma unroll
  for (int b = 0; b < TM; ++b) {
    const int m = m0 + wave_m * WM + b * 32 + frag_row;
    if (m >= M) continue;
    if constexpr (DUAL) {
#pragma unroll
      for (int a = 0; a < TN / 2; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = out_n0 + wave_n * (WN / 2) + a * 32 + j * 8 + frag_half * 4;
          if (c >= N) continue;
          float g[4], u[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            g[i] = acc[a][b][j * 4 + i];
            u[i] = acc[a + TN / 2][b][j * 4 + i];
          }
          epi(m, c, g, u, min(4, N - c));
        }
    } else {
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = out_n0 + wave_n * WN + a * 32 + j * 8 + frag_half * 4;
          if (n >= N) continue;
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[a][b][j * 4 + i];
          epi(m, n, v, min(4, N - n));
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Generic VALU kernel (fp32 accumulation), 64x64 tile, 4x4 outputs per thread
// ---------------------------------------------------------------------------
template <typename T, bool DUAL, class Epi>
__global__ void __launch_bounds__(256)
gemm_valu_kernel(const T* __restrict__ X, WRows<T> W, int M, int N, int K, Epi epi) {
  constexpr int BT = 64, BKv = 16;
  __shared__ float xs[BKv][BT + 4];
  __shared__ float ws[BKv][BT + 4];
  __shared__ float us[DUAL ? BKv : 1][BT + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n0 = blockIdx.x * BT, m0 = blockIdx.y * BT;
  float acc[4][4] = {}, acc2[4][4] = {};
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int xr = m0 + lrow, wr = n0 + lrow;
  const T* xrow = xr < M ? X + static_cast<int64_t>(xr) * K : nullptr;
  const T* wrow = nullptr;
  const T* urow = nullptr;
  if (wr < N) {
    if constexpr (DUAL) {
      wrow = W.p[0] + static_cast<int64_t>(wr) * W.ld;
      urow = W.p[1] + static_cast<int64_t>(wr) * W.ld;
    } else {
      wrow = W.row(wr);
    }
  }
  for (int k0 = 0; k0 < K; k0 += BKv) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kk = k0 + lk + e;
      xs[lk + e][lrow] = (xrow && kk < K) ? ld(xrow + kk) : 0.f;
      ws[lk + e][lrow] = (wrow && kk < K) ? ld(wrow + kk) : 0.f;
      if constexpr (DUAL) us[lk + e][lrow] = (urow && kk < K) ? ld(urow + kk) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKv; ++kk) {
      float a[4], b[4], u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = xs[kk][ty * 4 + i];
        b[i] = ws[kk][tx * 4 + i];
        if constexpr (DUAL) u[i] = us[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] += a[i] * b[j];
          if constexpr (DUAL) acc2[i][j] += a[i] * u[j];
        }
    }
    __syncthreads();
  }
  const int n = n0 + tx * 4;
  if (n >= N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    if constexpr (DUAL)
      epi(m, n, acc[i], acc2[i], min(4, N - n));
    else
      epi(m, n, acc[i], min(4, N - n));
  }
}

// ---------------------------------------------------------------------------
// split-K reduction + epilogue: one thread per 4 output columns of a row
// ---------------------------------------------------------------------------
template <bool DUAL, class Epi>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ part, int splits, int64_t split_stride, int M,
                     int N, int ldp, Epi epi) {
  const int groups = (N + 3) >> 2;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= static_cast<int64_t>(M) * groups) return;
  const int m = static_cast<int>(gid / groups);
  const int n = static_cast<int>(gid - static_cast<int64_t>(m) * groups) * 4;
  const int cnt = min(4, N - n);
  float v[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < splits; ++z) {
    const float* p = part + z * split_stride + static_cast<int64_t>(m) * ldp + n;
    for (int i = 0; i < cnt; ++i) {
      v[i] += p[i];
      if constexpr (DUAL) u[i] += p[N + i];
    }
  }
  if constexpr (DUAL)
    epi(m, n, v, u, cnt);
  else
    epi(m, n, v, cnt);
}

// ---------------------------------------------------------------------------
// dispatch helpers
// ---------------------------------------------------------------------------
struct Plan {
  bool mfma;
  bool big;       // 256x256 eight-wave kernel
  int bn, bm;     // MFMA tile (bn = weight rows per tile incl. both halves when dual)
  int splits;     // K splits (>1: partial sums + reduce)
  int k_per_split;
};

int ceil_div(int a, int b) { return (a + b - 1) / b; }

Plan make_plan(DType dt, int M, int N, int K, bool dual) {
  Plan p{};
  p.mfma = dt == DType::BF16 && K % 8 == 0;
  p.splits = 1;
  p.k_per_split = K;
  if (!p.mfma) return p;
  if (M >= 512) {
    p.bn = 256;
    p.bm = 256;
    p.big = K % kBK == 0;
    return p;
  }
  // few rows (decode): 64x64 tiles; split K until there are >= 512 workgroups
  p.bn = 64;
  p.bm = 64;
  const int n_logical = dual ? 2 * N : N;
  const int tiles = ceil_div(n_logical, 64) * ceil_div(M, 64);
  int splits = 1;
  while (tiles * splits < 512 && K / (splits * 2) >= 256) splits *= 2;
  p.splits = splits;
  p.k_per_split = ceil_div(ceil_div(K, splits), kBK) * kBK;
  p.splits = ceil_div(K, p.k_per_split);
  return p;
}

template <class F>
hipError_t with_epi(const GemmEpi& e, F&& f) {
  switch (e.kind) {
    case EpiKind::Store:
      if (e.out_dt == DType::F32) return f(EpiStore<float>{static_cast<float*>(e.out), e.ldo});
      return f(EpiStore<bf16_t>{static_cast<bf16_t*>(e.out), e.ldo});
    case EpiKind::Resid:
      if (e.out_dt == DType::F32)
        return f(EpiResid<float>{static_cast<float*>(e.out), static_cast<const float*>(e.resid), e.ldo});
      return f(EpiResid<bf16_t>{static_cast<bf16_t*>(e.out), static_cast<const bf16_t*>(e.resid), e.ldo});
    case EpiKind::Qkv:
      if (e.out_dt == DType::F32)
        return f(EpiQkv<float>{static_cast<float*>(e.q), static_cast<float*>(e.k),
                               static_cast<float*>(e.v), e.positions, e.nq_hd, e.nkv_hd, e.hd,
                               e.seq_len, e.kv_cap, *e.rope});
      return f(EpiQkv<bf16_t>{static_cast<bf16_t*>(e.q), static_cast<bf16_t*>(e.k),
                              static_cast<bf16_t*>(e.v), e.positions, e.nq_hd, e.nkv_hd, e.hd,
                              e.seq_len, e.kv_cap, *e.rope});
    default:
      return hipErrorInvalidValue;
  }
}

template <class F>
hipError_t with_silu(const GemmEpi& e, F&& f) {
  if (e.out_dt == DType::F32) return f(EpiSilu<float>{static_cast<float*>(e.out), e.ldo});
  return f(EpiSilu<bf16_t>{static_cast<bf16_t*>(e.out), e.ldo});
}

template <int BN, int BM, bool DUAL, class Epi>
hipError_t launch_mfma(const bf16_t* X, const WRows<bf16_t>& W, int M, int N, int K, int kps,
                       int splits, const Epi& epi, hipStream_t s) {
  const int tiles_m = ceil_div(M, BM);
  const int tiles_n = ceil_div(N, DUAL ? BN / 2 : BN);
  dim3 grid(tiles_m * tiles_n, 1, splits);
  hipLaunchKernelGGL((gemm_mfma_kernel<BN, BM, DUAL, Epi>), grid, dim3(256), 0, s, X, W, M, N, K,
                     kps, tiles_m, tiles_n, epi);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(DType dt, int M, int N, int K, bool dual) {
  Plan p = make_plan(dt, M, N, K, dual);
  if (!p.mfma || p.splits <= 1) return 0;
  const int n_logical = dual ? 2 * N : N;
  return static_cast<size_t>(p.splits) * M * n_logical * sizeof(float);
}

hipError_t launch_gemm(DType dt, const void* X, int M, int K, const WSeg& W, int N, bool dual,
                       const GemmEpi& epi, void* ws, size_t ws_bytes, hipStream_t s,
                       const char** kernel_name) {
  if (M == 0 || N == 0) return hipSuccess;
  const Plan p = make_plan(dt, M, N, K, dual);
  if (!p.mfma) {
    dim3 grid(ceil_div(N, 64), ceil_div(M, 64));
    if (kernel_name) *kernel_name = dual ? "gemm_valu_silu" : "gemm_valu";
    if (dt == DType::F32) {
      auto rows = make_rows<float>(W, K);
      const float* xp = static_cast<const float*>(X);
      if (dual)
        return with_silu(epi, [&](auto e) {
          hipLaunchKernelGGL((gemm_valu_kernel<float, true, decltype(e)>), grid, dim3(256), 0, s,
                             xp, rows, M, N, K, e);
          return hipGetLastError();
        });
      return with_epi(epi, [&](auto e) {
        hipLaunchKernelGGL((gemm_valu_kernel<float, false, decltype(e)>), grid, dim3(256), 0, s,
                           xp, rows, M, N, K, e);
        return hipGetLastError();
      });
    }
    auto rows = make_rows<bf16_t>(W, K);
    const bf16_t* xp = static_cast<const bf16_t*>(X);
    if (dual)
      return with_silu(epi, [&](auto e) {
        hipLaunchKernelGGL((gemm_valu_kernel<bf16_t, true, decltype(e)>), grid, dim3(256), 0, s,
                           xp, rows, M, N, K, e);
        return hipGetLastError();
      });
    return with_epi(epi, [&](auto e) {
      hipLaunchKernelGGL((gemm_valu_kernel<bf16_t, false, decltype(e)>), grid, dim3(256), 0, s,
                         xp, rows, M, N, K, e);
      return hipGetLastError();
    });
  }

  const bf16_t* xp = static_cast<const bf16_t*>(X);
  auto rows = make_rows<bf16_t>(W, K);
  if (p.splits <= 1) {
    if (kernel_name) *kernel_name = dual ? "gemm_mfma_gate_up_silu" : "gemm_mfma";
    if (p.big) {
      const int tiles_m = ceil_div(M, 256);
      const int tiles_n = ceil_div(N, dual ? 128 : 256);
      dim3 grid(tiles_m * tiles_n);
      if (dual)
        return with_silu(epi, [&](auto e) {
          hipLaunchKernelGGL((gemm_mfma8_kernel<true, decltype(e)>), grid, dim3(512), 0, s, xp, rows, M, N, K,
                             tiles_m, tiles_n, e);
          return hipGetLastError();
        });
      return with_epi(epi, [&](auto e) {
        hipLaunchKernelGGL((gemm_mfma8_kernel<false, decltype(e)>), grid, dim3(512), 0, s, xp, rows, M, N, K,
                           tiles_m, tiles_n, e);
        return hipGetLastError();
      });
    }
    if (p.bn == 256 && p.bm == 256) {
      if (dual)
        return with_silu(epi, [&](auto e) {
          return launch_mfma<256, 256, true>(xp, rows, M, N, K, K, 1, e, s);
        });
      return with_epi(epi, [&](auto e) { return launch_mfma<256, 256, false>(xp, rows, M, N, K, K, 1, e, s); });
    }
    if (dual)
      return with_silu(epi, [&](auto e) { return launch_mfma<128, 64, true>(xp, rows, M, N, K, K, 1, e, s); });
    return with_epi(epi, [&](auto e) { return launch_mfma<64, 64, false>(xp, rows, M, N, K, K, 1, e, s); });
  }

  // split-K: partial sums over logical N (gate rows then up rows when dual)
  const int n_logical = dual ? 2 * N : N;
  const size_t need = static_cast<size_t>(p.splits) * M * n_logical * sizeof(float);
  if (ws == nullptr || ws_bytes < need) return hipErrorInvalidValue;
  float* part = static_cast<float*>(ws);
  const int64_t split_stride = static_cast<int64_t>(M) * n_logical;
  EpiPartial pe{part, n_logical, split_stride};
  WRows<bf16_t> lrows = rows;
  if (dual) {  // gate rows [0, N), up rows [N, 2N)
    lrows.s1 = N;
    lrows.s2 = 0x7fffffff;
  }
  if (kernel_name) *kernel_name = dual ? "gemm_mfma_splitk_gate_up" : "gemm_mfma_splitk";
  hipError_t err = launch_mfma<64, 64, false>(xp, lrows, M, n_logical, K, p.k_per_split, p.splits, pe, s);
  if (err != hipSuccess) return err;
  const int64_t threads = static_cast<int64_t>(M) * ceil_div(N, 4);
  const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
  if (dual)
    return with_silu(epi, [&](auto e) {
      hipLaunchKernelGGL((splitk_reduce_kernel<true, decltype(e)>), dim3(blocks), dim3(256), 0, s,
                         part, p.splits, split_stride, M, N, n_logical, e);
      return hipGetLastError();
    });
  return with_epi(epi, [&](auto e) {
    hipLaunchKernelGGL((splitk_reduce_kernel<false, decltype(e)>), dim3(blocks), dim3(256), 0, s,
                       part, p.splits, split_stride, M, N, n_logical, e);
    return hipGetLastError();
  });
}

}  // namespace lb
