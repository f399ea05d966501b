// GEMMs of the block: acc[m][n] = sum_k X[m][k] * W[n][k] (both operands K-
// contiguous, weights stored [out, in] as nn.Linear stores them in "Llama
// Architecture: RMSNorm, SwiGLU, RoPE, GQA, and PyTorch Implementation",
// "Production PyTorch Implementation"), followed by a fused epilogue:
// RoPE + Q/K/V (cache) stores, SiLU(gate) * up, residual add, or a plain store.
//
// Kernels (bf16 operands on the CDNA4 matrix cores, v_mfma_f32_32x32x16_bf16,
// fp32 accumulation; the weight tile is the MFMA "A" operand and the
// activations the "B" operand, so each lane holds four consecutive output
// features of one token: RoPE pairs and 4-wide stores stay inside a lane):
// gemm_mfma_dma_kernel / gemm_mfma_rs_kernel: prefill (M >= 512, K % 64 == 0,
//   weight segments on 32-row boundaries).  256x256 tiles, one wavefront per
//   SIMD owning 128x128, XOR-swizzled LDS; operands loaded straight into LDS
//   one K step ahead (dma, K <= 12288) or through registers two steps ahead
//   (rs, longer K).
// gemm_skinny_kernel: decode (M <= 64, K % 256 == 0): streams the weights once
//   with whole-line loads, K split over the wavefronts and summed in LDS;
//   64 or 32 weight rows per workgroup, K also split over workgroups (fp32
//   partials + splitk_reduce_kernel) when the row blocks cannot fill the GPU.
// gemm_mfma_kernel: generic tiles (64x64 .. 256x256) for every other bf16
//   shape; with few rows it writes fp32 partial sums per K slice and
//   splitk_reduce_kernel sums them and applies the epilogue.
// gemm_valu_kernel: fp32-accumulating VALU kernel for the fp32 path and for
//   K % 8 != 0.
#include <type_traits>

#include "buffer_sizes.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace lb {

namespace {

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

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
// N so that tiles resident on one XCD share operand panels in its L2.  With
// 4 row tiles (32 resident tiles = 4 x 8 per XCD, 12 distinct panels as with
// 8 x 4) an XCD's range of the Llama-3-8B prefill products is one group, so
// all XCDs walk the weight columns in step and can share each weight panel
// through the last-level cache (measured on MI355X against 8: gate/up
// 1500-1508 -> 1485 us, o 267 -> 255, QKV 363-367 -> 357-360; 2 and 16 were
// slower than both).
__device__ __forceinline__ void tile_coords(int bid, int nblk, int tiles_m, int tiles_n,
                                            int* tm, int* tn) {
  int logical = bid;
  if ((nblk & 7) == 0) logical = (bid & 7) * (nblk >> 3) + (bid >> 3);
  constexpr int GROUP_M = 4;
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
// longest K (elements) the LDS-DMA prefill kernel takes (see launch_gemm)
constexpr int kDmaMaxK = 12288;
// compute units of the GPU the large-tile schedule is sized for, and the
// fewest K steps a split of the large-tile kernels keeps
constexpr int kCUs = 256;
constexpr int kBigSplitMinSteps = 16;


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

// a per-row key of lane t of the wavefront (32- or 64-bit)
__device__ __forceinline__ int shfl_key(int k, int t) { return __shfl(k, t, 64); }
__device__ __forceinline__ int64_t shfl_key(int64_t k, int t) {
  const int lo = __shfl(static_cast<int>(k & 0xffffffff), t, 64);
  const int hi = __shfl(static_cast<int>(k >> 32), t, 64);
  return static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo));
}

// ---------------------------------------------------------------------------
// Epilogue of the 256 x 256 tile kernels (4 wavefronts in a 2 x 2 grid, each
// holding 4 x 4 accumulator tiles of 32 x 32): register e of a 32x32 tile is
// feature row (e/4)*8 + half*4 + e%4 of the weight operand and token column
// lane%32.  `lds` is the K loop's LDS, free once every wavefront has passed
// the barrier at the top of the staged path.
// ---------------------------------------------------------------------------
template <bool DUAL, class Epi>
__device__ __forceinline__ void tile_epilogue(const f32x16 (&acc)[4][4], u32x4* lds, int m0, int out_n0, int M,
                                              int N, const Epi& epi) {
  constexpr int BN = 256, BM = 256, WN = 128, WM = 128, TN = 4, TM = 4;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wave_n = wid & 1, wave_m = wid >> 1;
  const int frag_row = lane & 31, frag_half = lane >> 5;
  if constexpr (!DUAL) {
    // Whole tile inside the output: the staged epilogue.  The K loop's LDS
    // buffers are free now; each wavefront passes its 128 x 128 block through
    // its own LDS region one 32-token block at a time, so that afterwards a
    // lane holds four consecutive columns of one token and each store (and
    // each load of pre(), e.g. the residual or the rotation table) covers
    // whole rows: 32 lanes x 16 bytes of one token, instead of 32 tokens x
    // 16 bytes.  The next block's pre() loads are issued before the current
    // block is stored.  Per-token keys (positions) are loaded once for all
    // four blocks and shared between lanes.
    if (m0 + BM <= M && out_n0 + BN <= N && epi.vec_ok()) {
      constexpr int SROW = WN + 4;  // floats per staged token row (16 lanes of a read hit 64 distinct banks)
      __syncthreads();              // every wavefront is done with the K loop's fragments
      // lane values derived from a copy made here, so that nothing of the
      // epilogue is computed before the K loop and kept live through it
      int le = lane;
      asm volatile("" : "+v"(le));
      float* stage = reinterpret_cast<float*>(lds) + wid * (32 * SROW);
      const int g = le & 31, hsel = le >> 5, srow = le & 31, shalf = le >> 5;
      const int n = out_n0 + wave_n * WN + g * 4;
      const int mw = m0 + wave_m * WM;
      // what depends on this lane's column group only, resolved once
      const typename Epi::Col col = epi.col(n);
      using Key = typename Epi::Key;
      Key key[TM];
#pragma unroll
      for (int b = 0; b < TM; ++b) key[b] = Epi::kRowKey ? epi.row_key(mw + b * 32 + g) : Key{};
      // row of token 2i + hsel of block b (iteration i: lanes 0-31 one token, 32-63 the next)
      auto row_of = [&](int b, int i) {
        const int t = 2 * i + hsel;
        return epi.row_from(mw + b * 32 + t, Epi::kRowKey ? shfl_key(key[b], t) : Key{});
      };
      // chunks of CH iterations (16 / CH per block); chunk c + 1's pre()
      // loads are issued before chunk c is stored.  CH is the largest that
      // leaves the K loop free of register spills for each epilogue.
      constexpr int CH = Epi::kRowKey ? 8 : 4, NCH = 16 / CH;
      f32x4 pre[2][CH];
      auto issue = [&](int c) {
#pragma unroll
        for (int i = 0; i < CH; ++i) pre[c & 1][i] = epi.pre(row_of(c / NCH, (c % NCH) * CH + i), col);
      };
      issue(0);
      // chunk c's accumulator tile acc[.][c / NCH] must be a compile-time
      // index (a runtime one puts all of acc in scratch memory), so the loop
      // is unrolled by template recursion rather than left to the unroller
      static_for<0, NCH * TM>([&](auto C) {
        constexpr int c = decltype(C)::value;
        constexpr int b = c / NCH, i0 = (c % NCH) * CH;
        if constexpr (i0 == 0) {
          // register e of tile (a, b): token frag_row, column a*32 + (e/4)*8 + frag_half*4 + e%4
#pragma unroll
          for (int a = 0; a < TN; ++a)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              f32x4 t = f32x4{acc[a][b][4 * j], acc[a][b][4 * j + 1], acc[a][b][4 * j + 2], acc[a][b][4 * j + 3]};
              asm volatile("" : "+v"(t));  // through VGPRs (left to itself the allocator spills in the K loop)
              *reinterpret_cast<f32x4*>(stage + srow * SROW + a * 32 + j * 8 + shalf * 4) = t;
            }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        f32x4 val[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i)
          val[i] = *reinterpret_cast<const f32x4*>(stage + (2 * (i0 + i) + hsel) * SROW + g * 4);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the next block overwrites it
        if constexpr (c + 1 < NCH * TM) issue(c + 1);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const float v[4] = {val[i][0], val[i][1], val[i][2], val[i][3]};
          epi.put(row_of(b, i0 + i), col, pre[c & 1][i], v);
        }
      });
      return;
    }
  }
  // per-fragment path (partial tiles, the fused gate/up product): the tile
  // indices a, b must be compile-time (a runtime index puts all of acc in
  // scratch memory), so the loops are unrolled by template recursion
  static_for<0, TM>([&](auto B) {
    constexpr int b = decltype(B)::value;
    const int m = m0 + wave_m * WM + b * 32 + frag_row;
    if (m >= M) return;
    if constexpr (DUAL) {
      static_for<0, TN / 2>([&](auto A) {
        constexpr int a = decltype(A)::value;
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
      });
    } else {
      static_for<0, TN>([&](auto A) {
        constexpr int a = decltype(A)::value;
        static_for<0, 4>([&](auto J) {
          constexpr int j = decltype(J)::value;
          const int n = out_n0 + wave_n * WN + a * 32 + j * 8 + frag_half * 4;
          if (n >= N) return;
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[a][b][j * 4 + i];
          epi(m, n, v, min(4, N - n));
        });
      });
    }
  });
}

// ---------------------------------------------------------------------------
// MFMA kernel, large tiles, register-staged buffer loads ("rs" kernel).
// 256 x 256 output tile, four wavefronts (one per SIMD) in a 2 x 2 grid, each
// owning 128 x 128 as 4 x 4 tiles of 32 x 32 (accumulators in AGPRs).
// K advances in steps of 64 so that every global load request covers a whole
// 128-byte line (8 lanes x 16 B of one row).  The operands are read with
// buffer loads: one SGPR resource per operand segment and a 32-bit per-lane
// offset, so rows past M or N come back as zeros from the hardware range
// check instead of being clamped.  Per K step kt each wavefront
//   * issues the global loads of step kt+2 into one register staging set,
//   * writes the staging set holding step kt+1 into the other LDS buffer,
//   * runs 4 sub-steps of 16 MFMAs with every memory instruction placed
//     between two MFMAs: the loads and LDS stores between the first ones,
//     the next sub-step's fragment reads one per MFMA after them,
//   * and crosses the end-of-step barrier half-way through the last
//     sub-step's MFMAs, then reads the first fragments of step kt+1.
// Requires K % 64 == 0 and weight-segment boundaries at multiples of 32 rows.
// ---------------------------------------------------------------------------
struct BufOperands {
  const bf16_t* x;        // activations [M, K]
  const bf16_t* w[3];     // weight segments, each [rows_i, K]
  int wrows[3];           // rows of each segment (bounds for the range check)
  int s1, s2;             // logical start rows of segments 1 and 2
};

template <bool DUAL, class Epi>
__global__ void __launch_bounds__(256, 1)
gemm_mfma_rs_kernel(BufOperands op, int M, int N, int K, int kps, int tiles_m, int tiles_n, Epi epi) {
  constexpr int BN = 256, BM = 256, WN = 128, WM = 128, TN = 4, TM = 4;
  constexpr int GROUPS = 8;  // row groups of 32 per operand
  __shared__ u32x4 lds[2][(BN + BM) * 8];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, &tm, &tn);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wave_n = wid & 1, wave_m = wid >> 1;
  const int out_n0 = tn * (DUAL ? BN / 2 : BN);
  const int m0 = tm * BM;
  // K steps [kt0, KT) of split blockIdx.z (kps steps per split)
  const int kt0 = blockIdx.z * kps;
  const int KT = min(K / kBK, kt0 + kps);
  const uint32_t row_bytes = static_cast<uint32_t>(K) * 2u;
  const int chunk = tid & 7, rbase = tid >> 3;
  const uint32_t voff = static_cast<uint32_t>(rbase) * row_bytes + static_cast<uint32_t>(chunk) * 16u;

  // Each 32-row group of an operand gets its own buffer resource whose base is
  // the group's first row and whose size ends at the group's last row (or the
  // operand's, if that comes first), so the per-lane offset is just (row
  // within group, chunk, K position); rows past the end read as zero.  A
  // group never reads past its 32 rows, so the size is clamped to them: the
  // byte count then stays below 2^32 however many rows the operand has.  The
  // resources are uniform (SALU arithmetic).
  auto group_rsrc = [&](const bf16_t* base, int first_row, int rows) {
    const uint32_t bytes = group_bytes(rows, first_row, row_bytes);
    const bf16_t* p = rows > first_row ? base + static_cast<int64_t>(first_row) * K : base;
    return make_rsrc(p, bytes);
  };
  auto w_rsrc = [&](int g) {
    if constexpr (DUAL) {
      const int r0 = 32 * g, wv = r0 / WN, rr0 = r0 % WN;
      const int c0 = out_n0 + wv * (WN / 2) + (rr0 % (WN / 2));
      return group_rsrc(rr0 >= WN / 2 ? op.w[1] : op.w[0], c0, N);
    } else {
      const int n0 = out_n0 + 32 * g;
      if (n0 < op.s1) return group_rsrc(op.w[0], n0, op.wrows[0]);
      if (n0 < op.s2) return group_rsrc(op.w[1], n0 - op.s1, op.wrows[1]);
      return group_rsrc(op.w[2], n0 - op.s2, op.wrows[2]);
    }
  };

  u32x4 wreg[2][GROUPS], xreg[2][GROUPS];
  auto gload = [&](int kt, int g, auto S) {
    constexpr int st = decltype(S)::value;
    const uint32_t vo = voff + static_cast<uint32_t>(kt) * (kBK * 2);
    wreg[st][g] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc(g), vo, 0, 0));
    xreg[st][g] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(group_rsrc(op.x, m0 + 32 * g, M), vo, 0, 0));
  };
  auto lstore = [&](int buf, int g, auto S) {
    constexpr int st = decltype(S)::value;
    lds[buf][lds_idx(rbase + 32 * g, chunk)] = wreg[st][g];
    lds[buf][BN * 8 + lds_idx(rbase + 32 * g, chunk)] = xreg[st][g];
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  const int frag_row = lane & 31, frag_half = lane >> 5;
  bf16x8 fa[2][TN], fb[2][TM];
  auto read_frags = [&](int buf, int sub, auto F) {
    constexpr int f = decltype(F)::value;
    const int ch = sub * 2 + frag_half;
#pragma unroll
    for (int a = 0; a < TN; ++a)
      fa[f][a] = __builtin_bit_cast(bf16x8, lds[buf][lds_idx(wave_n * WN + a * 32 + frag_row, ch)]);
#pragma unroll
    for (int b = 0; b < TM; ++b)
      fb[f][b] = __builtin_bit_cast(bf16x8, lds[buf][BN * 8 + lds_idx(wave_m * WM + b * 32 + frag_row, ch)]);
  };
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  auto barrier = [&]() {
    fence();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    fence();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;


  // One K step on LDS buffer BUF; staging set P holds step kt+1, set Q
  // receives step kt+2.  Every global load, LDS store and fragment read sits
  // between two MFMAs, so the matrix core is never left waiting while a burst
  // of memory instructions issues (4-5% faster than issuing them in groups).
  // Straight-line on purpose: loads, stores and fragment reads are issued
  // unconditionally (past the last K step the buffer range check returns
  // zeros or in-bounds data that is never consumed), so the compiler can
  // count outstanding loads exactly instead of waiting for the newest ones.
  auto rd = [&](int bufi, int sub, auto F, int i) {
    constexpr int f = decltype(F)::value;
    const int ch = sub * 2 + frag_half;
    if (i < TN)
      fa[f][i] = __builtin_bit_cast(bf16x8, lds[bufi][lds_idx(wave_n * WN + i * 32 + frag_row, ch)]);
    else
      fb[f][i - TN] = __builtin_bit_cast(bf16x8, lds[bufi][BN * 8 + lds_idx(wave_m * WM + (i - TN) * 32 + frag_row, ch)]);
  };
  auto mf = [&](auto F, int t) {
    constexpr int f = decltype(F)::value;
    acc[t / TM][t % TM] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[f][t / TM], fb[f][t % TM], acc[t / TM][t % TM], 0, 0, 0);
    fence();
  };
  auto kstep = [&](int kt, auto BUFc, auto P, auto Q) {
    constexpr int buf = decltype(BUFc)::value;
    // sub-steps 0..2: memory operations between MFMAs 0..3, the next
    // sub-step's fragment reads between MFMAs 4..11
    auto sub = [&](auto F, auto NF, int s) {
      if (s == 0) {
        mf(F, 0); gload(kt + 2, 0, Q); fence();
        mf(F, 1); gload(kt + 2, 1, Q); fence();
        mf(F, 2); mf(F, 3);
      } else {
        const int ga = 2 * s, gs = 2 * (s - 1);
        mf(F, 0); gload(kt + 2, ga, Q); fence();
        mf(F, 1); gload(kt + 2, ga + 1, Q); fence();
        mf(F, 2); lstore(buf ^ 1, gs, P); fence();
        mf(F, 3); lstore(buf ^ 1, gs + 1, P); fence();
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        mf(F, 4 + i);
        rd(buf, s + 1, NF, i);
        fence();
      }
#pragma unroll
      for (int t = 12; t < 16; ++t) mf(F, t);
    };
    sub(I0{}, I1{}, 0);
    sub(I1{}, I0{}, 1);
    sub(I0{}, I1{}, 2);
    // sub-step 3: loads and stores between MFMAs 0..7, the end-of-step
    // barrier, then the next step's first fragments between MFMAs 8..11
    mf(I1{}, 0); gload(kt + 2, 6, Q); fence();
    mf(I1{}, 1); gload(kt + 2, 7, Q); fence();
    mf(I1{}, 2); lstore(buf ^ 1, 4, P); fence();
    mf(I1{}, 3); lstore(buf ^ 1, 5, P); fence();
    mf(I1{}, 4); lstore(buf ^ 1, 6, P); fence();
    mf(I1{}, 5); lstore(buf ^ 1, 7, P); fence();
    mf(I1{}, 6);
    mf(I1{}, 7);
    barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rd(buf ^ 1, 0, I0{}, 2 * i);
      rd(buf ^ 1, 0, I0{}, 2 * i + 1);
      fence();
      mf(I1{}, 8 + i);
    }
#pragma unroll
    for (int t = 12; t < 16; ++t) mf(I1{}, t);
  };

  // prologue: step 0 in LDS buffer 0 (staging set 0), step 1 in flight (set 1)
#pragma unroll
  for (int g = 0; g < GROUPS; ++g) gload(kt0, g, I0{});
#pragma unroll
  for (int g = 0; g < GROUPS; ++g) gload(kt0 + 1, g, I1{});
#pragma unroll
  for (int g = 0; g < GROUPS; ++g) lstore(0, g, I0{});
  barrier();
  read_frags(0, 0, I0{});
  int kt = kt0;
  for (; kt + 1 < KT; kt += 2) {
    kstep(kt, I0{}, I1{}, I0{});
    kstep(kt + 1, I1{}, I0{}, I1{});
  }
  if (kt < KT) kstep(kt, I0{}, I1{}, I0{});

  tile_epilogue<DUAL>(acc, &lds[0][0], m0, out_n0, M, N, epi);
}

// ---------------------------------------------------------------------------
// MFMA kernel, large tiles, operands loaded straight into LDS ("dma" kernel).
// Tile, wavefront grid, LDS layout (XOR-swizzled 128-byte rows), fragment
// reads and epilogues are those of gemm_mfma_rs_kernel; the K loop differs.
// Each operand row is fetched with buffer_load_dwordx4 ... lds, which writes a
// wavefront's 64 x 16 bytes to 1 KB of LDS at M0 + 16 * lane without passing
// through VGPRs: the wavefronts issue no LDS stores and hold no staging
// registers.  Lane i of a load covers row i / 8 of an 8-row piece and LDS
// chunk i % 8, so it fetches the row's logical K chunk (i % 8) ^ swizzle
// (whole 128-byte lines per 8 lanes, as before).  Two 64 KB LDS buffers:
// while the MFMAs consume step kt from one, the 16 loads per wavefront of
// step kt+1 fill the other (issued between the first 32 MFMAs); every
// wavefront's loads of step kt+1 have landed at the barrier that ends step kt.
// Requires K % 64 == 0 and weight-segment boundaries at multiples of 32 rows.
// ---------------------------------------------------------------------------
template <bool DUAL, class Epi>
__global__ void __launch_bounds__(256, 1)
gemm_mfma_dma_kernel(BufOperands op, int M, int N, int K, int kps, int tiles_m, int tiles_n, Epi epi) {
  constexpr int BN = 256, WN = 128, WM = 128, TN = 4, TM = 4;
  __shared__ u32x4 lds[2][(BN + 256) * 8];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, &tm, &tn);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_n = wid & 1, wave_m = wid >> 1;
  const int out_n0 = tn * (DUAL ? BN / 2 : BN);
  const int m0 = tm * 256;
  // K steps [kt0, KT) of split blockIdx.z (kps steps per split)
  const int kt0 = blockIdx.z * kps;
  const int KT = min(K / kBK, kt0 + kps);
  const uint32_t row_bytes = static_cast<uint32_t>(K) * 2u;

  // buffer resource of a 32-row group: based at its first row, sized to its
  // rows (rows past the operand's end read as zero); uniform (SALU)
  auto group_rsrc = [&](const bf16_t* base, int first_row, int rows) {
    const uint32_t bytes = group_bytes(rows, first_row, row_bytes);
    const bf16_t* p = rows > first_row ? base + static_cast<int64_t>(first_row) * K : base;
    return make_rsrc(p, bytes);
  };
  auto w_rsrc = [&](int g) {
    if constexpr (DUAL) {
      const int r0 = 32 * g, wv = r0 / WN, rr0 = r0 % WN;
      const int c0 = out_n0 + wv * (WN / 2) + (rr0 % (WN / 2));
      return group_rsrc(rr0 >= WN / 2 ? op.w[1] : op.w[0], c0, N);
    } else {
      const int n0 = out_n0 + 32 * g;
      if (n0 < op.s1) return group_rsrc(op.w[0], n0, op.wrows[0]);
      if (n0 < op.s2) return group_rsrc(op.w[1], n0 - op.s1, op.wrows[1]);
      return group_rsrc(op.w[2], n0 - op.s2, op.wrows[2]);
    }
  };
  // this wavefront's groups: weight groups 2 wid, 2 wid + 1 and token groups
  // 2 wid, 2 wid + 1 (of 8 each), each as four pieces of 8 rows
  const __amdgpu_buffer_rsrc_t rs[4] = {w_rsrc(2 * wid), w_rsrc(2 * wid + 1),
                                        group_rsrc(op.x, m0 + 64 * wid, M),
                                        group_rsrc(op.x, m0 + 64 * wid + 32, M)};
  // row r = 32 g + 8 q + lane / 8 holds logical chunk c at LDS chunk
  // c ^ ((r >> 1) & 7) = c ^ (4 (q & 1) + lane / 16): lane i fetches logical
  // chunk (i % 8) ^ that
  const int r8 = lane >> 3, pc = lane & 7;
  const uint32_t voff0 = static_cast<uint32_t>(r8) * row_bytes + static_cast<uint32_t>(pc ^ (r8 >> 1)) * 16u;
  const uint32_t voff1 = static_cast<uint32_t>(r8) * row_bytes + static_cast<uint32_t>(pc ^ (4 + (r8 >> 1))) * 16u;
  // piece p = 0..15 of step kt into buffer BUF: operand p / 8, group p / 4 % 2, quarter p % 4
  auto dma = [&](auto BUFc, int kt, int p) {
    constexpr int buf = decltype(BUFc)::value;
    const int opnd = p >> 3, gi = (p >> 2) & 1, q = p & 3;
    const int row = 32 * (2 * wid + gi) + 8 * q;
    u32x4* dst = &lds[buf][(opnd ? BN * 8 : 0) + row * 8];
    const uint32_t soff = static_cast<uint32_t>(kt) * (kBK * 2) + static_cast<uint32_t>(8 * q) * row_bytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[opnd * 2 + gi], (__attribute__((address_space(3))) void*)dst, 16,
                                             (q & 1) ? voff1 : voff0, soff, 0, 0);
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  const int frag_row = lane & 31, frag_half = lane >> 5;
  bf16x8 fa[2][TN], fb[2][TM];
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  auto rd = [&](auto BUFc, int sub, auto F, int i) {
    constexpr int buf = decltype(BUFc)::value, f = decltype(F)::value;
    const int ch = sub * 2 + frag_half;
    if (i < TN)
      fa[f][i] = __builtin_bit_cast(bf16x8, lds[buf][lds_idx(wave_n * WN + i * 32 + frag_row, ch)]);
    else
      fb[f][i - TN] = __builtin_bit_cast(bf16x8, lds[buf][BN * 8 + lds_idx(wave_m * WM + (i - TN) * 32 + frag_row, ch)]);
  };
  auto mf = [&](auto F, int t) {
    constexpr int f = decltype(F)::value;
    acc[t / TM][t % TM] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[f][t / TM], fb[f][t % TM], acc[t / TM][t % TM], 0, 0, 0);
    fence();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // One K step on buffer CUR (fragments of sub-step 0 already read into set
  // 0): sub-steps 0 and 1 issue the next step's 16 loads into the other
  // buffer between their first 8 MFMAs, sub-steps 0..2 read the next
  // sub-step's fragments between MFMAs 8..15, and sub-step 3 waits for the
  // loads, crosses the barrier half-way and reads the next step's first
  // fragments between its last MFMAs.  Straight-line: the last step's loads
  // of a step past the end are issued too (they read in-bounds bytes of the
  // next row, or zeros past a group's last row, into the idle buffer, and
  // have landed at the step's final barrier, before the epilogue reuses LDS);
  // its fragment reads past the end are never used.
  auto kstep = [&](int kt, auto CUR) {
    constexpr int cur = decltype(CUR)::value;
    using NXT = std::integral_constant<int, 1 - cur>;
    // the 16 loads spread over sub-steps 0..2, one after every third MFMA,
    // so they reach the texture addresser no faster than it drains them
    auto sub = [&](auto F, auto NF, int s) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        mf(F, t);
        const int slot = 16 * s + t;
        if (slot % 3 == 0 && slot / 3 < 16) {
          dma(NXT{}, kt + 1, slot / 3);
          fence();
        }
        if (t >= 8) {
          rd(CUR, s + 1, NF, t - 8);
          fence();
        }
      }
    };
    sub(I0{}, I1{}, 0);
    sub(I1{}, I0{}, 1);
    sub(I0{}, I1{}, 2);
#pragma unroll
    for (int t = 0; t < 8; ++t) mf(I1{}, t);
    fence();
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    fence();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rd(NXT{}, 0, I0{}, 2 * i);
      rd(NXT{}, 0, I0{}, 2 * i + 1);
      fence();
      mf(I1{}, 8 + i);
    }
#pragma unroll
    for (int t = 12; t < 16; ++t) mf(I1{}, t);
  };

  // prologue: step 0 into buffer 0
#pragma unroll
  for (int p = 0; p < 16; ++p) dma(I0{}, kt0, p);
  fence();
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  fence();
#pragma unroll
  for (int i = 0; i < 8; ++i) rd(I0{}, 0, I0{}, i);
  int kt = kt0;
  for (; kt + 1 < KT; kt += 2) {
    kstep(kt, I0{});
    kstep(kt + 1, I1{});
  }
  if (kt < KT) kstep(kt, I0{});
  tile_epilogue<DUAL>(acc, &lds[0][0], m0, out_n0, M, N, epi);
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
  const float* p0 = part + static_cast<int64_t>(m) * ldp + n;
  if (cnt == 4 && (ldp & 3) == 0 && (N & 3) == 0 && (split_stride & 3) == 0) {
    // whole 16-byte groups: all splits' loads issued before the sums
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, c = {0.f, 0.f, 0.f, 0.f};
    int z = 0;
    for (; z + 4 <= splits; z += 4) {
      f32x4 t[4], tu[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        t[i] = *reinterpret_cast<const f32x4*>(p0 + (z + i) * split_stride);
        if constexpr (DUAL) tu[i] = *reinterpret_cast<const f32x4*>(p0 + (z + i) * split_stride + N);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a += t[i];
        if constexpr (DUAL) c += tu[i];
      }
    }
    for (; z < splits; ++z) {
      a += *reinterpret_cast<const f32x4*>(p0 + z * split_stride);
      if constexpr (DUAL) c += *reinterpret_cast<const f32x4*>(p0 + z * split_stride + N);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      u[i] = c[i];
    }
  } else {
    for (int z = 0; z < splits; ++z) {
      const float* p = p0 + z * split_stride;
      for (int i = 0; i < cnt; ++i) {
        v[i] += p[i];
        if constexpr (DUAL) u[i] += p[N + i];
      }
    }
  }
  if constexpr (DUAL)
    epi(m, n, v, u, cnt);
  else
    epi(m, n, v, cnt);
}

// ---------------------------------------------------------------------------
// split-K reduction + residual + the RMSNorm of the result, one workgroup per
// token row (few rows: the decode step's O projection followed by the FFN
// pre-norm, "LLaMA Architecture" block structure: h = x + attention output,
// then RMSNorm(h) feeds the FFN).  h = resid + sum of the fp32 partials, with
// the additions of splitk_reduce_kernel and its residual epilogue in the same
// order (splits in turn from zero, then the residual); then, with the row held in
// registers, f = h * (mean(h^2) + eps)^-1/2 * gamma as the RMSNorm kernels
// compute it (sum of squares per lane, then over the wavefront, then over the
// four wavefronts in order).  Wavefront w covers columns [w d/4, (w+1) d/4),
// lane l the four columns w d/4 + 4 (l + 64 c), c < V = d / 1024.  One
// memory round trip per row for all loads (partials, residual, gamma) instead
// of two kernels with one each.  h may be resid itself (each lane reads its
// residual elements before it writes them).
// ---------------------------------------------------------------------------
template <int V>
__global__ void __launch_bounds__(256)
splitk_resid_norm_kernel(const float* __restrict__ part, int splits, int64_t split_stride, int d,
                         const float* resid, float* h, const bf16_t* __restrict__ gamma,
                         bf16_t* __restrict__ f, float eps) {
  __shared__ float red[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * d;
  const int c0 = wid * (d >> 2);
  float a[V][4], r[V][4], g[V][4];
#pragma unroll
  for (int c = 0; c < V; ++c) {
    const int n = c0 + 4 * (lane + 64 * c);
    Vec4<float>::load(resid + row + n, r[c]);
    Vec4<bf16_t>::load(gamma + n, g[c]);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[c][e] = 0.f;
  }
  // four splits' loads in flight at once, added in split order
  const float* pr = part + row + c0 + 4 * lane;
  int z = 0;
  for (; z + 4 <= splits; z += 4) {
    float t[4][V][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < V; ++c) Vec4<float>::load(pr + (z + i) * split_stride + 256 * c, t[i][c]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < V; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) a[c][e] += t[i][c][e];
  }
  for (; z < splits; ++z) {
#pragma unroll
    for (int c = 0; c < V; ++c) {
      float t[4];
      Vec4<float>::load(pr + z * split_stride + 256 * c, t);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[c][e] += t[e];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < V; ++c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[c][e] = r[c][e] + a[c][e];
      ss += a[c][e] * a[c][e];
    }
    Vec4<float>::store(h + row + c0 + 4 * (lane + 64 * c), a[c]);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wid] = ss;
  __syncthreads();
  const float tot = ((red[0] + red[1]) + red[2]) + red[3];
  const float inv = rsqrtf(tot / static_cast<float>(d) + eps);
#pragma unroll
  for (int c = 0; c < V; ++c) {
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = a[c][e] * inv * g[c][e];
    Vec4<bf16_t>::store(f + row + c0 + 4 * (lane + 64 * c), o);
  }
}

// ---------------------------------------------------------------------------
// Skinny MFMA kernel for few token rows (decode: M <= 64).  The product is
// bound by streaming the weights once, so the kernel is built around that
// stream: a workgroup owns 64 weight rows (for the fused gate/up product 32
// gate rows and the same 32 up rows) and all M <= 64 tokens over a K range
// split four ways between its wavefronts.  Each wavefront works alone on its
// K range: per step of 64 K elements it loads its 64 weight rows and the 64
// token rows with whole 128-byte lines per row (eight lanes per row), one
// step ahead into registers; stores them into its own LDS region (16-byte
// chunks XOR-swizzled by (row / 2) % 8) and reads the MFMA fragments back,
// so the next step's loads are in flight during this step's products.  The
// four wavefronts' 64 x 64 tiles are then summed through LDS and the epilogue
// (or, with a K split across workgroups, an fp32 partial store for
// splitk_reduce_kernel) runs on whole rows.  Needs K / splits % 256 == 0.
// ---------------------------------------------------------------------------
constexpr int kSkStep = 64;  // K elements per step

__device__ __forceinline__ int sk_idx(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

// FB: 32-row weight blocks per workgroup (2, or 1 for a product with too few
// row blocks of 64 to fill the GPU without a K split; the fused gate/up
// product always takes one gate and one up block).
template <bool DUAL, int FB, class Epi>
__global__ void __launch_bounds__(256, 2)
gemm_skinny_kernel(const bf16_t* __restrict__ X, BufOperands op, int M, int N, int K, int ks, Epi epi) {
  static_assert(FB == 2 || (FB == 1 && !DUAL), "one or two 32-row weight blocks");
  constexpr int WROWS = 32 * FB;  // weight rows of the workgroup
  // per wavefront: 64 weight rows + 64 token rows of one step (128 B each);
  // reused afterwards for the cross-wavefront sum
  __shared__ u32x4 lds[4][2][64 * 8];
  // The wavefront index is made visibly uniform: the K offsets derived from
  // it are the buffer loads' scalar offsets, which would otherwise be taken
  // for per-lane values and every load wrapped in a read-first-lane loop.
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t row_bytes = static_cast<uint32_t>(K) * 2u;

  // buffer resources of the two 32-row weight blocks of this workgroup
  __amdgpu_buffer_rsrc_t wr[FB];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb) {
    const bf16_t* base;
    int left;
    if (DUAL) {
      const int f0 = blockIdx.x * 32;
      base = op.w[fb] + static_cast<int64_t>(f0) * K;
      left = op.wrows[fb] - f0;
    } else {
      const int r0 = blockIdx.x * WROWS + fb * 32;
      const int seg = r0 < op.s1 ? 0 : r0 < op.s2 ? 1 : 2;
      const int start = seg == 0 ? 0 : seg == 1 ? op.s1 : op.s2;
      base = op.w[seg] + static_cast<int64_t>(r0 - start) * K;
      left = op.wrows[seg] - (r0 - start);
    }
    // clamped on the vector unit (no scalar min/max of three), hence made
    // visibly uniform again, like the wavefront index above
    left = __builtin_amdgcn_readfirstlane(max(0, min(left, 32)));
    wr[fb] = make_rsrc(base, static_cast<uint32_t>(left) * row_bytes);
  }
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, static_cast<uint32_t>(M) * row_bytes);

  const int kw = ks / 4;  // K elements of this wavefront
  const int k0 = blockIdx.z * ks + w * kw;
  const int nsteps = kw / kSkStep;
  // load pattern: instruction i covers rows 8i .. 8i+7, lane = (row % 8) * 8 + chunk
  const int lrow = lane >> 3, lchunk = lane & 7;
  const uint32_t voff = static_cast<uint32_t>(lrow) * row_bytes + lchunk * 16u;
  struct Stage {
    u32x4 w[4 * FB], x[8];
  };
  auto gload = [&](Stage& g, int step) {
    const uint32_t soff = static_cast<uint32_t>(k0 + min(step, nsteps - 1) * kSkStep) * 2u;
#pragma unroll
    for (int i = 0; i < 4 * FB; ++i) g.w[i] = buffer_load16(wr[i >> 2], voff + static_cast<uint32_t>(i & 3) * 8u * row_bytes, soff);
#pragma unroll
    for (int i = 0; i < 8; ++i) g.x[i] = buffer_load16(xr, voff + static_cast<uint32_t>(i) * 8u * row_bytes, soff);
  };
  u32x4* lw = lds[w][0];
  u32x4* lx = lds[w][1];
  auto lstore = [&](const Stage& g) {
#pragma unroll
    for (int i = 0; i < 4 * FB; ++i) lw[sk_idx(i * 8 + lrow, lchunk)] = g.w[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) lx[sk_idx(i * 8 + lrow, lchunk)] = g.x[i];
  };
  f32x16 acc[FB][2];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[fb][tb][e] = 0.f;
  const int fr = lane & 31, fh = lane >> 5;
  auto compute = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x8 a[FB], b[2];
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) a[fb] = __builtin_bit_cast(bf16x8, lw[sk_idx(fb * 32 + fr, 2 * i + fh)]);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) b[tb] = __builtin_bit_cast(bf16x8, lx[sk_idx(tb * 32 + fr, 2 * i + fh)]);
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fb], b[tb], acc[fb][tb], 0, 0, 0);
    }
  };
  // Two register stages: the loads of the next two steps are in flight
  // while a step multiplies out of LDS (the wavefronts of a short product
  // have only a few steps each, so one step of lookahead leaves most of the
  // load latency exposed).  LDS accesses of one wavefront execute in order,
  // so a step's stores may follow the previous step's fragment reads without
  // a barrier.  Loads past the last step re-read it (cache hits).
  Stage g0, g1;
  gload(g0, 0);
  gload(g1, 1);
  lstore(g0);
  int st = 0;
  for (; st + 1 < nsteps; st += 2) {
    // LDS holds step st, g1 step st + 1
    gload(g0, st + 2);
    compute();
    lstore(g1);
    gload(g1, st + 3);
    compute();
    lstore(g0);
  }
  if (st < nsteps) compute();  // an odd step count's last step

  // sum the four wavefronts' tiles: C register e is row (e/4)*8 + fh*4 + e%4
  // of a 32-row block and token fr of a 32-token block.  The sum buffer is
  // [wave][token][16 chunks of 4 rows], chunks XOR-swizzled by token % 16.
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(&lds[0][0][0]);
  auto rix = [](int wv, int tok, int chunk) { return (wv * 64 + tok) * 16 + (chunk ^ (tok & 15)); };
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        red[rix(w, tb * 32 + fr, fb * 8 + j * 2 + fh)] =
            f32x4{acc[fb][tb][4 * j], acc[fb][tb][4 * j + 1], acc[fb][tb][4 * j + 2], acc[fb][tb][4 * j + 3]};
  __syncthreads();
  const int m = tid >> 2, q = tid & 3;
  if (m >= M) return;
  auto sum4 = [&](int row) {
    f32x4 v = red[rix(0, m, row >> 2)];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) v += red[rix(ww, m, row >> 2)];
    return v;
  };
  if constexpr (DUAL) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int row = q * 8 + g * 4;
      const int c = blockIdx.x * 32 + row;
      if (c >= N) continue;
      const f32x4 g4 = sum4(row), u4 = sum4(32 + row);
      const float gv[4] = {g4[0], g4[1], g4[2], g4[3]};
      const float uv[4] = {u4[0], u4[1], u4[2], u4[3]};
      epi(m, c, gv, uv, min(4, N - c));
    }
  } else {
    // thread (m, q): rows q * WROWS / 4 + 4 g of the workgroup's block
#pragma unroll
    for (int g = 0; g < FB * 2; ++g) {
      const int row = q * (WROWS / 4) + g * 4;
      const int n = blockIdx.x * WROWS + row;
      if (n >= N) continue;
      const f32x4 v4 = sum4(row);
      const float v[4] = {v4[0], v4[1], v4[2], v4[3]};
      epi(m, n, v, min(4, N - n));
    }
  }
}

// ---------------------------------------------------------------------------
// dispatch helpers
// ---------------------------------------------------------------------------
struct Plan {
  bool mfma;
  bool big;       // 256x256 four-wave kernel (gemm_mfma_rs_kernel)
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
    if (p.big) {
      // Too few 256x256 tiles to give every CU one (e.g. 2048 tokens against
      // 4096 features: 128 tiles): split K so the grid reaches one workgroup
      // per CU, each split keeping at least kBigSplitMinSteps K steps; fp32
      // partial sums, then splitk_reduce_kernel applies the epilogue.
      const int tiles = ceil_div(M, 256) * ceil_div(N, dual ? 128 : 256);
      const int KT = K / kBK;
      int splits = 1;
      while (tiles * splits * 2 <= kCUs && KT / (splits * 2) >= kBigSplitMinSteps) splits *= 2;
      p.k_per_split = ceil_div(KT, splits) * kBK;
      p.splits = ceil_div(K, p.k_per_split);
    }
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
                               e.seq_len, e.kv_cap, e.rope_cs, e.rope_base});
      return f(EpiQkv<bf16_t>{static_cast<bf16_t*>(e.q), static_cast<bf16_t*>(e.k),
                              static_cast<bf16_t*>(e.v), e.positions, e.nq_hd, e.nkv_hd, e.hd,
                              e.seq_len, e.kv_cap, e.rope_cs, e.rope_base});
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


// The buffer-load kernels need every 32-row group of a tile inside one weight
// segment and a group's byte size and offsets inside 32 bits (K bounded).
bool rs_ok(const WSeg& w, int K) {
  for (int i = 1; i < w.nseg; ++i)
    if (w.start[i] % kGroupRows != 0) return false;
  return K <= kMaxGroupK;
}

BufOperands buf_operands(const bf16_t* x, const WSeg& w, int N, bool dual) {
  BufOperands op{};
  op.x = x;
  for (int i = 0; i < 3; ++i) op.w[i] = static_cast<const bf16_t*>(w.ptr[i < w.nseg ? i : 0]);
  if (dual) {
    op.wrows[0] = N;
    op.wrows[1] = N;
    op.wrows[2] = 0;
    op.s1 = op.s2 = 0x7fffffff;
  } else {
    for (int i = 0; i < 3; ++i) op.wrows[i] = i < w.nseg ? w.start[i + 1] - w.start[i] : 0;
    op.s1 = w.nseg > 1 ? w.start[1] : 0x7fffffff;
    op.s2 = w.nseg > 2 ? w.start[2] : 0x7fffffff;
  }
  return op;
}

// The skinny kernel takes bf16 products with M <= 64 tokens, K a multiple of
// 256 and weight segments starting on 32-row boundaries.
bool skinny_shape(DType dt, int M, int K) { return dt == DType::BF16 && M <= 64 && K % 256 == 0; }

// K splits across workgroups, keeping K / splits a multiple of 256: with
// more than 32 token rows until there are >= 192 workgroups, with fewer until
// there are >= 384 (measured on the Llama-3-8B decode step: 64 rows, O and
// down at 4 splits instead of 8 and QKV at 2 instead of 4, step 334.5 ->
// 327.0-328.5 us; 8 rows, the same splits cost 3 us per step)
int skinny_target(int M) { return M > 32 ? 192 : 384; }
int skinny_splits(int n_logical, int K, int M) {
  const int nb = ceil_div(n_logical, 64);
  const int target = skinny_target(M);
  int splits = 1;
  while (nb * splits < target && K % (splits * 2 * 256) == 0) splits *= 2;
  return splits;
}

}  // namespace

size_t gemm_workspace_bytes(DType dt, int M, int N, int K, bool dual) {
  Plan p = make_plan(dt, M, N, K, dual);
  const int n_logical = dual ? 2 * N : N;
  size_t need = 0;
  if (p.mfma && p.splits > 1) need = static_cast<size_t>(p.splits) * M * n_logical * sizeof(float);
  if (skinny_shape(dt, M, K)) {
    const int sk = skinny_splits(n_logical, K, M);
    if (sk > 1) need = std::max(need, static_cast<size_t>(sk) * M * n_logical * sizeof(float));
  }
  return need;
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
  if (skinny_shape(dt, M, K) && rs_ok(W, K)) {
    const int n_logical = dual ? 2 * N : N;
    const int splits = skinny_splits(n_logical, K, M);
    const int ks = K / splits;
    if (!dual && splits > 1 && ceil_div(N, 32) >= skinny_target(M)) {
      // enough 32-row weight blocks to fill the GPU: no K split, so the
      // epilogue (e.g. the rotation and cache append of QKV) runs here and
      // no partials go through HBM (Llama-3-8B decode QKV: 192 workgroups)
      if (kernel_name) *kernel_name = "gemm_skinny_narrow";
      BufOperands op = buf_operands(xp, W, N, false);
      return with_epi(epi, [&](auto e) {
        hipLaunchKernelGGL((gemm_skinny_kernel<false, 1, decltype(e)>), dim3(ceil_div(N, 32)), dim3(256), 0, s, xp,
                           op, M, N, K, K, e);
        return hipGetLastError();
      });
    }
    if (splits == 1) {
      if (kernel_name) *kernel_name = dual ? "gemm_skinny_gate_up_silu" : "gemm_skinny";
      BufOperands op = buf_operands(xp, W, N, dual);
      dim3 grid(ceil_div(n_logical, 64), 1, 1);
      if (dual)
        return with_silu(epi, [&](auto e) {
          hipLaunchKernelGGL((gemm_skinny_kernel<true, 2, decltype(e)>), grid, dim3(256), 0, s, xp, op, M, N, K, ks, e);
          return hipGetLastError();
        });
      return with_epi(epi, [&](auto e) {
        hipLaunchKernelGGL((gemm_skinny_kernel<false, 2, decltype(e)>), grid, dim3(256), 0, s, xp, op, M, N, K, ks, e);
        return hipGetLastError();
      });
    }
    // fp32 partials over the logical rows (gate rows then up rows when dual)
    const size_t need = static_cast<size_t>(splits) * M * n_logical * sizeof(float);
    if (ws == nullptr || ws_bytes < need) return hipErrorInvalidValue;
    if (kernel_name) *kernel_name = dual ? "gemm_skinny_splitk_gate_up" : "gemm_skinny_splitk";
    float* part = static_cast<float*>(ws);
    const int64_t split_stride = static_cast<int64_t>(M) * n_logical;
    EpiPartial pe{part, n_logical, split_stride};
    BufOperands op = buf_operands(xp, W, n_logical, false);
    hipLaunchKernelGGL((gemm_skinny_kernel<false, 2, EpiPartial>), dim3(ceil_div(n_logical, 64), 1, splits), dim3(256),
                       0, s, xp, op, M, n_logical, K, ks, pe);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t threads = static_cast<int64_t>(M) * ceil_div(N, 4);
    const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
    if (dual)
      return with_silu(epi, [&](auto e) {
        hipLaunchKernelGGL((splitk_reduce_kernel<true, decltype(e)>), dim3(blocks), dim3(256), 0, s,
                           part, splits, split_stride, M, N, n_logical, e);
        return hipGetLastError();
      });
    return with_epi(epi, [&](auto e) {
      hipLaunchKernelGGL((splitk_reduce_kernel<false, decltype(e)>), dim3(blocks), dim3(256), 0, s,
                         part, splits, split_stride, M, N, n_logical, e);
      return hipGetLastError();
    });
  }
  if (p.big && rs_ok(W, K)) {
    if (kernel_name) *kernel_name = dual ? "gemm_mfma_gate_up_silu" : "gemm_mfma";
    const int tiles_m = ceil_div(M, 256);
    const int tiles_n = ceil_div(N, dual ? 128 : 256);
    const int kps = p.k_per_split / kBK;
    dim3 grid(tiles_m * tiles_n, 1, p.splits);
    BufOperands op = buf_operands(xp, W, N, dual);
    // Operands straight into LDS for K up to kDmaMaxK; past it the
    // register-staged kernel, whose loads run two K steps ahead instead of
    // one (measured on MI355X: gate/up 1475 against 1519 us, QKV 398
    // against 412, o equal, the Llama-7B down partials at K = 11008 184-187
    // against 190-194 us, but down at K = 14336 880 against 752 us, with
    // more L2 misses left exposed and a busier texture addresser; equal at
    // K = 22016)
    const bool dma = K <= kDmaMaxK;
    auto go = [&](auto kern, auto e) {
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, op, M, N, K, kps, tiles_m, tiles_n, e);
      return hipGetLastError();
    };
    if (p.splits == 1) {
      if (dual)
        return with_silu(epi, [&](auto e) {
          using E = decltype(e);
          return dma ? go(gemm_mfma_dma_kernel<true, E>, e) : go(gemm_mfma_rs_kernel<true, E>, e);
        });
      return with_epi(epi, [&](auto e) {
        using E = decltype(e);
        return dma ? go(gemm_mfma_dma_kernel<false, E>, e) : go(gemm_mfma_rs_kernel<false, E>, e);
      });
    }
    // K split: fp32 partials over the logical rows (gate then up), then the reduction applies the epilogue
    const int n_logical = dual ? 2 * N : N;
    const size_t need = static_cast<size_t>(p.splits) * M * n_logical * sizeof(float);
    if (ws == nullptr || ws_bytes < need) return hipErrorInvalidValue;
    if (kernel_name) *kernel_name = dual ? "gemm_mfma_splitk_big_gate_up" : "gemm_mfma_splitk_big";
    float* part = static_cast<float*>(ws);
    const int64_t split_stride = static_cast<int64_t>(M) * n_logical;
    EpiPartial pe{part, n_logical, split_stride, N};
    hipError_t err = dual ? (dma ? go(gemm_mfma_dma_kernel<true, EpiPartial>, pe) : go(gemm_mfma_rs_kernel<true, EpiPartial>, pe))
                          : (dma ? go(gemm_mfma_dma_kernel<false, EpiPartial>, pe) : go(gemm_mfma_rs_kernel<false, EpiPartial>, pe));
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
  if (p.splits <= 1) {
    if (kernel_name) *kernel_name = dual ? "gemm_mfma_gate_up_silu" : "gemm_mfma";
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

bool resid_norm_fused(DType dt, DType rdt, int M, int K, const WSeg& W, int N) {
  if (M <= 0 || rdt != DType::F32 || !skinny_shape(dt, M, K) || !rs_ok(W, K)) return false;
  if (N % 1024 != 0) return false;
  const int v = N / 1024;
  if (v != 1 && v != 2 && v != 4 && v != 8) return false;
  return skinny_splits(N, K, M) > 1;
}

hipError_t launch_gemm_partials(DType dt, const void* X, int M, int K, const WSeg& W, int N, void* ws,
                                size_t ws_bytes, hipStream_t s, const char** kernel_name) {
  if (!resid_norm_fused(dt, DType::F32, M, K, W, N)) return hipErrorInvalidValue;
  const int splits = skinny_splits(N, K, M);
  const size_t need = static_cast<size_t>(splits) * M * N * sizeof(float);
  if (ws == nullptr || ws_bytes < need) return hipErrorInvalidValue;
  if (kernel_name) *kernel_name = "gemm_skinny_splitk";
  const bf16_t* xp = static_cast<const bf16_t*>(X);
  EpiPartial pe{static_cast<float*>(ws), N, static_cast<int64_t>(M) * N};
  BufOperands op = buf_operands(xp, W, N, false);
  hipLaunchKernelGGL((gemm_skinny_kernel<false, 2, EpiPartial>), dim3(ceil_div(N, 64), 1, splits), dim3(256), 0, s,
                     xp, op, M, N, K, K / splits, pe);
  return hipGetLastError();
}

hipError_t launch_resid_norm(int M, int K, int N, const void* ws, const void* resid, void* h, const void* gamma,
                             void* f, float eps, hipStream_t s, const char** kernel_name) {
  if (M <= 0) return hipSuccess;
  if (N % 1024 != 0 || N > 8192 || K % 256 != 0) return hipErrorInvalidValue;
  const int splits = skinny_splits(N, K, M);
  if (kernel_name) *kernel_name = "splitk_resid_norm";
  const float* part = static_cast<const float*>(ws);
  const int64_t stride = static_cast<int64_t>(M) * N;
  const float* r = static_cast<const float*>(resid);
  float* hp = static_cast<float*>(h);
  const bf16_t* g = static_cast<const bf16_t*>(gamma);
  bf16_t* fp = static_cast<bf16_t*>(f);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(M), dim3(256), 0, s, part, splits, stride, N, r, hp, g, fp, eps);
    return hipGetLastError();
  };
  switch (N / 1024) {
    case 1: return go(splitk_resid_norm_kernel<1>);
    case 2: return go(splitk_resid_norm_kernel<2>);
    case 4: return go(splitk_resid_norm_kernel<4>);
    case 8: return go(splitk_resid_norm_kernel<8>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lb
