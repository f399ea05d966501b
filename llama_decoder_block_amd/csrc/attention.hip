// Causal grouped-query attention: o = softmax(q.k / sqrt(hd) over visible
// slots) . V, query head h reading KV head floor(h / (n_q/n_kv))
// ("Llama Architecture: RMSNorm, SwiGLU, RoPE, GQA, and PyTorch Implementation"
// §4 GQA equation; "LLaMA-3 8B 现代 LLM 架构、计算规模与能耗" §4.4-4.7, which also
// notes that the shared K/V need not be copied per query head and that a
// tiled on-chip softmax gives the same result as the full matrix).
//
// attn_flash_kernel (bf16, hd = 128, prefill): one workgroup per (sequence,
//   KV group, tile of 128 query rows) where the rows are the R = n_q/n_kv
//   heads of the group times 128/R tokens.  Each K/V tile of 64 slots goes
//   once from HBM straight into LDS (buffer loads with LDS destination) and
//   is used by all R heads.  Four wavefronts own 32 query rows each.  Scores
//   are computed transposed (S^T = K Q^T on v_mfma_f32_32x32x16_bf16) so that
//   every lane holds 32 scores of ONE query row: the online-softmax max/sum
//   need only one cross-lane exchange, and the probabilities already sit in
//   the register layout of the B operand of O^T = V^T P^T, whose A operand
//   comes from V's [slot][hd] tile through transposing LDS reads
//   (ds_read_b64_tr_b16).  S^T of tile j+1 is issued beside the softmax of
//   tile j.  Accumulators, running max and sum are fp32; P is rounded to bf16
//   for the MFMA.  Only tiles at or below each workgroup's last visible slot
//   are read.
// attn_decode3_kernel (bf16, hd = 128, one query token per sequence): one
//   workgroup per (sequence, KV group) whose wavefronts split the visible
//   slots; each streams its K/V rows once for the R query heads of the group
//   (scores on v_mfma_f32_16x16x32_bf16 with K rows loaded straight into
//   A-operand registers), and the workgroup merges the partial softmax
//   states in LDS.  attn_decode2_kernel + attn_decode_combine_kernel do the
//   same with chunks spread over workgroups and merged through HBM when there
//   are too few (sequence, KV group) pairs to fill the chip.
// attn_decode_kernel (fp32 or hd = 64): split-K over 256-slot chunks, one
//   workgroup per (sequence, KV group, chunk), merged by the combine kernel.
// attn_valu_kernel: generic fp32-accumulating kernel (one wavefront per query
//   row, online softmax over 64-slot chunks) for fp32 and other shapes.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace lb {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ===========================================================================
// generic VALU kernel
// ===========================================================================
template <typename T>
__global__ void __launch_bounds__(256)
attn_valu_kernel(AttnArgs a) {
  __shared__ float qs[4][256];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rid = static_cast<int64_t>(blockIdx.x) * 4 + w;  // (b, t, h), h fastest
  const int64_t nrows = static_cast<int64_t>(a.B) * a.Tq * a.nq;
  const bool active = rid < nrows;
  const int h = active ? static_cast<int>(rid % a.nq) : 0;
  const int64_t bt = active ? rid / a.nq : 0;
  const int b = static_cast<int>(bt / a.Tq), t = static_cast<int>(bt % a.Tq);
  const T* q = static_cast<const T*>(a.q) + rid * a.hd;
  if (active)
    for (int d = lane; d < a.hd; d += 64) qs[w][d] = ld(q + d);
  __syncthreads();
  if (!active) return;
  const int g = h / (a.nq / a.nkv);
  const int vis = min(a.positions ? a.positions[bt] : t, a.S - 1);
  const T* kb = static_cast<const T*>(a.k) + (static_cast<int64_t>(b) * a.S * a.nkv + g) * a.hd;
  const T* vb = static_cast<const T*>(a.v) + (static_cast<int64_t>(b) * a.S * a.nkv + g) * a.hd;
  const int64_t kstride = static_cast<int64_t>(a.nkv) * a.hd;
  const float c = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 <= vis; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j <= vis) {
      const T* kr = kb + j * kstride;
      float acc = 0.f;
      for (int d = 0; d < a.hd; ++d) acc += qs[w][d] * ld(kr + d);
      s = acc * c;
    }
    const float mx = wave_max(s);
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    const float p = j <= vis ? exp2f(s - mn) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] *= alpha;
    const int cnt = min(64, vis - j0 + 1);
    for (int jj = 0; jj < cnt; ++jj) {
      const float pj = __shfl(p, jj, 64);
      const T* vr = vb + (j0 + jj) * kstride;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        if (d < a.hd) o[i] += pj * ld(vr + d);
      }
    }
    m = mn;
  }
  T* out = static_cast<T*>(a.out) + rid * a.hd;
  const float inv = 1.f / l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = lane + 64 * i;
    if (d < a.hd) st(out + d, o[i] * inv);
  }
}

// ===========================================================================
// flash prefill kernel (bf16, hd = 128)
// ===========================================================================
constexpr int kFHd = 128;
constexpr int kFRows = 128;              // query rows per workgroup
constexpr int kFKeys = 64;               // key slots per tile
constexpr int kTileBytes = kFKeys * kFHd * 2;  // one K or V tile: 64 slots x 256 bytes

// LDS layout of a K or V tile: four column blocks of 32 hd (64 bytes of each
// slot row), block-major, slot rows of 64 bytes inside a block.  In K tiles
// the 16-byte chunk c of row r sits at chunk c ^ ((r >> 2) & 3), so the 16
// rows read by 16 lanes at one logical chunk fall on 16 distinct bank groups;
// V tiles are unswizzled (a transposing read takes 8 consecutive rows x 64
// bytes, a contiguous 512 bytes).
__device__ __forceinline__ int kswz(int r) { return (r >> 2) & 3; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint8_t lds_byte;

template <int R>
__global__ void __launch_bounds__(256, 2)
attn_flash_kernel(AttnArgs a, int n_qtiles) {
  constexpr int TQ = kFRows / R;  // tokens per workgroup
  // two K and two V tiles, as four arrays so that every access names its
  // buffer at compile time
  __shared__ __attribute__((aligned(1024))) uint8_t k0s[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t k1s[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v0s[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v1s[kTileBytes];
  __shared__ int vis_s[kFRows];
  auto kbuf = [&](auto I) -> uint8_t* { if constexpr (decltype(I)::value == 0) return k0s; else return k1s; };
  auto vbuf = [&](auto I) -> uint8_t* { if constexpr (decltype(I)::value == 0) return v0s; else return v1s; };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // Heavy tiles (late query tokens) first across all (sequence, KV group)
  // pairs, so the last workgroups to start are the light ones; consecutive
  // workgroups take consecutive pairs, so with workgroups placed on the XCDs
  // in turn each XCD's L2 serves few KV heads.
  const int n_bg = static_cast<int>(gridDim.x) / n_qtiles;
  const int qt = n_qtiles - 1 - static_cast<int>(blockIdx.x) / n_bg;
  const int bg = static_cast<int>(blockIdx.x) % n_bg;
  const int g = bg % a.nkv, b = bg / a.nkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = qt * TQ;
  const int my_row = w * 32 + (lane & 31);
  const int my_hi = my_row / TQ, my_t = t0 + my_row % TQ;
  const int my_h = g * R + my_hi;
  const int half = lane >> 5;

  bf16x8 qf[8];
  {
    const int tq = min(my_t, a.Tq - 1);
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) +
                       ((static_cast<int64_t>(b) * a.Tq + tq) * a.nq + my_h) * kFHd;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16 + half * 8);
    // Consume the Q fragments before the tile loop, so their wait is not
    // placed inside it, where (the counter being in order) it would also
    // wait for the next tile's loads.
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) asm volatile("" ::"v"(qf[kk]));
  }

  if (tid < kFRows) {
    const int t = t0 + tid % TQ;
    int vis = -1;
    // a position past the cache sees the whole cache (as in the decode
    // kernels), so the tile count stays bounded by the cache length
    if (t < a.Tq) vis = min(a.positions ? a.positions[static_cast<int64_t>(b) * a.Tq + t] : t, a.S - 1);
    vis_s[tid] = vis;
  }
  __syncthreads();
  int maxvis = -1;
  for (int i = 0; i < kFRows; ++i) maxvis = max(maxvis, vis_s[i]);
  const int my_vis = vis_s[my_row];
  int wave_min = 0x7fffffff;
  for (int i = 0; i < 32; ++i) {
    const int v = vis_s[w * 32 + i];
    wave_min = min(wave_min, v < 0 ? 0x7fffffff : v);
  }
  const int nkt = maxvis < 0 ? 0 : maxvis / kFKeys + 1;

  const int64_t kvrow = static_cast<int64_t>(a.nkv) * kFHd;
  const bf16_t* kbase = static_cast<const bf16_t*>(a.k) + (static_cast<int64_t>(b) * a.S * a.nkv + g) * kFHd;
  const bf16_t* vbase = static_cast<const bf16_t*>(a.v) + (static_cast<int64_t>(b) * a.S * a.nkv + g) * kFHd;
  const uint32_t kv_bytes = static_cast<uint32_t>((static_cast<int64_t>(a.S - 1) * kvrow + kFHd) * 2);
  const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(kbase, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(vbase, kv_bytes);
  const uint32_t row_bytes = static_cast<uint32_t>(kvrow) * 2;

  // Tile loads: wavefront w fills column block w (bytes 64 w .. 64 w + 63
  // of each slot row), 16 rows per instruction; lane i writes LDS chunk i % 4
  // of row 16 q + i / 4, i.e. the logical chunk (i % 4) ^ swizzle, where the K
  // swizzle of that row, (row >> 2) & 3, is i / 16 for every q.
  const uint32_t kvo = (lane >> 2) * row_bytes + static_cast<uint32_t>(((lane & 3) ^ (lane >> 4)) << 4);
  const uint32_t vvo = (lane >> 2) * row_bytes + static_cast<uint32_t>((lane & 3) << 4);
  auto tile_load = [&](__amdgpu_buffer_rsrc_t rs, uint32_t vo, uint8_t* dst, bool ktile, int kt) {
    const int base = kt * kFKeys;
    lds_byte* d = (lds_byte*)(dst + w * 4096);
    if (base + kFKeys - 1 <= maxvis) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t soff = static_cast<uint32_t>(base + 16 * q) * row_bytes + static_cast<uint32_t>(w * 64);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(d + q * 1024), 16,
                                                 vo, soff, 0, 0);
      }
    } else {
      // the tile holding the workgroup's last visible slot: later slots are
      // read as that slot (their weights are exactly 0, and a cache row past
      // the written positions may hold anything, NaN included)
      const int lc = ktile ? ((lane & 3) ^ (lane >> 4)) : (lane & 3);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t j = static_cast<uint32_t>(min(base + 16 * q + (lane >> 2), maxvis));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(d + q * 1024), 16,
                                                 j * row_bytes + static_cast<uint32_t>(w * 64 + (lc << 4)), 0, 0, 0);
      }
    }
  };

  // K fragment of chunk kk (hd 16 kk + 8 half .. + 7, logical chunk
  // 2 (kk % 2) + half of block kk / 2) of row h2 * 32 + lane % 32: a per-lane
  // offset for even and odd kk, the rest immediate.
  uint32_t ka[2];
#pragma unroll
  for (int o = 0; o < 2; ++o)
    ka[o] = static_cast<uint32_t>((lane & 31) * 64 + (((2 * o + half) ^ kswz(lane & 31)) << 4));
  // V^T fragment of hd block d for the 16 slots of (h2, hh): two transposing
  // reads r = 0, 1 of 4 slots each (slots 16 hh + 8 r + 4 half + 0..3 of the
  // 32-slot half h2, the order in which this lane holds the weights); source
  // lane i of each 16-lane group reads slot + i / 4, hd 16 ((lane / 16) % 2)
  // + 4 (i % 4) .. + 3 of block d.
  const uint32_t va = static_cast<uint32_t>((4 * half + ((lane & 15) >> 2)) * 64 + 32 * ((lane >> 4) & 1) +
                                            8 * (lane & 3));

  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[d][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale * kLog2e;

  // S^T = K Q^T of one tile from K buffer KB (the two 32-slot halves
  // alternate so consecutive MFMAs are independent)
  auto qk = [&](auto KB, f32x16 (&s)[2]) {
    const uint8_t* kb = kbuf(KB);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[h2][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + (kk >> 1) * 4096 + h2 * 2048 + ka[kk & 1]);
        s[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[h2], 0, 0, 0);
      }
  };
  auto wait_all_barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // One tile kt whose scores sit in `cur`: the loads of K kt + 2 and V kt + 1,
  // masking, the running maximum and rescale, then S^T of tile kt + 1 into
  // `nxt` beside the weights of tile kt, and O^T += V^T P^T.  Buffers: K kt in
  // KB P (free: its scores were computed a tile earlier), K kt + 1 in KB 1-P,
  // V kt in VB P, V kt + 1 into VB 1-P (free since the previous tile).
  auto step = [&](int kt, auto P, f32x16 (&cur)[2], f32x16 (&nxt)[2], auto NEXT) {
    constexpr int p = decltype(P)::value;
    constexpr bool next = decltype(NEXT)::value;
    using NP = std::integral_constant<int, 1 - p>;
    wait_all_barrier();
    if (kt + 2 < nkt) tile_load(krsrc, kvo, kbuf(P), true, kt + 2);
    if (kt + 1 < nkt) tile_load(vrsrc, vvo, vbuf(NP{}), false, kt + 1);

    const bool need_mask = kt * kFKeys + kFKeys - 1 > wave_min;
    if (need_mask) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = kt * kFKeys + h2 * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
          if (j > my_vis) cur[h2][e] = -INFINITY;
        }
    }
    // From here to the end of the tile the code is one basic block, so the
    // next tile's score MFMAs interleave with this tile's maximum and
    // rescale, and the PV MFMAs with the weights.
    if constexpr (next) qk(NP{}, nxt);
    float tmax = -INFINITY;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, cur[h2][e]);
    // lanes l and l ^ 32 hold the two key halves of one query: combine them
    // with the VALU half swap rather than a round trip through LDS
    {
      const auto hv = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(hv[0]), __uint_as_float(hv[1])) * c;
    }
    // Online softmax: each row's reference m_run is its running maximum
    // (rows whose maximum did not move rescale by exactly exp2(0) = 1).  The
    // weights exp2(score * c - m_run) are rounded to bf16 for the PV product,
    // so a reference equal to the row maximum keeps the largest weight
    // exactly 1 and free of rounding error, as in the softmax that subtracts
    // the row maximum; only weights of tiles seen before the maximum are
    // rounded against an earlier reference.  (A row with nothing visible yet
    // keeps -inf, and its factor 1 leaves its zero accumulators at zero.)
    {
      const float m_new = fmaxf(m_run, tmax);
      // the factors are all exactly 1 unless some row's maximum moved
      if (__builtin_amdgcn_ballot_w64(m_new != m_run) != 0) {
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[d][e] *= alpha;
      }
      m_run = m_new;
    }

    const float neg_m = -m_run;
    float psum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 pk;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float p0 = fast_exp2(__builtin_fmaf(cur[h2][hh * 8 + 2 * e2], c, neg_m));
          const float p1 = fast_exp2(__builtin_fmaf(cur[h2][hh * 8 + 2 * e2 + 1], c, neg_m));
          psum += p0 + p1;
          pk[e2] = pack_bf16x2(p0, p1);
        }
        pf[h2][hh] = __builtin_bit_cast(bf16x8, pk);
      }
    l_run += psum;

    const uint8_t* vb = vbuf(P);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          lds_byte* vt = (lds_byte*)vb + d * 4096 + (h2 * 32 + hh * 16) * 64 + va;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)vt);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(vt + 8 * 64));
          const s16x8 vv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf[h2][hh], oacc[d],
                                                            0, 0, 0);
        }
  };

  f32x16 sa[2], sb[2];
  if (nkt > 0) {
    tile_load(krsrc, kvo, k0s, true, 0);
    tile_load(vrsrc, vvo, v0s, false, 0);
    if (nkt > 1) tile_load(krsrc, kvo, k1s, true, 1);
    wait_all_barrier();
    qk(I0{}, sa);
  }
  // tile kt (even) starts with its scores in sa and its K/V in buffers 0
  using Yes = std::true_type;
  using No = std::false_type;
  int kt = 0;
  for (; kt + 2 < nkt; kt += 2) {
    step(kt, I0{}, sa, sb, Yes{});
    step(kt + 1, I1{}, sb, sa, Yes{});
  }
  if (kt + 1 < nkt) {
    step(kt, I0{}, sa, sb, Yes{});
    step(kt + 1, I1{}, sb, sa, No{});
  } else if (kt < nkt) {
    step(kt, I0{}, sa, sb, No{});
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (my_t < a.Tq && my_vis >= 0) {
    const float inv = 1.f / l_tot;
    bf16_t* op = static_cast<bf16_t*>(a.out) + ((static_cast<int64_t>(b) * a.Tq + my_t) * a.nq + my_h) * kFHd;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = oacc[d][j * 4 + i] * inv;
        Vec4<bf16_t>::store(op + d * 32 + j * 8 + half * 4, v);
      }
  }
}

// ===========================================================================
// split-K decode kernel + combine
// ===========================================================================
constexpr int kDChunk = 256;  // key slots per chunk of attn_decode_kernel (and the minimum split-K chunk)

template <typename T> struct VecN;            // 16-byte vector of T
template <> struct VecN<bf16_t> { static constexpr int N = 8; };
template <> struct VecN<float> { static constexpr int N = 4; };

template <typename T>
__device__ __forceinline__ void unpack16(const u32x4& r, float* out) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(r[i] << 16);
      out[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(r[i]);
  }
}

// Workgroup: 256 threads.  A K/V row of HD elements is read by L = HD/EPL
// lanes (16 bytes each); a wavefront covers 64/L slots per load and the
// workgroup 256/L; each thread issues kDChunk*L/256 loads for K and as many
// for V.
template <typename T, int HD, int R>
__global__ void __launch_bounds__(256)
attn_decode_kernel(AttnArgs a, int n_chunks, float* __restrict__ part_o,
                   float* __restrict__ part_ml) {
  constexpr int EPL = VecN<T>::N;
  constexpr int L = HD / EPL;               // lanes per slot row
  constexpr int SLOTS_PER_PASS = 256 / L;   // slots per workgroup load
  constexpr int PASSES = kDChunk / SLOTS_PER_PASS;
  static_assert(L >= 1 && L <= 64 && (64 % L) == 0, "bad HD");
  __shared__ float s_sc[R][kDChunk];
  __shared__ float s_red[R][256 / L > 0 ? 4 : 1][HD];
  __shared__ float s_ml[R][2];

  const int chunk = blockIdx.x % n_chunks;
  const int bg = blockIdx.x / n_chunks;
  const int g = bg % a.nkv, b = bg / a.nkv;
  const int vis = min(a.positions ? a.positions[b] : 0, a.S - 1);  // q_len == 1
  const int j0 = chunk * kDChunk;
  if (j0 > vis) return;  // nothing visible in this chunk (combine skips it)
  const int jn = min(kDChunk, vis - j0 + 1);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sub = tid % L;           // element group within the row
  const int slot_in_pass = tid / L;  // 0 .. SLOTS_PER_PASS-1
  const int64_t kvrow = static_cast<int64_t>(a.nkv) * HD;
  const T* kb = static_cast<const T*>(a.k) + (static_cast<int64_t>(b) * a.S * a.nkv + g) * HD + sub * EPL;
  const T* vb = static_cast<const T*>(a.v) + (static_cast<int64_t>(b) * a.S * a.nkv + g) * HD + sub * EPL;

  // issue every K and V load of this thread
  u32x4 kr[PASSES], vr[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int jl = p * SLOTS_PER_PASS + slot_in_pass;
    const int j = j0 + min(jl, jn - 1);
    kr[p] = *reinterpret_cast<const u32x4*>(kb + j * kvrow);
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int jl = p * SLOTS_PER_PASS + slot_in_pass;
    const int j = j0 + min(jl, jn - 1);
    vr[p] = *reinterpret_cast<const u32x4*>(vb + j * kvrow);
  }

  // this lane's slice of the R query vectors
  float qv[R][EPL];
  const T* qb = static_cast<const T*>(a.q) + (static_cast<int64_t>(b) * a.nq + g * R) * HD + sub * EPL;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const u32x4 t = *reinterpret_cast<const u32x4*>(qb + r * HD);
    unpack16<T>(t, qv[r]);
  }
  const float c = a.scale * kLog2e;

  // scores
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    float kv[EPL];
    unpack16<T>(kr[p], kv);
    const int jl = p * SLOTS_PER_PASS + slot_in_pass;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc += qv[r][e] * kv[e];
#pragma unroll
      for (int off = L / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
      if (sub == 0) s_sc[r][jl] = jl < jn ? acc * c : -INFINITY;
    }
  }
  __syncthreads();

  // per-head softmax over the chunk (wave w handles heads w, w+4, ...)
  for (int r = w; r < R; r += 4) {
    float mx = -INFINITY;
    for (int i = lane; i < kDChunk; i += 64) mx = fmaxf(mx, s_sc[r][i]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int i = lane; i < kDChunk; i += 64) {
      const float p = fast_exp2(s_sc[r][i] - mx);
      s_sc[r][i] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      s_ml[r][0] = mx;
      s_ml[r][1] = sum;
    }
  }
  __syncthreads();

  // P V: each thread accumulates its element group over its slots
  float o[R][EPL];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[r][e] = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    float vv[EPL];
    unpack16<T>(vr[p], vv);
    const int jl = p * SLOTS_PER_PASS + slot_in_pass;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float pr = jl < jn ? s_sc[r][jl] : 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[r][e] += pr * vv[e];
    }
  }
  // reduce over the slots handled by different lanes of a wavefront
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = o[r][e];
#pragma unroll
      for (int off = 32; off >= L; off >>= 1) v += __shfl_xor(v, off, 64);
      o[r][e] = v;
    }
  if (lane < L) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_red[r][w][sub * EPL + e] = o[r][e];
  }
  __syncthreads();
  // reduce over the four wavefronts and write the partial
  const int64_t pbase = (static_cast<int64_t>(b) * a.nq + g * R) * n_chunks + chunk;
  for (int i = tid; i < R * HD; i += 256) {
    const int r = i / HD, d = i % HD;
    const float v = s_red[r][0][d] + s_red[r][1][d] + s_red[r][2][d] + s_red[r][3][d];
    part_o[(pbase + static_cast<int64_t>(r) * n_chunks) * HD + d] = v;
  }
  if (tid < R) {
    part_ml[(pbase + static_cast<int64_t>(tid) * n_chunks) * 2 + 0] = s_ml[tid][0];
    part_ml[(pbase + static_cast<int64_t>(tid) * n_chunks) * 2 + 1] = s_ml[tid][1];
  }
}

// ===========================================================================
// decode kernel v2 (bf16, hd = 128): one wavefront per (sequence, KV group,
// chunk of 256 slots).  The chunk is walked in sub-steps of 32 slots:
//   * scores S = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16): K rows
//     are loaded straight into A-operand registers (lane l: slot l%16 of a
//     16-slot block, 8 head-dim elements at (l/16)*8 + 32 s), Q^T is the B
//     operand with the R query heads of the group as columns (other columns
//     zero);
//   * online softmax per query column in registers (lanes l%16 < R);
//   * the weights go through a small per-wavefront LDS buffer to the PV lanes,
//     which read V coalesced (16 lanes per 256-byte row) and accumulate
//     o[r][8 elements] with fp32 FMAs.
// Writes a partial (max, sum, o) per chunk; attn_decode_combine_kernel merges.
// ===========================================================================
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kDSub = 32;  // slots per step of the decode wavefront

// Sum / max over the four 16-lane rows of a wavefront (lanes l, l^16, l^32,
// l^48): v_permlane32_swap then v_permlane16_swap exchange the rows on the
// VALU (no LDS round trip).
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// K/V registers of one 32-slot step: K as two 16-slot MFMA A blocks x 4
// head-dim steps, V as 8 slots per lane group (16 lanes per 256-byte row).
// With the 8-bit cache (KV8) a lane holds 32 E4M3 codes of each K row block
// (the four head-dim steps), 8 codes of each V row and the fp32 row scales of
// the eight slots whose scores it computes.
template <bool KV8>
struct DecRegsT {
  u32x4 k[2][4];
  u32x4 v[8];
};
template <>
struct DecRegsT<true> {
  u32x4 k[2][2];
  u32x2 v[8];
  float sc;  // lane l < 32: k scale of slot js + l; l >= 32: v scale of slot js + l - 32
};
using DecRegs = DecRegsT<false>;

__device__ __forceinline__ void dec_load(DecRegs& r, const bf16_t* kbase, const bf16_t* vbase,
                                         int64_t kvrow, int js, int jend, int col, int grp) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int j = min(js + blk * 16 + col, jend);
#pragma unroll
    for (int s = 0; s < 4; ++s) r.k[blk][s] = *reinterpret_cast<const u32x4*>(kbase + j * kvrow + s * 32 + grp * 8);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = min(js + grp + 4 * i, jend);
    r.v[i] = *reinterpret_cast<const u32x4*>(vbase + j * kvrow + col * 8);
  }
}

// 8-bit cache rows: codes [n_kv][S][128] per sequence (the slots of one KV
// head are contiguous 128-byte rows), scales [n_kv][S].  Lane (col, grp) loads the 32
// codes grp*32 .. grp*32+31 of K row js + blk*16 + col (head-dim steps s use
// codes s*8 .. s*8+7 of them, so the Q fragments take the same permutation of
// the head dimension) and the 8 codes col*8 .. col*8+7 of V row js + grp + 4i.
// The rows of one (sequence, KV head) are read through buffer resources that
// end after its last visible slot: rows past the end read as zero (their
// scores are masked), so no clamping runs per load.  The range check covers
// the per-lane offset only (not the scalar one), so each load's offset is
// the lane's fixed row offset plus the step's js * row stride.
struct Dec8Src {
  __amdgpu_buffer_rsrc_t k, v;
  uint32_t row;      // bytes between slots (128)
  uint32_t koff[2];  // lane offsets of the two 16-slot K blocks
  uint32_t voff[8];  // lane offsets of the eight V rows
  const float* ksb;
  const float* vsb;

  __device__ __forceinline__ void init(const uint8_t* k8, const uint8_t* v8, const float* ks, const float* vs,
                                       int vis, int col, int grp) {
    row = 128u;
    const uint32_t bytes = vis >= 0 ? static_cast<uint32_t>(vis) * row + 128u : 0u;
    k = make_rsrc(k8, bytes);
    v = make_rsrc(v8, bytes);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) koff[blk] = static_cast<uint32_t>(blk * 16 + col) * row + grp * 32;
#pragma unroll
    for (int i = 0; i < 8; ++i) voff[i] = static_cast<uint32_t>(grp + 4 * i) * row + col * 8;
    ksb = ks;
    vsb = vs;
  }
};

__device__ __forceinline__ void dec_load8(DecRegsT<true>& r, const Dec8Src& src, int js, int jend, int col,
                                          int grp) {
  const uint32_t so = static_cast<uint32_t>(js) * src.row;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    r.k[blk][0] = buffer_load16(src.k, src.koff[blk] + so, 0);
    r.k[blk][1] = buffer_load16(src.k, src.koff[blk] + so + 16u, 0);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    r.v[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(src.v, src.voff[i] + so, 0, 0));
  // the step's 32 k scales and 32 v scales, one per lane (masked slots read a
  // visible one); step() hands them to the score lanes through LDS
  const int l = col + 16 * grp;
  r.sc = (l < 32 ? src.ksb : src.vsb)[min(js + (l & 31), jend)];
}

// Eight E4M3 codes (the lowest byte first) -> eight bf16 / fp32 values.  The
// conversion is exact: every E4M3 value is a bf16 value.  To bf16: gfx950's
// scaled pair conversion with scale 1, one instruction per two codes (an
// in-bounds probe matched it, for every code in each byte position, to the
// fp32 conversion's upper halves).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t d0, uint32_t d1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.f, true));
  return __builtin_bit_cast(bf16x8_t, r);
}
__device__ __forceinline__ void fp8x8_to_f32(uint32_t d0, uint32_t d1, float v[8]) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(d0, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(d0, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(d1, false), e = __builtin_amdgcn_cvt_pk_f32_fp8(d1, true);
  v[0] = a[0]; v[1] = a[1]; v[2] = b[0]; v[3] = b[1];
  v[4] = c[0]; v[5] = c[1]; v[6] = e[0]; v[7] = e[1];
}

// Paged cache: slot j of sequence b is row j % P of page table[j / P] in a
// pool [n_pages, P, n_kv, hd].  P is a multiple of the 32-slot step and steps
// start on multiples of 32, so one table entry serves a whole step; entries
// outside [0, n_pages) are clamped into the pool (a valid table never has
// them for visible slots; the clamp only keeps a bad table inside memory).
// The loops read the next step's table entry before this step's loads, so
// the indirection adds no dependent round trip.
__device__ __forceinline__ void dec_load_paged(DecRegs& r, const bf16_t* kpool, const bf16_t* vpool, int page,
                                               int P, int64_t n_pages, int64_t kvrow, int js, int jend, int col,
                                               int grp) {
  const int64_t pg = page < 0 ? 0 : (page >= n_pages ? n_pages - 1 : page);
  const int64_t base = (pg * P + (js % P)) * kvrow;
  dec_load(r, kpool + base, vpool + base, kvrow, 0, jend - js, col, grp);
}

template <int R>
struct DecState {
  static constexpr int RP = R > 4 ? R : 4;
  float m_run, l_run;  // per query column (score lanes)
  float o[R][8];       // head-dim elements col*8 .. +7, summed over lane groups at the end

  __device__ __forceinline__ void init() {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] = 0.f;
  }

  // one 32-slot step: scores on the matrix cores, online softmax, PV on the VALU.
  // With the 8-bit cache a score is k_scale * (q . codes) and a weight enters
  // PV as p * v_scale (the softmax sum uses p itself).
  template <bool KV8>
  __device__ __forceinline__ void step(const DecRegsT<KV8>& kv, const bf16x8_t (&qf)[4], float c, int js, int jend,
                                       int col, int grp, float (*s_p)[RP], float* s_alpha) {
    f32x4 ks[2], vs[2];
    if constexpr (KV8) {
      // the weight buffer (>= 64 floats) first passes the scales: score lane
      // (col, grp) needs those of slots blk*16 + grp*4 .. +3.  LDS accesses of
      // a wavefront run in order, so the previous step's weight reads are done
      // and this step's weight writes come after these reads.
      float* sbuf = &s_p[0][0];
      sbuf[col + 16 * grp] = kv.sc;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        ks[blk] = *reinterpret_cast<const f32x4*>(sbuf + blk * 16 + grp * 4);
        vs[blk] = *reinterpret_cast<const f32x4*>(sbuf + 32 + blk * 16 + grp * 4);
      }
      __builtin_amdgcn_wave_barrier();
    }
    f32x4 sc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      sc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8_t kf;
        if constexpr (KV8) {
          const u32x4 src = kv.k[blk][s >> 1];
          kf = fp8x8_to_bf16(src[(s & 1) * 2], src[(s & 1) * 2 + 1]);
        } else {
          kf = __builtin_bit_cast(bf16x8_t, kv.k[blk][s]);
        }
        sc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sc[blk], 0, 0, 0);
      }
      if constexpr (KV8) sc[blk] *= ks[blk];
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = js + blk * 16 + grp * 4 + i;
        if (j > jend) sc[blk][i] = -INFINITY;
        tmax = fmaxf(tmax, sc[blk][i]);
      }
    tmax = rows_max(tmax) * c;
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(__builtin_fmaf(sc[blk][i], c, -m_new));
        psum += p;
        float pv = p;
        if constexpr (KV8) pv *= vs[blk][i];
        if (col < R) s_p[blk * 16 + grp * 4 + i][col] = pv;
      }
    l_run = l_run * alpha + rows_sum(psum);
    if (grp == 0 && col < R) s_alpha[col] = alpha;
    __builtin_amdgcn_wave_barrier();
    float al[R];
#pragma unroll
    for (int r = 0; r < R; ++r) al[r] = s_alpha[r];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] *= al[r];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v[8];
      if constexpr (KV8) {
        fp8x8_to_f32(kv.v[i][0], kv.v[i][1], v);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] = __uint_as_float(kv.v[i][q] << 16);
          v[2 * q + 1] = __uint_as_float(kv.v[i][q] & 0xffff0000u);
        }
      }
      const int sl = grp + 4 * i;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float p = s_p[sl][r];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[r][e] = __builtin_fmaf(p, v[e], o[r][e]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
};

template <int R, bool KV8, bool PAGED = false>
__global__ void __launch_bounds__(256)
attn_decode2_kernel(AttnArgs a, int n_chunks, int chunk_len, float* __restrict__ part_o,
                    float* __restrict__ part_ml) {
  constexpr int HD = 128, SUB = kDSub;
  const int CHUNK = chunk_len;
  using St = DecState<R>;
  __shared__ float s_p[4][SUB][St::RP];   // weights [slot][query] per wavefront
  __shared__ float s_alpha[4][St::RP];
  // the wavefront index made visibly uniform: the task, and with it the
  // buffer resources of the 8-bit cache rows, derive from it (a per-lane
  // resource would wrap every load in a read-first-lane loop)
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int task = blockIdx.x * 4 + w;
  if (task >= a.B * a.nkv * n_chunks) return;
  const int chunk = task % n_chunks;
  const int bg = task / n_chunks;
  const int g = bg % a.nkv, b = bg / a.nkv;
  const int vis = min(a.positions ? a.positions[b] : 0, a.S - 1);
  const int j0 = chunk * CHUNK;
  if (j0 > vis) return;  // nothing visible (the combine skips this chunk)
  const int jend = min(vis, j0 + CHUNK - 1);

  // K/V rows of (b, g): bf16 elements, or E4M3 codes (one byte each) plus
  // the fp32 row scales [n_kv][S] of the sequence
  const int64_t kvrow = static_cast<int64_t>(a.nkv) * HD;
  // (paged: the pool base at KV head g; the table picks the page per step)
  const int64_t kvoff = PAGED ? static_cast<int64_t>(g) * HD : (static_cast<int64_t>(b) * a.S * a.nkv + g) * HD;
  const bf16_t* kbase = static_cast<const bf16_t*>(a.k) + kvoff;
  const bf16_t* vbase = static_cast<const bf16_t*>(a.v) + kvoff;
  const int32_t* table = PAGED ? a.block_table + static_cast<int64_t>(b) * a.max_pages : nullptr;
  const int col = lane & 15, grp = lane >> 4;
  Dec8Src src8;
  if constexpr (KV8) {
    const int64_t hs = (static_cast<int64_t>(b) * a.nkv + g) * a.S;  // (sequence, KV head) slot base
    src8.init(static_cast<const uint8_t*>(a.k) + hs * HD, static_cast<const uint8_t*>(a.v) + hs * HD,
              a.k_scale + hs, a.v_scale + hs, vis, col, grp);
  }

  // Q^T fragments (B operand): column = query head col (< R), k = head dim
  bf16x8_t qf[4];
  {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + (static_cast<int64_t>(b) * a.nq + g * R + (col < R ? col : 0)) * HD;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // head-dim step s, lane group grp: elements s*32 + grp*8 .. +7, or with
      // the 8-bit cache grp*32 + s*8 .. +7 (the permutation of its K codes)
      u32x4 t = *reinterpret_cast<const u32x4*>(qp + (KV8 ? grp * 32 + s * 8 : s * 32 + grp * 8));
      if (col >= R) t = u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8_t, t);
    }
  }
  const float c = a.scale * kLog2e;
  St st;
  st.init();
  if constexpr (KV8) {
    // half the bytes per slot: the next step's loads are issued before this
    // step's arithmetic so that each wavefront keeps two steps in flight
    // (loads past the end re-read the last visible slot)
    DecRegsT<true> ra, rb;
    if (j0 <= jend) dec_load8(ra, src8, j0, jend, col, grp);
    for (int js = j0; js <= jend; js += 2 * SUB) {
      dec_load8(rb, src8, js + SUB, jend, col, grp);
      st.step(ra, qf, c, js, jend, col, grp, s_p[w], s_alpha[w]);
      if (js + SUB > jend) break;
      dec_load8(ra, src8, js + 2 * SUB, jend, col, grp);
      st.step(rb, qf, c, js + SUB, jend, col, grp, s_p[w], s_alpha[w]);
    }
  } else {
    int page = PAGED && j0 <= jend ? table[j0 / a.page_size] : 0;
    for (int js = j0; js <= jend; js += SUB) {
      DecRegs rr;
      if constexpr (PAGED) {
        const int next = table[min(js + SUB, jend) / a.page_size];
        dec_load_paged(rr, kbase, vbase, page, a.page_size, a.n_pages, kvrow, js, jend, col, grp);
        page = next;
      } else {
        dec_load(rr, kbase, vbase, kvrow, js, jend, col, grp);
      }
      st.step(rr, qf, c, js, jend, col, grp, s_p[w], s_alpha[w]);
    }
  }

  // reduce o over the 4 lane groups, then lanes 0..15 write the partial
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      st.o[r][e] = rows_sum(st.o[r][e]);
    }
  const int64_t pbase = (static_cast<int64_t>(b) * a.nq + g * R) * n_chunks + chunk;
  if (grp == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float* po = part_o + (pbase + static_cast<int64_t>(r) * n_chunks) * HD + col * 8;
      *reinterpret_cast<f32x4*>(po) = f32x4{st.o[r][0], st.o[r][1], st.o[r][2], st.o[r][3]};
      *reinterpret_cast<f32x4*>(po + 4) = f32x4{st.o[r][4], st.o[r][5], st.o[r][6], st.o[r][7]};
    }
  }
  if (lane < R) {
    part_ml[(pbase + static_cast<int64_t>(lane) * n_chunks) * 2 + 0] = st.m_run;
    part_ml[(pbase + static_cast<int64_t>(lane) * n_chunks) * 2 + 1] = st.l_run;
  }
}

// ===========================================================================
// decode kernel, workgroup-combined (bf16, hd = 128): one workgroup of NW
// wavefronts per (sequence, KV head).  Wavefront w walks slots
// [w*per, (w+1)*per) of the visible range exactly as attn_decode2_kernel does
// (MFMA scores, online softmax, VALU PV), leaves its (max, sum, o) in LDS, and
// after one barrier the workgroup merges the NW partials and writes the R
// output rows.  NW is chosen on the host so that all wavefronts of the launch
// are resident at once; nothing goes through HBM but K, V, q and the output.
// ===========================================================================
// At most 16 wavefronts per workgroup (8 for R = 8, whose accumulators need
// more than the 128 registers a 16-wavefront workgroup leaves per lane, and
// for the 8-bit cache, whose two steps of registers in flight need more too).
template <int R, bool KV8, bool PAGED = false>
__global__ void __launch_bounds__(R >= 8 || KV8 ? 512 : 1024)
attn_decode3_kernel(AttnArgs a) {
  constexpr int HD = 128, SUB = kDSub;
  using St = DecState<R>;
  constexpr int RP = St::RP;
  extern __shared__ float dsm[];
  const int nw = blockDim.x >> 6;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float(*s_p)[SUB][RP] = reinterpret_cast<float(*)[SUB][RP]>(dsm);
  float* s_ml = dsm + nw * SUB * RP;  // [nw][R][2]
  float* s_o = s_ml + nw * R * 2;     // [nw][R][HD]
  const int g = blockIdx.x % a.nkv, b = blockIdx.x / a.nkv;
  const int vis = min(a.positions ? a.positions[b] : 0, a.S - 1);
  const int per = ((vis + nw) / nw + SUB - 1) / SUB * SUB;  // slots per wavefront, whole steps
  const int j0 = w * per;
  const int jend = min(vis, j0 + per - 1);

  // K/V rows of (b, g): bf16 elements, or E4M3 codes (one byte each) plus
  // the fp32 row scales [n_kv][S] of the sequence
  const int64_t kvrow = static_cast<int64_t>(a.nkv) * HD;
  // (paged: the pool base at KV head g; the table picks the page per step)
  const int64_t kvoff = PAGED ? static_cast<int64_t>(g) * HD : (static_cast<int64_t>(b) * a.S * a.nkv + g) * HD;
  const bf16_t* kbase = static_cast<const bf16_t*>(a.k) + kvoff;
  const bf16_t* vbase = static_cast<const bf16_t*>(a.v) + kvoff;
  const int32_t* table = PAGED ? a.block_table + static_cast<int64_t>(b) * a.max_pages : nullptr;
  const int col = lane & 15, grp = lane >> 4;
  Dec8Src src8;
  if constexpr (KV8) {
    const int64_t hs = (static_cast<int64_t>(b) * a.nkv + g) * a.S;  // (sequence, KV head) slot base
    src8.init(static_cast<const uint8_t*>(a.k) + hs * HD, static_cast<const uint8_t*>(a.v) + hs * HD,
              a.k_scale + hs, a.v_scale + hs, vis, col, grp);
  }
  bf16x8_t qf[4];
  {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + (static_cast<int64_t>(b) * a.nq + g * R + (col < R ? col : 0)) * HD;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // head-dim step s, lane group grp: elements s*32 + grp*8 .. +7, or with
      // the 8-bit cache grp*32 + s*8 .. +7 (the permutation of its K codes)
      u32x4 t = *reinterpret_cast<const u32x4*>(qp + (KV8 ? grp * 32 + s * 8 : s * 32 + grp * 8));
      if (col >= R) t = u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8_t, t);
    }
  }
  const float c = a.scale * kLog2e;
  St st;
  st.init();
  float* my_alpha = s_ml + w * R * 2;  // scratch for the step's rescale factors (before the final write)
  if constexpr (KV8) {
    // half the bytes per slot: the next step's loads are issued before this
    // step's arithmetic so that each wavefront keeps two steps in flight
    // (loads past the end re-read the last visible slot)
    DecRegsT<true> ra, rb;
    if (j0 <= jend) dec_load8(ra, src8, j0, jend, col, grp);
    for (int js = j0; js <= jend; js += 2 * SUB) {
      dec_load8(rb, src8, js + SUB, jend, col, grp);
      st.step(ra, qf, c, js, jend, col, grp, s_p[w], my_alpha);
      if (js + SUB > jend) break;
      dec_load8(ra, src8, js + 2 * SUB, jend, col, grp);
      st.step(rb, qf, c, js + SUB, jend, col, grp, s_p[w], my_alpha);
    }
  } else {
    int page = PAGED && j0 <= jend ? table[j0 / a.page_size] : 0;
    for (int js = j0; js <= jend; js += SUB) {
      DecRegs rr;
      if constexpr (PAGED) {
        const int next = table[min(js + SUB, jend) / a.page_size];
        dec_load_paged(rr, kbase, vbase, page, a.page_size, a.n_pages, kvrow, js, jend, col, grp);
        page = next;
      } else {
        dec_load(rr, kbase, vbase, kvrow, js, jend, col, grp);
      }
      st.step(rr, qf, c, js, jend, col, grp, s_p[w], my_alpha);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) st.o[r][e] = rows_sum(st.o[r][e]);
  if (grp == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float* po = s_o + (w * R + r) * HD + col * 8;
      *reinterpret_cast<f32x4*>(po) = f32x4{st.o[r][0], st.o[r][1], st.o[r][2], st.o[r][3]};
      *reinterpret_cast<f32x4*>(po + 4) = f32x4{st.o[r][4], st.o[r][5], st.o[r][6], st.o[r][7]};
    }
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < R) {
    s_ml[(w * R + lane) * 2 + 0] = st.m_run;
    s_ml[(w * R + lane) * 2 + 1] = st.l_run;
  }
  __syncthreads();
  bf16_t* out = static_cast<bf16_t*>(a.out) + (static_cast<int64_t>(b) * a.nq + g * R) * HD;
  for (int idx = threadIdx.x; idx < R * HD; idx += blockDim.x) {
    const int r = idx / HD, d = idx - r * HD;
    float mx = -INFINITY;
    for (int w2 = 0; w2 < nw; ++w2) mx = fmaxf(mx, s_ml[(w2 * R + r) * 2]);
    float l = 0.f, o = 0.f;
    for (int w2 = 0; w2 < nw; ++w2) {
      const float f = fast_exp2(s_ml[(w2 * R + r) * 2] - mx);
      l += s_ml[(w2 * R + r) * 2 + 1] * f;
      o += s_o[(w2 * R + r) * HD + d] * f;
    }
    out[idx] = f32_to_bf16(o / l);
  }
}

size_t decode3_lds_bytes(int R, int nw) {
  const int rp = R > 4 ? R : 4;
  return static_cast<size_t>(nw) * (kDSub * rp + R * 2 + R * 128) * sizeof(float);
}

// one wavefront per (b, h): merge the visible chunks.  The chunk maxima and
// sums are reduced across lanes; each lane then owns HD/64 consecutive output
// elements and accumulates the chunks with all their loads independent.
template <typename T, int HD>
__global__ void __launch_bounds__(256)
attn_decode_combine_kernel(AttnArgs a, int n_chunks, int chunk_len, const float* __restrict__ part_o,
                           const float* __restrict__ part_ml) {
  constexpr int E = HD / 64 > 0 ? HD / 64 : 1;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t bh = static_cast<int64_t>(blockIdx.x) * 4 + w;
  if (bh >= static_cast<int64_t>(a.B) * a.nq) return;
  const int b = static_cast<int>(bh / a.nq);
  const int vis = min(a.positions ? a.positions[b] : 0, a.S - 1);
  const int nvalid = vis < 0 ? 0 : min(n_chunks, vis / chunk_len + 1);
  const float* ml = part_ml + bh * n_chunks * 2;
  float mx = -INFINITY;
  for (int ch = lane; ch < nvalid; ch += 64) mx = fmaxf(mx, ml[2 * ch]);
  mx = wave_max(mx);
  float lsum = 0.f;
  for (int ch = lane; ch < nvalid; ch += 64) lsum += ml[2 * ch + 1] * fast_exp2(ml[2 * ch] - mx);
  lsum = wave_sum(lsum);
  float o[E] = {};
  const float* po = part_o + bh * n_chunks * HD + lane * E;
#pragma unroll 8
  for (int ch = 0; ch < nvalid; ++ch) {
    const float f = fast_exp2(ml[2 * ch] - mx);
#pragma unroll
    for (int i = 0; i < E; ++i) o[i] += po[ch * HD + i] * f;
  }
  const float inv = 1.f / lsum;
  T* out = static_cast<T*>(a.out) + bh * HD + lane * E;
  if (lane * E < HD) {
#pragma unroll
    for (int i = 0; i < E; ++i) st(out + i, o[i] * inv);
  }
}

int decode_chunks(int S) { return (S + kDChunk - 1) / kDChunk; }

int device_cus() {
  static thread_local int cached_dev = -1, cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached_dev = dev;
    cached_cus = n;
  }
  return cached_cus;
}

constexpr size_t kD3MaxLds = 64 * 1024;

template <int R, bool KV8>
constexpr int d3_max_waves() { return R >= 8 || KV8 ? 8 : 16; }

// Workgroups of attn_decode3_kernel<R> with nw wavefronts that one CU holds
// at once (register, LDS and wave-slot limits), cached per device.
template <int R, bool KV8, bool PAGED>
int d3_blocks_per_cu(int nw) {
  static thread_local int cached_dev = -1;
  static thread_local int cache[17];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev != cached_dev) {
    for (int& c : cache) c = -1;
    cached_dev = dev;
  }
  if (cache[nw] < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_decode3_kernel<R, KV8, PAGED>, 64 * nw,
                                                     decode3_lds_bytes(R, nw)) != hipSuccess)
      n = 0;
    cache[nw] = n;
  }
  return cache[nw];
}

// Wavefronts in flight for the bf16 decode kernels: about 6 per CU.  On
// MI355X the K/V stream of the B=64, 4097-slot workload measured 5.75 TB/s
// with 6 wavefronts per CU (1536 streams), against 5.2-5.5 TB/s with 4, 8, 10
// or 16: more concurrent streams than that cost HBM page locality, fewer
// leave bandwidth idle.
constexpr int kDecWavesPerCu = 6;
// The 8-bit cache's rows are half as long and each wavefront keeps two steps
// in flight; its sweep on the same workload: 4 / 6 / 8 / 10 / 12 / 16 per CU
// gave 131 / 115 / 109 / 121 / 119 / 120 us.
constexpr int kDecWavesPerCuFp8 = 8;
// The split path (few pairs, long histories) sizes its chunks for one
// four-wavefront workgroup per CU: on MI355X, 8 sequences x 8 KV heads at
// 32768 slots took 288 / 209 / 190 / 240 / 210 / 207 / 211 us with chunks for
// 2 / 3 / 4 / 5 / 6 / 8 / 12 wavefronts per CU (fewer than one workgroup per
// CU leaves CUs idle, a fraction more leaves a tail).
constexpr int kDecSplitWavesPerCu = 4;

// Wavefronts per (sequence, KV head) workgroup of attn_decode3_kernel: close
// to the target count, all workgroups resident in one round, within LDS.
template <int R, bool KV8, bool PAGED>
int d3_pick_waves(int64_t pairs, int64_t target) {
  const int cus = device_cus();
  int nw = static_cast<int>(std::min<int64_t>(d3_max_waves<R, KV8>(), std::max<int64_t>(1, (target + pairs / 2) / pairs)));
  while (nw > 1 && (decode3_lds_bytes(R, nw) > kD3MaxLds ||
                    pairs > static_cast<int64_t>(d3_blocks_per_cu<R, KV8, PAGED>(nw)) * cus))
    --nw;
  return nw;
}

template <int R, bool KV8, bool PAGED = false>
hipError_t launch_decode_bf16(const AttnArgs& a, void* ws, hipStream_t s, const char** kernel_name) {
  constexpr int HD = 128;
  const int64_t pairs = static_cast<int64_t>(a.B) * a.nkv;
  const int64_t target = static_cast<int64_t>(device_cus()) * (KV8 ? kDecWavesPerCuFp8 : kDecWavesPerCu);
  const int nw = d3_pick_waves<R, KV8, PAGED>(pairs, target);
  if (pairs * nw * 2 >= target && pairs * 4 >= 3 * static_cast<int64_t>(device_cus())) {
    // one workgroup per (sequence, KV head) reaches at least half the target
    // and keeps at least 3/4 of the CUs streaming: a CU alone moves far less
    // than its share of HBM bandwidth, however many wavefronts it holds.  On
    // MI355X (32K-slot histories, 8 KV heads) 128 pairs ran 534 us this way
    // against 395 us split; 192 pairs 162 us against 171 us split.
    if (kernel_name) *kernel_name = KV8 ? "attn_decode_wg_fp8kv" : PAGED ? "attn_decode_wg_paged" : "attn_decode_wg";
    hipLaunchKernelGGL((attn_decode3_kernel<R, KV8, PAGED>), dim3(static_cast<unsigned>(pairs)), dim3(64 * nw),
                       decode3_lds_bytes(R, nw), s, a);
    return hipGetLastError();
  }
  // few pairs (long contexts, small batches): split the slots of each pair
  // into chunks across wavefronts of their own, then merge the partials
  if (kernel_name)
    *kernel_name = KV8 ? "attn_decode_splitk_fp8kv" : PAGED ? "attn_decode_splitk_paged" : "attn_decode_splitk";
  const int64_t want = std::max<int64_t>(1, static_cast<int64_t>(device_cus()) * kDecSplitWavesPerCu / pairs);
  int chunk = static_cast<int>(((a.S + want - 1) / want + kDSub - 1) / kDSub * kDSub);
  chunk = std::max(chunk, kDChunk);  // never more chunks than the workspace holds
  const int nch = (a.S + chunk - 1) / chunk;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o + static_cast<int64_t>(a.B) * a.nq * nch * HD;
  hipLaunchKernelGGL((attn_decode2_kernel<R, KV8, PAGED>), dim3(static_cast<unsigned>((pairs * nch + 3) / 4)), dim3(256), 0, s,
                     a, nch, chunk, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t waves = static_cast<int64_t>(a.B) * a.nq;
  hipLaunchKernelGGL((attn_decode_combine_kernel<bf16_t, HD>), dim3(static_cast<unsigned>((waves + 3) / 4)),
                     dim3(256), 0, s, a, nch, chunk, part_o, part_ml);
  return hipGetLastError();
}

// Generic decode (fp32, or hd = 64): attn_decode_kernel over 256-slot chunks
// plus the merge.
template <typename T, int HD>
hipError_t launch_decode_t(const AttnArgs& a, void* ws, hipStream_t s, const char** kernel_name) {
  const int R = a.nq / a.nkv;
  if (sizeof(T) == 2 && HD == 128) {
    switch (R) {
      case 1: return launch_decode_bf16<1, false>(a, ws, s, kernel_name);
      case 2: return launch_decode_bf16<2, false>(a, ws, s, kernel_name);
      case 4: return launch_decode_bf16<4, false>(a, ws, s, kernel_name);
      case 8: return launch_decode_bf16<8, false>(a, ws, s, kernel_name);
      default: return hipErrorInvalidValue;
    }
  }
  if (kernel_name) *kernel_name = "attn_decode_splitk";
  const int nch = decode_chunks(a.S);
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o + static_cast<int64_t>(a.B) * a.nq * nch * HD;
  dim3 grid(a.B * a.nkv * nch);
  switch (R) {
    case 1: hipLaunchKernelGGL((attn_decode_kernel<T, HD, 1>), grid, dim3(256), 0, s, a, nch, part_o, part_ml); break;
    case 2: hipLaunchKernelGGL((attn_decode_kernel<T, HD, 2>), grid, dim3(256), 0, s, a, nch, part_o, part_ml); break;
    case 4: hipLaunchKernelGGL((attn_decode_kernel<T, HD, 4>), grid, dim3(256), 0, s, a, nch, part_o, part_ml); break;
    case 8: hipLaunchKernelGGL((attn_decode_kernel<T, HD, 8>), grid, dim3(256), 0, s, a, nch, part_o, part_ml); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t waves = static_cast<int64_t>(a.B) * a.nq;
  hipLaunchKernelGGL((attn_decode_combine_kernel<T, HD>), dim3(static_cast<unsigned>((waves + 3) / 4)),
                     dim3(256), 0, s, a, nch, kDChunk, part_o, part_ml);
  return hipGetLastError();
}

bool decode_supported(DType dt, const AttnArgs& a) {
  const int R = a.nq / a.nkv;
  const bool r_ok = R == 1 || R == 2 || R == 4 || R == 8;
  return a.Tq == 1 && r_ok && (a.hd == 64 || a.hd == 128);
  (void)dt;
}

bool flash_supported(DType dt, const AttnArgs& a) {
  const int R = a.nq / a.nkv;
  // (the K/V buffer resources address one sequence's cache with 32-bit offsets)
  return dt == DType::BF16 && a.Tq > 1 && a.hd == kFHd &&
         (R == 1 || R == 2 || R == 4 || R == 8) &&
         static_cast<int64_t>(a.S) * a.nkv * a.hd * 2 < (int64_t(1) << 31);
}

}  // namespace

size_t attention_workspace_bytes(DType dt, int B, int Tq, int S, int nq, int nkv, int hd) {
  AttnArgs a{};
  a.B = B; a.Tq = Tq; a.S = S; a.nq = nq; a.nkv = nkv; a.hd = hd;
  if (!decode_supported(dt, a)) return 0;
  const int nch = decode_chunks(S);
  return static_cast<size_t>(B) * nq * nch * (hd + 2) * sizeof(float);
}

size_t attention_fp8kv_workspace_bytes(int B, int S, int nq, int nkv) {
  return static_cast<size_t>(B) * nq * decode_chunks(S) * (128 + 2) * sizeof(float);
}

hipError_t launch_attention_fp8kv(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s,
                                  const char** kernel_name) {
  if (a.B == 0) return hipSuccess;
  if (a.Tq != 1 || a.hd != 128 || !a.k_scale || !a.v_scale) return hipErrorInvalidValue;
  if (ws_bytes < attention_fp8kv_workspace_bytes(a.B, a.S, a.nq, a.nkv)) return hipErrorInvalidValue;
  // (the buffer resources address one KV head's rows with 32-bit offsets)
  if (static_cast<int64_t>(a.S) * 128 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  switch (a.nq / a.nkv) {
    case 1: return launch_decode_bf16<1, true>(a, ws, s, kernel_name);
    case 2: return launch_decode_bf16<2, true>(a, ws, s, kernel_name);
    case 4: return launch_decode_bf16<4, true>(a, ws, s, kernel_name);
    case 8: return launch_decode_bf16<8, true>(a, ws, s, kernel_name);
    default: return hipErrorInvalidValue;
  }
}

size_t attention_paged_workspace_bytes(int B, int S, int nq) {
  return static_cast<size_t>(B) * nq * decode_chunks(S) * (128 + 2) * sizeof(float);
}

hipError_t launch_attention_paged(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t s,
                                  const char** kernel_name) {
  if (a.B == 0) return hipSuccess;
  if (a.Tq != 1 || a.hd != 128 || !a.block_table || a.page_size <= 0 || a.page_size % kDSub != 0 ||
      a.n_pages <= 0)
    return hipErrorInvalidValue;
  if (ws_bytes < attention_paged_workspace_bytes(a.B, a.S, a.nq)) return hipErrorInvalidValue;
  switch (a.nq / a.nkv) {
    case 1: return launch_decode_bf16<1, false, true>(a, ws, s, kernel_name);
    case 2: return launch_decode_bf16<2, false, true>(a, ws, s, kernel_name);
    case 4: return launch_decode_bf16<4, false, true>(a, ws, s, kernel_name);
    case 8: return launch_decode_bf16<8, false, true>(a, ws, s, kernel_name);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention(DType dt, const AttnArgs& a, void* ws, size_t ws_bytes,
                            hipStream_t s, const char** kernel_name) {
  if (a.B == 0 || a.Tq == 0) return hipSuccess;
  if (decode_supported(dt, a)) {
    if (ws_bytes < attention_workspace_bytes(dt, a.B, a.Tq, a.S, a.nq, a.nkv, a.hd))
      return hipErrorInvalidValue;
    if (dt == DType::BF16)
      return a.hd == 128 ? launch_decode_t<bf16_t, 128>(a, ws, s, kernel_name)
                         : launch_decode_t<bf16_t, 64>(a, ws, s, kernel_name);
    return a.hd == 128 ? launch_decode_t<float, 128>(a, ws, s, kernel_name)
                       : launch_decode_t<float, 64>(a, ws, s, kernel_name);
  }
  if (flash_supported(dt, a)) {
    const int R = a.nq / a.nkv;
    const int TQ = kFRows / R;
    const int n_qtiles = (a.Tq + TQ - 1) / TQ;
    dim3 grid(a.B * a.nkv * n_qtiles);
    if (kernel_name) *kernel_name = "attn_flash_prefill";
    switch (R) {
      case 1: hipLaunchKernelGGL((attn_flash_kernel<1>), grid, dim3(256), 0, s, a, n_qtiles); break;
      case 2: hipLaunchKernelGGL((attn_flash_kernel<2>), grid, dim3(256), 0, s, a, n_qtiles); break;
      case 4: hipLaunchKernelGGL((attn_flash_kernel<4>), grid, dim3(256), 0, s, a, n_qtiles); break;
      default: hipLaunchKernelGGL((attn_flash_kernel<8>), grid, dim3(256), 0, s, a, n_qtiles); break;
    }
    return hipGetLastError();
  }
  if (a.hd > 256) return hipErrorInvalidValue;
  const int64_t rows = static_cast<int64_t>(a.B) * a.Tq * a.nq;
  dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  if (kernel_name) *kernel_name = "attn_valu";
  if (dt == DType::F32)
    hipLaunchKernelGGL((attn_valu_kernel<float>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_valu_kernel<bf16_t>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lb
