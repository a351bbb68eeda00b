// fa_bwd.hip -- gradients of exact attention for MI355X (gfx950, CDNA4), C ABI in include/fa.h.
//
// For one head, with kept pairs (i, j) as in the forward pass (j <= i when
// causal), s_ij = scale <q_i, k_j>, P_ij = exp(s_ij - lse_i) and an upstream
// gradient dO:
//   dV_j = sum_i P_ij dO_i,   dP_ij = <dO_i, v_j>,   delta_i = <dO_i, O_i>,
//   dS_ij = P_ij (dP_ij - delta_i),
//   dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i.
// P is never stored: every kernel recomputes it tile by tile from the row
// log-sum-exp the forward pass wrote, the statistic a recomputing backward pass
// keeps ("FlashAttention" (ai360xpert), section "Recomputation in the
// backward pass"); delta_i = sum_j P_ij dP_ij reduces to <dO_i, O_i> because
// O_i = sum_j P_ij v_j.
//
// Three kernels per call (plus a summing kernel when split), no atomics, so
// the result is bitwise reproducible:
//  * attn_bwd_prep: per row, nl = -lse/scale and nd = -delta (fp32) into the
//    caller's workspace (rows padded to a multiple of 32 with zeros).  These
//    are the initial accumulators of the score and dP products below, so
//    S + nl and dP - delta come out of the matrix core directly.
//  * attn_bwd_dkdv: a workgroup owns 128 keys (32 per wave) of one head, with
//    its K and V rows held in registers, and streams 32-row tiles of Q and dO
//    through double-buffered LDS.  S = Q K^T and dP = dO V^T are computed in
//    (query x key) orientation, so each lane owns one key column and its P and
//    dS values are already the B operand of dV^T += dO^T P and
//    dK^T += Q^T dS; dO^T and Q^T are read out of the same LDS tiles with
//    ds_read_b64_tr_b16 (the V^T reads of the forward kernel).  Tiles read
//    both ways are row-major with a chunk swizzle that keeps both kinds of
//    read free of bank conflicts.
//  * attn_bwd_dq: a workgroup owns 256 query rows (128 at d = 64; 32 per
//    wave) with Q and dO in registers and streams 64-key tiles of K and V, like the forward pass:
//    S^T = K Q^T, dP^T = V dO^T, then dQ^T += K^T dS^T with K^T read by the
//    transpose instruction.
// All products run on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulators;
// P and dS are rounded to the input type before their products.  fp32 inputs
// take their own kernels (attn_bwd_*_f32, on v_mfma_f32_32x32x2_f32), and
// grids too small to fill the GPU share each block's tiles over several
// workgroups whose fp32 partial sums attn_bwd_sum_* adds in a fixed order.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <initializer_list>

#include "fa.h"
#include "fa_device.h"

namespace {

using namespace fa_dev;

// widen one 16-bit element to fp32
template <class TT>
__device__ __forceinline__ float widen(uint16_t x);
template <>
__device__ __forceinline__ float widen<Bf16>(uint16_t x) {
  return __uint_as_float((unsigned)x << 16);
}
template <>
__device__ __forceinline__ float widen<F16>(uint16_t x) {
  return (float)__builtin_bit_cast(_Float16, x);
}

constexpr int kRowPad = 32;  // statistic rows are padded to this multiple

// The streamed tiles that are read both as rows and transposed (Q and dO in
// the dK/dV kernel, K in the dQ kernel) use the swizzled row-major layout of
// TileLayout::s_src: 1 KB blocks of 16 rows x 4 sixteen-byte chunks, block
// (rg, cg) at (rg * D/32 + cg) KB, row ri chunk ci in slot 4ri + (ci ^ ri/4).
__device__ __forceinline__ int swz_slot(int ri, int ci) { return 4 * ri + (ci ^ (ri >> 2)); }

// Byte offset, inside such a tile, of the 16 bytes lane (row, hf) supplies as
// the A operand of a 32x32x16 product over head-dim chunk c: elements
// [16c + 8hf, 16c + 8hf + 8) of row `row`.  A 16-lane group reads 16 rows of
// one chunk: 16 distinct slots modulo 16, so no bank conflicts.
template <int D>
__device__ __forceinline__ int rowmajor_a(int row, int hf, int c) {
  const int t = 2 * c + hf;  // 16-byte chunk of the row
  return ((row >> 4) * (D / 32) + (t >> 2)) * 1024 + swz_slot(row & 15, t & 3) * 16;
}

// Lane parts of the transpose read (ds_read_b64_tr_b16) of one such block:
// the reads at offsets lo and hi give lane (x = lane % 32, h = lane / 32)
// rows {4h .. 4h+3} and {8 + 4h .. 8 + 4h + 3} of column x of the block's
// 32 columns -- the A-operand order that matches a B operand packed from
// accumulator registers 0..7 (rows 8(r/4) + 4h + r%4).  Each lane reads 8
// bytes of row r (first read: r in 0..7, second: r + 8), chunk ch.
struct TrLane {
  int lo, hi;
};
__device__ __forceinline__ TrLane tr_lane(int lane) {
  const int i = lane & 15, grp = lane >> 4;
  const int r = 4 * (grp >> 1) + (i >> 2), ch = 2 * (grp & 1) + ((i & 3) >> 1), half = 8 * (i & 1);
  return TrLane{swz_slot(r, ch) * 16 + half, swz_slot(r + 8, ch) * 16 + half};
}

__device__ __forceinline__ u32x4 tr_read(const uint8_t* blk, TrLane t) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(blk + t.lo));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(blk + t.hi));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
}

// Store a wave's 32 x D transposed accumulator (block b, register r of lane
// (x, h) = element [row x][32b + 8(r/4) + 4h + r%4]) times `mul`, rounded to
// the element type, to rows row0 .. row0+31 of `out` (rows >= n_valid are
// skipped).  Passes through the wave's own LDS area `stg` (32 rows x 144
// bytes) so that each store writes whole 128-byte row segments.
template <class TT, int D>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[D / 32], float mul, uint8_t* stg,
                                           uint16_t* out, int row0, int n_valid, int lane) {
  constexpr int kRow = 144;
  const int x = lane & 31, h = lane >> 5;
#pragma unroll
  for (int r = 0; r < D / 64; ++r) {
#pragma unroll
    for (int bl = 0; bl < 2; ++bl)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = acc[2 * r + bl];
        const u32x2 w = {TT::pack(a[4 * g + 0] * mul, a[4 * g + 1] * mul),
                         TT::pack(a[4 * g + 2] * mul, a[4 * g + 3] * mul)};
        *(u32x2*)(stg + x * kRow + 2 * (32 * bl + 8 * g + 4 * h)) = w;
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 8 * i + (lane >> 3);
      const u32x4 v = *(const u32x4*)(stg + row * kRow + 16 * (lane & 7));
      if (row0 + row < n_valid) *(u32x4*)(out + (size_t)(row0 + row) * D + 64 * r + 8 * (lane & 7)) = v;
    }
  }
}

// Store a wave's 32 x D transposed accumulator (block b, register 4g+e of
// lane (x, h) = element [row x][32b + 8g + 4h + e]) times `mul`, in fp32, to
// rows row0 .. row0+31 of `out` (rows >= n_valid are skipped): the partial
// sums of a split, one 16-byte store per register group.
template <int D>
__device__ __forceinline__ void store_rows_f32(const f32x16 (&acc)[D / 32], float mul, float* out,
                                               int row0, int n_valid, int lane) {
  const int x = lane & 31, h = lane >> 5;
  if (row0 + x >= n_valid) return;
  float* row = out + (size_t)(row0 + x) * D + 4 * h;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(f32x4*)(row + 32 * b + 8 * g) = f32x4{acc[b][4 * g] * mul, acc[b][4 * g + 1] * mul,
                                               acc[b][4 * g + 2] * mul, acc[b][4 * g + 3] * mul};
}

// ---------------------------------------------------------------------------
// Row statistics.  TPR = D/8 threads per row, 8 elements each.
template <class TT, int D>
__global__ __launch_bounds__(256) void attn_bwd_prep(const uint16_t* __restrict__ O,
                                                     const uint16_t* __restrict__ dO,
                                                     const float* __restrict__ LSE,
                                                     float* __restrict__ NL, float* __restrict__ ND,
                                                     int N, int H, const int* __restrict__ q_len,
                                                     int n_pad, long long padded_rows,
                                                     float inv_scale) {
  // N: query rows per head (the rows of O, dO and lse); rows from the batch's
  // valid query count on are padding: P = 0 there (nl = -inf), never read
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  const int t = threadIdx.x % TPR;
  const long long prow = (long long)blockIdx.x * RPB + threadIdx.x / TPR;  // padded row id
  if (prow >= padded_rows) return;  // whole rows only: TPR divides the wave
  const long long bh = prow / n_pad;
  const int i = (int)(prow % n_pad);
  const int nq = q_len ? min(max(q_len[bh / H], 0), N) : N;
  float acc = 0.f, nl = i < N ? -INFINITY : 0.f;
  if (i < nq) {
    const size_t row = (size_t)bh * N + i;
    const u32x4 a = *(const u32x4*)(O + row * D + 8 * t);
    const u32x4 b = *(const u32x4*)(dO + row * D + 8 * t);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(widen<TT>((uint16_t)(a[w] & 0xffffu)), widen<TT>((uint16_t)(b[w] & 0xffffu)), acc);
      acc = fmaf(widen<TT>((uint16_t)(a[w] >> 16)), widen<TT>((uint16_t)(b[w] >> 16)), acc);
    }
    // a row that kept no key (lse = -inf) keeps P = 0 without an infinite step
    const float l = LSE[row];
    nl = l == -INFINITY ? -INFINITY : -l * inv_scale;
  }
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m, TPR);
  if (t == 0) {
    NL[prow] = nl;
    ND[prow] = -acc;
  }
}

// ---------------------------------------------------------------------------
// dK, dV.  NW = 4 waves x 32 keys; query tiles of 32 rows.
//
// Register layouts (DK = head dim of Q and K, DV = of V, O and dO; lane
// (x = lane % 32, h = lane / 32)):
//   K and V rows (whole kernel): lane holds row[key0 + x][16c + 8h .. +7]
//     for c = 0..DK/16-1 (K) or DV/16-1 (V), the B operand of S = Q K^T and
//     dP = dO V^T.
//   S, dP (accumulators, 32 queries x 32 keys): register r of lane (x, h) is
//     query 8(r/4) + 4h + r%4 of the tile and key key0 + x.
//   dK^T, dV^T (accumulators): block b, register r of lane (x, h) is
//     d-column 32b + 8(r/4) + 4h + r%4 of key key0 + x.
// Occupancy (both main kernels): two waves per SIMD, three at d = 64 (they fit
// 168 registers there; measured 9% faster on the d = 64 workload).
template <class TT, int DK, int DV, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(DK + DV == 128 ? 3 : 2, DK + DV == 128 ? 3 : 2))) void attn_bwd_dkdv(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ NL, const float* __restrict__ ND,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Nq, int Nk, int H,
    const int* __restrict__ k_len, const int* __restrict__ q_len, int n_pad, int n_kblocks, int total, float scale, int n_split,
    float* __restrict__ part, long long kstride, long long vstride) {
  constexpr int BQ = 32, CGK = DK / 32, CGV = DV / 32;
  // 1 KB blocks and bytes of one 32-row Q tile and one dO tile
  constexpr int TBLKQ = 2 * CGK, TBQ = TBLKQ * 1024, TBLKD = 2 * CGV, TBD = TBLKD * 1024;
  // [buffer][Q tile, dO tile, nl of its rows (1 KB), nd of its rows (1 KB)];
  // the epilogue reuses it as the waves' output staging
  constexpr int BUF = TBQ + TBD + 2048;
  constexpr int SMEM = 2 * BUF > NW * 32 * 144 ? 2 * BUF : NW * 32 * 144;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int x = lane & 31, h = lane >> 5;
  const int item = xcd_remap(blockIdx.x, total);
  // split (small grids): this workgroup takes one of n_split shares of the
  // block's query tiles and writes fp32 partial sums to `part`
  const int split = item % n_split, work = item / n_split;
  const int bh = work / n_kblocks;
  const int kb = work % n_kblocks;  // ascending: causal key blocks near 0 see the most queries
  // as in the forward: key j is kept for query i < nq iff j < nk and, when
  // causal, j <= i + diag; query rows from nq on are padding
  const int nk = k_len ? min(max(k_len[bh / H], 0), Nk) : Nk;
  const int nq = q_len ? min(max(q_len[bh / H], 0), Nq) : Nq;
  const int diag = nk - nq;
  const size_t head = (size_t)bh * Nq * DK, ohead = (size_t)bh * Nq * DV;
  const size_t khead = (size_t)bh * Nk * DK, vhead = (size_t)bh * Nk * DV;
  const int k0 = kb * 32 * NW;              // the block's first key
  const int kw = k0 + 32 * wave;            // this wave's first key
  const int my_k = kw + x;

  u32x4 kf[DK / 16], vf[DV / 16];
  {
    const uint16_t* kr = K + khead + (size_t)my_k * DK + 8 * h;
    const uint16_t* vr = V + vhead + (size_t)my_k * DV + 8 * h;
    if constexpr (DK == DV) {
#pragma unroll
      for (int c = 0; c < DK / 16; ++c) {
        kf[c] = my_k < nk ? *(const u32x4*)(kr + 16 * c) : u32x4{0, 0, 0, 0};
        vf[c] = my_k < nk ? *(const u32x4*)(vr + 16 * c) : u32x4{0, 0, 0, 0};
      }
    } else {
#pragma unroll
      for (int c = 0; c < DK / 16; ++c)
        kf[c] = my_k < nk ? *(const u32x4*)(kr + 16 * c) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < DV / 16; ++c)
        vf[c] = my_k < nk ? *(const u32x4*)(vr + 16 * c) : u32x4{0, 0, 0, 0};
    }
  }
  f32x16 dk[DK / 32], dv[DV / 32];
#pragma unroll
  for (int b = 0; b < DK / 32; ++b) dk[b] = f32x16{};
#pragma unroll
  for (int b = 0; b < DV / 32; ++b) dv[b] = f32x16{};
  const float c2 = scale * kLog2e;
  const float* nl_row = NL + (size_t)bh * n_pad;
  const float* nd_row = ND + (size_t)bh * n_pad;

  const int nqt = (nq + BQ - 1) / BQ;
  // first tile holding a query that keeps a key of this block (q + diag >= k0);
  // a block wholly past the valid keys has none and only writes zeros
  const int qt0 = k0 >= nk ? nqt : CAUSAL ? max(0, k0 - diag) / BQ : 0;
  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  auto load = [&](int t, int buf) {
    const int r0 = t * BQ;
    const unsigned base = lds0 + buf * BUF;
    // the rows' statistics: one wave-wide load each, 128 bytes of data (the
    // rest of the 1 KB reads past the descriptor's end and lands as zeros)
    if (wave < 2) {
      const float* src = (wave == 0 ? nl_row : nd_row) + r0;
      dma16(buffer_desc(src, BQ * 4), base + TBQ + TBD + 1024 * wave, lane * 16);
    }
    // rows past nq read as zero (never loaded)
    const u32x4 dq = buffer_desc(Q + head + (size_t)r0 * DK, (unsigned)(nq - r0) * DK * 2);
    const u32x4 dd = buffer_desc(dO + ohead + (size_t)r0 * DV, (unsigned)(nq - r0) * DV * 2);
    if constexpr (DK == DV) {  // the same block pattern in both tiles
#pragma unroll
      for (int i = 0; i < (TBLKQ + NW - 1) / NW; ++i) {
        const int blk = wave + i * NW;
        if (blk < TBLKQ) {  // with more waves than blocks, some waves load none
          const int el = TileLayout<DK>::s_src(blk, lane);
          dma16(dq, base + blk * 1024, el * 2);
          dma16(dd, base + TBQ + blk * 1024, el * 2);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < (TBLKQ + NW - 1) / NW; ++i) {
        const int blk = wave + i * NW;
        if (blk < TBLKQ) dma16(dq, base + blk * 1024, TileLayout<DK>::s_src(blk, lane) * 2);
      }
#pragma unroll
      for (int i = 0; i < (TBLKD + NW - 1) / NW; ++i) {
        const int blk = wave + i * NW;
        if (blk < TBLKD) dma16(dd, base + TBQ + blk * 1024, TileLayout<DV>::s_src(blk, lane) * 2);
      }
    }
  };
  const TrLane trl = tr_lane(lane);

  const int qs = qt0 + (int)((long long)(nqt - qt0) * split / n_split);
  const int qe = qt0 + (int)((long long)(nqt - qt0) * (split + 1) / n_split);
  if (qs < qe) load(qs, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  for (int t = qs; t < qe; ++t) {
    const int buf = (t - qs) & 1;
    if (t + 1 < qe) load(t + 1, buf ^ 1);
    const int q0 = t * BQ;
    // nothing kept when this wave's keys are all padding, or all above the
    // last query row of the tile
    if (kw < nk && (!CAUSAL || q0 + BQ - 1 + diag >= kw)) {
      const uint8_t* qt = smem + buf * BUF;
      const uint8_t* dt = qt + TBQ;
      f32x16 s, dp;
      // initial accumulators: -lse/scale and -delta of the tile's rows
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 a = *(const f32x4*)(qt + TBQ + TBD + 4 * (8 * g + 4 * h));
        const f32x4 b = *(const f32x4*)(qt + TBQ + TBD + 1024 + 4 * (8 * g + 4 * h));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[4 * g + e] = a[e];
          dp[4 * g + e] = b[e];
        }
      }
      if constexpr (DK == DV) {
#pragma unroll
        for (int c = 0; c < DK / 16; ++c) {
          s = TT::mma(*(const u32x4*)(qt + rowmajor_a<DK>(x, h, c)), kf[c], s);
          dp = TT::mma(*(const u32x4*)(dt + rowmajor_a<DV>(x, h, c)), vf[c], dp);
        }
      } else {
#pragma unroll
        for (int c = 0; c < DK / 16; ++c) s = TT::mma(*(const u32x4*)(qt + rowmajor_a<DK>(x, h, c)), kf[c], s);
#pragma unroll
        for (int c = 0; c < DV / 16; ++c) dp = TT::mma(*(const u32x4*)(dt + rowmajor_a<DV>(x, h, c)), vf[c], dp);
      }
      // P = exp(scale s - lse); dS = P (dP - delta); a tile across the
      // diagonal or the end of the valid keys keeps key <= query + diag and
      // key < nk only: its other scores become -inf before the exponentials
      // (P = 0 exactly), in a branch that only such tiles take
      const bool mask = (CAUSAL && q0 + diag < kw + 31) || kw + 31 >= nk;
      if (mask) {
        const int lim = my_k >= nk ? 0x7fffffff : CAUSAL ? my_k - diag : -0x7fffffff;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (q0 + 8 * (r >> 2) + 4 * h + (r & 3) < lim) s[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(s[r] * c2);
        s[r] = p;
        dp[r] = p * dp[r];
      }
      u32x4 pf[2], df[2];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int r0 = 8 * kc;
        pf[kc] = u32x4{TT::pack(s[r0 + 0], s[r0 + 1]), TT::pack(s[r0 + 2], s[r0 + 3]),
                       TT::pack(s[r0 + 4], s[r0 + 5]), TT::pack(s[r0 + 6], s[r0 + 7])};
        df[kc] = u32x4{TT::pack(dp[r0 + 0], dp[r0 + 1]), TT::pack(dp[r0 + 2], dp[r0 + 3]),
                       TT::pack(dp[r0 + 4], dp[r0 + 5]), TT::pack(dp[r0 + 6], dp[r0 + 7])};
      }
      // d = 64 (three waves per SIMD): the wave issuing its dV/dK products
      // is served before the others' vector work (measured 0.5-6% faster on
      // d = 64 shapes; 1% slower at d = 128, which keeps the default)
      if constexpr (DK + DV == 128) __builtin_amdgcn_s_setprio(1);
      // dV^T += dO^T P and dK^T += Q^T dS over the tile's 32 queries
      if constexpr (DK == DV) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
          for (int b = 0; b < DV / 32; ++b) {
            const int off = (kc * CGV + b) * 1024;
            dv[b] = TT::mma(tr_read(dt + off, trl), pf[kc], dv[b]);
            dk[b] = TT::mma(tr_read(qt + off, trl), df[kc], dk[b]);
          }
      } else {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
          for (int b = 0; b < DV / 32; ++b)
            dv[b] = TT::mma(tr_read(dt + (kc * CGV + b) * 1024, trl), pf[kc], dv[b]);
#pragma unroll
          for (int b = 0; b < DK / 32; ++b)
            dk[b] = TT::mma(tr_read(qt + (kc * CGK + b) * 1024, trl), df[kc], dk[b]);
        }
      }
    }
    if constexpr (DK + DV == 128) __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }
  // the tile buffers are free after the last barrier
  // every key row is written, those past the valid keys as zeros
  if (part) {  // split: the dK parts, then the dV parts
    store_rows_f32<DK>(dk, scale, part + (size_t)split * kstride + khead, kw, Nk, lane);
    store_rows_f32<DV>(dv, 1.f, part + (size_t)n_split * kstride + (size_t)split * vstride + vhead, kw,
                       Nk, lane);
    return;
  }
  uint8_t* stg = smem + wave * 32 * 144;
  store_rows<TT, DV>(dv, 1.f, stg, dV + vhead, kw, Nk, lane);
  store_rows<TT, DK>(dk, scale, stg, dK + khead, kw, Nk, lane);
}

// ---------------------------------------------------------------------------
// dQ.  NW = 8 waves x 32 queries (4 at d = 64); key tiles of 64 keys: K swizzled row-major
// (read as rows and, transposed, as K^T), V chunk-major (read as rows).
//
// Register layouts (lane (x, h)):
//   Q and dO rows (whole kernel): row[q_first + x][16c + 8h .. +7], the B
//     operands of S^T = K Q^T and dP^T = V dO^T.
//   S^T, dP^T (accumulators, per 32-key block): register r of lane (x, h) is
//     key 8(r/4) + 4h + r%4 of the block and query q_first + x.
//   dQ^T (accumulator): block b, register r is d-column 32b + 8(r/4) + 4h + r%4.
template <class TT, int DK, int DV, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(DK + DV == 128 ? 3 : 2, DK + DV == 128 ? 3 : 2))) void attn_bwd_dq(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ NL, const float* __restrict__ ND,
    uint16_t* __restrict__ dQ, int Nq, int Nk, int H, const int* __restrict__ k_len, const int* __restrict__ q_len, int n_pad,
    int n_qblocks, int total, float scale, int n_split, float* __restrict__ part,
    long long qstride) {
  // DK: head dim of Q, K and dQ; DV: of V and dO
  constexpr int BR = 32 * NW, BC = 64, CGK = DK / 32, CGV = DV / 32;
  using LK = TileLayout<DK>;
  using LV = TileLayout<DV>;
  constexpr int TBK = LK::BYTES, TBV = LV::BYTES, SB = TBK + TBV;
  static_assert(LK::BLOCKS % NW == 0 && LV::BLOCKS % NW == 0, "tile blocks split evenly over the waves");
  // [buffer][K, V]; the epilogue reuses it as the waves' output staging
  constexpr int SMEM = 2 * SB > NW * 32 * 144 ? 2 * SB : NW * 32 * 144;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int x = lane & 31, h = lane >> 5;
  const int item = xcd_remap(blockIdx.x, total);
  // split (small grids): one of n_split shares of the block's key tiles,
  // fp32 partial sums to `part`
  const int split = item % n_split, work = item / n_split;
  const int bh = work / n_qblocks;
  int qb = work % n_qblocks;
  if (CAUSAL) qb = n_qblocks - 1 - qb;  // longest rows first
  const int nk = k_len ? min(max(k_len[bh / H], 0), Nk) : Nk;  // as in the dK/dV kernel
  const int nq = q_len ? min(max(q_len[bh / H], 0), Nq) : Nq;
  const int diag = nk - nq;
  const size_t head = (size_t)bh * Nq * DK, ohead = (size_t)bh * Nq * DV;
  const size_t khead = (size_t)bh * Nk * DK, vhead = (size_t)bh * Nk * DV;
  const int q_first = qb * BR + 32 * wave;
  const int my_q = q_first + x;

  u32x4 qf[DK / 16], of[DV / 16];
  {
    const uint16_t* qr = Q + head + (size_t)my_q * DK + 8 * h;
    const uint16_t* dr = dO + ohead + (size_t)my_q * DV + 8 * h;
    if constexpr (DK == DV) {
#pragma unroll
      for (int c = 0; c < DK / 16; ++c) {
        qf[c] = my_q < nq ? *(const u32x4*)(qr + 16 * c) : u32x4{0, 0, 0, 0};
        of[c] = my_q < nq ? *(const u32x4*)(dr + 16 * c) : u32x4{0, 0, 0, 0};
      }
    } else {
#pragma unroll
      for (int c = 0; c < DK / 16; ++c)
        qf[c] = my_q < nq ? *(const u32x4*)(qr + 16 * c) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < DV / 16; ++c)
        of[c] = my_q < nq ? *(const u32x4*)(dr + 16 * c) : u32x4{0, 0, 0, 0};
    }
  }
  const float c2 = scale * kLog2e;
  // rows from nq on get no weight (P = 0) and store dQ = 0; rows past Nq are
  // never stored (the block's last rows may lie past the row padding)
  const float nl2 = my_q < nq ? NL[(size_t)bh * n_pad + my_q] * c2 : -INFINITY;
  const float nd = my_q < nq ? ND[(size_t)bh * n_pad + my_q] : 0.f;
  // -delta of the lane's row in every register: the initial accumulator of
  // each dP^T block, so dP - delta comes out of the matrix core
  f32x16 ndb;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndb[r] = nd;
  f32x16 dq[DK / 32];
#pragma unroll
  for (int b = 0; b < DK / 32; ++b) dq[b] = f32x16{};

  const int kv_end = qb * BR >= nq ? 0 : CAUSAL ? min(nk, min((qb + 1) * BR, nq) + diag) : nk;
  const int T = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
  const int last_key = q_first + 31 + diag;  // this wave's last kept key (causal)
  // a wave whose rows all lie past nq only helps load the tiles
  const int my_T = q_first >= nq ? 0 : CAUSAL ? (last_key < 0 ? 0 : min(T, last_key / BC + 1)) : T;
  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  auto load = [&](int j, int buf) {
    const int k0 = j * BC;
    const unsigned base = lds0 + buf * SB;
    const unsigned rows = (unsigned)(nk - k0);
    dma_tile_swz<DK, NW>(buffer_desc(K + khead + (size_t)k0 * DK, rows * DK * 2), base, wave, lane);
    dma_tile<DV, false, NW>(buffer_desc(V + vhead + (size_t)k0 * DV, rows * DV * 2), base + TBK, 0,
                            wave, lane);
  };
  const TrLane trl = tr_lane(lane);
  // A operand of V (chunk-major block layout), as in the forward kernel
  const int v_lane = (x >> 4) * CGV * 1024 + (h * 16 + (x & 15)) * 16;

  const int js = (int)((long long)T * split / n_split), je = (int)((long long)T * (split + 1) / n_split);
  if (js < je) load(js, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  for (int j = js; j < je; ++j) {
    const int buf = (j - js) & 1;
    if (j + 1 < je) load(j + 1, buf ^ 1);
    if (j < my_T) {
      const uint8_t* kt = smem + buf * SB;
      const uint8_t* vt = kt + TBK;
      const int k0 = j * BC;
      // keys past the row (causal) or past the valid keys get no weight: such
      // a key has zero K and V rows, but its weight exp(-lse) need not be finite
      const bool masked = (CAUSAL && k0 + BC - 1 > q_first + diag) || (k0 + BC > nk);
#pragma unroll
      for (int kb2 = 0; kb2 < BC / 32; ++kb2) {
        f32x16 st = f32x16{}, dpt = ndb;
        auto vop = [&](int c) {
          return *(const u32x4*)(vt + v_lane + (2 * kb2 * CGV + (c >> 1)) * 1024 + (c & 1) * 512);
        };
        if constexpr (DK == DV) {
#pragma unroll
          for (int c = 0; c < DK / 16; ++c) {
            st = TT::mma(*(const u32x4*)(kt + rowmajor_a<DK>(32 * kb2 + x, h, c)), qf[c], st);
            dpt = TT::mma(vop(c), of[c], dpt);
          }
        } else {
#pragma unroll
          for (int c = 0; c < DK / 16; ++c)
            st = TT::mma(*(const u32x4*)(kt + rowmajor_a<DK>(32 * kb2 + x, h, c)), qf[c], st);
#pragma unroll
          for (int c = 0; c < DV / 16; ++c) dpt = TT::mma(vop(c), of[c], dpt);
        }
        // masked scores become -inf before the exponentials (P = 0 exactly), in
        // a branch that only the tiles across the diagonal or the end take
        if (masked) {
          const int lim = min(CAUSAL ? my_q + diag : nk - 1, nk - 1) - (k0 + 32 * kb2 + 4 * h);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) > lim) st[r] = -INFINITY;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = fast_exp2(fmaf(st[r], c2, nl2)) * dpt[r];
        u32x4 df[2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const int r0 = 8 * kc;
          df[kc] = u32x4{TT::pack(st[r0 + 0], st[r0 + 1]), TT::pack(st[r0 + 2], st[r0 + 3]),
                         TT::pack(st[r0 + 4], st[r0 + 5]), TT::pack(st[r0 + 6], st[r0 + 7])};
        }
        if constexpr (DK + DV == 128) __builtin_amdgcn_s_setprio(1);  // as in the dK/dV kernel
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
          for (int b = 0; b < DK / 32; ++b)
            dq[b] = TT::mma(tr_read(kt + ((2 * kb2 + kc) * CGK + b) * 1024, trl), df[kc], dq[b]);
      }
    }
    if constexpr (DK + DV == 128) __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }
  if (part) {
    store_rows_f32<DK>(dq, scale, part + (size_t)split * qstride + head, q_first, Nq, lane);
    return;
  }
  uint8_t* stg = smem + wave * 32 * 144;
  store_rows<TT, DK>(dq, scale, stg, dQ + head, q_first, Nq, lane);
}

// ---------------------------------------------------------------------------
// fp32 gradients.  Like the fp32 forward kernel: v_mfma_f32_32x32x2_f32, each
// lane supplying one element per operand, operands read from global memory
// (L2) straight into registers in operand order, no LDS staging.  A
// workgroup has DS waves; wave w owns head-dim columns [w*DSL, (w+1)*DSL),
// and the partial S and dP of the waves are summed through LDS in fixed
// wave order, so every wave sees bitwise the same values.
//   S-type products contract column w*DSL + 8u + 4h + v at step (u, v): lane
//     (x, h) supplies row x's element of it (16-byte loads).
//   The products over 32 rows of the tile (dV^T, dK^T, dQ^T) take step r =
//     accumulator register r (row 8(r/4) + 4h + r%4); their output block b,
//     row i is column w*DSL + NB*i + b (NB = DSL/32), so one lane's NB values
//     of a row are contiguous.

// Row statistics from fp32 O and dO: TPR threads per row (at most a wave).
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_f32(const float* __restrict__ O,
                                                         const float* __restrict__ dO,
                                                         const float* __restrict__ LSE,
                                                         float* __restrict__ NL, float* __restrict__ ND,
                                                         int N, int H, const int* __restrict__ q_len,
                                                         int n_pad, long long padded_rows,
                                                         float inv_scale) {
  constexpr int TPR = D / 4 < 64 ? D / 4 : 64, RPB = 256 / TPR, CH = D / (4 * TPR);
  const int t = threadIdx.x % TPR;
  const long long prow = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  if (prow >= padded_rows) return;  // whole rows only: TPR divides the wave
  const long long bh = prow / n_pad;
  const int i = (int)(prow % n_pad);
  const int nq = q_len ? min(max(q_len[bh / H], 0), N) : N;  // as in the 16-bit kernel
  float acc = 0.f, nl = i < N ? -INFINITY : 0.f;
  if (i < nq) {
    const size_t row = (size_t)bh * N + i;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const f32x4 a = *(const f32x4*)(O + row * D + 4 * (t + TPR * c));
      const f32x4 b = *(const f32x4*)(dO + row * D + 4 * (t + TPR * c));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(a[e], b[e], acc);
    }
    const float l = LSE[row];
    nl = l == -INFINITY ? -INFINITY : -l * inv_scale;
  }
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m, TPR);
  if (t == 0) {
    NL[prow] = nl;
    ND[prow] = -acc;
  }
}

// load NB contiguous floats (zeros when !ok)
template <int NB>
__device__ __forceinline__ void load_nb(const float* p, bool ok, float (&out)[NB]) {
  if (!ok) {
#pragma unroll
    for (int b = 0; b < NB; ++b) out[b] = 0.f;
    return;
  }
  if constexpr (NB == 8) {
    const f32x4 t = *(const f32x4*)p, u = *(const f32x4*)(p + 4);
    out[0] = t[0]; out[1] = t[1]; out[2] = t[2]; out[3] = t[3];
    out[4] = u[0]; out[5] = u[1]; out[6] = u[2]; out[7] = u[3];
  } else if constexpr (NB == 4) {
    const f32x4 t = *(const f32x4*)p;
    out[0] = t[0]; out[1] = t[1]; out[2] = t[2]; out[3] = t[3];
  } else if constexpr (NB == 2) {
    const f32x2 t = *(const f32x2*)p;
    out[0] = t[0]; out[1] = t[1];
  } else {
#pragma unroll
    for (int b = 0; b < NB; ++b) out[b] = p[b];
  }
}

// Sum of the DS waves' partial s and dp (fixed wave order).
template <int DS>
__device__ __forceinline__ void sum_waves(f32x16* red, f32x16& s, f32x16& dp, int wave, int lane) {
  if constexpr (DS > 1) {
    red[wave * 64 + lane] = s;
    red[(DS + wave) * 64 + lane] = dp;
    __syncthreads();
    s = red[lane];
    dp = red[DS * 64 + lane];
#pragma unroll
    for (int w = 1; w < DS; ++w) {
      s += red[w * 64 + lane];
      dp += red[(DS + w) * 64 + lane];
    }
    __syncthreads();
  }
}

// dK, dV of 32 keys per workgroup.  S and dP in (query x key) orientation:
// register r of lane (x, h) is query q0 + 8(r/4) + 4h + r%4, key k0 + x.
// DSL, DSLV: a wave's columns of Q/K and of V/dO (DS waves each).
template <int DSL, int DSLV, int DS, bool CAUSAL>
__global__ __launch_bounds__(DS * 64) void attn_bwd_dkdv_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ NL, const float* __restrict__ ND,
    float* __restrict__ dK, float* __restrict__ dV, int Nq, int Nk, int H,
    const int* __restrict__ k_len, const int* __restrict__ q_len, int n_pad, int n_kblocks, int total, float scale, int n_split,
    float* __restrict__ part, long long kstride, long long vstride) {
  constexpr int D = DSL * DS, DV = DSLV * DS, NB = DSL / 32, NBV = DSLV / 32;
  __shared__ f32x16 red[DS > 1 ? 2 * DS * 64 : 1];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int x = lane & 31, h = lane >> 5;
  const int item = xcd_remap(blockIdx.x, total);
  const int split = item % n_split, work = item / n_split;  // a block's splits are neighbours
  const int bh = work / n_kblocks, kb = work % n_kblocks;
  const int nk = k_len ? min(max(k_len[bh / H], 0), Nk) : Nk;  // as in the 16-bit kernels
  const int nq = q_len ? min(max(q_len[bh / H], 0), Nq) : Nq;
  const int diag = nk - nq;
  const size_t head = (size_t)bh * Nq * D, khead = (size_t)bh * Nk * D;
  const size_t ohead = (size_t)bh * Nq * DV, vhead = (size_t)bh * Nk * DV;
  const int k0 = kb * 32, my_k = k0 + x, col0 = wave * DSL, colv0 = wave * DSLV;

  // The block's K and V rows are held in registers for the whole kernel when
  // a wave's share is 128 columns or fewer; with 256 columns each 16-byte
  // piece is read from L2 where a product uses it, to stay within the wave's
  // 512 registers.
  constexpr bool HOLD = DSL <= 128 && DSLV <= 128;
  constexpr int NF = HOLD ? DSL / 8 : 1, NFV = HOLD ? DSLV / 8 : 1;
  const float* kr = K + khead + (size_t)my_k * D + col0 + 4 * h;
  const float* vr = V + vhead + (size_t)my_k * DV + colv0 + 4 * h;
  f32x4 kf[NF], vf[NFV];
  if (HOLD) {
    if constexpr (DSL == DSLV) {
#pragma unroll
      for (int u = 0; u < NF; ++u) {
        kf[u] = my_k < nk ? *(const f32x4*)(kr + 8 * u) : f32x4{0, 0, 0, 0};
        vf[u] = my_k < nk ? *(const f32x4*)(vr + 8 * u) : f32x4{0, 0, 0, 0};
      }
    } else {
#pragma unroll
      for (int u = 0; u < NF; ++u) kf[u] = my_k < nk ? *(const f32x4*)(kr + 8 * u) : f32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < NFV; ++u) vf[u] = my_k < nk ? *(const f32x4*)(vr + 8 * u) : f32x4{0, 0, 0, 0};
    }
  }
  f32x16 dk[NB], dv[NBV];
  if constexpr (DSL == DSLV) {
#pragma unroll
    for (int b = 0; b < NB; ++b) dk[b] = dv[b] = f32x16{};
  } else {
#pragma unroll
    for (int b = 0; b < NB; ++b) dk[b] = f32x16{};
#pragma unroll
    for (int b = 0; b < NBV; ++b) dv[b] = f32x16{};
  }
  const float c2 = scale * kLog2e;
  const float* nl_row = NL + (size_t)bh * n_pad;
  const float* nd_row = ND + (size_t)bh * n_pad;
  const int nqt = (nq + 31) / 32;
  const int qt_first = k0 >= nk ? nqt : CAUSAL ? max(0, k0 - diag) / 32 : 0;
  // this workgroup's share of the block's query tiles (all of them unsplit)
  const int span = nqt - qt_first;
  const int qt0 = qt_first + (int)((long long)span * split / n_split);
  const int qt1 = qt_first + (int)((long long)span * (split + 1) / n_split);
  const bool edge_k = k0 + 31 >= nk;  // some keys of the block are padding
  const int lim = my_k >= nk ? 0x7fffffff : CAUSAL ? my_k - diag : -0x7fffffff;

  for (int t = qt0; t < qt1; ++t) {
    const int q0 = t * 32;
    f32x16 s = f32x16{}, dp = f32x16{};
    {
      const bool ok = q0 + x < nq;
      const float* qr = Q + head + (size_t)(q0 + x) * D + col0 + 4 * h;
      const float* gr = dO + ohead + (size_t)(q0 + x) * DV + colv0 + 4 * h;
      if constexpr (DSL == DSLV) {
#pragma unroll
        for (int u = 0; u < DSL / 8; ++u) {
          const f32x4 qa = ok ? *(const f32x4*)(qr + 8 * u) : f32x4{0, 0, 0, 0};
          const f32x4 ga = ok ? *(const f32x4*)(gr + 8 * u) : f32x4{0, 0, 0, 0};
          const f32x4 ka = HOLD ? kf[HOLD ? u : 0]
                                : (my_k < nk ? *(const f32x4*)(kr + 8 * u) : f32x4{0, 0, 0, 0});
          const f32x4 va = HOLD ? vf[HOLD ? u : 0]
                                : (my_k < nk ? *(const f32x4*)(vr + 8 * u) : f32x4{0, 0, 0, 0});
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[v], ka[v], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x2f32(ga[v], va[v], dp, 0, 0, 0);
          }
        }
      } else {  // unequal widths: both fit in registers (at most 128 columns)
#pragma unroll
        for (int u = 0; u < DSL / 8; ++u) {
          const f32x4 qa = ok ? *(const f32x4*)(qr + 8 * u) : f32x4{0, 0, 0, 0};
#pragma unroll
          for (int v = 0; v < 4; ++v) s = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[v], kf[u][v], s, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < DSLV / 8; ++u) {
          const f32x4 ga = ok ? *(const f32x4*)(gr + 8 * u) : f32x4{0, 0, 0, 0};
#pragma unroll
          for (int v = 0; v < 4; ++v) dp = __builtin_amdgcn_mfma_f32_32x32x2f32(ga[v], vf[u][v], dp, 0, 0, 0);
        }
      }
    }
    sum_waves<DS>(red, s, dp, wave, lane);
    // P = exp(scale s - lse), dS = P (dP - delta); keys past the valid ones or
    // past a row's causal limit get no weight
    const bool mask = (CAUSAL && q0 + diag < k0 + 31) || edge_k;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 a = *(const f32x4*)(nl_row + q0 + 8 * g + 4 * h);
      const f32x4 b = *(const f32x4*)(nd_row + q0 + 8 * g + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float p = fast_exp2((s[r] + a[e]) * c2);
        if (mask && q0 + 8 * g + 4 * h + e < lim) p = 0.f;
        s[r] = p;
        dp[r] = p * (dp[r] + b[e]);
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS over the tile's 32 rows
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = q0 + 8 * (r >> 2) + 4 * h + (r & 3);
      float gv[NBV], qv[NB];
      load_nb<NBV>(dO + ohead + (size_t)q * DV + colv0 + NBV * x, q < nq, gv);
      load_nb<NB>(Q + head + (size_t)q * D + col0 + NB * x, q < nq, qv);
      if constexpr (DSL == DSLV) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          dv[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(gv[b], s[r], dv[b], 0, 0, 0);
          dk[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(qv[b], dp[r], dk[b], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int b = 0; b < NBV; ++b) dv[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(gv[b], s[r], dv[b], 0, 0, 0);
#pragma unroll
        for (int b = 0; b < NB; ++b) dk[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(qv[b], dp[r], dk[b], 0, 0, 0);
      }
    }
  }
  if (my_k < Nk) {  // every key row, those past the valid keys as zeros
    // split: partial sums to the workspace, the dK parts then the dV parts
    float* kout = part ? part + (size_t)split * kstride : dK;
    float* vout = part ? part + (size_t)n_split * kstride + (size_t)split * vstride : dV;
    float* kr = kout + khead + (size_t)my_k * D + col0;
    float* vr = vout + vhead + (size_t)my_k * DV + colv0;
    if constexpr (DSL == DSLV) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          kr[NB * i + b] = dk[b][r] * scale;
          vr[NB * i + b] = dv[b][r];
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int b = 0; b < NB; ++b) kr[NB * i + b] = dk[b][r] * scale;
#pragma unroll
        for (int b = 0; b < NBV; ++b) vr[NBV * i + b] = dv[b][r];
      }
    }
  }
}

// dQ of 32 query rows per workgroup.  S^T and dP^T: register r of lane (x, h)
// is key k0 + 8(r/4) + 4h + r%4, query q0 + x.
template <int DSL, int DSLV, int DS, bool CAUSAL>
__global__ __launch_bounds__(DS * 64) void attn_bwd_dq_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ NL, const float* __restrict__ ND,
    float* __restrict__ dQ, int Nq, int Nk, int H, const int* __restrict__ k_len, const int* __restrict__ q_len, int n_pad,
    int n_qblocks, int total, float scale, int n_split, float* __restrict__ part,
    long long part_stride) {
  constexpr int D = DSL * DS, DV = DSLV * DS, NB = DSL / 32;
  __shared__ f32x16 red[DS > 1 ? 2 * DS * 64 : 1];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int x = lane & 31, h = lane >> 5;
  const int item = xcd_remap(blockIdx.x, total);
  const int split = item % n_split, work = item / n_split;
  const int bh = work / n_qblocks;
  int qb = work % n_qblocks;
  if (CAUSAL) qb = n_qblocks - 1 - qb;  // longest rows first
  const int nk = k_len ? min(max(k_len[bh / H], 0), Nk) : Nk;
  const int nq = q_len ? min(max(q_len[bh / H], 0), Nq) : Nq;
  const int diag = nk - nq;
  const size_t head = (size_t)bh * Nq * D, khead = (size_t)bh * Nk * D;
  const size_t ohead = (size_t)bh * Nq * DV, vhead = (size_t)bh * Nk * DV;
  const int q0 = qb * 32, my_q = q0 + x, col0 = wave * DSL, colv0 = wave * DSLV;

  // Q and dO rows in registers, or read where used with 256 columns per wave
  // (as K and V in the dK/dV kernel)
  constexpr bool HOLD = DSL <= 128 && DSLV <= 128;
  constexpr int NF = HOLD ? DSL / 8 : 1, NFV = HOLD ? DSLV / 8 : 1;
  const float* qrow = Q + head + (size_t)my_q * D + col0 + 4 * h;
  const float* grow = dO + ohead + (size_t)my_q * DV + colv0 + 4 * h;
  f32x4 qf[NF], gf[NFV];
  if (HOLD) {
    if constexpr (DSL == DSLV) {
#pragma unroll
      for (int u = 0; u < NF; ++u) {
        qf[u] = my_q < nq ? *(const f32x4*)(qrow + 8 * u) : f32x4{0, 0, 0, 0};
        gf[u] = my_q < nq ? *(const f32x4*)(grow + 8 * u) : f32x4{0, 0, 0, 0};
      }
    } else {
#pragma unroll
      for (int u = 0; u < NF; ++u) qf[u] = my_q < nq ? *(const f32x4*)(qrow + 8 * u) : f32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < NFV; ++u) gf[u] = my_q < nq ? *(const f32x4*)(grow + 8 * u) : f32x4{0, 0, 0, 0};
    }
  }
  const float c2 = scale * kLog2e;
  // padding rows (from nq on) get no weight and store dQ = 0
  const float nl2 = my_q < nq ? NL[(size_t)bh * n_pad + my_q] * c2 : -INFINITY;
  const float nd = my_q < nq ? ND[(size_t)bh * n_pad + my_q] : 0.f;
  f32x16 dq[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) dq[b] = f32x16{};
  const int kv_end = q0 >= nq ? 0 : CAUSAL ? min(nk, min(q0 + 32, nq) + diag) : nk;
  const int T = kv_end > 0 ? (kv_end + 31) / 32 : 0;
  const int j0 = (int)((long long)T * split / n_split), j1 = (int)((long long)T * (split + 1) / n_split);
  const int lim = min(CAUSAL ? my_q + diag : nk - 1, nk - 1);

  for (int j = j0; j < j1; ++j) {
    const int k0 = j * 32;
    f32x16 st = f32x16{}, dpt = f32x16{};
    {
      const bool ok = k0 + x < nk;
      const float* kr = K + khead + (size_t)(k0 + x) * D + col0 + 4 * h;
      const float* vr = V + vhead + (size_t)(k0 + x) * DV + colv0 + 4 * h;
      if constexpr (DSL == DSLV) {
#pragma unroll
        for (int u = 0; u < DSL / 8; ++u) {
          const f32x4 ka = ok ? *(const f32x4*)(kr + 8 * u) : f32x4{0, 0, 0, 0};
          const f32x4 va = ok ? *(const f32x4*)(vr + 8 * u) : f32x4{0, 0, 0, 0};
          const f32x4 qa = HOLD ? qf[HOLD ? u : 0]
                                : (my_q < nq ? *(const f32x4*)(qrow + 8 * u) : f32x4{0, 0, 0, 0});
          const f32x4 ga = HOLD ? gf[HOLD ? u : 0]
                                : (my_q < nq ? *(const f32x4*)(grow + 8 * u) : f32x4{0, 0, 0, 0});
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            st = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[v], qa[v], st, 0, 0, 0);
            dpt = __builtin_amdgcn_mfma_f32_32x32x2f32(va[v], ga[v], dpt, 0, 0, 0);
          }
        }
      } else {  // unequal widths: both fit in registers (at most 128 columns)
#pragma unroll
        for (int u = 0; u < DSL / 8; ++u) {
          const f32x4 ka = ok ? *(const f32x4*)(kr + 8 * u) : f32x4{0, 0, 0, 0};
#pragma unroll
          for (int v = 0; v < 4; ++v) st = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[v], qf[u][v], st, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < DSLV / 8; ++u) {
          const f32x4 va = ok ? *(const f32x4*)(vr + 8 * u) : f32x4{0, 0, 0, 0};
#pragma unroll
          for (int v = 0; v < 4; ++v) dpt = __builtin_amdgcn_mfma_f32_32x32x2f32(va[v], gf[u][v], dpt, 0, 0, 0);
        }
      }
    }
    sum_waves<DS>(red, st, dpt, wave, lane);
    const bool masked = (CAUSAL && k0 + 31 > q0 + diag) || (k0 + 32 > nk);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = fast_exp2(fmaf(st[r], c2, nl2));
      if (masked && k0 + 8 * (r >> 2) + 4 * h + (r & 3) > lim) p = 0.f;
      st[r] = p * (dpt[r] + nd);
    }
    // dQ^T += K^T dS^T over the tile's 32 keys
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
      float kv[NB];
      load_nb<NB>(K + khead + (size_t)key * D + col0 + NB * x, key < nk, kv);
#pragma unroll
      for (int b = 0; b < NB; ++b) dq[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[b], st[r], dq[b], 0, 0, 0);
    }
  }
  if (my_q < Nq) {
    float* qout = part ? part + (size_t)split * part_stride : dQ;  // split: a partial sum
    float* qr = qout + head + (size_t)my_q * D + col0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
      for (int b = 0; b < NB; ++b) qr[NB * i + b] = dq[b][r] * scale;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
size_t padded_rows(long long BH, int N) { return (size_t)BH * (size_t)((N + kRowPad - 1) / kRowPad * kRowPad); }

// out = sum of n_split partial tensors of n floats each (stride apart), added
// in split order so the result does not depend on timing.
__global__ __launch_bounds__(256) void attn_bwd_sum_f32(const float* __restrict__ part,
                                                        float* __restrict__ out, long long n,
                                                        long long stride, int n_split) {
  const long long n4 = n / 4;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4;
       i += (long long)gridDim.x * 256) {
    f32x4 acc = ((const f32x4*)part)[i];
    for (int sp = 1; sp < n_split; ++sp) acc += ((const f32x4*)(part + sp * stride))[i];
    ((f32x4*)out)[i] = acc;
  }
}

// The same for 16-bit outputs: the fp32 partial sums added in split order,
// then rounded once to the element type (8 elements per thread).
template <class TT>
__global__ __launch_bounds__(256) void attn_bwd_sum_sp(const float* __restrict__ part,
                                                       uint16_t* __restrict__ out, long long n,
                                                       long long stride, int n_split) {
  const long long n8 = n / 8;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n8;
       i += (long long)gridDim.x * 256) {
    f32x4 a = ((const f32x4*)part)[2 * i], b = ((const f32x4*)part)[2 * i + 1];
    for (int sp = 1; sp < n_split; ++sp) {
      a += ((const f32x4*)(part + sp * stride))[2 * i];
      b += ((const f32x4*)(part + sp * stride))[2 * i + 1];
    }
    ((u32x4*)out)[i] = u32x4{TT::pack(a[0], a[1]), TT::pack(a[2], a[3]), TT::pack(b[0], b[1]),
                             TT::pack(b[2], b[3])};
  }
}

// Problems with fewer key (query) blocks than the GPU holds at once split
// each block's query (key) tiles over `kv` (`q`) workgroups; their partial dK
// and dV (dQ) go to the workspace after the row statistics, in fp32, and are
// summed by attn_bwd_sum_f32 / attn_bwd_sum_sp.  Each split keeps at least
// two tiles.
struct BwdSplit {
  int kv = 1, q = 1;
  size_t bytes = 0;  // partial sums
};

// Waves per workgroup of the 16-bit dQ kernel (32 query rows each): eight
// above d = 64, where one workgroup fills a CU's two waves per SIMD and each
// K/V tile in LDS serves 256 rows; four at d = 64, whose three waves per SIMD
// (12 per CU) take three four-wave workgroups.  Measured on d = 128 gradients
// against four waves: 1.5-4.5% faster, bitwise equal (the dK/dV kernel with
// eight waves was 1.8% slower on causal shapes: more of its waves idle at the
// diagonal; eight-wave dQ at d = 64, two waves per SIMD instead of three, was
// 2.5-9.5% slower).
constexpr int bwd_dq_waves(int dk, int dv) { return dk + dv == 128 ? 4 : 8; }

// dk, dv: head dims of Q/K and of V/dO
BwdSplit plan_bwd_split(long long BH, int Nq, int Nk, int dk, int dv, int dtype) {
  BwdSplit p;
  int cus = 0;
  if (compute_units(&cus) != hipSuccess) return p;
  // at least two tiles per share for the 16-bit kernels; one for fp32, whose
  // small grids are latency-bound (one head of 256 rows at d = 128:
  // 64.5 -> 48.4 us against two-tile shares)
  auto pick = [&](long long blocks, long long tiles, long long slots) {
    if (blocks >= slots) return 1;
    const long long per = dtype == FA_DTYPE_FP32 ? tiles : tiles / 2;
    const long long sp = std::min<long long>((slots + blocks - 1) / blocks, per);
    return sp < 2 ? 1 : (int)sp;
  };
  if (dtype == FA_DTYPE_FP32) {  // 32-row blocks of keys and of queries, one workgroup per CU
    const long long nkb = (Nk + 31) / 32, nqb = (Nq + 31) / 32;
    p.kv = pick(nkb * BH, nqb, cus);
    p.q = pick(nqb * BH, nkb, cus);
  } else if (dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_FP16) {
    // 32-row blocks per wave; a CU holds 8 waves (12 at d = 64); the dK/dV
    // kernel streams 32-row query tiles, the dQ kernel 64-key tiles
    const long long waves = (long long)cus * (dk + dv == 128 ? 12 : 8);
    const int qw = bwd_dq_waves(dk, dv);
    p.kv = pick((Nk + 127) / 128 * BH, (Nq + 31) / 32, waves / 4);
    p.q = pick((Nq + 32 * qw - 1) / (32 * qw) * BH, (Nk + 63) / 64, waves / qw);
  } else {
    return p;
  }
  if (p.kv > 1) p.bytes += (size_t)p.kv * BH * Nk * (size_t)(dk + dv) * sizeof(float);
  if (p.q > 1) p.bytes += (size_t)p.q * BH * Nq * (size_t)dk * sizeof(float);
  return p;
}

template <class TT, int DK, int DV>
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int BH, int H, int Nq, int Nk,
                      const int* k_len, const int* q_len, float scale, bool causal, float* ws,
                      const BwdSplit& sp,
                      hipStream_t st) {
  const int n_pad = (Nq + kRowPad - 1) / kRowPad * kRowPad;
  const long long prow = (long long)BH * n_pad;
  float* nl = ws;
  float* nd = ws + prow;
  {
    constexpr int RPB = 256 / (DV / 8);  // delta = <dO, O> over the value dim
    hipLaunchKernelGGL((attn_bwd_prep<TT, DV>), dim3((unsigned)((prow + RPB - 1) / RPB)), dim3(256), 0,
                       st, (const uint16_t*)o, (const uint16_t*)dout, lse, nl, nd, Nq, H, q_len, n_pad, prow,
                       1.f / scale);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  // 4 waves (128 keys, 128 query rows) per workgroup; 8 were measured slower
  // on every workload shape, though they halve the re-streamed tiles
  constexpr int NWK = 4, NWQ = bwd_dq_waves(DK, DV);
  const int nkb = (Nk + 32 * NWK - 1) / (32 * NWK), nqb = (Nq + 32 * NWQ - 1) / (32 * NWQ);
  const int tk = nkb * BH * sp.kv, tq = nqb * BH * sp.q;
  const long long kstride = (long long)BH * Nk * DK, vstride = (long long)BH * Nk * DV;
  const long long qstride = (long long)BH * Nq * DK;
  float* kvpart = sp.kv > 1 ? ws + 2 * prow : nullptr;
  float* qpart = sp.q > 1 ? ws + 2 * prow + (sp.kv > 1 ? sp.kv * (kstride + vstride) : 0) : nullptr;
  const dim3 bk(64 * NWK), bq(64 * NWQ);
  if (causal) {
    hipLaunchKernelGGL((attn_bwd_dkdv<TT, DK, DV, true, NWK>), dim3(tk), bk, 0, st, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, nl, nd,
                       (uint16_t*)dk, (uint16_t*)dv, Nq, Nk, H, k_len, q_len, n_pad, nkb, tk, scale,
                       sp.kv, kvpart, kstride, vstride);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_bwd_dq<TT, DK, DV, true, NWQ>), dim3(tq), bq, 0, st, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, nl, nd,
                       (uint16_t*)dq, Nq, Nk, H, k_len, q_len, n_pad, nqb, tq, scale, sp.q, qpart,
                       qstride);
  } else {
    hipLaunchKernelGGL((attn_bwd_dkdv<TT, DK, DV, false, NWK>), dim3(tk), bk, 0, st, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, nl, nd,
                       (uint16_t*)dk, (uint16_t*)dv, Nq, Nk, H, k_len, q_len, n_pad, nkb, tk, scale,
                       sp.kv, kvpart, kstride, vstride);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_bwd_dq<TT, DK, DV, false, NWQ>), dim3(tq), bq, 0, st, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, nl, nd,
                       (uint16_t*)dq, Nq, Nk, H, k_len, q_len, n_pad, nqb, tq, scale, sp.q, qpart,
                       qstride);
  }
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  auto sum = [&](const float* part, void* out, long long n, int n_split) {
    const long long blocks = std::min<long long>((n / 8 + 255) / 256, 8192);
    hipLaunchKernelGGL((attn_bwd_sum_sp<TT>), dim3((unsigned)blocks), dim3(256), 0, st, part,
                       (uint16_t*)out, n, n, n_split);
    return hipGetLastError();
  };
  if (sp.kv > 1) {
    if (hipError_t e = sum(kvpart, dk, kstride, sp.kv); e != hipSuccess) return e;
    if (hipError_t e = sum(kvpart + sp.kv * kstride, dv, vstride, sp.kv); e != hipSuccess) return e;
  }
  if (sp.q > 1)
    if (hipError_t e = sum(qpart, dq, qstride, sp.q); e != hipSuccess) return e;
  return hipSuccess;
}

// DSL, DSLV, DS: the dK/dV kernel's columns per wave and waves; QDS: the dQ
// kernel's waves, over the same head dims; KDS2: waves of a second dK/dV
// arrangement for grids too small to fill the GPU at DS waves.
// At d = 128 the dQ kernel runs two waves of 64 columns (216 registers, two
// waves per SIMD, against 280 and one for a single wave of 128), and the
// dK/dV kernel one wave of 128 columns, or two of 64 when its grid holds
// fewer than 4 workgroups per compute unit (8 with the causal mask, which
// halves the work): both arrangements run one wave per SIMD (384 and 288
// registers), so two waves per workgroup double the waves at work on a small
// grid and shorten its longest block, at the price of the LDS exchange of
// partial S and dP, which a full grid does not recover.  Measured on fp32
// d = 128 gradients: 7-31% faster below those grid sizes, 12-17% slower
// above them.
template <int DSL, int DSLV, int DS, int QDS = DS, int KDS2 = DS>
hipError_t launch_bwd_f32(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv, int BH,
                          int H, int Nq, int Nk, const int* k_len, const int* q_len, float scale,
                          bool causal, float* ws, const BwdSplit& sp, hipStream_t st) {
  constexpr int D = DSL * DS, DV = DSLV * DS;
  static_assert(D % QDS == 0 && DV % QDS == 0 && D % KDS2 == 0 && DV % KDS2 == 0, "whole column shares");
  const int n_pad = (Nq + kRowPad - 1) / kRowPad * kRowPad;
  const long long prow = (long long)BH * n_pad;
  float* nl = ws;
  float* nd = ws + prow;
  {
    constexpr int TPR = DV / 4 < 64 ? DV / 4 : 64, RPB = 256 / TPR;  // delta over the value dim
    hipLaunchKernelGGL((attn_bwd_prep_f32<DV>), dim3((unsigned)((prow + RPB - 1) / RPB)), dim3(256),
                       0, st, (const float*)o, (const float*)dout, lse, nl, nd, Nq, H, q_len, n_pad, prow,
                       1.f / scale);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  const int nkb = (Nk + 31) / 32, nqb = (Nq + 31) / 32;
  const int tk = nkb * BH * sp.kv, tq = nqb * BH * sp.q;
  const long long kstride = (long long)BH * Nk * D, vstride = (long long)BH * Nk * DV;
  const long long qstride = (long long)BH * Nq * D;
  float* kvpart = sp.kv > 1 ? ws + 2 * prow : nullptr;
  float* qpart = sp.q > 1 ? ws + 2 * prow + (sp.kv > 1 ? sp.kv * (kstride + vstride) : 0) : nullptr;
  bool kv_wide = false;  // the dK/dV kernel with KDS2 waves
  if constexpr (KDS2 != DS) {
    int cus = 0;
    if (hipError_t e = compute_units(&cus); e != hipSuccess) return e;
    kv_wide = (long long)tk * (causal ? 1 : 2) < 8LL * cus;
  }
  auto dkdv = [&](auto kernel, int waves) {
    hipLaunchKernelGGL(kernel, dim3(tk), dim3(64 * waves), 0, st, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)dout, nl, nd, (float*)dk, (float*)dv, Nq, Nk, H, k_len,
                       q_len, n_pad, nkb, tk, scale, sp.kv, kvpart, kstride, vstride);
  };
  auto dqk = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(tq), dim3(64 * QDS), 0, st, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)dout, nl, nd, (float*)dq, Nq, Nk, H, k_len, q_len,
                       n_pad, nqb, tq, scale, sp.q, qpart, qstride);
  };
  if (causal) {
    if (kv_wide) dkdv(attn_bwd_dkdv_f32<D / KDS2, DV / KDS2, KDS2, true>, KDS2);
    else dkdv(attn_bwd_dkdv_f32<DSL, DSLV, DS, true>, DS);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    dqk(attn_bwd_dq_f32<D / QDS, DV / QDS, QDS, true>);
  } else {
    if (kv_wide) dkdv(attn_bwd_dkdv_f32<D / KDS2, DV / KDS2, KDS2, false>, KDS2);
    else dkdv(attn_bwd_dkdv_f32<DSL, DSLV, DS, false>, DS);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    dqk(attn_bwd_dq_f32<D / QDS, DV / QDS, QDS, false>);
  }
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  auto sum = [&](const float* part, void* out, long long n, int n_split) {
    const long long blocks = std::min<long long>((n / 4 + 255) / 256, 8192);
    hipLaunchKernelGGL(attn_bwd_sum_f32, dim3((unsigned)blocks), dim3(256), 0, st, part,
                       (float*)out, n, n, n_split);
    return hipGetLastError();
  };
  if (sp.kv > 1) {
    if (hipError_t e = sum(kvpart, dk, kstride, sp.kv); e != hipSuccess) return e;
    if (hipError_t e = sum(kvpart + sp.kv * kstride, dv, vstride, sp.kv); e != hipSuccess) return e;
  }
  if (sp.q > 1)
    if (hipError_t e = sum(qpart, dq, qstride, sp.q); e != hipSuccess) return e;
  return hipSuccess;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

namespace {

template <class TT>
hipError_t launch_bwd_dims(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           int bh, int H, int Nq, int Nk, const int* k_len, const int* q_len,
                           float scale,
                           bool causal, int d_qk, int d_v, float* ws, const BwdSplit& sp,
                           hipStream_t st) {
  if (d_qk == 64)
    return d_v == 64 ? launch_bwd<TT, 64, 64>(q, k, v, o, dout, lse, dq, dk, dv, bh, H, Nq, Nk, k_len, q_len, scale, causal, ws, sp, st)
                     : launch_bwd<TT, 64, 128>(q, k, v, o, dout, lse, dq, dk, dv, bh, H, Nq, Nk, k_len, q_len, scale, causal, ws, sp, st);
  return d_v == 64 ? launch_bwd<TT, 128, 64>(q, k, v, o, dout, lse, dq, dk, dv, bh, H, Nq, Nk, k_len, q_len, scale, causal, ws, sp, st)
                   : launch_bwd<TT, 128, 128>(q, k, v, o, dout, lse, dq, dk, dv, bh, H, Nq, Nk, k_len, q_len, scale, causal, ws, sp, st);
}

}  // namespace

extern "C" {

int fa_bwd_supported(int d, int dtype, int causal) {
  if (causal != 0 && causal != 1) return 0;
  if (dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_FP16) return d == 64 || d == 128;
  if (dtype == FA_DTYPE_FP32) return d == 64 || d == 128 || d == 256 || d == 512 || d == 1024;
  return 0;
}

int fa_bwd_gen_supported(int d_qk, int d_v, int dtype, int causal) {
  if (d_qk == d_v) return fa_bwd_supported(d_qk, dtype, causal);
  if (causal != 0 && causal != 1) return 0;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_FP32) return 0;
  return (d_qk == 64 || d_qk == 128) && (d_v == 64 || d_v == 128);
}

size_t fa_bwd_gen_workspace_size(int B, int H, int Nq, int Nk, int d_qk, int d_v, int causal,
                                 int dtype) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || !fa_bwd_gen_supported(d_qk, d_v, dtype, causal))
    return 0;
  const long long BH = (long long)B * H;
  if (BH > (1LL << 24) || BH * Nq > 0x7fffffffLL || BH * Nk > 0x7fffffffLL) return 0;
  return 2 * padded_rows(BH, Nq) * sizeof(float) +
         plan_bwd_split(BH, Nq, Nk, d_qk, d_v, dtype).bytes;
}

size_t fa_bwd_ex_workspace_size(int B, int H, int Nq, int Nk, int d, int causal, int dtype) {
  return fa_bwd_gen_workspace_size(B, H, Nq, Nk, d, d, causal, dtype);
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d, int causal, int dtype) {
  return fa_bwd_ex_workspace_size(B, H, N, N, d, causal, dtype);
}

int fa_bwd_gen(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
               int d_qk, int d_v, float scale, int causal, int dtype, const int* k_len,
               const int* q_len, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d_qk <= 0 || d_v <= 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  const long long BH = (long long)B * H;
  if (BH > (1LL << 24) || BH * Nq > 0x7fffffffLL || BH * Nk > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  if ((((long long)Nq + 127) / 128 + ((long long)Nk + 127) / 128) * BH > 0x7fffffffLL)
    return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16)
    return FA_ERR_UNSUPPORTED;
  if (!fa_bwd_gen_supported(d_qk, d_v, dtype, causal)) return FA_ERR_UNSUPPORTED;
  // per-head byte offsets (plus one tile of slack) fit the 32-bit buffer offsets
  const long long elem = dtype == FA_DTYPE_FP32 ? 4 : 2;
  const long long dmax = d_qk > d_v ? d_qk : d_v;
  if (((long long)(Nq > Nk ? Nq : Nk) + 128) * dmax * elem > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  if (!workspace ||
      workspace_bytes < fa_bwd_gen_workspace_size(B, H, Nq, Nk, d_qk, d_v, causal, dtype))
    return FA_ERR_INVALID_ARG;
  for (const void* p : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv,
                        (const void*)workspace})
    if (!aligned16(p)) return FA_ERR_UNSUPPORTED;
  if (((uintptr_t)k_len & 3u) != 0 || ((uintptr_t)q_len & 3u) != 0) return FA_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  const int bh = (int)BH;
  float* ws = (float*)workspace;
  const BwdSplit sp = plan_bwd_split(BH, Nq, Nk, d_qk, d_v, dtype);
  hipError_t e;
  if (dtype == FA_DTYPE_BF16) {
    e = launch_bwd_dims<Bf16>(q, k, v, o, dout, lse, dq, dk, dv, bh, H, Nq, Nk, k_len, q_len, scale, causal, d_qk, d_v, ws, sp, st);
  } else if (dtype == FA_DTYPE_FP16) {
    e = launch_bwd_dims<F16>(q, k, v, o, dout, lse, dq, dk, dv, bh, H, Nq, Nk, k_len, q_len, scale, causal, d_qk, d_v, ws, sp, st);
  } else if (d_qk != d_v) {
    e = d_qk == 64 ? launch_bwd_f32<64, 128, 1>(q, k, v, o, dout, lse, dq, dk, dv, bh, H, Nq, Nk, k_len, q_len, scale, causal, ws, sp, st)
                   : launch_bwd_f32<128, 64, 1>(q, k, v, o, dout, lse, dq, dk, dv, bh, H, Nq, Nk, k_len, q_len, scale, causal, ws, sp, st);
  } else {
    switch (d_qk) {
      case 64: e = launch_bwd_f32<64, 64, 1>(q, k, v, o, dout, lse, dq, dk, dv, bh, H, Nq, Nk, k_len, q_len, scale, causal, ws, sp, st); break;
      case 128: e = launch_bwd_f32<128, 128, 1, 2, 2>(q, k, v, o, dout, lse, dq, dk, dv, bh, H, Nq, Nk, k_len, q_len, scale, causal, ws, sp, st); break;
      case 256: e = launch_bwd_f32<128, 128, 2>(q, k, v, o, dout, lse, dq, dk, dv, bh, H, Nq, Nk, k_len, q_len, scale, causal, ws, sp, st); break;
      case 512: e = launch_bwd_f32<128, 128, 4>(q, k, v, o, dout, lse, dq, dk, dv, bh, H, Nq, Nk, k_len, q_len, scale, causal, ws, sp, st); break;
      default: e = launch_bwd_f32<256, 256, 4>(q, k, v, o, dout, lse, dq, dk, dv, bh, H, Nq, Nk, k_len, q_len, scale, causal, ws, sp, st); break;
    }
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d,
              float scale, int causal, int dtype, const int* k_len, void* workspace,
              size_t workspace_bytes, void* stream) {
  return fa_bwd_gen(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, d, d, scale, causal, dtype,
                    k_len, nullptr, workspace, workspace_bytes, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
           float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
           void* stream) {
  return fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, N, d, scale, causal, dtype, nullptr,
                   workspace, workspace_bytes, stream);
}

}  // extern "C"
