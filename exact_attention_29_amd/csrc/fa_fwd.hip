// fa_fwd.hip -- FlashAttention forward for MI355X (gfx950, CDNA4), C ABI in include/fa.h.
//
// What is computed: O = softmax(scale * Q K^T) V per (batch, head), plus the
// per-row log-sum-exp, one key/value tile at a time with the online-softmax
// recurrence -- running row max m, running denominator l, and an unnormalized
// accumulator rescaled by exp(m_old - m_new) when a tile raises the max, then
// one divide by l at the end ("Deep Learning - Flash Attention", section "An
// Example", steps 4-6; "The Details of Flash Attention", sections "Online
// Softmax" and "Tiling the Loop").  One workgroup owns a block of query rows
// and streams every key/value tile through it (the query-block worker of "An
// Example", step 7).  The N x N score matrix never leaves registers.
//
// Kernels:
//  * attn_fwd_sp<T>: bf16 / fp16 inputs, head dims 64 or 128 (Q/K and V/O
//    each).  4 (d = 64) or 8 (d = 128) waves x 32 query rows per workgroup,
//    persistent at d = 128; K and V tiles of 64
//    keys double-buffered in LDS and filled by buffer loads that write
//    straight to LDS; both products on v_mfma_f32_32x32x16_{bf16,f16} with
//    fp32 accumulators.  The score tile is computed transposed (S^T = K Q^T)
//    so that each lane owns one query column: the row max and row sum are
//    in-lane plus one swap between the two 32-lane halves, and the
//    probabilities are already in the B-operand layout of the P V product
//    (O^T = V^T P^T).  V is read out of its row-major LDS blocks with
//    ds_read_b64_tr_b16, which hands each lane four keys of one head-dim
//    column.  Each wave software-pipelines the score product of the next
//    tile against the softmax of the current one.
//  * attn_fwd_f32: fp32 inputs, head dim 64..1024, on v_mfma_f32_32x32x2_f32.
//    Head dims above 128 are split across the waves of a workgroup (64
//    columns each, 128 at d = 1024; at d = 128 on the small grids that take
//    the key split); the partial scores are summed through LDS in a fixed
//    wave order, so every wave sees bitwise the same scores and softmax.
//    Q stays in registers; each wave's slice of the next K tile is loaded
//    straight into LDS while the current tile's products run.
//  * attn_combine_sp / attn_combine_f32: grids too small to fill the GPU
//    split each query block's keys over several workgroups; these merge the
//    partial results of the key ranges in a fixed order.
//
// Exponentials are exp2 of scores pre-multiplied by scale*log2(e) (v_exp_f32);
// the log-sum-exp is converted back to natural-log units at the end.
//
// Built with FA_SYNC_PHASES defined (a separate check library, never the
// product), the 16-bit kernel waits for every tile load and meets the whole
// workgroup at a barrier before each tile's LDS reads and around each
// epilogue staging phase, and the fp32 kernel waits for all of a tile's
// loads (K and V) before its score products: the same arithmetic with no
// overlap of loads, reads and writes, which must give bitwise the same
// results.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>

#include "fa.h"
#include "fa_device.h"

namespace {

using namespace fa_dev;

// Dynamic work distribution for the persistent bf16 / fp16 kernel.  The
// items of a launch (a head and a block of query rows each) are split into 8
// contiguous ranges, one per XCD, in the order xcd_remap gives: the query
// blocks of one head go to one XCD's L2, longest first.  A workgroup takes
// the next unclaimed item of its own XCD's range with an atomic counter, and
// once that range is exhausted takes items from the other ranges, so no XCD
// idles while another still has work.
//
// The counters live in one of kWorkSlots slots in the code object, chosen
// round-robin by the host.  A slot belongs to one launch at a time: the
// launch's tag (a hash of its dispatch packet's address and its dispatch id,
// which together differ between any two launches in flight) is stored in
// the slot's state word beside a count of the workgroups using it.  A
// workgroup that finds the slot free or owned by its own launch joins it and
// claims items from its counters; the last one to leave clears the counters,
// records the tag as finished and frees the slot.  A workgroup that finds
// the slot owned by another launch (a captured launch replayed beside a
// later call that drew the same slot, or more than kWorkSlots launches in
// flight) does not touch the counters: it runs the items of its own id,
// blockIdx.x, blockIdx.x + gridDim.x, ..., so that its launch's items are
// all computed whether or not any of its workgroups got the slot (an item
// computed twice is written twice with the same bits).  A workgroup that
// arrives after its launch has already finished every item exits.
constexpr int kWorkSlots = 64;
struct WorkSlot {
  unsigned long long state;     // tag << 16 | workgroups using the slot; 0 when free
  unsigned long long done_tag;  // tag of the last launch that finished in this slot
  unsigned next_rank[8];        // per XCD: next item rank to hand out
};
__device__ WorkSlot g_slots[kWorkSlots];

enum { kJoinDynamic = 0, kJoinStatic = 1, kJoinDone = 2 };

// dispatch id of the running launch: the index of its packet in its queue
extern "C" __device__ unsigned long long fa_llvm_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

// 48-bit, non-zero tag of this launch (splitmix64 finaliser over the packet
// address and the dispatch id)
__device__ __forceinline__ unsigned long long launch_tag() {
  const unsigned long long p = (unsigned long long)(uintptr_t)__builtin_amdgcn_dispatch_ptr();
  unsigned long long h = (p >> 6) * 0x9E3779B97F4A7C15ull ^ (fa_llvm_dispatch_id() + 0x632BE59BD9B4E019ull);
  h ^= h >> 30;
  h *= 0xBF58476D1CE4E5B9ull;
  h ^= h >> 27;
  h *= 0x94D049BB133111EBull;
  h ^= h >> 31;
  h &= 0xFFFFFFFFFFFFull;
  return h ? h : 1;
}

__device__ __forceinline__ int xcd_id() {
  // hardware register XCC_ID (id 20), bits [3:0]
  return (int)(__builtin_amdgcn_s_getreg((15 << 11) | 20) & 7u);
}

// Called once per workgroup by one thread, before its first claim.  Only
// the first workgroup of a launch exchanges the free state for its own
// (compare-and-swap); the others add themselves with one fetch-add, so the
// start of a launch costs each workgroup a few atomics, not a contended loop.
__device__ __forceinline__ int join_launch(int slot, unsigned long long tag) {
  WorkSlot& w = g_slots[slot];
  unsigned long long st = __hip_atomic_load(&w.state, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
  for (int tries = 0; tries < 64; ++tries) {  // the bound only guarantees an end: static is always correct
    if (st == 0) {
      if (__hip_atomic_load(&w.done_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag) return kJoinDone;
      if (__hip_atomic_compare_exchange_strong(&w.state, &st, (tag << 16) | 1ull, __ATOMIC_ACQ_REL,
                                               __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT))
        return kJoinDynamic;
      continue;  // st now holds the state another workgroup installed
    }
    if ((st >> 16) != tag)
      return __hip_atomic_load(&w.done_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag ? kJoinDone
                                                                                               : kJoinStatic;
    const unsigned long long old =
        __hip_atomic_fetch_add(&w.state, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if ((old >> 16) == tag) return kJoinDynamic;
    // The slot changed between the load and the add (this launch had
    // finished and freed it, and it may have a new owner): take the count
    // back.  If that leaves a new owner with no workgroup, its workgroups
    // have all left (one of them saw this one's count and did not free the
    // slot), so free it on their behalf.
    const unsigned long long prev =
        __hip_atomic_fetch_sub(&w.state, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if ((prev & 0xFFFFull) == 1ull && (prev >> 16) != 0) {
      unsigned long long dead = prev - 1;
      __hip_atomic_store(&w.done_tag, prev >> 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int y = 0; y < 8; ++y)
        __hip_atomic_store(&w.next_rank[y], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_compare_exchange_strong(&w.state, &dead, 0ull, __ATOMIC_ACQ_REL, __ATOMIC_ACQUIRE,
                                           __HIP_MEMORY_SCOPE_AGENT);
    }
    st = __hip_atomic_load(&w.state, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
  }
  return kJoinStatic;
}

__device__ __forceinline__ int take_item(int slot, int xcd, int total) {
  for (int i = 0; i < 8; ++i) {
    const int y = (xcd + i) & 7;
    const unsigned lo = (unsigned)((long long)y * total / 8);
    const unsigned n = (unsigned)((long long)(y + 1) * total / 8) - lo;
    unsigned* ctr = &g_slots[slot].next_rank[y];
    if (n == 0) continue;
    const unsigned t = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t < n) return (int)(lo + t);
  }
  return -1;
}

// The next item of a workgroup: from the slot's counters (joined), or the
// next of its own stride (static).
__device__ __forceinline__ int next_item(int mode, int slot, int xcd, int total, int cur) {
  if (mode == kJoinDynamic) return take_item(slot, xcd, total);
  const long long n = (long long)cur + gridDim.x;
  return n < total ? (int)n : -1;
}

// Called once per joined workgroup by one thread, after its last claim (the
// counters are exhausted, so every item of the launch has been claimed).  The
// workgroup that takes the count to zero clears the counters, records the
// launch as finished and frees the slot; should a late workgroup of the same
// launch join in between, the exchange fails and that workgroup frees it
// when it leaves (it finds the counters cleared and computes items again,
// with the same results).
__device__ __forceinline__ void leave_launch(int slot, unsigned long long tag) {
  WorkSlot& w = g_slots[slot];
  __threadfence();
  const unsigned long long old =
      __hip_atomic_fetch_sub(&w.state, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  if ((old & 0xFFFFull) != 1ull) return;
  unsigned long long mine = old - 1;  // this launch's tag with no workgroup left
  __hip_atomic_store(&w.done_tag, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int y = 0; y < 8; ++y)
    __hip_atomic_store(&w.next_rank[y], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_compare_exchange_strong(&w.state, &mine, 0ull, __ATOMIC_ACQ_REL, __ATOMIC_ACQUIRE,
                                       __HIP_MEMORY_SCOPE_AGENT);
}

// At d = 64 the steady step takes its exponentials against the row's
// reference without the tile's row max; a lane whose weights of the tile sum
// past this bound (or not to a finite value) sends the tile to the exact path.
// Below it every weight is at most 2^15: finite in fp32, bf16 and fp16.
constexpr float kSumLimit = 32768.0f;

// ---------------------------------------------------------------------------
// bf16 / fp16 kernel, software-pipelined
//
// A wave issues in order, so its matrix-core work overlaps its vector work
// only when the two are interleaved in its instruction stream (an MFMA runs
// for 32 cycles while the wave keeps issuing independent VALU).  Each
// iteration j therefore pairs independent work:
//   step A: S_{j+1} = K_{j+1} Q^T (MFMA)  with  exponentials, sums and packing
//           of tile j's probabilities P_j (VALU);
//   step B: O += P_j V_j (MFMA)           with  mask, max and reference update
//           of tile j+1 (VALU); a rare rescale of O follows the product.
// At d = 64, whose step is bound by the vector unit, step B takes no row max:
// tile j's exponentials are taken against the row's current reference, and a
// lane whose weights of the tile sum past kSumLimit (or not to a finite
// value) sends tile j to the exact path before its product (scores computed
// again from K in global memory, max, reference move, rescale).
// LDS stage j holds (K_{j+1}, V_j) in buffer j % 2 (block layout above),
// loaded by all waves during iteration j-1; one barrier per iteration.
// Tiles that need a mask (diagonal, sequence tail) and each wave's last tile
// take a general path without the interleaving constraints.
//
// Register layouts (D = head dim, BC = 64 keys per tile, 32 queries per wave):
//   Q fragment (registers, whole kernel): lane (q = lane%32, h = lane/32) holds
//     Q[q][16c + 8h .. 16c + 8h + 7] for c = 0..D/16-1 (the MFMA B operand).
//   K tile (LDS blocks, chunk-major): A operand of S^T = K Q^T, lane
//     (key = lane%32, h) reads K[key][16c + 8h .. +7].
//   S^T block (accumulator): lane (q, h), register r holds key
//     8*(r/4) + 4h + r%4 of the 32-key block, for query q.
//   P^T B operand of O^T += V^T P^T, 16-key chunk c: registers 8(c%2)..+7 of
//     block c/2, i.e. lane (q, h) element t is key 16c + 8(t/4) + 4h + t%4.
//   V tile (LDS blocks, row-major): two ds_read_b64_tr_b16 per A operand
//     give lane (d = lane%32, h) the same eight keys for its column d.
//   O^T (accumulator): block b, register r of lane (q, h) holds
//     O[q][32b + 8*(r/4) + 4h + r%4].
// Occupancy: two waves per SIMD (256 registers each), three at d = 64.
//
// Key split (SPLIT, for grids smaller than the GPU; never persistent): item
// (query block, split s) covers the s-th of n_split equal shares of the
// block's key tiles and writes, per row, its output normalised by its own
// weight sum (fp32, Opart[s]) and the log2 weight of the share,
// mc + log2(l) (Lpart[s]); attn_combine_sp merges them.  A share with no
// kept key of a row writes 0 and -inf.
template <class TT, int DK, int DV, bool CAUSAL, int NW, int NS, bool PERSIST, bool SPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(DK + DV == 128 ? 3 : 2, DK + DV == 128 ? 3 : 2))) void attn_fwd_sp(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int Nq, int Nk, int H, const int* __restrict__ k_len, const int* __restrict__ q_len,
    int n_qtiles, int total_items, int slot, float scale, int n_split, float* __restrict__ Opart,
    float* __restrict__ Lpart) {
  static_assert(!(SPLIT && PERSIST), "a split launch has one workgroup per item");
  // DK: head dim of Q and K (the scores); DV: head dim of V and O
  constexpr int BR = 32 * NW, BC = 64;
  using LK = TileLayout<DK>;
  using LV = TileLayout<DV>;
  constexpr int TBK = LK::BYTES, TBV = LV::BYTES, CGK = LK::CG, CGV = LV::CG;
  constexpr int SB = TBK + TBV;  // bytes of one stage (K tile, then V tile)
  // DMA instructions one wave issues for a K tile and for a V tile
  constexpr int NDK = LK::BLOCKS / NW, NDV = LV::BLOCKS / NW;
  static_assert(LK::BLOCKS % NW == 0 && LV::BLOCKS % NW == 0 && NS >= 2,
                "stages split evenly over the waves");
  static_assert(DK == DV || NS == 2, "more than two stages only with equal head dims");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * SB];  // [stage buffer][K, V]
  // O staging in the epilogue: per wave 32 rows x 64 columns (bf16) at a
  // 144-byte row stride (16-byte aligned rows, writes spread over the banks)
  constexpr int kOStageRow = 144, kOStageBytes = 32 * kOStageRow;
  static_assert(NW * kOStageBytes <= NS * SB && DV % 64 == 0, "O staging fits the stage buffers");

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hf = lane >> 5;
  // O is divided by the fp32 sum l of the unrounded weights, the running
  // denominator of the online softmax ("Deep Learning - Flash Attention",
  // "An Example", the final division by l).
  // Work loop.  Persistent: the workgroup claims items until none is left;
  // thread 0 claims the next item during the current one's last tile.
  // Otherwise the workgroup runs the one item its id maps to.  Every item
  // ends with a barrier after its last LDS read, so the next item's first
  // tile loads may overwrite the stage buffers.
  __shared__ int s_item;
  // thread 0 alone joins the launch's counter slot and claims items; it keeps
  // the launch tag and its join mode here rather than in registers
  __shared__ unsigned long long s_tag;
  __shared__ int s_mode;
  const int xcd = xcd_id();
  if (tid == 0) {
    if (PERSIST) {
      const unsigned long long tag = launch_tag();
      const int mode = join_launch(slot, tag);
      s_tag = tag;
      s_mode = mode;
      s_item = mode == kJoinDynamic ? take_item(slot, xcd, total_items)
                                    : mode == kJoinStatic && (int)blockIdx.x < total_items ? (int)blockIdx.x : -1;
    } else {
      s_item = xcd_remap(blockIdx.x, total_items);
    }
  }
  __syncthreads();
  int work = __builtin_amdgcn_readfirstlane(s_item);
  while (work >= 0) {
    int next = -1;
    const int split = SPLIT ? work % n_split : 0;  // the shares of a block are neighbours
    const int wq = SPLIT ? work / n_split : work;
    const int bh = wq / n_qtiles;
    int qt = wq % n_qtiles;
    if (CAUSAL) qt = n_qtiles - 1 - qt;  // longest rows first
    // keys kept for query i < nq: j < nk and, when causal, j <= i + diag (the
    // last valid query row is aligned with the last valid key); rows from nq
    // on are padding and keep no key
    const int nk = k_len ? min(max(k_len[bh / H], 0), Nk) : Nk;
    const int nq = q_len ? min(max(q_len[bh / H], 0), Nq) : Nq;
    const int diag = nk - nq;
    const size_t qhead = (size_t)bh * Nq * DK, ohead = (size_t)bh * Nq * DV;
    const size_t khead = (size_t)bh * Nk * DK, vhead = (size_t)bh * Nk * DV;
    const int q_first = qt * BR + 32 * wave;
    const int my_q = q_first + lq;

    u32x4 qf[DK / 16];

    const int kv_end = qt * BR >= nq ? 0 : CAUSAL ? min(nk, min((qt + 1) * BR, nq) + diag) : nk;
    const int T_all = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
    // this workgroup's tiles: [tile0, tile0 + T) of the block's T_all (all of
    // them unsplit); tile t below is key tile tile0 + t
    const int tile0 = SPLIT ? (int)((long long)T_all * split / n_split) : 0;
    const int T = SPLIT ? (int)((long long)T_all * (split + 1) / n_split) - tile0 : T_all;
    const int last_key = q_first + 31 + diag;  // this wave's last kept key (causal)
    const int my_T_all = CAUSAL ? (last_key < 0 ? 0 : min(T_all, last_key / BC + 1)) : T_all;
    // A wave whose rows all lie past nq (the ragged last block, padding; a
    // single decoding query leaves seven of eight waves so) only helps load
    // the tiles and meets the barriers.  Not at d = 64, whose three-wave
    // occupancy leaves no registers for the extra control flow.
    const bool idle = DK + DV > 128 && q_first >= nq;
    const int my_T = idle ? 0 : SPLIT ? min(T, max(0, my_T_all - tile0)) : my_T_all;

    const uint16_t* const kbase = K + khead;
    const uint16_t* const vbase = V + vhead;
    const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
    // stage st in [-1, T-1] = (K tile st+1, V tile st) into buffer (st+1) % NS.
    // Each tile gets a descriptor starting at its first key row (scalar
    // arithmetic), so the per-lane offsets are the same for every tile; the
    // record count ends at the last valid key, so rows past it read as zero.
    auto load_stage = [&](int st) {
      const unsigned base = lds0 + ((st + 1) % NS) * SB;
      if (st + 1 < T) {
        const int k0 = (tile0 + st + 1) * BC;
        dma_tile<DK, false, NW>(buffer_desc(kbase + (size_t)k0 * DK, (unsigned)(nk - k0) * DK * 2), base, 0, wave, lane);
      }
      if (st >= 0) {
        const int k0 = (tile0 + st) * BC;
        dma_tile<DV, true, NW>(buffer_desc(vbase + (size_t)k0 * DV, (unsigned)(nk - k0) * DV * 2), base + TBK, 0, wave, lane);
      }
    };
    auto stage_buf = [&](int st) { return (st + 1) % NS; };
    const int k_lane = (lq >> 4) * CGK * 1024 + (hf * 16 + (lq & 15)) * 16;
    const int tr_i = lane & 15, tr_grp = lane >> 4;
    const int v_lane = (4 * (tr_grp >> 1) + (tr_i >> 2)) * 64 + (2 * (tr_grp & 1) + ((tr_i & 3) >> 1)) * 16 +
                       8 * (tr_i & 1);

    f32x16 o[DV / 32];
#pragma unroll
    for (int b = 0; b < DV / 32; ++b) o[b] = f32x16{};
    // running state: row max m, its scaled reference mc (exponents are taken
    // against mc) and the fp32 sum l of the weights
    float m_run = -INFINITY, mc_run = -INFINITY, l_run = 0.f;
    // the exponentials' offset: mc, or 0 while a row has no reference yet
    // (its scores are then all -inf), kept beside mc as it changes
    float off_run = 0.f;
    const float c2 = scale * kLog2e;
    u32x4 pf[BC / 16];  // P_j packed, B operand of the P V product

    auto qk = [&](const uint8_t* kt, f32x16 (&acc)[BC / 32]) {
#pragma unroll
      for (int b = 0; b < BC / 32; ++b) {
        acc[b] = f32x16{};
#pragma unroll
        for (int c = 0; c < DK / 16; ++c) {
          const u32x4 a = *(const u32x4*)(kt + k_lane + (2 * b * CGK + (c >> 1)) * 1024 + (c & 1) * 512);
          acc[b] = TT::mma(a, qf[c], acc[b]);
        }
      }
    };
    auto pv = [&](const uint8_t* vt) {
#pragma unroll
      for (int cc = 0; cc < BC / 16; ++cc)
#pragma unroll
        for (int b = 0; b < DV / 32; ++b) {
          const uint8_t* va = vt + v_lane + (cc * CGV + b) * 1024;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(va));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(va + 512));
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
          o[b] = TT::mma(u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}, pf[cc], o[b]);
        }
    };
    // Tile t's mask (if any), row max and reference move.  Returns the factor
    // for O, which the caller applies after O has received the previous tile;
    // l is rescaled here.  `resc` tells whether any row moved.
    auto part1 = [&](f32x16 (&sv)[BC / 32], int t, bool masked, bool& resc) -> float {
      if (masked) {
        const int k0 = (tile0 + t) * BC;
#pragma unroll
        for (int b = 0; b < BC / 32; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * b + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool keep = key < nk && (!CAUSAL || key <= my_q + diag);
            if (!keep) sv[b][r] = -INFINITY;
          }
      }
      float mt = sv[0][0];
#pragma unroll
      for (int b = 0; b < BC / 32; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sv[b][r]);
      mt = half_max(mt);
      m_run = fmaxf(m_run, mt);
      const float mc_cand = (m_run == -INFINITY) ? -INFINITY : m_run * c2;
      resc = __builtin_amdgcn_ballot_w64(mc_cand > mc_run + kLazyRescale) != 0;
      // 0 for a row's first finite tile; a still fully masked row keeps alpha 1
      const float alpha = (!resc || mc_cand == -INFINITY) ? 1.f : fast_exp2(mc_run - mc_cand);
      mc_run = resc ? mc_cand : mc_run;
      off_run = (mc_run == -INFINITY) ? 0.f : mc_run;
      l_run *= alpha;
      return alpha;
    };
    // Exponentials against the current reference, their sum, and P packed.
    auto part2 = [&](f32x16 (&sv)[BC / 32]) {
      const float off = off_run;
      float ls[2] = {0.f, 0.f};
#pragma unroll
      for (int b = 0; b < BC / 32; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sv[b][r], c2, -off));
          sv[b][r] = p;
          ls[r & 1] += p;
        }
#pragma unroll
      for (int c = 0; c < BC / 16; ++c) {
        const int r0 = 8 * (c & 1);
        const f32x16& sb = sv[c >> 1];
        pf[c] = u32x4{TT::pack(sb[r0 + 0], sb[r0 + 1]), TT::pack(sb[r0 + 2], sb[r0 + 3]),
                      TT::pack(sb[r0 + 4], sb[r0 + 5]), TT::pack(sb[r0 + 6], sb[r0 + 7])};
      }
      l_run += ls[0] + ls[1];
    };
    auto tile_masked = [&](int t) {
      const int k0 = (tile0 + t) * BC;
      return (CAUSAL && k0 + BC - 1 > q_first + diag) || (k0 + BC > nk);
    };
    // d = 64: tile t's scores computed again from K in global memory (the
    // same operands and products as from the LDS copy, so the same bits)
    // and the exact path run on them: mask, row max, reference move, O and l
    // rescaled, exponentials again
    constexpr bool NOMAX = DK + DV == 128;
    auto redo = [&](f32x16 (&sv)[BC / 32], int t) {
      const int k0 = (tile0 + t) * BC;
#pragma unroll
      for (int b = 0; b < BC / 32; ++b) {
        sv[b] = f32x16{};
        const int key = k0 + 32 * b + lq;
        const uint16_t* krow = kbase + (size_t)key * DK + 8 * hf;
#pragma unroll
        for (int c = 0; c < DK / 16; ++c) {
          const u32x4 a = key < nk ? *(const u32x4*)(krow + 16 * c) : u32x4{0, 0, 0, 0};
          sv[b] = TT::mma(a, qf[c], sv[b]);
        }
      }
      bool resc;
      const float alpha = part1(sv, t, tile_masked(t), resc);
      if (resc) {
#pragma unroll
        for (int bb = 0; bb < DV / 32; ++bb) o[bb] *= alpha;
      }
      part2(sv);
    };

    // One steady-state step (tile j's softmax and product, tile j+1's scores
    // and, above d = 64, statistics), written in issue order and fenced so that every MFMA is
    // followed by the independent vector work that hides it.
    auto steady = [&](f32x16 (&cur)[BC / 32], f32x16 (&nxt)[BC / 32], const uint8_t* kt,
                      const uint8_t* vt, int t_next, bool mask_next) {
      constexpr int NQK = BC / 32 * DK / 16, NPV = BC / 16 * DV / 32;
      constexpr int ELEM = BC / 2;  // scores of a tile held by one lane
      const float off = off_run;
      float ls0 = 0.f, ls1 = 0.f;
      // ---- step A: S_{j+1} (MFMA) with exp / sums / packing of tile j (VALU)
      auto kaddr = [&](int i) {
        const int bb = i / (DK / 16), c = i % (DK / 16);
        return (const u32x4*)(kt + k_lane + (2 * bb * CGK + (c >> 1)) * 1024 + (c & 1) * 512);
      };
      constexpr int KP = 4;  // K operands in flight ahead of the matrix core
      u32x4 kop[KP + 1];
#pragma unroll
      for (int i = 0; i < KP && i < NQK; ++i) kop[i] = *kaddr(i);
      __builtin_amdgcn_sched_barrier(0);
      constexpr int EPM = ELEM / NQK;  // elements of tile j per MFMA (2 at d = 128, 4 at d = 64)
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        if (i + KP < NQK) kop[(i + KP) % (KP + 1)] = *kaddr(i + KP);
        const int bb = i / (DK / 16), c = i % (DK / 16);
        nxt[bb] = TT::mma(kop[i % (KP + 1)], qf[c], c == 0 ? f32x16{} : nxt[bb]);
#pragma unroll
        for (int e = EPM * i; e < EPM * (i + 1); ++e) {
          const float pe = fast_exp2(fmaf(cur[e >> 4][e & 15], c2, -off));
          cur[e >> 4][e & 15] = pe;
          if (e & 1) ls1 += pe; else ls0 += pe;
          if ((e & 7) == 7) {  // a 16-key chunk's probabilities are complete: pack them
            const int cc = e >> 3, r0 = 8 * (cc & 1);
            const f32x16& sb = cur[cc >> 1];
            pf[cc] = u32x4{TT::pack(sb[r0 + 0], sb[r0 + 1]), TT::pack(sb[r0 + 2], sb[r0 + 3]),
                           TT::pack(sb[r0 + 4], sb[r0 + 5]), TT::pack(sb[r0 + 6], sb[r0 + 7])};
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (NOMAX) {
        const float ts = ls0 + ls1;
        if (__builtin_amdgcn_ballot_w64(!(ts <= kSumLimit)) != 0) redo(cur, t_next - 1);
        else l_run += ts;
      } else {
        l_run += ls0 + ls1;
      }
      // ---- step B: O += P_j V_j (MFMA) with tile j+1's row max (VALU)
      auto vaddr = [&](int i) {
        const int cc = i / (DV / 32), bb = i % (DV / 32);
        return vt + v_lane + (cc * CGV + bb) * 1024;
      };
      constexpr int VP = 4;  // V operands in flight ahead of the matrix core
      u32x4 vop[VP + 1];
      auto vload = [&](int i) {
        const uint8_t* va = vaddr(i);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(va));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(va + 512));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
      };
#pragma unroll
      for (int i = 0; i < VP && i < NPV; ++i) vop[i] = vload(i);
      if (mask_next) {
        // keys past the row (causal) or past the valid keys score -inf: lane
        // (q, h) keeps key offsets 32b + 8(r/4) + r%4 <= lim within tile t_next
        const int lim = min(CAUSAL ? my_q + diag : nk - 1, nk - 1) - ((tile0 + t_next) * BC + 4 * hf);
#pragma unroll
        for (int b = 0; b < BC / 32; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * b + 8 * (r >> 2) + (r & 3) > lim) nxt[b][r] = -INFINITY;
      }
      // Raised wave priority while this wave feeds the matrix core: when the
      // other wave on the SIMD is in its exponential-heavy step, the arbiter
      // issues this wave's MFMAs first instead of letting them queue behind
      // vector instructions.
      __builtin_amdgcn_s_setprio(2);
      __builtin_amdgcn_sched_barrier(0);
      float mt0 = -INFINITY, mt1 = -INFINITY;
      constexpr int MPM = (ELEM / 2 + NPV - 3) / (NPV - 2);  // score pairs per MFMA from the third on
      int e = 0;
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        if (i + VP < NPV) vop[(i + VP) % (VP + 1)] = vload(i + VP);
        const int cc = i / (DV / 32), bb = i % (DV / 32);
        o[bb] = TT::mma(vop[i % (VP + 1)], pf[cc], o[bb]);
        if (!NOMAX && i >= 2) {
#pragma unroll
          for (int k = 0; k < MPM; ++k) {
            if (e < ELEM / 2) {  // two scores of tile j+1 per max3
              const int e0 = 2 * e, e1 = 2 * e + 1;
              if (e & 1) mt1 = max3(mt1, nxt[e0 >> 4][e0 & 15], nxt[e1 >> 4][e1 & 15]);
              else mt0 = max3(mt0, nxt[e0 >> 4][e0 & 15], nxt[e1 >> 4][e1 & 15]);
              ++e;
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      if constexpr (NOMAX) return;
      // tile j+1's statistics; a row whose keys in this tile are all masked
      // keeps its max (the kept keys are a prefix, so tile 0 gave every row
      // with a kept key a finite one; a row without any stays at -inf)
      const float mt = half_max(max3(mt0, mt1, mt1));
      m_run = fmaxf(m_run, mt);
      const float mc_cand = m_run * c2;
      const bool resc = __builtin_amdgcn_ballot_w64(mc_cand > mc_run + kLazyRescale) != 0;
      if (resc) {
        const float alpha = mc_cand == -INFINITY ? 1.f : fast_exp2(mc_run - mc_cand);
        mc_run = mc_cand;
        off_run = (mc_run == -INFINITY) ? 0.f : mc_run;
        l_run *= alpha;
#pragma unroll
        for (int bb = 0; bb < DV / 32; ++bb) o[bb] *= alpha;
      }
    };

    // Stages are issued AHEAD = NS-1 iterations early: iteration j issues stage
    // j + AHEAD into the buffer of stage j - 1, which iteration j - 1 finished
    // reading before its closing barrier.  Before that barrier, iteration j
    // waits until stage j + 1 (read next) has landed while stages j + 2 ..
    // j + AHEAD stay in flight.  vmcnt retires in issue order, so "at most n
    // outstanding" (n = this wave's loads of those younger stages) means every
    // older load is done.
    constexpr int AHEAD = NS - 1;
    static_assert((NS & (NS - 1)) == 0 && NS <= 4, "power-of-two stage count, at most 4");
    auto issue_for = [&](int j) {
      if (j + AHEAD < T) load_stage(j + AHEAD);
#ifdef FA_SYNC_PHASES
      // check build: every stage has landed and every wave has arrived
      // before any wave reads a tile, so no load overlaps any LDS read
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
#endif
    };
    // loads one wave issues for stage st: K tile (if st+1 < T) and V tile (if st >= 0)
    auto stage_loads = [&](int st) {
      return st >= T ? 0 : (st + 1 < T ? NDK : 0) + (st >= 0 ? NDV : 0);
    };
    // s_waitcnt takes an immediate, so each reachable count (a multiple of half
    // a stage, at most NS-2 full stages) gets its own instruction
    auto wait_keep = [&](int keep) {
      constexpr int HS = NDK;  // loads of half a stage (NDK = NDV when NS > 2)
      static_assert((NS - 2) * (NDK + NDV) <= 63, "vmcnt is a 6-bit count");
      if constexpr (NS >= 4) {
        if (keep >= 4 * HS) { __builtin_amdgcn_s_waitcnt(wait_vmcnt(4 * HS)); return; }
        if (keep == 3 * HS) { __builtin_amdgcn_s_waitcnt(wait_vmcnt(3 * HS)); return; }
      }
      if constexpr (NS >= 3) {
        if (keep >= 2 * HS) { __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * HS)); return; }
        if (keep == HS) { __builtin_amdgcn_s_waitcnt(wait_vmcnt(HS)); return; }
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    };
    auto end_iter = [&](int j) {
      int keep = 0;
#pragma unroll
      for (int st = 2; st <= AHEAD; ++st) keep += stage_loads(j + st);
      wait_keep(keep);
      __syncthreads();
    };

    // prologue: stages -1 (K_0), 0 (K_1, V_0), ..., NS-2; S_0 and its statistics
    f32x16 sA[BC / 32], sB[BC / 32];
    load_stage(-1);
#pragma unroll
    for (int st = 0; st <= NS - 2; ++st)
      if (st < T) load_stage(st);
    // Q after the first stages: its latency overlaps theirs
    if (my_q < nq) {
      const uint16_t* qrow = Q + qhead + (size_t)my_q * DK + 8 * hf;
#pragma unroll
      for (int c = 0; c < DK / 16; ++c) qf[c] = *(const u32x4*)(qrow + 16 * c);
    } else {
#pragma unroll
      for (int c = 0; c < DK / 16; ++c) qf[c] = u32x4{0, 0, 0, 0};
    }
    // stages -1 and 0 must be in; stages 1 .. NS-2 may stay in flight
    {
      int keep = 0;
#pragma unroll
      for (int st = 1; st <= NS - 2; ++st) keep += stage_loads(st);
      wait_keep(keep);
    }
    __syncthreads();
    // Every wave with rows below nq scores tile 0 when the block has one, even
    // a wave whose rows keep no key (causal, more queries than keys): its
    // scores are then all masked, so the steady steps below see -inf instead
    // of stale registers.  An idle wave runs no steady step at all.
    if (0 < T && !idle) {
      bool resc;
      qk(smem + stage_buf(-1) * SB, sA);
      part1(sA, 0, tile_masked(0), resc);  // O is still zero: its factor is not needed
    }
    __syncthreads();  // every wave is done with stage -1's buffer before it is refilled

    // Steady steps run in pairs while both tiles have a successor, masking the
    // next tile's scores where it crosses the diagonal or the end of the
    // sequence; the last one or two tiles take the general path.
    int j = 0;
    // two tiles per trip so the score registers swap roles
    for (; j + 2 < T; j += 2) {
      issue_for(j);
      {
        const uint8_t* kt = smem + stage_buf(j) * SB;
        if (!idle) steady(sA, sB, kt, kt + TBK, j + 1, tile_masked(j + 1));
      }
      end_iter(j);
      issue_for(j + 1);
      {
        const uint8_t* kt = smem + stage_buf(j + 1) * SB;
        if (!idle) steady(sB, sA, kt, kt + TBK, j + 2, tile_masked(j + 2));
      }
      end_iter(j + 1);
    }
    // At d = 64 the last steady step hands tile j's scores on without their
    // row max: take it here (mask, max, reference move, rescale) before the
    // general path takes the exponentials
    if constexpr (NOMAX) {
      if (j > 0 && j < T && !idle) {
        bool resc;
        const float alpha = part1(sA, j, tile_masked(j), resc);
        if (resc) {
#pragma unroll
          for (int b = 0; b < DV / 32; ++b) o[b] *= alpha;
        }
      }
    }
    // remaining tiles: general path (a wave skips tiles past its last row)
    for (; j < T; ++j) {
      issue_for(j);
      // claim the next item during the last tile: claiming earlier would
      // reserve work that an idle workgroup could have started sooner
      if (PERSIST && tid == 0 && j == T - 1) next = next_item(s_mode, slot, xcd, total_items, work);
      const uint8_t* kt = smem + stage_buf(j) * SB;  // K_{j+1}
      const uint8_t* vt = kt + TBK;                   // V_j
      if (j < my_T) {
        part2(sA);
        pv(vt);
        if (j + 1 < my_T) {
          bool resc;
          qk(kt, sB);
          const float alpha = part1(sB, j + 1, tile_masked(j + 1), resc);
          if (resc) {
#pragma unroll
            for (int b = 0; b < DV / 32; ++b) o[b] *= alpha;
          }
#pragma unroll
          for (int b = 0; b < BC / 32; ++b) sA[b] = sB[b];
        }
      }
      end_iter(j);
    }
    // An item without key tiles (a block of padding rows, no valid keys, or
    // causal rows that all precede the first key) runs no tile above, so its
    // successor is claimed here.
    if (PERSIST && tid == 0 && T == 0) next = next_item(s_mode, slot, xcd, total_items, work);

    // Epilogue.  A lane holds 8-byte pieces of its row at 16-byte strides, so
    // storing straight from registers would make every store instruction
    // touch 32 rows; instead each wave passes its normalised, rounded rows
    // through its own LDS area (the stage buffers are free after the last
    // barrier) and stores whole 128-byte row segments, 8 lanes per segment.
    // a padding row (my_q >= nq) stores the empty sum: O = 0, lse = -inf
    const bool pad = my_q >= nq;
    const float l_tot = pad ? 0.f : half_sum(l_run);
    if constexpr (SPLIT) {
      // this share's output and weights, fp32, straight from the registers
      // (block b, register 4g+e of lane (q, h) is column 32b + 8g + 4h + e)
      const float inv = l_tot > 0.f ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
      if (my_q < Nq) {
        const size_t rows = (size_t)(total_items / (n_qtiles * n_split)) * Nq;
        const size_t row = (size_t)split * rows + (size_t)bh * Nq + my_q;
        float* orow = Opart + row * DV + 4 * hf;
#pragma unroll
        for (int b = 0; b < DV / 32; ++b)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(f32x4*)(orow + 32 * b + 8 * g) = f32x4{o[b][4 * g] * inv, o[b][4 * g + 1] * inv,
                                                     o[b][4 * g + 2] * inv, o[b][4 * g + 3] * inv};
        if (hf == 0) Lpart[row] = l_tot > 0.f ? mc_run + __builtin_amdgcn_logf(l_tot) : -INFINITY;
      }
    } else {
      // a row without kept keys has l = 0 and O = 0 (rows past Nq: not stored)
      const float inv = l_tot > 0.f ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
      uint8_t* stg = smem + wave * kOStageBytes;
#pragma unroll
      for (int r = 0; r < DV / 64; ++r) {
#ifdef FA_SYNC_PHASES
        __syncthreads();  // check build: a barrier around every staging phase
#endif
#pragma unroll
        for (int bl = 0; bl < 2; ++bl)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16& ob = o[2 * r + bl];
            const u32x2 w = {TT::pack(ob[4 * g + 0] * inv, ob[4 * g + 1] * inv),
                             TT::pack(ob[4 * g + 2] * inv, ob[4 * g + 3] * inv)};
            *(u32x2*)(stg + lq * kOStageRow + 2 * (32 * bl + 8 * g + 4 * hf)) = w;
          }
#ifdef FA_SYNC_PHASES
        __syncthreads();
#endif
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 8 * i + (lane >> 3);
          const u32x4 v = *(const u32x4*)(stg + row * kOStageRow + 16 * (lane & 7));
          if (q_first + row < Nq)
            *(u32x4*)(O + ohead + (size_t)(q_first + row) * DV + 64 * r + 8 * (lane & 7)) = v;
        }
      }
      // a row without kept keys: -inf + ln 0 = -inf, the log of the empty sum
      if (hf == 0 && my_q < Nq) LSE[(size_t)bh * Nq + my_q] = (mc_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    if (tid == 0) s_item = next;
    __syncthreads();
    work = __builtin_amdgcn_readfirstlane(s_item);
  }
  if (PERSIST && tid == 0 && s_mode == kJoinDynamic) leave_launch(slot, s_tag);
}

// splits whose partial results one merge thread has in flight at once
constexpr int kCombineBatch = 8;

// Merge of the 16-bit kernel's key shares, per row: with b_s = mc_s +
// log2(l_s) the log2 weight of share s, O = sum_s 2^(b_s) O_s / sum_s 2^(b_s)
// and lse = ln sum_s 2^(b_s), the rule by which partial softmax results over
// disjoint key sets combine ("FlashAttention Engine", "Core FlashAttention
// Mechanics", item 3).  DV/8 threads per row, 8 columns each; shares are
// added in order.
template <class TT, int DV>
__global__ __launch_bounds__(256) void attn_combine_sp(const float* __restrict__ Opart,
                                                       const float* __restrict__ Lpart,
                                                       uint16_t* __restrict__ O,
                                                       float* __restrict__ LSE, long long rows,
                                                       int n_split) {
  constexpr int TPR = DV / 8, RPB = 256 / TPR;  // threads per row, rows per block
  const int t = threadIdx.x % TPR;
  // row blocks on XCDs as the split kernel's blocks were (see attn_combine_f32)
  const long long row = (long long)xcd_remap(blockIdx.x, gridDim.x) * RPB + threadIdx.x / TPR;
  if (row >= rows) return;
  // shares read kCombineBatch at a time, as in attn_combine_f32 (one batch:
  // the max from its own loads)
  const bool one = n_split <= kCombineBatch;
  float bmax = -INFINITY;
  for (int s0 = 0; !one && s0 < n_split; s0 += kCombineBatch) {
    float l[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i)
      l[i] = s0 + i < n_split ? Lpart[(size_t)(s0 + i) * rows + row] : -INFINITY;
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) bmax = fmaxf(bmax, l[i]);
  }
  uint16_t* orow = O + (size_t)row * DV + 8 * t;
  float wsum = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_split; s0 += kCombineBatch) {
    float l[kCombineBatch];
    f32x4 op0[kCombineBatch], op1[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const bool in = s0 + i < n_split;
      const f32x4* op = (const f32x4*)(Opart + ((size_t)(s0 + i) * rows + row) * DV + 8 * t);
      l[i] = in ? Lpart[(size_t)(s0 + i) * rows + row] : -INFINITY;
      op0[i] = in ? op[0] : f32x4{0.f, 0.f, 0.f, 0.f};
      op1[i] = in ? op[1] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (one) {
#pragma unroll
      for (int i = 0; i < kCombineBatch; ++i) bmax = fmaxf(bmax, l[i]);
    }
    if (bmax == -INFINITY) {  // no share kept a key of this row: the empty sum
      *(u32x4*)orow = u32x4{0, 0, 0, 0};
      if (t == 0) LSE[row] = -INFINITY;
      return;
    }
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      if (s0 + i < n_split) {
        const float e = fast_exp2(l[i] - bmax);  // 0 for a share without kept keys
        wsum += e;
        acc0 += e * op0[i];
        acc1 += e * op1[i];
      }
    }
  }
  const float inv = 1.f / wsum;
  *(u32x4*)orow = u32x4{TT::pack(acc0[0] * inv, acc0[1] * inv), TT::pack(acc0[2] * inv, acc0[3] * inv),
                        TT::pack(acc1[0] * inv, acc1[1] * inv), TT::pack(acc1[2] * inv, acc1[3] * inv)};
  if (t == 0) LSE[row] = (bmax + __builtin_amdgcn_logf(wsum)) * kLn2;
}

// ---------------------------------------------------------------------------
// fp32 kernel
//
// A workgroup owns 32 query rows and DS waves; wave w owns head-dim columns
// [w*DSL, (w+1)*DSL).  Keys go 32 per tile.  With the 32x32x2 fp32 MFMA each
// lane supplies one element per operand, so K and V are read from global
// memory (L2) straight into registers in operand order:
//   S^T = K Q^T : step (u, v) contracts column  w*DSL + 8u + 4h + v,
//                 lane (key, h) gives K[key][..], lane (q, h) gives Q[q][..].
//   O^T += V^T P^T : step r contracts key 8(r/4) + 4h + r%4 (register r of
//                 the score block); output block bb row i is column
//                 w*DSL + NB*i + bb (NB = DSL/32 blocks), so one lane's NB
//                 values of a V row are contiguous.
//
// Key split (SPLIT): work item (query block, split s) covers key tiles
// [s*tps, (s+1)*tps) only and writes its own normalised output and
// log-sum-exp over those keys to Opart[s] / LSEpart[s] (rows*D and rows
// floats per split); attn_combine_f32 merges the splits.  A split that holds
// no kept key of a row writes 0 and -inf for it.
// A raw buffer resource for compiler-visible buffer loads, its base and
// record count read from the first lane (wave-uniform by construction), so
// that the compiler keeps it in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)base;
  const uint64_t u = (uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)a) |
                     ((uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32)) << 32);
  return __builtin_amdgcn_make_buffer_rsrc((void*)u, 0, __builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
}

// With 64 V columns a wave fits two waves per SIMD; the hint keeps the
// compiler there (without it the 128/64 split takes 267 registers).
template <int DSL, int DSLV, int DS, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(DS * 64) __attribute__((amdgpu_waves_per_eu(DSLV == 64 ? 2 : 1))) void attn_fwd_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int Nq, int Nk, int H,
    const int* __restrict__ k_len, const int* __restrict__ q_len, int n_qtiles, int total_wg,
    float scale, int n_split, int tps, float* __restrict__ Opart, float* __restrict__ LSEpart) {
  // D: head dim of Q and K (DSL columns per wave); DV: of V and O (DSLV per wave)
  constexpr int D = DSL * DS, DV = DSLV * DS, NB = DSLV / 32, BC = 32;
  // partial scores exchanged between the waves: slot w, slice c of every
  // lane, CH = 16/DS floats each, lanes contiguous (no bank conflicts)
  constexpr int CH = 16 / DS;
  __shared__ __attribute__((aligned(16))) float red[DS > 1 ? DS * DS * 64 * CH : 1];
  // Each wave's slice of a K tile (32 keys x DSL columns, read by that wave
  // only) is loaded straight into LDS by buffer loads, 16 bytes per lane:
  // 1 KB blocks of 8 rows x 8 chunks (one 128-byte line of each row), block
  // (rg, cg) = rows 8rg.., chunks 8cg.. at (rg * DSL/32 + cg) KB, and chunk
  // ci of row ri in slot ri * 8 + (ci ^ ri ^ (rg & 1)).  A load instruction
  // then reads 8 whole lines, and the 16 rows a 16-lane group reads for one
  // operand fall in 16 distinct slots of a 256-byte bank row.
  static_assert(DSL % 32 == 0, "K slices are whole 8-chunk blocks");
  __shared__ __attribute__((aligned(1024))) float ksm[DS * 32 * DSL];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lq = lane & 31, hf = lane >> 5;
  const int item = xcd_remap(blockIdx.x, total_wg);
  const int split = SPLIT ? item % n_split : 0;  // the splits of a block are neighbours
  const int work = SPLIT ? item / n_split : item;
  const int bh = work / n_qtiles;
  int qt = work % n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;
  // as in the 16-bit kernel; read from the first lane so that the compiler
  // keeps them (and the buffer descriptors made from them) scalar
  const int nk = __builtin_amdgcn_readfirstlane(k_len ? min(max(k_len[bh / H], 0), Nk) : Nk);
  const int nq = __builtin_amdgcn_readfirstlane(q_len ? min(max(q_len[bh / H], 0), Nq) : Nq);
  const int diag = nk - nq;
  const size_t head = (size_t)bh * Nq * D, khead = (size_t)bh * Nk * D;
  const size_t vhead = (size_t)bh * Nk * DV, ohead = (size_t)bh * Nq * DV;
  const int q_first = qt * 32;
  const int my_q = q_first + lq;
  const int col0 = wave * DSL, colv0 = wave * DSLV;

  f32x4 qf[DSL / 8];  // Q rows, loaded below
  f32x16 o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) o[b] = f32x16{};
  // running state as in the 16-bit kernel: raw max, exponent reference, sum
  float m_run = -INFINITY, mc_run = -INFINITY, l_run = 0.f;
  const float c2 = scale * kLog2e;
  const int kv_end = q_first >= nq ? 0 : CAUSAL ? min(nk, min(q_first + 32, nq) + diag) : nk;
  const int ntiles = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
  const int j_begin = SPLIT ? split * tps : 0;
  const int j_end = SPLIT ? min(ntiles, j_begin + tps) : ntiles;

  // K tile j into this wave's LDS slice, through one descriptor per tile
  // based at its first key row and this wave's first column and ending at
  // the last valid key row (rows past it read 0); lane L of block (rg, cg)
  // reads row 8rg + L/8, chunk 8cg + ((L%8) ^ (L/8) ^ (rg & 1)).
  constexpr int CG = DSL / 32;
  float* const kw = ksm + wave * 32 * DSL;
  const unsigned kw_lds = (unsigned)(uintptr_t)(__attribute__((address_space(3))) float*)kw;
  const int dma_lane0 = ((lane >> 3) * D + 4 * ((lane & 7) ^ (lane >> 3))) * 4;
  const int dma_lane1 = ((lane >> 3) * D + 4 * ((lane & 7) ^ (lane >> 3) ^ 1)) * 4;
  auto dma_k = [&](int j) {
    const int k0 = j * BC;
    const u32x4 desc = buffer_desc(K + khead + (size_t)k0 * D + col0, (unsigned)min(nk - k0, BC) * D * 4);
#pragma unroll
    for (int blk = 0; blk < 4 * CG; ++blk) {
      const int rg = blk / CG, cg = blk % CG;
      dma16(desc, kw_lds + blk * 1024, (rg & 1 ? dma_lane1 : dma_lane0) + (8 * rg * D + 32 * cg) * 4);
    }
  };
  // where lane (key, h) reads chunk 2u + h of its key row
  const int krg = lq >> 3, kri = lq & 7;
  const float* const kread = kw + (krg * CG * 64 + kri * 8) * 4;
  auto kslot = [&](int u) {
    const int c = 2 * u + hf;
    return kread + ((c >> 3) * 64 + ((c & 7) ^ kri ^ (krg & 1))) * 4;
  };
  // V rows of a tile: step r takes key 8(r/4) + 4h + r%4.  Buffer loads
  // through one descriptor per tile based at its first key and ending at the
  // last valid key (rows past it read 0), one instruction per step, so that
  // the wait for a tile's K below can count them.
  const int v_lane = (4 * hf * DV + colv0 + NB * lq) * 4;  // row 4h of the tile, this lane's columns
  float vv[16][NB];
  auto v_res = [&](int j) {
    return uniform_rsrc(V + vhead + (size_t)j * BC * DV, min(nk - j * BC, BC) * DV * 4);
  };
  auto load_v = [&](__amdgpu_buffer_rsrc_t vres, int r) {
    const int voff = v_lane + (8 * (r >> 2) + (r & 3)) * DV * 4;
    if constexpr (NB == 4) {
      const f32x4 t = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(vres, voff, 0, 0));
      vv[r][0] = t[0]; vv[r][1] = t[1]; vv[r][2] = t[2]; vv[r][3] = t[3];
    } else {
      static_assert(NB == 2, "V rows are 64 or 128 columns per wave");
      const f32x2 t = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(vres, voff, 0, 0));
      vv[r][0] = t[0]; vv[r][1] = t[1];
    }
  };
  // Q rows in registers: lane (q, h) holds Q[q][col0 + 8u + 4h .. +3],
  // staged through this wave's LDS slice in the K layout (whole-line loads)
  {
    const u32x4 desc = buffer_desc(Q + head + (size_t)q_first * D + col0,
                                   (unsigned)min(max(nq - q_first, 0), 32) * D * 4);
#pragma unroll
    for (int blk = 0; blk < 4 * CG; ++blk) {
      const int rg = blk / CG, cg = blk % CG;
      dma16(desc, kw_lds + blk * 1024, (rg & 1 ? dma_lane1 : dma_lane0) + (8 * rg * D + 32 * cg) * 4);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
    for (int u = 0; u < DSL / 8; ++u) qf[u] = *(const f32x4*)kslot(u);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slice is read before K overwrites it
  }
  // first K tile; waited for before the first V rows are requested (V is
  // not needed before the first P V product)
  if (j_begin < j_end) dma_k(j_begin);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  if (j_begin < j_end) {
    const __amdgpu_buffer_rsrc_t vres = v_res(j_begin);
#pragma unroll
    for (int r = 0; r < 16; ++r) load_v(vres, r);
  }
  for (int j = j_begin; j < j_end; ++j) {
    const int k0 = j * BC;
    // this tile's K: issued before its 16 V loads, so done at vmcnt <= 16
#ifdef FA_SYNC_PHASES
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#else
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(16));
#endif
    // partial S^T over this wave's columns
    f32x16 s = f32x16{};
#pragma unroll
    for (int u = 0; u < DSL / 8; ++u) {
      const f32x4 ka = *(const f32x4*)kslot(u);
#pragma unroll
      for (int v = 0; v < 4; ++v) s = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[v], qf[u][v], s, 0, 0, 0);
    }
    // The V rows have arrived (they were requested first; waiting here also
    // tells the compiler so, and it adds no wait later that would count the
    // K loads below); this wave's reads of its K slice are done (consumed by
    // the products above), so the next tile's K can go into it.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (j + 1 < j_end) dma_k(j + 1);

    if constexpr (DS > 1) {
      // Full scores = the DS partials summed in wave order, each element once:
      // wave w sums slice w (registers CH*w .. CH*w+CH-1) of every wave's
      // partial and publishes it in its own slot at position w; every wave
      // then reads the DS sums.  Position w of slot w is never written with a
      // partial (wave w keeps that slice in registers), so the next tile's
      // partials cannot overwrite a sum another wave may still be reading.
      auto at = [&](int slot, int c) { return red + ((slot * DS + c) * 64 + lane) * CH; };
#pragma unroll
      for (int c = 0; c < DS; ++c)
        if (c != wave) {
#pragma unroll
          for (int i = 0; i < CH; ++i) at(wave, c)[i] = s[CH * c + i];
        }
      __syncthreads();
      float sum[CH];
#pragma unroll
      for (int w = 0; w < DS; ++w) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          float part = 0.f;
#pragma unroll
          for (int c = 0; c < DS; ++c)  // this wave's own slice, from registers
            if (c == wave) part = s[CH * c + i];
          if (w != wave) part = at(w, wave)[i];
          sum[i] = w == 0 ? part : sum[i] + part;
        }
      }
#pragma unroll
      for (int i = 0; i < CH; ++i) at(wave, wave)[i] = sum[i];
      __syncthreads();
#pragma unroll
      for (int c = 0; c < DS; ++c) {
#pragma unroll
        for (int i = 0; i < CH; ++i) s[CH * c + i] = c == wave ? sum[i] : at(c, c)[i];
      }
    }
    const bool need_mask = (CAUSAL && k0 + BC - 1 > q_first + diag) || (k0 + BC > nk);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (!(key < nk && (!CAUSAL || key <= my_q + diag))) s[r] = -INFINITY;
      }
    }
    float mt = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
    mt = half_max(mt);
    m_run = fmaxf(m_run, mt);
    // the reference moves (and O and l are rescaled) only when some row's max
    // has grown past it by more than kLazyRescale powers of two, as in the
    // 16-bit kernel; a row's first finite tile always moves it
    const float mc_cand = (m_run == -INFINITY) ? -INFINITY : m_run * c2;
    if (__builtin_amdgcn_ballot_w64(mc_cand > mc_run + kLazyRescale) != 0) {
      // 0 for a row's first finite tile; a still fully masked row keeps alpha 1
      const float alpha = mc_cand == -INFINITY ? 1.f : fast_exp2(mc_run - mc_cand);
      mc_run = mc_cand;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b] *= alpha;
    }
    const float off = (mc_run == -INFINITY) ? 0.f : mc_run;
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(fmaf(s[r], c2, -off));
      s[r] = p;
      lsum += p;
    }
    l_run += lsum;
    // O^T += V^T P^T; the next tile's V rows of step r go into that step's
    // registers four steps later, so the loads spread over the products and
    // never wait for a product that still has to read the registers
    constexpr int LAG = 4;
    const bool more = j + 1 < j_end;
    const __amdgpu_buffer_rsrc_t vnext = v_res(more ? j + 1 : j);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[r][b], s[r], o[b], 0, 0, 0);
      if (more && r >= LAG) load_v(vnext, r - LAG);
    }
    if (more) {
#pragma unroll
      for (int r = 16 - LAG; r < 16; ++r) load_v(vnext, r);
    }
  }

  const float l_sum = half_sum(l_run);
  const float l_tot = my_q < nq ? l_sum : 0.f;  // a padding row: the empty sum
  if (my_q < Nq) {
    // a split may hold no kept key of this row: weight 0, lse -inf
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = (SPLIT ? Opart + (size_t)split * ((size_t)Nq * DV * (total_wg / (n_qtiles * n_split))) : O) +
                  ohead + (size_t)my_q * DV + colv0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * hf + (r & 3);
      if constexpr (NB == 4 && DSLV <= DSL) {
        // Staged in this wave's K area (no load is pending into it), row
        // lq's 16-byte chunk i in slot i ^ lq, then stored whole rows at a
        // time below: a direct store from these registers would write 32 B
        // to each of 32 rows per instruction.
        *(f32x4*)(kw + lq * DSLV + 4 * (i ^ lq)) =
            f32x4{o[0][r] * inv, o[1][r] * inv, o[2][r] * inv, o[3][r] * inv};
      } else if constexpr (NB == 4) {
        *(f32x4*)(orow + 4 * i) = f32x4{o[0][r] * inv, o[1][r] * inv, o[2][r] * inv, o[3][r] * inv};
      } else if constexpr (NB == 2) {
        *(f32x2*)(orow + 2 * i) = f32x2{o[0][r] * inv, o[1][r] * inv};
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) orow[NB * i + b] = o[b][r] * inv;
      }
    }
    if (hf == 0 && wave == 0) {
      const float lse_row = l_tot > 0.f ? (mc_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
      if (SPLIT)
        LSEpart[(size_t)split * Nq * (total_wg / (n_qtiles * n_split)) + (size_t)bh * Nq + my_q] = lse_row;
      else
        LSE[(size_t)bh * Nq + my_q] = lse_row;
    }
  }
  if constexpr (NB == 4 && DSLV <= DSL) {
    // whole rows out, two per store: lane (c, h) takes chunk c of row 2t + h
    float* obase = (SPLIT ? Opart + (size_t)split * ((size_t)Nq * DV * (total_wg / (n_qtiles * n_split))) : O) +
                   ohead + colv0;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int row = 2 * t + hf, c = lq;
      const f32x4 val = *(const f32x4*)(kw + row * DSLV + 4 * (c ^ row));
      if (q_first + row < Nq) *(f32x4*)(obase + (size_t)(q_first + row) * DV + 4 * c) = val;
    }
  }
}

// Merge of the key splits: for each row, lse = ln sum_s exp(lse_s) and
// O = sum_s exp(lse_s - lse) O_s -- the rule by which two partial softmax
// results over disjoint key sets combine ("FlashAttention Engine", "Core
// FlashAttention Mechanics", item 3).  D/4 threads per row, 4 columns each;
// splits are summed in order, so the result is reproducible.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_f32(const float* __restrict__ Opart,
                                                        const float* __restrict__ LSEpart,
                                                        float* __restrict__ O,
                                                        float* __restrict__ LSE, int rows,
                                                        int n_split) {
  constexpr int TPR = D / 4, RPB = TPR >= 256 ? 1 : 256 / TPR;  // threads per row, rows per block
  const int t = threadIdx.x % TPR;
  // Row blocks go to XCDs in contiguous ranges, as the split kernel's query
  // blocks did, so that a row's partials are mostly read from the L2 of the
  // XCD that wrote them.
  const long long row = (long long)xcd_remap(blockIdx.x, gridDim.x) * RPB + threadIdx.x / TPR;
  if (threadIdx.x / TPR >= RPB || row >= rows) return;
  // The splits are read kCombineBatch at a time, all loads of a batch issued
  // before any is used; the sums still run over the splits in order.  Up to
  // kCombineBatch splits take one batch, and the max comes from its loads
  // (one round trip to memory); more take a first pass for the max.
  const bool one = n_split <= kCombineBatch;
  float m = -INFINITY;
  for (int s0 = 0; !one && s0 < n_split; s0 += kCombineBatch) {
    float l[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i)
      l[i] = s0 + i < n_split ? LSEpart[(size_t)(s0 + i) * rows + row] : -INFINITY;
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) m = fmaxf(m, l[i]);
  }
  float sum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_split; s0 += kCombineBatch) {
    float l[kCombineBatch];
    f32x4 op[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const bool in = s0 + i < n_split;
      l[i] = in ? LSEpart[(size_t)(s0 + i) * rows + row] : -INFINITY;
      op[i] = in ? *(const f32x4*)(Opart + ((size_t)(s0 + i) * rows + row) * D + 4 * t) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (one) {
#pragma unroll
      for (int i = 0; i < kCombineBatch; ++i) m = fmaxf(m, l[i]);
    }
    if (m == -INFINITY) {  // no split kept a key of this row: the empty sum
      *(f32x4*)(O + (size_t)row * D + 4 * t) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t == 0) LSE[row] = -INFINITY;
      return;
    }
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      if (s0 + i < n_split) {
        const float w = __expf(l[i] - m);  // 0 for an empty split
        sum += w;
        acc += w * op[i];
      }
    }
  }
  const float inv = 1.f / sum;
  *(f32x4*)(O + (size_t)row * D + 4 * t) = acc * inv;
  if (t == 0) LSE[row] = m + __logf(sum);
}

// ---------------------------------------------------------------------------
// host side

// Shape of one call: Nq query rows and Nk key rows per head, optional
// per-batch valid key and query counts (device arrays, clamped to [0, Nk]
// and [0, Nq] on the GPU).
struct Shape {
  int BH, H, Nq, Nk;
  const int* k_len;
  const int* q_len = nullptr;
};

// Key-split plan for grids too small to fill the GPU.  fp32: about one
// workgroup per CU, at least one key tile (of 32) per split, `tps` tiles each
// (its kernel runs one dependent chain of products per tile, so a tiny grid
// is latency-bound and gains even from one-tile ranges: 20.6 -> 12.1 us on
// one head of 128 rows at d = 64).
// 16-bit: about as many workgroups as the CUs hold at once (one at d = 128,
// three at d = 64), at least 4 key tiles (of 64) per share, each query
// block's tiles cut into n_split equal shares.  n_split = 1: none.
struct SplitPlan {
  int n_split = 1, tps = 0;
  size_t bytes = 0;  // workspace: partial O (n_split*rows*dv floats), then the rows' weights
};

SplitPlan plan_split(long long BH, int Nq, int Nk, int dk, int dv, int dtype) {
  SplitPlan p;
  int cus = 0;
  if (compute_units(&cus) != hipSuccess) return p;
  const size_t rows = (size_t)BH * Nq;
  if (dtype == FA_DTYPE_FP32) {
    const long long items = (long long)((Nq + 31) / 32) * BH, ntiles = (Nk + 31) / 32;
    if (items >= cus) return p;
    long long sp = std::min<long long>((cus + items - 1) / items, ntiles);
    if (sp < 2) return p;
    p.tps = (int)((ntiles + sp - 1) / sp);
    p.n_split = (int)((ntiles + p.tps - 1) / p.tps);
    if (p.n_split < 2) return SplitPlan{};
    p.bytes = (size_t)p.n_split * rows * (size_t)(dv + 1) * sizeof(float);
    return p;
  }
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16) return p;
  const bool wide = dk == 128 || dv == 128;
  const long long br = wide ? 256 : 128, slots = (long long)cus * (wide ? 1 : 3);
  const long long items = (Nq + br - 1) / br * BH, ntiles = (Nk + 63) / 64;
  if (items >= slots) return p;
  const long long sp = std::min<long long>((slots + items - 1) / items, ntiles / 4);
  if (sp < 2) return p;
  p.n_split = (int)sp;
  p.bytes = (size_t)p.n_split * rows * (size_t)(dv + 1) * sizeof(float);
  return p;
}

template <class TT, int DK, int DV>
hipError_t launch_sp(const void* q, const void* k, const void* v, void* o, float* lse,
                     const Shape& sh, float scale, bool causal, hipStream_t st,
                     const SplitPlan& plan, void* ws) {
  // d = 128: 8 waves (256 query rows) per workgroup halve the K/V tile
  // loads per FLOP, and one persistent workgroup per CU claims work items
  // (no gap between items, no idle XCD at the end).  d = 64: 4 waves, three
  // waves per SIMD (the kernel fits 168 registers; measured 6% faster than
  // two), one workgroup per item.  Unequal head dims take the d = 128
  // arrangement.
  constexpr bool WIDE = DK == 128 || DV == 128;
  constexpr int NW = WIDE ? 8 : 4, NS = 2;
  constexpr bool PERSIST = WIDE;
  static std::atomic<unsigned> launches{0};
  const int nq = (sh.Nq + 32 * NW - 1) / (32 * NW);
  if (plan.n_split > 1) {
    const int total = nq * sh.BH * plan.n_split;
    const long long rows = (long long)sh.BH * sh.Nq;
    float* opart = (float*)ws;
    float* lpart = opart + (size_t)plan.n_split * rows * DV;
    const dim3 grid(total), block(64 * NW);
    if (causal)
      hipLaunchKernelGGL((attn_fwd_sp<TT, DK, DV, true, NW, NS, false, true>), grid, block, 0, st,
                         (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o,
                         lse, sh.Nq, sh.Nk, sh.H, sh.k_len, sh.q_len, nq, total, 0, scale, plan.n_split,
                         opart, lpart);
    else
      hipLaunchKernelGGL((attn_fwd_sp<TT, DK, DV, false, NW, NS, false, true>), grid, block, 0, st,
                         (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o,
                         lse, sh.Nq, sh.Nk, sh.H, sh.k_len, sh.q_len, nq, total, 0, scale, plan.n_split,
                         opart, lpart);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    constexpr int RPB = 256 / (DV / 8);
    hipLaunchKernelGGL((attn_combine_sp<TT, DV>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256),
                       0, st, (const float*)opart, (const float*)lpart, (uint16_t*)o, lse, rows,
                       plan.n_split);
    return hipGetLastError();
  }
  const int total = nq * sh.BH;
  int grid_wg = total, slot = 0;
  if (PERSIST) {
    int cus = 0;
    if (hipError_t e = compute_units(&cus); e != hipSuccess) return e;
    grid_wg = std::min(total, cus);
    slot = (int)(launches.fetch_add(1, std::memory_order_relaxed) % kWorkSlots);
  }
  const dim3 grid(grid_wg), block(64 * NW);
  if (causal)
    hipLaunchKernelGGL((attn_fwd_sp<TT, DK, DV, true, NW, NS, PERSIST, false>), grid, block, 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse,
                       sh.Nq, sh.Nk, sh.H, sh.k_len, sh.q_len, nq, total, slot, scale, 1, nullptr, nullptr);
  else
    hipLaunchKernelGGL((attn_fwd_sp<TT, DK, DV, false, NW, NS, PERSIST, false>), grid, block, 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse,
                       sh.Nq, sh.Nk, sh.H, sh.k_len, sh.q_len, nq, total, slot, scale, 1, nullptr, nullptr);
  return hipGetLastError();
}

template <int DSL, int DSLV, int DS>
hipError_t launch32(const void* q, const void* k, const void* v, void* o, float* lse,
                    const Shape& sh, float scale, bool causal, hipStream_t st,
                    const SplitPlan& plan, void* ws) {
  constexpr int D = DSLV * DS;  // the width of O
  const int nq = (sh.Nq + 31) / 32;
  if (plan.n_split > 1) {
    const int total = nq * sh.BH * plan.n_split;
    float* opart = (float*)ws;
    float* lpart = opart + (size_t)plan.n_split * sh.BH * sh.Nq * D;
    const dim3 grid(total), block(DS * 64);
    if (causal)
      hipLaunchKernelGGL((attn_fwd_f32<DSL, DSLV, DS, true, true>), grid, block, 0, st, (const float*)q,
                         (const float*)k, (const float*)v, (float*)o, lse, sh.Nq, sh.Nk, sh.H,
                         sh.k_len, sh.q_len, nq, total, scale, plan.n_split, plan.tps, opart, lpart);
    else
      hipLaunchKernelGGL((attn_fwd_f32<DSL, DSLV, DS, false, true>), grid, block, 0, st, (const float*)q,
                         (const float*)k, (const float*)v, (float*)o, lse, sh.Nq, sh.Nk, sh.H,
                         sh.k_len, sh.q_len, nq, total, scale, plan.n_split, plan.tps, opart, lpart);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    constexpr int RPB = D / 4 >= 256 ? 1 : 256 / (D / 4);
    const int rows = sh.BH * sh.Nq;
    hipLaunchKernelGGL((attn_combine_f32<D>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, st,
                       (const float*)opart, (const float*)lpart, (float*)o, lse, rows,
                       plan.n_split);
    return hipGetLastError();
  }
  const int total = nq * sh.BH;
  const dim3 grid(total), block(DS * 64);
  if (causal)
    hipLaunchKernelGGL((attn_fwd_f32<DSL, DSLV, DS, true, false>), grid, block, 0, st, (const float*)q,
                       (const float*)k, (const float*)v, (float*)o, lse, sh.Nq, sh.Nk, sh.H,
                       sh.k_len, sh.q_len, nq, total, scale, 1, 0, nullptr, nullptr);
  else
    hipLaunchKernelGGL((attn_fwd_f32<DSL, DSLV, DS, false, false>), grid, block, 0, st, (const float*)q,
                       (const float*)k, (const float*)v, (float*)o, lse, sh.Nq, sh.Nk, sh.H,
                       sh.k_len, sh.q_len, nq, total, scale, 1, 0, nullptr, nullptr);
  return hipGetLastError();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

// Scratch of the allocation-free entry point: the key-split partial outputs
// and weights (the workspace fa_fwd_gen takes from the caller), held in the
// code object on every device the library runs on, for the life of the
// process.  Host code never passes the array's name to a kernel (on the host
// it is only a stand-in for the symbol); it passes the device address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

int fa_fwd_supported(int d, int dtype, int causal) {
  if (causal != 0 && causal != 1) return 0;
  if (dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_FP16) return d == 64 || d == 128;
  if (dtype == FA_DTYPE_FP32) return d == 64 || d == 128 || d == 256 || d == 512 || d == 1024;
  return 0;
}

int fa_fwd_gen_supported(int d_qk, int d_v, int dtype, int causal) {
  if (d_qk == d_v) return fa_fwd_supported(d_qk, dtype, causal);
  if (causal != 0 && causal != 1) return 0;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_FP32) return 0;
  return (d_qk == 64 || d_qk == 128) && (d_v == 64 || d_v == 128);
}

}  // extern "C"

namespace {

// Argument checks shared by the entry points (no HIP call).
int check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
               int B, int H, int Nq, int Nk, int dk, int dv, float scale, int causal,
               int dtype) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || dk <= 0 || dv <= 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  const long long BH = (long long)B * H;
  if (BH > (1LL << 24)) return FA_ERR_INVALID_ARG;
  const long long nq_max = (Nq + 31) / 32;  // most query tiles any kernel uses
  if (nq_max * BH > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  if (BH * Nq > 0x7fffffffLL || BH * Nk > 0x7fffffffLL) return FA_ERR_INVALID_ARG;  // row ids
  if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16)
    return FA_ERR_UNSUPPORTED;
  if (!fa_fwd_gen_supported(dk, dv, dtype, causal)) return FA_ERR_UNSUPPORTED;
  // per-head byte offsets (plus one tile of slack) must fit the 32-bit
  // offsets of the buffer loads
  const long long elem = dtype == FA_DTYPE_FP32 ? 4 : 2;
  if (((long long)std::max(Nq, Nk) + 128) * std::max(dk, dv) * elem > 0x7fffffffLL)
    return FA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

template <class TT>
hipError_t launch_sp_dims(const void* q, const void* k, const void* v, void* o, float* lse,
                          const Shape& sh, int dk, int dv, float scale, bool c, hipStream_t st,
                          const SplitPlan& plan, void* ws) {
  if (dk == 64) return dv == 64 ? launch_sp<TT, 64, 64>(q, k, v, o, lse, sh, scale, c, st, plan, ws)
                                : launch_sp<TT, 64, 128>(q, k, v, o, lse, sh, scale, c, st, plan, ws);
  return dv == 64 ? launch_sp<TT, 128, 64>(q, k, v, o, lse, sh, scale, c, st, plan, ws)
                  : launch_sp<TT, 128, 128>(q, k, v, o, lse, sh, scale, c, st, plan, ws);
}

// dk, dv: head dims of Q/K and of V/O (a supported pair)
int dispatch(const void* q, const void* k, const void* v, void* o, float* lse, const Shape& sh,
             int dk, int dv, float scale, int causal, int dtype, const SplitPlan& plan, void* ws,
             void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const bool c = causal != 0;
  hipError_t e = hipSuccess;
  if (dtype == FA_DTYPE_BF16) {
    e = launch_sp_dims<Bf16>(q, k, v, o, lse, sh, dk, dv, scale, c, st, plan, ws);
  } else if (dtype == FA_DTYPE_FP16) {
    e = launch_sp_dims<F16>(q, k, v, o, lse, sh, dk, dv, scale, c, st, plan, ws);
  } else if (dk != dv) {
    e = dk == 64 ? launch32<64, 128, 1>(q, k, v, o, lse, sh, scale, c, st, plan, ws)
                 : launch32<128, 64, 1>(q, k, v, o, lse, sh, scale, c, st, plan, ws);
  } else {
    // Columns per wave: 64 wherever the waves then fit two per SIMD (about
    // 210 registers, against 340-360 with 128 columns), which at d = 256
    // and 512 is faster on every grid measured (4-31%).  At d = 128 one
    // wave of 128 columns needs no exchange of partial scores and is faster
    // on grids that fill the GPU (8-17%); two waves of 64 are 16-26% faster
    // on the small grids that take the key split.  d = 1024 keeps 128
    // columns: sixteen waves' K slices and partial scores would not fit in
    // the LDS.
    switch (dk) {
      case 64: e = launch32<64, 64, 1>(q, k, v, o, lse, sh, scale, c, st, plan, ws); break;
      case 128:
        e = plan.n_split > 1 ? launch32<64, 64, 2>(q, k, v, o, lse, sh, scale, c, st, plan, ws)
                             : launch32<128, 128, 1>(q, k, v, o, lse, sh, scale, c, st, plan, ws);
        break;
      case 256: e = launch32<64, 64, 4>(q, k, v, o, lse, sh, scale, c, st, plan, ws); break;
      case 512: e = launch32<64, 64, 8>(q, k, v, o, lse, sh, scale, c, st, plan, ws); break;
      default: e = launch32<128, 128, 8>(q, k, v, o, lse, sh, scale, c, st, plan, ws); break;
    }
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

size_t fa_fwd_gen_workspace_size(int B, int H, int Nq, int Nk, int d_qk, int d_v, int causal,
                                 int dtype) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || (causal != 0 && causal != 1)) return 0;
  if (!fa_fwd_gen_supported(d_qk, d_v, dtype, causal)) return 0;
  const long long BH = (long long)B * H;
  if (BH > (1LL << 24) || BH * Nq > 0x7fffffffLL || BH * Nk > 0x7fffffffLL) return 0;
  return plan_split(BH, Nq, Nk, d_qk, d_v, dtype).bytes;
}

size_t fa_fwd_ex_workspace_size(int B, int H, int Nq, int Nk, int d, int causal, int dtype) {
  return fa_fwd_gen_workspace_size(B, H, Nq, Nk, d, d, causal, dtype);
}

int fa_fwd_gen(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int Nq, int Nk, int d_qk, int d_v, float scale, int causal, int dtype,
               const int* k_len, const int* q_len, void* workspace, size_t workspace_bytes,
               void* stream) {
  if (int err = check_args(q, k, v, o, lse, B, H, Nq, Nk, d_qk, d_v, scale, causal, dtype);
      err != FA_OK)
    return err;
  if (((uintptr_t)k_len & 3u) != 0 || ((uintptr_t)q_len & 3u) != 0) return FA_ERR_UNSUPPORTED;
  const Shape sh{B * H, H, Nq, Nk, k_len, q_len};
  if (workspace == nullptr || workspace_bytes == 0)
    return dispatch(q, k, v, o, lse, sh, d_qk, d_v, scale, causal, dtype, SplitPlan{}, nullptr,
                    stream);
  const SplitPlan plan = plan_split((long long)B * H, Nq, Nk, d_qk, d_v, dtype);
  if (workspace_bytes < plan.bytes) return FA_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return FA_ERR_UNSUPPORTED;
  return dispatch(q, k, v, o, lse, sh, d_qk, d_v, scale, causal, dtype, plan, workspace, stream);
}

int fa_fwd_gen_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int Nq, int Nk, int d_qk, int d_v, float scale, int causal, int dtype,
                       const int* k_len, const int* q_len, void* stream) {
  if (int err = check_args(q, k, v, o, lse, B, H, Nq, Nk, d_qk, d_v, scale, causal, dtype);
      err != FA_OK)
    return err;
  if (((uintptr_t)k_len & 3u) != 0 || ((uintptr_t)q_len & 3u) != 0) return FA_ERR_UNSUPPORTED;
  const Shape sh{B * H, H, Nq, Nk, k_len, q_len};
  const SplitPlan plan = plan_split((long long)B * H, Nq, Nk, d_qk, d_v, dtype);
  if (plan.bytes > kScratchBytes) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (plan.n_split > 1 && scratch_address(&ws) != hipSuccess) return FA_ERR_HIP;
  return dispatch(q, k, v, o, lse, sh, d_qk, d_v, scale, causal, dtype, plan, ws, stream);
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int Nq, int Nk, int d, float scale, int causal, int dtype, const int* k_len,
              void* workspace, size_t workspace_bytes, void* stream) {
  return fa_fwd_gen(q, k, v, o, lse, B, H, Nq, Nk, d, d, scale, causal, dtype, k_len, nullptr,
                    workspace, workspace_bytes, stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int N, int d, float scale, int causal, int dtype, void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, N, N, d, scale, causal, dtype, nullptr, nullptr, 0,
                   stream);
}

size_t fa_fwd_workspace_size(int B, int H, int N, int d, int causal, int dtype) {
  return fa_fwd_ex_workspace_size(B, H, N, N, d, causal, dtype);
}

int fa_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int N, int d, float scale, int causal, int dtype, void* workspace,
              size_t workspace_bytes, void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, N, N, d, scale, causal, dtype, nullptr, workspace,
                   workspace_bytes, stream);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dim, dtype or alignment";
    case FA_ERR_HIP: return "HIP launch error";
    case FA_ERR_SCRATCH: return "problem needs more split scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int fa_version(void) { return 400; }

}  // extern "C"
