// fa_device.h -- device helpers shared by the forward and backward kernels of
// libfa.so (gfx950): vector types, constants, element-type traits for the
// 16-bit MFMA, cross-half reductions, the XCD-aware id remap, the LDS tile
// layout and the buffer loads that write straight to LDS; on the host, the
// device's compute-unit count.
#ifndef FA_DEVICE_H
#define FA_DEVICE_H

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>

namespace fa_dev {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The exponent reference of a row moves only when its max has grown past it
// by more than this many powers of two (probabilities stay <= 256).
constexpr float kLazyRescale = 8.0f;
// Word 3 of a raw buffer descriptor on gfx9-class GPUs: 32-bit data format,
// no swizzle, no stride; reads past num_records return zero.
constexpr int kBufferFlags = 0x00020000;
// s_waitcnt operand that waits for vmcnt = 0 only (expcnt 7, lgkmcnt 15)
constexpr int kWaitVmcnt0 = 0x0F70;
// ... and for vmcnt <= n (n < 64: low 4 bits in 3:0, high 2 bits in 15:14)
constexpr int wait_vmcnt(int n) { return kWaitVmcnt0 | (n & 15) | ((n >> 4) << 14); }

// ---------------------------------------------------------------------------
// element-type traits for the 16-bit kernels
struct Bf16 {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two fp32 -> one dword of two round-to-nearest-even bf16 (x in the low half)
  static __device__ __forceinline__ unsigned pack(float x, float y) {
    bf16x2 v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(unsigned, v);
  }
};
struct F16 {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack(float x, float y) {
    f16x2 v = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(unsigned, v);
  }
};

// {x[lane], x[lane ^ 32]} with the lower-half lane's value first in both
// halves, so a max or sum of the pair is bitwise identical across halves.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max(a, b, c) in one v_max3_f32.  fmaxf would first canonicalise each input
// (one extra instruction per score); the scores fed here are finite MFMA
// results, for which canonicalising changes nothing.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Map the hardware workgroup id to a work item.  Workgroups are handed to the
// 8 XCDs round-robin (id % 8); giving XCD x the contiguous range
// [x*W/8, (x+1)*W/8) of work items keeps the query tiles of one head -- which
// all stream the same K and V -- inside one XCD's L2.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  const int per = total / 8;
  if (wg >= per * 8) return wg;
  return (wg % 8) * per + wg / 8;
}

// ---------------------------------------------------------------------------
// LDS tile layout of the bf16 / fp16 kernels
//
// A K or V tile is 64 keys x D elements (2D bytes per key row), stored as
// 1 KB blocks of 16 rows x 4 sixteen-byte chunks: block (rg, cg) holds rows
// 16rg..16rg+15 and chunks 4cg..4cg+3, at byte (rg * D/32 + cg) * 1024.
//   K blocks are chunk-major inside (chunk ci, row ri at (ci*16 + ri)*16), so
//     the 16 rows one 16-lane group reads for an A operand are 16 consecutive
//     16-byte slots: no bank conflicts.
//   V blocks are row-major inside (row ri, chunk ci at (ri*4 + ci)*16), so a
//     16-lane group's ds_read_b64_tr_b16 (4 rows x 32 bytes) spans 256
//     distinct bytes.
// Each block is filled by one wave-wide buffer load that writes straight to
// LDS (lane L's 16 bytes land at block + 16L; rows past N read as zero), and
// every operand read is a lane constant plus a compile-time offset.
template <int D>
struct TileLayout {
  static constexpr int CG = D / 32;               // chunk groups per row
  static constexpr int BLOCKS = 4 * CG;           // 1 KB blocks per tile
  static constexpr int BYTES = BLOCKS * 1024;     // = 64 * D * 2
  // source element offset (within the tile's first row) of lane L in block `blk`
  static __device__ __forceinline__ int k_src(int blk, int L) {
    const int rg = blk / CG, cg = blk % CG;
    return (16 * rg + (L & 15)) * D + 8 * (4 * cg + (L >> 4));
  }
  static __device__ __forceinline__ int v_src(int blk, int L) {
    const int rg = blk / CG, cg = blk % CG;
    return (16 * rg + (L >> 2)) * D + 8 * (4 * cg + (L & 3));
  }
  // Swizzled row-major block (for a tile read both as rows and transposed):
  // row ri keeps its four chunks in slots 4ri .. 4ri+3, chunk ci in slot
  // 4ri + (ci ^ (ri / 4)).  Sixteen rows of one chunk (an A-operand read)
  // then fall in sixteen distinct 16-byte bank groups, while each row's 64
  // bytes stay together for the transposing reads.
  static __device__ __forceinline__ int s_src(int blk, int L) {
    const int rg = blk / CG, cg = blk % CG;
    const int ri = L >> 2, ci = (L & 3) ^ (ri >> 2);
    return (16 * rg + ri) * D + 8 * (4 * cg + ci);
  }
};

// A raw buffer descriptor as four SGPRs: 48-bit base, no stride,
// num_records bytes, reads past the end return zero.
__device__ __forceinline__ u32x4 buffer_desc(const void* base, unsigned bytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4{(unsigned)__builtin_amdgcn_readfirstlane((unsigned)a),
               (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xffffu),
               (unsigned)__builtin_amdgcn_readfirstlane(bytes), (unsigned)kBufferFlags};
}

// One wave-wide 16-byte-per-lane buffer load straight into LDS: lane L's
// bytes land at LDS byte address lds_addr + 16 L.  Written as inline asm so
// that the compiler does not wait for it at every LDS read and barrier: the
// caller waits (vmcnt) before the barrier that precedes the first read of
// the data.  The statement sets M0, the LDS base the load reads, and keeps
// one wait state between that SALU write of M0 and the load that reads it
// (the ISA asks for it before an LDS-writing memory instruction).  M0 is
// named as clobbered so that the compiler's hazard checks see the write, and
// keep a wait state before whatever follows (the compiler reserves M0 and
// warns about the clobber; nothing else in these kernels touches M0).
__device__ __forceinline__ void dma16(u32x4 desc, unsigned lds_addr, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voffset), "s"(desc)
               : "memory", "m0");
}

// This wave's share of one K (or V) tile: blocks wave, wave + NW, ... (the
// same count for every wave) of the tile whose first key row is key0.
template <int D, bool IS_V, int NW>
__device__ __forceinline__ void dma_tile(u32x4 desc, unsigned lds_tile, int key0, int wave,
                                         int lane) {
  using L = TileLayout<D>;
  static_assert(L::BLOCKS % NW == 0, "tile blocks split evenly over the waves");
#pragma unroll
  for (int i = 0; i < L::BLOCKS / NW; ++i) {
    const int blk = wave + i * NW;
    const int el = key0 * D + (IS_V ? L::v_src(blk, lane) : L::k_src(blk, lane));
    dma16(desc, lds_tile + blk * 1024, el * 2);
  }
}

// The same for a tile in the swizzled row-major layout (TileLayout::s_src).
template <int D, int NW>
__device__ __forceinline__ void dma_tile_swz(u32x4 desc, unsigned lds_tile, int wave, int lane) {
  using L = TileLayout<D>;
  static_assert(L::BLOCKS % NW == 0, "tile blocks split evenly over the waves");
#pragma unroll
  for (int i = 0; i < L::BLOCKS / NW; ++i) {
    const int blk = wave + i * NW;
    dma16(desc, lds_tile + blk * 1024, L::s_src(blk, lane) * 2);
  }
}

// host side
// Compute units of the current device, queried once per device.
inline hipError_t compute_units(int* cus) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && (*cus = cache[dev].load(std::memory_order_relaxed)) > 0)
    return hipSuccess;
  if (hipError_t e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
      e != hipSuccess)
    return e;
  if (*cus <= 0) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(*cus, std::memory_order_relaxed);
  return hipSuccess;
}

}  // namespace fa_dev

#endif  // FA_DEVICE_H
