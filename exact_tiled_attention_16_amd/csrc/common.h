// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Matrix-core layout facts used throughout (v_mfma_f32_32x32x16_{bf16,f16}
// and v_mfma_f32_32x32x64_f8f6f4, wave64):
//   * operand A (M x K): lane l holds row l%32 and eight (fp8: thirty-two)
//     K-consecutive elements; operand B (K x N): lane l holds column l%32 and
//     the same K slots.  Lanes l and l+32 hold the two halves of K.  Any
//     permutation of K applied identically to A and B leaves the product
//     unchanged, which the kernels use to pick convenient key orders.
//   * accumulator (32 x 32, 16 floats per lane): register r of lane l holds
//     row 8*(r/4) + 4*(l/32) + r%4 and column l%32.
//   * ds_read_b64_tr_b16: inside each 16-lane group, lane j receives, as its
//     element e (0..3), element j%4 of the 8-byte chunk addressed by lane
//     4*e + j/4 of the same group.  With 4 x 4 lanes addressing rows r0+e and
//     column groups c0+4*(j/4) of a row-major tile, lane j gets the column
//     c0 + j of four consecutive rows: a transposed 16-bit read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- 16-bit types

// Element-type traits: DT 0 = bf16, 1 = fp16.
template <int DT> struct Elem;

template <> struct Elem<0> {
  typedef bf16x8_t v8;
  static __device__ __forceinline__ f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Two fp32 values -> packed pair, round to nearest even.
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  }
};

template <> struct Elem<1> {
  typedef f16x8_t v8;
  static __device__ __forceinline__ f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  }
};

// ---------------------------------------------------------------- cross-lane

// Combine a per-lane value with the one held 32 lanes away (same query row in
// the accumulator layout).  permlane32_swap(x, x) returns the low half of x in
// both halves of the first result and the high half in both of the second.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// True in every lane when the predicate holds in at least one lane.
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Lazy softmax reference: the running row maximum used as the exp2 reference
// is raised only when one lane's partial row sum of a tile's probabilities
// (computed against the current reference) exceeds kLazySum, or is not
// finite.  Below the bound every probability is at most kLazySum, and the
// reference never exceeds the running maximum, so the result stays exact and
// needs no per-tile maximum.
constexpr float kLazySum = 1024.0f;

// ---------------------------------------------------------------- memory

__device__ __forceinline__ u32x4_t ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ u32x4_t ld_lds16(const FA_LDS void* p) {
  return *reinterpret_cast<const FA_LDS u32x4_t*>(p);
}

__device__ __forceinline__ s16x4_t ld_lds_tr16(const FA_LDS void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<FA_LDS s16x4_t*>(const_cast<FA_LDS void*>(p)));
}

// Buffer resource for `bytes` bytes at `base` (wave-uniform): base address in
// dwords 0-1 (stride 0), byte count in dword 2, format word in dword 3.
// Loads through it at offsets at or past `bytes` return zeros instead of
// touching memory.  The fields pass through readfirstlane so that the
// descriptor lives in scalar registers.
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  u32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) & 0xffffu;
  r[2] = __builtin_amdgcn_readfirstlane((uint32_t)bytes);
  r[3] = 0x00020000u;
  return r;
}

// Buffer -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane i
// reads `voff` bytes into the resource and writes bytes [16 i, 16 i + 16) of the
// 1 KiB block at `lds_block` (wave-uniform, placed in M0 by the compiler).  Out-of-range lanes
// write zeros.  Issued as inline assembly on purpose: the compiler cannot
// prove that later LDS reads miss the copy's destination and would otherwise
// wait for every copy to land right after issuing it.  Completion is
// therefore tracked only by the explicit vector-memory waits below, which
// also order the compiler's own loads correctly (vector-memory operations
// complete in issue order).
// The statement also supplies its own wait states: a vector-memory
// instruction reading an SGPR that a vector ALU instruction wrote (the
// descriptor fields pass through v_readfirstlane, or come back from a spill
// by v_readlane) needs five, and an LDS-DMA load after a scalar write of M0
// needs one.  The compiler inserts these before its own memory instructions
// but cannot see into an asm statement, so without them the load may take a
// stale base address or M0.  s_nop 4 gives five; NOP = 0 (one) serves the
// later copies of a batch that share the first one's descriptor.
template <int NOP = 4>
__device__ __forceinline__ void dma16_buf(u32x4_t r, uint32_t voff, FA_LDS void* lds_block) {
  static_assert(NOP == 0 || NOP == 4, "wait states");
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_block);
  if constexpr (NOP == 4)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 : : "v"(voff), "s"(r), "{m0}"(m0) : "memory");
  else
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 : : "v"(voff), "s"(r), "{m0}"(m0) : "memory");
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Waits until at most PENDING of this wave's vector-memory operations (DMA
// copies included) are outstanding, then a workgroup barrier makes every
// wave's completed copies visible.  No memory fence: the asm statements only
// keep the compiler from moving LDS accesses across.
template <int PENDING>
__device__ __forceinline__ void dma_sync() {
  wait_vmcnt<PENDING>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- scheduling

// Persistent heaviest-first (longest-processing-time) schedule over
// nheads x ntiles work units whose cost depends only on their tile's rank:
// rank 0 is the heaviest.  The grid's G workgroups take the units, heaviest
// rank first across all heads, in rounds of G whose direction alternates
// (round r: workgroup w takes unit r G + w when r is even, r G + G - 1 - w
// when odd), so that each workgroup's heavy and light units pair up and all
// end with nearly the same total.  With `pin` (heads and grid both split
// evenly over the 8 XCDs) each XCD keeps its own heads: head x + 8 i runs on
// XCD x (workgroups w with w % 8 == x), so a head's operands stay in one L2.
// run(head, rank, next_head, next_rank) is called once per unit of this
// workgroup, with the workgroup's following unit (-1, -1 after its last):
// unit indices grow with the round, so the next one is the next round's.
template <typename F>
__device__ __forceinline__ void lpt_units(int ntiles, int nheads, bool pin, F&& run) {
  constexpr int kXcd = 8;
  const int w = blockIdx.x;
  const int G = gridDim.x;
  int v, g, heads, x;
  if (pin) {
    x = w % kXcd;
    v = w / kXcd;
    g = G / kXcd;
    heads = nheads / kXcd;
  } else {
    x = 0;
    v = w;
    g = G;
    heads = nheads;
  }
  const int units = heads * ntiles;
  auto unit_of = [&](int r) { return r * g + ((r & 1) ? g - 1 - v : v); };
  auto head_of = [&](int k) { return pin ? x + kXcd * (k % heads) : k % heads; };
  for (int r = 0; r * g < units; ++r) {
    const int k = unit_of(r);
    if (k < units) {
      const int kn = unit_of(r + 1);
      const bool more = kn < units;  // (one call site: the unit is inlined once)
      run(head_of(k), k / heads, more ? head_of(kn) : -1, more ? kn / heads : -1);
    }
  }
}

// Workgroups of `Kernel` (with `threads` threads) resident at once on the
// current device, cached per device and kernel (the kernel is a template
// argument, so each instantiation has its own cache: kernels of one
// signature may differ in registers and LDS); 0 if it cannot be queried.
template <auto Kernel>
int resident_slots(int threads) {
  constexpr int kMaxDev = 64;
  static int cache[kMaxDev];  // written once per device with the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDev && __atomic_load_n(&cache[dev], __ATOMIC_RELAXED) > 0)
    return __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, Kernel, threads, 0) != hipSuccess)
    return 0;
  const int slots = cus * per_cu;
  if (dev < kMaxDev) __atomic_store_n(&cache[dev], slots, __ATOMIC_RELAXED);
  return slots;
}

// MI355X dispatches consecutive workgroup ids round-robin over its 8 XCDs,
// each with a private L2.  Remap so that a contiguous range of logical ids
// (the query tiles of one head, which stream the same K/V) runs on one XCD.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  constexpr int kXcd = 8;
  const int full = (nwg / kXcd) * kXcd;
  if (bid >= full) return bid;
  return (bid % kXcd) * (nwg / kXcd) + bid / kXcd;
}

}  // namespace fa
