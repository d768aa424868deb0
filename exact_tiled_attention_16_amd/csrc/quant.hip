// FP8 (e4m3) quantisation with block scales and optional incoherent
// processing ("FlashAttention-3: Fast and Accurate Attention with Asynchrony
// and Low-precision", abstract: block quantization and incoherent processing;
// its reference list points to Hadamard-based incoherence).
//
//   x' = H_d (s o x)  when signs are given (H_d: unnormalised Sylvester
//        Hadamard matrix, applied by the fast Walsh-Hadamard transform in
//        fp32 with half-widths 1, 2, ..., d/2 in that order; each level maps
//        the pair (x[i], x[i+h]), i & h == 0, to (x[i] + x[i+h], x[i] - x[i+h]))
//   scale = amax(|x'| over the block) / 448   (1 when the amax is 0), or in
//           the power-of-two mode that value rounded up to a power of two
//   code  = e4m3_rne(clamp(x' / scale, -448, 448)),  stored = scale * scale_mul
//
// A block is FA_FP8_BLOCK = 128 rows of one (b, h), all d columns.  Each row is
// held by d/16 consecutive lanes, 16 elements per lane; butterflies of
// half-width < 16 stay inside a lane, wider ones pair lane t with lane
// t ^ (h/16).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace fa {

namespace {

constexpr int kBlock = 128;
constexpr int kEl = 16;  // elements per lane: 16 consecutive of one row
// Threads per workgroup: one per 16-element chunk of the block, at most 1024.
// (Workgroups of 256 or 512 threads, with more chunks per thread, measured
// faster only for some modes and head dimensions.)
template <int D>
constexpr int quant_threads() {
  return kBlock * (D / kEl) < 1024 ? kBlock * (D / kEl) : 1024;
}
constexpr int kReduceThreads = 1024;

template <int DT> __device__ __forceinline__ float elem_to_f32(uint32_t bits16);
template <> __device__ __forceinline__ float elem_to_f32<0>(uint32_t b) {
  return __uint_as_float(b << 16);
}
template <> __device__ __forceinline__ float elem_to_f32<1>(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Value of the lane `hl` away inside a 16-lane row (hl = 4, 8) by data
// parallel row shifts (no LDS traffic): a lane whose bit hl is clear reads
// lane + hl, one whose bit is set reads lane - hl.
template <int HL>
__device__ __forceinline__ float lane_xor_in_row(float v, bool upper) {
  const int b = __builtin_bit_cast(int, v);
  const int from_above = __builtin_amdgcn_update_dpp(0, b, 0x100 + HL, 0xF, 0xF, false);
  const int from_below = __builtin_amdgcn_update_dpp(0, b, 0x110 + HL, 0xF, 0xF, false);
  return __builtin_bit_cast(float, upper ? from_below : from_above);
}
// Value of the lane `hl` away for hl = 1, 2: a quad permutation.
template <int HL>
__device__ __forceinline__ float lane_xor_in_quad(float v) {
  constexpr int ctrl = HL == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF,
                                                        0xF, false));
}

// Smallest power of two >= s for a positive finite fp32 s, from its bits: a
// power of two keeps its value; a normal value goes to the next exponent; a
// subnormal one to the next power of two above its mantissa (2^-126 at most).
__device__ __forceinline__ float pow2_ceil_f32(float s) {
  const uint32_t b = __float_as_uint(s);
  const uint32_t man = b & 0x007fffffu;
  const uint32_t ex = b & 0x7f800000u;
  if (ex != 0) return man == 0 ? s : __uint_as_float(ex + 0x00800000u);
  if ((man & (man - 1u)) == 0) return s;
  return __uint_as_float(1u << (32 - __builtin_clz(man)));
}

// MODE 0: block scales, quantise.  MODE 1: write the block amax only.
// MODE 2: quantise with the amax found in scales[slot] (per-tensor mode).
// MODE 3: block scales rounded up to a power of two, quantise.
template <int D, int DT, int MODE>
__global__ void __launch_bounds__(quant_threads<D>())
quant_kernel(QuantArgs a) {
  constexpr int NT = quant_threads<D>();
  constexpr int TPR = D / kEl;             // lanes per row (4, 8 or 16)
  constexpr int TASKS = kBlock * TPR;      // 16-element chunks per block
  static_assert(TASKS % NT == 0, "");
  constexpr int CPT = TASKS / NT;
  static_assert(TPR >= 2 && TPR <= 16, "cross-lane levels stay inside a 16-lane row");

  const int tid = threadIdx.x;
  const int slot = blockIdx.x;             // (b*H + h) * nblk + blk
  const int bh = slot / a.nblk;
  const int blk = slot % a.nblk;
  const int N = a.N;
  const int row0 = blk * kBlock;
  const int64_t base = (int64_t)bh * N * D;

  float x[CPT][kEl];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + i * NT;
    const int r = c / TPR;
    const int col = (c % TPR) * kEl;
    const int row = row0 + r;
    u32x4_t raw[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    if (row < N) {
      const uint16_t* src = static_cast<const uint16_t*>(a.x) + base + (int64_t)row * D + col;
      raw[0] = ld_global16(src);
      raw[1] = ld_global16(src + 8);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[i][2 * j] = elem_to_f32<DT>(raw[j >> 2][j & 3] & 0xffffu);
      x[i][2 * j + 1] = elem_to_f32<DT>(raw[j >> 2][j & 3] >> 16);
    }
    if (a.signs != nullptr) {
#pragma unroll
      for (int e = 0; e < kEl; ++e) x[i][e] *= a.signs[col + e];
      // Half-widths 1, 2, 4, 8: inside the lane.
#pragma unroll
      for (int h = 1; h < kEl; h <<= 1) {
#pragma unroll
        for (int e = 0; e < kEl; ++e) {
          if ((e & h) == 0) {
            const float lo = x[i][e], hi = x[i][e + h];
            x[i][e] = lo + hi;
            x[i][e + h] = lo - hi;
          }
        }
      }
      // Half-widths 16 .. D/2: partner lane t ^ (h/16) of the row's lanes, by
      // data-parallel moves.  The lower lane of a pair keeps mine + other,
      // the upper one other - mine; for the quad permutations as one fused
      // multiply-add with +-1, which rounds exactly like the sum or the
      // difference.
      const int t = c % TPR;
      auto level = [&](auto hl_tag) {
        constexpr int HL = decltype(hl_tag)::value;
        const bool upper = (t & HL) != 0;
        const float sgn = upper ? -1.0f : 1.0f;
#pragma unroll
        for (int e = 0; e < kEl; ++e) {
          const float mine = x[i][e];
          if constexpr (HL < 4) {
            x[i][e] = fmaf(sgn, mine, lane_xor_in_quad<HL>(mine));
          } else {
            const float other = lane_xor_in_row<HL>(mine, upper);
            x[i][e] = upper ? (other - mine) : (mine + other);
          }
        }
      };
      level(std::integral_constant<int, 1>{});
      level(std::integral_constant<int, 2>{});
      if constexpr (TPR > 4) level(std::integral_constant<int, 4>{});
      if constexpr (TPR > 8) level(std::integral_constant<int, 8>{});
    }
    if (row < N) {
#pragma unroll
      for (int e = 0; e < kEl; ++e) amax = fmaxf(amax, fabsf(x[i][e]));
    }
  }

  float block_amax;
  if (MODE == 2) {
    block_amax = a.scales[slot];
  } else {
    // Workgroup max: wave reduction, then across the waves through LDS.
    __shared__ float red[NT / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    block_amax = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) block_amax = fmaxf(block_amax, red[w]);
    if (MODE == 1) {
      if (tid == 0) a.scales[slot] = block_amax;
      return;
    }
  }

  float scale = block_amax > 0.f ? block_amax / 448.0f : 1.0f;
  if constexpr (MODE == 3) scale = pow2_ceil_f32(scale);  // x' / scale then exact
  // x / scale correctly rounded (IEEE division) from the correctly rounded
  // reciprocal and one residual step: for q0 within 1 ulp of x / scale and
  // rinv within half an ulp of 1 / scale, q0 + fma(-q0, scale, x) * rinv is
  // the correctly rounded quotient (Markstein, IBM J. Res. Dev. 34(1), 1990)
  // outside the subnormal range, where every code is zero anyway.  The
  // quotient has the sign of x' (scale > 0); the residual step alone would
  // turn -0 into +0, so the sign is put back.
  const float rinv = 1.0f / scale;
  auto quotient = [&](float v) {
    const float q0 = v * rinv;
    return __builtin_copysignf(fmaf(fmaf(-q0, scale, v), rinv, q0), v);
  };
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + i * NT;
    const int r = c / TPR;
    const int col = (c % TPR) * kEl;
    const int row = row0 + r;
    if (row >= N) continue;
    u32x4_t out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        y[e] = fminf(fmaxf(quotient(x[i][4 * j + e]), -448.0f), 448.0f);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
      out[j] = (uint32_t)w;
    }
    *reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(a.x8) + base + (int64_t)row * D + col) = out;
  }
  if (MODE == 2) __syncthreads();  // every lane has read scales[slot]
  if (tid == 0) a.scales[slot] = scale * a.scale_mul;
}

// Max over n values, written back to all n (one workgroup).
__global__ void __launch_bounds__(kReduceThreads)
reduce_max_kernel(float* v, int n) {
  __shared__ float red[kReduceThreads / 64];
  float m = 0.f;
  for (int i = threadIdx.x; i < n; i += kReduceThreads) m = fmaxf(m, v[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kReduceThreads / 64; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kReduceThreads) v[i] = m;
}

template <int D, int DT>
hipError_t launch_d(const QuantArgs& a, int BH, int mode, hipStream_t s) {
  const int64_t grid = (int64_t)BH * a.nblk;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (mode != 1) {
    if (mode == 2)
      hipLaunchKernelGGL((quant_kernel<D, DT, 3>), dim3((unsigned)grid), dim3(quant_threads<D>()),
                         0, s, a);
    else
      hipLaunchKernelGGL((quant_kernel<D, DT, 0>), dim3((unsigned)grid), dim3(quant_threads<D>()),
                         0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((quant_kernel<D, DT, 1>), dim3((unsigned)grid), dim3(quant_threads<D>()), 0, s,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reduce_max_kernel, dim3(1), dim3(kReduceThreads), 0, s, a.scales, (int)grid);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((quant_kernel<D, DT, 2>), dim3((unsigned)grid), dim3(quant_threads<D>()), 0, s,
                     a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dtype(const QuantArgs& a, int BH, int d, int mode, hipStream_t s) {
  switch (d) {
    case 64: return launch_d<64, DT>(a, BH, mode, s);
    case 128: return launch_d<128, DT>(a, BH, mode, s);
    case 256: return launch_d<256, DT>(a, BH, mode, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_quant_fp8(const QuantArgs& a, int B, int H, int d, int dtype, int mode,
                            hipStream_t stream) {
  const int BH = B * H;
  return dtype == 0 ? launch_dtype<0>(a, BH, d, mode, stream)
                    : launch_dtype<1>(a, BH, d, mode, stream);
}

}  // namespace fa
