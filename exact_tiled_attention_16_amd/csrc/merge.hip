// Log-sum-exp merge of partial attention results (gfx950).
//
// Attention over a key set that is split into parts can be computed part by
// part: each part p gives O_p (normalised over its own keys) and its
// log-sum-exp L_p, and the whole is
//     L = log sum_p exp(L_p),    O = sum_p exp(L_p - L) O_p,
// the same rescaling that the online softmax applies from one key tile to the
// next (FlashAttention-4 related-papers page, online-softmax snippet: a
// running maximum and normaliser).  The reference list of "FlashAttention-3:
// Fast and Accurate Attention with Asynchrony and Low-precision" names Ring
// Attention and Lean Attention, which combine per-device and per-split
// partial results this way.  A part with no visible key has L_p = -inf and
// weight 0; a row with no visible key anywhere gets O = 0 and L = -inf.
//
// Memory-bound: one pass over the partial outputs.  D/4 lanes per row, each
// with a 16-byte load per part; the part weights are recomputed per lane.
#include "common.h"
#include "kernels.h"

namespace fa {

namespace {

template <int D, int DT>
__global__ void __launch_bounds__(256) merge_kernel(MergeArgs a) {
  using E = Elem<DT>;
  constexpr int TPR = D / 4;         // lanes per row
  constexpr int RPB = 256 / TPR;     // rows per workgroup
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (row >= a.rows) return;
  const int S = a.n_parts;
  float m = -INFINITY;
  for (int p = 0; p < S; ++p) m = fmaxf(m, a.lse_parts[p * a.rows + row]);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int p = 0; p < S; ++p) {
      const float w = fast_exp2((a.lse_parts[p * a.rows + row] - m) * kLog2e);
      if (w > 0.f) {  // empty parts may hold anything in O
        wsum += w;
        acc += w * *reinterpret_cast<const f32x4_t*>(a.o_parts + (p * a.rows + row) * D + 4 * c);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  u32x2_t out;
  out[0] = E::pack2(acc[0] * inv, acc[1] * inv);
  out[1] = E::pack2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.o) + row * D + 4 * c) = out;
  if (c == 0 && a.lse != nullptr) a.lse[row] = m + __logf(wsum);  // -inf when empty
}

template <int DT>
hipError_t launch_dt(const MergeArgs& a, int d, hipStream_t s) {
  auto go = [&](auto kern, int tpr) {
    const int64_t blocks = (a.rows * tpr + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
  };
  switch (d) {
    case 64: return go(merge_kernel<64, DT>, 16);
    case 128: return go(merge_kernel<128, DT>, 32);
    case 256: return go(merge_kernel<256, DT>, 64);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int d, int dtype, hipStream_t stream) {
  return dtype == 0 ? launch_dt<0>(a, d, stream) : launch_dt<1>(a, d, stream);
}

}  // namespace fa
