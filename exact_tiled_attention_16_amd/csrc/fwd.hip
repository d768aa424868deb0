// Attention forward for gfx950: exact softmax attention computed tile by tile
// with an online softmax ("FlashAttention: Fast and Memory-Efficient Exact
// Attention with IO-Awareness", abstract: tiling between HBM and on-chip
// memory; FlashAttention-4 related-papers page, online-softmax snippet:
// running row maximum and normaliser; FlashAttention-3 review page, Appendix B
// fragment: exp2, row sum and output rescaling between the two products).
//
// Work unit: one workgroup = NW waves = 32*NW query rows of one (b, h).  Each
// wave keeps its 32 query rows in registers for the whole key loop.  Key and
// value tiles of BN rows stream through LDS, double buffered: tile j+1 is
// fetched from HBM into registers while tile j is consumed from LDS, then
// written to the other LDS buffer; one barrier per tile.
//
// Per tile and wave:
//   S^T = K_j Q^T on 32x32x16 matrix cores (keys are accumulator rows, the
//     wave's 32 queries are columns, so one lane owns one query row and its
//     row reductions are in-lane plus one exchange with the lane 32 away);
//   online softmax in the exp2 domain (scores pre-multiplied by
//     scale*log2(e)); probabilities rounded to the input type;
//   O^T += V_j^T P^T on matrix cores, with V read from LDS by transposed
//     16-bit reads so it can stay row-major; the accumulator of O^T again has
//     one query per lane, so the rescale by alpha is a per-lane multiply.
#include "common.h"
#include "kernels.h"

namespace fa {

namespace {

template <int D, int BN, int NW, bool CAUSAL, int DT>
__global__ void __launch_bounds__(NW * 64)
fwd_kernel(FwdArgs a) {
  using E = Elem<DT>;
  using v8 = typename E::v8;
  constexpr int NT = NW * 64;
  constexpr int BM = 32 * NW;
  constexpr int KSTR = D + 8;     // LDS row stride of K (elements): conflict-free 16 B reads
  constexpr int VSTR = D + 32;    // LDS row stride of V: conflict-free transposed reads
  constexpr int K_ELEMS = BN * KSTR;
  constexpr int STAGE = K_ELEMS + BN * VSTR;
  constexpr int CH_ROW = D / 8;   // 16-byte chunks per row
  constexpr int CH = BN * CH_ROW;
  static_assert(CH % NT == 0, "tile chunks must divide evenly over threads");
  constexpr int CPT = CH / NT;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
  FA_LDS uint16_t* lds = (FA_LDS uint16_t*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;   // which half of K slots / accumulator rows
  const int l32 = lane & 31;
  const int N = a.N;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / a.n_qtiles;
  int qt = logical % a.n_qtiles;
  if (CAUSAL) qt = a.n_qtiles - 1 - qt;  // longest key ranges first
  const int64_t base = (int64_t)bh * N * D;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q) + base;
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + base;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + base;

  const int q0 = qt * BM;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;

  // Q^T operand: lane holds query qrow, head-dim slots dc*16 + 8*hl + [0, 8).
  v8 qf[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    u32x4_t raw = {0u, 0u, 0u, 0u};
    if (qrow < N) raw = ld_global16(Q + (int64_t)qrow * D + dc * 16 + 8 * hl);
    qf[dc] = __builtin_bit_cast(v8, raw);
  }

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_run = -INFINITY;  // running max, log2 units
  float l_run = 0.f;        // this lane's share of the running normaliser

  u32x4_t kreg[CPT], vreg[CPT];
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      const int r = c / CH_ROW;
      const int col = (c % CH_ROW) * 8;
      const int key = t * BN + r;
      if (key < N) {
        kreg[i] = ld_global16(K + (int64_t)key * D + col);
        vreg[i] = ld_global16(V + (int64_t)key * D + col);
      } else {
        kreg[i] = u32x4_t{0u, 0u, 0u, 0u};
        vreg[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto stash = [&](int stage) {
    FA_LDS uint16_t* ks = lds + stage * STAGE;
    FA_LDS uint16_t* vs = ks + K_ELEMS;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      const int r = c / CH_ROW;
      const int col = (c % CH_ROW) * 8;
      st_lds16(ks + r * KSTR + col, kreg[i]);
      st_lds16(vs + r * VSTR + col, vreg[i]);
    }
  };

  // Lane roles in the transposed V read (see common.h).
  const int tr_row = (lane & 15) >> 2;              // e: row within a group of 4
  const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;

  fetch(0);
  stash(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < ntiles) fetch(t + 1);

    const int kbase = t * BN;
    const bool active = (qw0 < N) && (!CAUSAL || kbase <= qw0 + 31);
    if (active) {
      const FA_LDS uint16_t* ks = lds + stage * STAGE;
      const FA_LDS uint16_t* vs = ks + K_ELEMS;

      f32x16_t sacc[BN / 32];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
          const v8 kf = __builtin_bit_cast(
              v8, ld_lds16(ks + (kb * 32 + l32) * KSTR + dc * 16 + 8 * hl));
          sacc[kb] = E::mfma(kf, qf[dc], sacc[kb]);
        }
      }

      // Scale to log2 units, mask, running max.
      const bool need_mask = (kbase + BN > N) || (CAUSAL && kbase + BN - 1 > qw0);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float s = sacc[kb][r] * a.scale_log2;
          if (need_mask) {
            const int key = kbase + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (key >= N || (CAUSAL && key > qrow)) s = -INFINITY;
          }
          sacc[kb][r] = s;
          mx = fmaxf(mx, s);
        }
      }
      mx = max_halves(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(sacc[kb][r] - m_use);
          sacc[kb][r] = p;
          psum += p;
        }
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;

      // O^T += V^T P^T, 16 keys per instruction.  Chunk c of the tile uses
      // accumulator registers 8*(c%2)..+7 of block c/2, i.e. keys
      // 16c + 8*(s/4) + 4*hl + s%4 for slot s; the V operand is read for the
      // same keys.
#pragma unroll
      for (int c = 0; c < BN / 16; ++c) {
        const f32x16_t& sb = sacc[c >> 1];
        const int r0 = 8 * (c & 1);
        u32x4_t pw;
        pw[0] = E::pack2(sb[r0 + 0], sb[r0 + 1]);
        pw[1] = E::pack2(sb[r0 + 2], sb[r0 + 3]);
        pw[2] = E::pack2(sb[r0 + 4], sb[r0 + 5]);
        pw[3] = E::pack2(sb[r0 + 6], sb[r0 + 7]);
        const v8 pf = __builtin_bit_cast(v8, pw);
        const FA_LDS uint16_t* vrow0 = vs + (c * 16 + 4 * hl + tr_row) * VSTR + tr_col;
        const FA_LDS uint16_t* vrow1 = vrow0 + 8 * VSTR;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const s16x4_t lo = ld_lds_tr16(vrow0 + db * 32);
          const s16x4_t hi = ld_lds_tr16(vrow1 + db * 32);
          const v8 vf = __builtin_bit_cast(
              v8, u32x4_t{__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                          __builtin_bit_cast(u32x2_t, hi)[0], __builtin_bit_cast(u32x2_t, hi)[1]});
          oacc[db] = E::mfma(vf, pf, oacc[db]);
        }
      }
    }

    if (t + 1 < ntiles) stash(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: normalise, round, store; LSE in natural log.
  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + base + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2_t w;
        w[0] = E::pack2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
        w[1] = E::pack2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2_t*>(orow + db * 32 + 8 * g + 4 * hl) = w;
      }
    }
    if (hl == 0 && a.lse != nullptr)
      a.lse[(int64_t)bh * N + qrow] = m_run * kLn2 + __logf(l_tot);
  }
}

template <int D, int BN, int NW, bool CAUSAL, int DT>
hipError_t launch_one(const FwdArgs& a, int BH, hipStream_t stream) {
  constexpr int BM = 32 * NW;
  FwdArgs args = a;
  args.n_qtiles = (a.N + BM - 1) / BM;
  const int64_t grid = (int64_t)args.n_qtiles * BH;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_kernel<D, BN, NW, CAUSAL, DT>), dim3((unsigned)grid), dim3(NW * 64),
                     0, stream, args);
  return hipGetLastError();
}

template <int D, int BN, int NW, int DT>
hipError_t launch_causal(const FwdArgs& a, int BH, bool causal, hipStream_t s) {
  return causal ? launch_one<D, BN, NW, true, DT>(a, BH, s)
                : launch_one<D, BN, NW, false, DT>(a, BH, s);
}

template <int DT>
hipError_t launch_dtype(const FwdArgs& a, int BH, int d, bool causal, hipStream_t s) {
  switch (d) {
    case 64: return launch_causal<64, 64, 8, DT>(a, BH, causal, s);
    case 128: return launch_causal<128, 64, 8, DT>(a, BH, causal, s);
    case 256: return launch_causal<256, 32, 4, DT>(a, BH, causal, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int B, int H, int d, int dtype, bool causal,
                      hipStream_t stream) {
  const int BH = B * H;
  return dtype == 0 ? launch_dtype<0>(a, BH, d, causal, stream)
                    : launch_dtype<1>(a, BH, d, causal, stream);
}

}  // namespace fa
