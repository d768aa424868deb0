// Attention backward for gfx950, by recomputation from the saved log-sum-exp.
//
// The pages state that FlashAttention trains models (so a backward exists)
// but do not spell it out ("FlashAttention: Fast and Memory-Efficient Exact
// Attention with IO-Awareness", abstract).  What is computed is the gradient
// of <dO, O> with the softmax Jacobian:
//     P = exp(scale * Q K^T - LSE),  D = rowsum(dO o O),
//     dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
//     dK = scale * dS^T Q,  dQ = scale * dS K.
//
// Kernels:
//   bwd_pre_kernel  D = rowsum(dO o O) in fp32 (O is the stored forward
//                   output) and dQ := 0.
//   bwd_kernel      one workgroup per (b, h, tile of 32*NW keys); each wave
//                   owns 32 keys and keeps K and V rows for them in registers
//                   and dK, dV accumulators for them in registers.  Query
//                   tiles of BQ rows (Q, dO, LSE, D) stream through LDS,
//                   double buffered.  Per query tile and wave:
//                     S = Q K^T and dP = dO V^T on 32x32x16 matrix cores with
//                       keys as accumulator columns (one key per lane);
//                     P, dS in fp32 (scale folded into dS);
//                     dV^T += dO^T P and dK^T += Q^T dS, with dO and Q read
//                       from LDS by transposed 16-bit reads;
//                     dS^T goes to LDS; after the barrier the workgroup forms
//                       dQ_tile = dS K (both operands by transposed reads) and
//                       adds it to the fp32 dQ with hardware float atomics.
#include "common.h"
#include "kernels.h"

namespace fa {

namespace {

template <int DT> __device__ __forceinline__ float to_f32(uint16_t x);
template <> __device__ __forceinline__ float to_f32<0>(uint16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}
template <> __device__ __forceinline__ float to_f32<1>(uint16_t x) {
  return (float)__builtin_bit_cast(_Float16, x);
}

// D[row] = sum_c dO[row][c] * O[row][c]; dQ[row][:] = 0.  D/8 threads per row.
template <int D, int DT>
__global__ void __launch_bounds__(256)
bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
               float* __restrict__ Dsum, float* __restrict__ dQ, int64_t rows) {
  constexpr int TPR = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / TPR;
  const int c = (int)(gid % TPR);
  float acc = 0.f;
  if (row < rows) {
    const u32x4_t o = ld_global16(O + row * D + c * 8);
    const u32x4_t g = ld_global16(dO + row * D + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += to_f32<DT>((uint16_t)(o[i] & 0xffff)) * to_f32<DT>((uint16_t)(g[i] & 0xffff));
      acc += to_f32<DT>((uint16_t)(o[i] >> 16)) * to_f32<DT>((uint16_t)(g[i] >> 16));
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (row < rows) {
    if (c == 0) Dsum[row] = acc;
    f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4_t*>(dQ + row * D + c * 8) = z;
    *reinterpret_cast<f32x4_t*>(dQ + row * D + c * 8 + 4) = z;
  }
}

template <int D, int NW, int BQ, bool CAUSAL, int DT>
__global__ void __launch_bounds__(NW * 64)
bwd_kernel(BwdArgs a) {
  using E = Elem<DT>;
  using v8 = typename E::v8;
  constexpr int NT = NW * 64;
  constexpr int BKV = 32 * NW;       // keys per workgroup
  constexpr int KSTR = D + 32;       // K tile rows: transposed reads
  constexpr int QSTR = D + 8;        // Q / dO rows: 16-byte reads and transposed reads
  constexpr int SSTR = BQ + 8;       // dS^T rows (one per key)
  constexpr int Q_ELEMS = BQ * QSTR;
  constexpr int S_ELEMS = BKV * SSTR;
  constexpr int CH_ROW = D / 8;
  constexpr int QCH = BQ * CH_ROW;   // 16-byte chunks per Q (or dO) tile
  static_assert(QCH % NT == 0, "Q tile chunks must divide evenly");
  constexpr int CPT = QCH / NT;
  static_assert(BQ % 32 == 0 && BQ <= NT, "query tile");
  constexpr int NQB = BQ / 32;
  constexpr int NDB = D / 32;

  __shared__ __attribute__((aligned(16))) uint16_t smem_k[BKV * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t smem_q[2][Q_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t smem_do[2][Q_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t smem_ds[2][S_ELEMS];
  __shared__ __attribute__((aligned(16))) float smem_lse[2][BQ];
  __shared__ __attribute__((aligned(16))) float smem_dd[2][BQ];
  FA_LDS uint16_t* ks = (FA_LDS uint16_t*)smem_k;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int N = a.N;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / a.n_ktiles;
  const int kt = logical % a.n_ktiles;  // tile 0 (most query tiles when causal) first
  const int64_t base = (int64_t)bh * N * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.q) + base;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + base;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v) + base;
  const uint16_t* dOg = static_cast<const uint16_t*>(a.dout) + base;
  const float* lseg = a.lse + (int64_t)bh * N;
  const float* ddg = a.dsum + (int64_t)bh * N;
  float* dQg = a.dq + base;

  const int k0 = kt * BKV;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;

  // K and V rows of this lane's key as matrix-core B operands (head-dim slots
  // dc*16 + 8*hl + [0, 8)); the whole key tile of K also goes to LDS for dQ.
  v8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    u32x4_t rk = {0u, 0u, 0u, 0u}, rv = {0u, 0u, 0u, 0u};
    if (key < N) {
      rk = ld_global16(Kg + (int64_t)key * D + dc * 16 + 8 * hl);
      rv = ld_global16(Vg + (int64_t)key * D + dc * 16 + 8 * hl);
    }
    kf[dc] = __builtin_bit_cast(v8, rk);
    vf[dc] = __builtin_bit_cast(v8, rv);
  }
  for (int c = tid; c < BKV * CH_ROW; c += NT) {
    const int r = c / CH_ROW;
    const int col = (c % CH_ROW) * 8;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (k0 + r < N) v = ld_global16(Kg + (int64_t)(k0 + r) * D + col);
    st_lds16(ks + r * KSTR + col, v);
  }

  f32x16_t dvacc[NDB], dkacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dvacc[i][r] = 0.f;
      dkacc[i][r] = 0.f;
    }

  const int nq = (N + BQ - 1) / BQ;
  const int i0 = CAUSAL ? (k0 / BQ) : 0;

  u32x4_t qreg[CPT], oreg[CPT];
  float lreg = 0.f, dreg = 0.f;
  auto fetch = [&](int it) {
    const int q0 = it * BQ;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      const int r = c / CH_ROW;
      const int col = (c % CH_ROW) * 8;
      if (q0 + r < N) {
        qreg[i] = ld_global16(Qg + (int64_t)(q0 + r) * D + col);
        oreg[i] = ld_global16(dOg + (int64_t)(q0 + r) * D + col);
      } else {
        qreg[i] = u32x4_t{0u, 0u, 0u, 0u};
        oreg[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    if (tid < BQ) {
      const bool ok = q0 + tid < N;
      lreg = ok ? lseg[q0 + tid] * kLog2e : INFINITY;  // rows past N get P = 0
      dreg = ok ? ddg[q0 + tid] : 0.f;
    }
  };
  auto stash = [&](int st) {
    FA_LDS uint16_t* qs = (FA_LDS uint16_t*)smem_q[st];
    FA_LDS uint16_t* os = (FA_LDS uint16_t*)smem_do[st];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      const int r = c / CH_ROW;
      const int col = (c % CH_ROW) * 8;
      st_lds16(qs + r * QSTR + col, qreg[i]);
      st_lds16(os + r * QSTR + col, oreg[i]);
    }
    if (tid < BQ) {
      smem_lse[st][tid] = lreg;
      smem_dd[st][tid] = dreg;
    }
  };

  const int tr_row = (lane & 15) >> 2;
  const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;

  if (i0 < nq) {
    fetch(i0);
    stash(0);
  }
  __syncthreads();

  for (int it = i0; it < nq; ++it) {
    const int st = (it - i0) & 1;
    if (it + 1 < nq) fetch(it + 1);
    const int q0 = it * BQ;
    const FA_LDS uint16_t* qs = (const FA_LDS uint16_t*)smem_q[st];
    const FA_LDS uint16_t* os = (const FA_LDS uint16_t*)smem_do[st];
    FA_LDS uint16_t* dss = (FA_LDS uint16_t*)smem_ds[st];

#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qb0 = q0 + qb * 32;
      // Any (query, key) pair of this 32x32 block visible?
      const bool active = (kw0 < N) && (qb0 < N) && (!CAUSAL || qb0 + 31 >= kw0);
      u32x2_t dsw[4];
      if (active) {
        f32x16_t sacc, dpacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[r] = 0.f;
          dpacc[r] = 0.f;
        }
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
          const int off = (qb * 32 + l32) * QSTR + dc * 16 + 8 * hl;
          const v8 qa = __builtin_bit_cast(v8, ld_lds16(qs + off));
          const v8 oa = __builtin_bit_cast(v8, ld_lds16(os + off));
          sacc = E::mfma(qa, kf[dc], sacc);
          dpacc = E::mfma(oa, vf[dc], dpacc);
        }
        const bool need_mask = (kw0 + 31 >= N) || (CAUSAL && kw0 + 31 > qb0);
        float p[16], ds[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qo = qb * 32 + 8 * g + 4 * hl;
          const f32x4_t l4 = *(const FA_LDS f32x4_t*)(smem_lse[st] + qo);
          const f32x4_t d4 = *(const FA_LDS f32x4_t*)(smem_dd[st] + qo);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int r = 4 * g + t;
            float pv = fast_exp2(sacc[r] * a.scale_log2 - l4[t]);
            if (need_mask) {
              const int q = q0 + qo + t;
              if (key >= N || (CAUSAL && key > q)) pv = 0.f;
            }
            p[r] = pv;
            ds[r] = pv * (dpacc[r] - d4[t]) * a.scale;
          }
        }
        // P and dS as B operands, 16 queries per chunk (slot s of half hl is
        // query 16c + 8*(s/4) + 4*hl + s%4 of the block).
        v8 pf[2], df[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          u32x4_t pw, dw;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pw[j] = E::pack2(p[8 * c + 2 * j], p[8 * c + 2 * j + 1]);
            dw[j] = E::pack2(ds[8 * c + 2 * j], ds[8 * c + 2 * j + 1]);
          }
          pf[c] = __builtin_bit_cast(v8, pw);
          df[c] = __builtin_bit_cast(v8, dw);
          dsw[2 * c] = u32x2_t{dw[0], dw[1]};
          dsw[2 * c + 1] = u32x2_t{dw[2], dw[3]};
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int row0 = (qb * 32 + c * 16 + 4 * hl + tr_row) * QSTR + tr_col;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const s16x4_t olo = ld_lds_tr16(os + row0 + db * 32);
            const s16x4_t ohi = ld_lds_tr16(os + row0 + 8 * QSTR + db * 32);
            const s16x4_t qlo = ld_lds_tr16(qs + row0 + db * 32);
            const s16x4_t qhi = ld_lds_tr16(qs + row0 + 8 * QSTR + db * 32);
            const u32x2_t ol = __builtin_bit_cast(u32x2_t, olo), oh = __builtin_bit_cast(u32x2_t, ohi);
            const u32x2_t ql = __builtin_bit_cast(u32x2_t, qlo), qh = __builtin_bit_cast(u32x2_t, qhi);
            dvacc[db] = E::mfma(__builtin_bit_cast(v8, u32x4_t{ol[0], ol[1], oh[0], oh[1]}), pf[c],
                                dvacc[db]);
            dkacc[db] = E::mfma(__builtin_bit_cast(v8, u32x4_t{ql[0], ql[1], qh[0], qh[1]}), df[c],
                                dkacc[db]);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) dsw[j] = u32x2_t{0u, 0u};
      }
      // dS^T row of this lane's key: queries qb*32 + 8g + 4*hl + [0, 4).
      // dsw[2c + j] holds registers 8c + 4j .. +3, i.e. g = 2c + j.
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(FA_LDS u32x2_t*)(dss + (wave * 32 + l32) * SSTR + qb * 32 + 8 * g + 4 * hl) = dsw[g];
    }

    if (it + 1 < nq) stash(st ^ 1);
    __syncthreads();

    // dQ tile = dS (BQ x BKV) K (BKV x D): 32x32 output blocks spread over waves.
    for (int blk = wave; blk < NQB * NDB; blk += NW) {
      const int qb = blk / NDB;
      const int db = blk % NDB;
      if (q0 + qb * 32 >= N) continue;
      f32x16_t acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int kc = 0; kc < BKV / 16; ++kc) {
        const int srow = (kc * 16 + 4 * hl + tr_row);
        const s16x4_t slo = ld_lds_tr16(dss + srow * SSTR + qb * 32 + tr_col);
        const s16x4_t shi = ld_lds_tr16(dss + (srow + 8) * SSTR + qb * 32 + tr_col);
        const s16x4_t klo = ld_lds_tr16(ks + srow * KSTR + db * 32 + tr_col);
        const s16x4_t khi = ld_lds_tr16(ks + (srow + 8) * KSTR + db * 32 + tr_col);
        const u32x2_t sl = __builtin_bit_cast(u32x2_t, slo), sh = __builtin_bit_cast(u32x2_t, shi);
        const u32x2_t kl = __builtin_bit_cast(u32x2_t, klo), kh = __builtin_bit_cast(u32x2_t, khi);
        acc = E::mfma(__builtin_bit_cast(v8, u32x4_t{sl[0], sl[1], sh[0], sh[1]}),
                      __builtin_bit_cast(v8, u32x4_t{kl[0], kl[1], kh[0], kh[1]}), acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + qb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (q < N) unsafeAtomicAdd(dQg + (int64_t)q * D + db * 32 + l32, acc[r]);
      }
    }
  }

  // dK (scale already folded into dS) and dV for this lane's key.
  if (key < N) {
    uint16_t* dkrow = static_cast<uint16_t*>(a.dk) + base + (int64_t)key * D;
    uint16_t* dvrow = static_cast<uint16_t*>(a.dv) + base + (int64_t)key * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hl;
        u32x2_t w;
        w[0] = E::pack2(dkacc[db][4 * g + 0], dkacc[db][4 * g + 1]);
        w[1] = E::pack2(dkacc[db][4 * g + 2], dkacc[db][4 * g + 3]);
        *reinterpret_cast<u32x2_t*>(dkrow + d0) = w;
        w[0] = E::pack2(dvacc[db][4 * g + 0], dvacc[db][4 * g + 1]);
        w[1] = E::pack2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
        *reinterpret_cast<u32x2_t*>(dvrow + d0) = w;
      }
    }
  }
}

template <int D, int NW, int BQ, int DT>
hipError_t launch_d(const BwdArgs& a0, int BH, bool causal, hipStream_t s) {
  BwdArgs a = a0;
  const int64_t rows = (int64_t)BH * a.N;
  constexpr int TPR = D / 8;
  const int64_t pre_blocks = (rows * TPR + 255) / 256;
  if (pre_blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_pre_kernel<D, DT>), dim3((unsigned)pre_blocks), dim3(256), 0, s,
                     static_cast<const uint16_t*>(a.o), static_cast<const uint16_t*>(a.dout),
                     a.dsum, a.dq, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int BKV = 32 * NW;
  a.n_ktiles = (a.N + BKV - 1) / BKV;
  const int64_t grid = (int64_t)a.n_ktiles * BH;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (causal)
    hipLaunchKernelGGL((bwd_kernel<D, NW, BQ, true, DT>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       s, a);
  else
    hipLaunchKernelGGL((bwd_kernel<D, NW, BQ, false, DT>), dim3((unsigned)grid), dim3(NW * 64),
                       0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dtype(const BwdArgs& a, int BH, int d, bool causal, hipStream_t s) {
  switch (d) {
    case 64: return launch_d<64, 4, 64, DT>(a, BH, causal, s);
    case 128: return launch_d<128, 4, 32, DT>(a, BH, causal, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool bwd_supported(int d) { return d == 64 || d == 128; }

hipError_t launch_bwd(const BwdArgs& a, int B, int H, int d, int dtype, bool causal,
                      hipStream_t stream) {
  const int BH = B * H;
  return dtype == 0 ? launch_dtype<0>(a, BH, d, causal, stream)
                    : launch_dtype<1>(a, BH, d, causal, stream);
}

}  // namespace fa
