// FP8 (e4m3) attention forward for gfx950 ("FlashAttention-3: Fast and
// Accurate Attention with Asynchrony and Low-precision", abstract: FP8 with
// block quantization and incoherent processing).  Operands come from
// fa_quant_fp8: Q and K rotated by the same signed Hadamard transform (1/d
// folded into Q's scales), V unrotated, one fp32 scale per 128-row block.
//
// Same tiling as the 16-bit forward (query rows in registers, K/V tiles
// double buffered through LDS, S^T layout with one query per lane), with:
//   * S^T = K8 Q8^T on v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, fp32 acc);
//     the product of the query block's and key block's scales, the softmax
//     scale and log2(e) is one fp32 multiplier per tile (a key tile lies in
//     one 128-row scale block, a wave's 32 queries likewise);
//   * probabilities P~ = exp2(s - m) in [0, 1] are rounded to e4m3 (round to
//     nearest even) for O += P V; the row normaliser is summed from the fp32
//     P~;
//   * the output accumulator is kept in units of the current value block's
//     scale: moving to a tile whose V scale differs multiplies it by
//     alpha * vs_prev / vs_new (exact in real arithmetic), and the epilogue
//     multiplies by vs_last / l;
//   * V8 stays row-major in LDS and is read transposed with ds_read_b64_tr_b8
//     (inside a 16-lane group, lane j's byte e is byte j%8 of the chunk
//     addressed by lane 2e + j/8); 8-byte units of a V row are XOR-swizzled
//     so that the eight rows those reads touch fall in distinct LDS banks.
#include "common.h"
#include "kernels.h"

namespace fa {

namespace {

typedef int i32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16_t mfma_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
  // Format code 0 = e4m3 for both operands; no per-block hardware scaling.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x2_t ld_lds_tr8(const FA_LDS void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      reinterpret_cast<FA_LDS i32x2_t*>(const_cast<FA_LDS void*>(p)));
}

// XOR applied to the 8-byte unit index of V row `row` (multiple of 4, so
// 16-byte chunks stay contiguous and aligned).
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  const int g = ((row >> 1) & 1) | (((row >> 3) & 1) << 1);
  return (4 * g) & (D / 8 - 4);
}

template <int D, int BN, int NW, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64)
fwd_fp8_kernel(Fp8Args a) {
  constexpr int NT = NW * 64;
  constexpr int BM = 32 * NW;
  constexpr int KSTR = D + 16;       // bytes; conflict-free 16-byte reads by 16 rows
  constexpr int VSTR = D;            // bytes; swizzled
  constexpr int K_BYTES = BN * KSTR;
  constexpr int STAGE = K_BYTES + BN * VSTR;
  constexpr int CH_ROW = D / 16;     // 16-byte chunks per row
  constexpr int CH = BN * CH_ROW;
  static_assert(CH % NT == 0, "tile chunks must divide evenly over threads");
  constexpr int CPT = CH / NT;
  static_assert(BN == 64, "one 32x32x64 product per pair of 32-key blocks");
  static_assert(128 % BN == 0 && 128 % 32 == 0, "tiles inside one scale block");
  constexpr int NDC = D / 64;        // 64-wide head-dim chunks of S
  constexpr int NDB = D / 32;

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  FA_LDS uint8_t* lds = (FA_LDS uint8_t*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int N = a.N;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / a.n_qtiles;
  int qt = logical % a.n_qtiles;
  if (CAUSAL) qt = a.n_qtiles - 1 - qt;
  const int64_t base = (int64_t)bh * N * D;
  const uint8_t* Q = static_cast<const uint8_t*>(a.q8) + base;
  const uint8_t* K = static_cast<const uint8_t*>(a.k8) + base;
  const uint8_t* V = static_cast<const uint8_t*>(a.v8) + base;
  const float* qsc = a.q_scale + (int64_t)bh * a.nblk;
  const float* ksc = a.k_scale + (int64_t)bh * a.nblk;
  const float* vsc = a.v_scale + (int64_t)bh * a.nblk;

  const int q0 = qt * BM;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;
  const float q_scale = qsc[min(qw0, N - 1) / 128];

  // Q8^T operand: lane holds query qrow, head-dim bytes dc*64 + 32*hl + [0, 32).
  i32x8_t qf[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
    u32x4_t lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (qrow < N) {
      const uint8_t* p = Q + (int64_t)qrow * D + dc * 64 + 32 * hl;
      lo = ld_global16(p);
      hi = ld_global16(p + 16);
    }
    qf[dc] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }

  f32x16_t oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  float vs_cur = 1.f;  // V scale the accumulator is expressed in

  u32x4_t kreg[CPT], vreg[CPT];
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      const int r = c / CH_ROW;
      const int col = (c % CH_ROW) * 16;
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
    FA_LDS uint8_t* ks = lds + stage * STAGE;
    FA_LDS uint8_t* vs = ks + K_BYTES;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      const int r = c / CH_ROW;
      const int cc = c % CH_ROW;
      st_lds16(ks + r * KSTR + cc * 16, kreg[i]);
      st_lds16(vs + r * VSTR + (((2 * cc) ^ v_swz<D>(r)) * 8), vreg[i]);
    }
  };

  // Lane roles in the transposed byte reads: supplier lane 2e + c of each
  // 16-lane group addresses row e of the group's eight and unit c of two.
  const int tr_e = (lane & 15) >> 1;
  const int tr_c = lane & 1;
  const int tr_unit = ((lane >> 4) & 1) * 2 + tr_c;   // within a 32-byte column block
  // Row (within a 64-key tile) of read rd for this supplier: keys in the
  // order the S^T accumulator hands probabilities to the product.
  auto tr_row = [&](int rd) { return 16 * rd + 8 * (tr_e >> 2) + 4 * hl + (tr_e & 3); };

  fetch(0);
  stash(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < ntiles) fetch(t + 1);
    const int kbase = t * BN;
    const bool active = (qw0 < N) && (!CAUSAL || kbase <= qw0 + 31);
    if (active) {
      const FA_LDS uint8_t* ks = lds + stage * STAGE;
      const FA_LDS uint8_t* vs = ks + K_BYTES;
      const float k_scale = ksc[kbase / 128];
      const float v_scale = vsc[kbase / 128];
      const float mult = q_scale * k_scale * a.scale_log2;

      f32x16_t sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const FA_LDS uint8_t* p = ks + (kb * 32 + l32) * KSTR + dc * 64 + 32 * hl;
          const u32x4_t lo = ld_lds16(p), hi = ld_lds16(p + 16);
          const i32x8_t kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          sacc[kb] = mfma_fp8(kf, qf[dc], sacc[kb]);
        }
      }

      const bool need_mask = (kbase + BN > N) || (CAUSAL && kbase + BN - 1 > qw0);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float s = sacc[kb][r] * mult;
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
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(sacc[kb][r] - m_use);
          sacc[kb][r] = p;
          psum += p;
        }
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const float ofac = alpha * (vs_cur / v_scale);
      vs_cur = v_scale;
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= ofac;

      // P^T operand: byte s = 16*kb + r holds the probability of key
      // 32*kb + 8*(r/4) + 4*hl + r%4.
      i32x8_t pf;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int s0 = 4 * w;
        const f32x16_t& sb = sacc[s0 >> 4];
        const int r0 = s0 & 15;
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(sb[r0], sb[r0 + 1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(sb[r0 + 2], sb[r0 + 3], word, true);
        pf[w] = word;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int unit = db * 4 + tr_unit;
        i32x8_t vf;
#pragma unroll
        for (int rd = 0; rd < 4; ++rd) {
          const int row = tr_row(rd);
          const i32x2_t v2 = ld_lds_tr8(vs + row * VSTR + ((unit ^ v_swz<D>(row)) * 8));
          vf[2 * rd] = v2[0];
          vf[2 * rd + 1] = v2[1];
        }
        oacc[db] = mfma_fp8(vf, pf, oacc[db]);
      }
    }
    if (t + 1 < ntiles) stash(stage ^ 1);
    __syncthreads();
  }

  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.f ? vs_cur / l_tot : 0.f;
  if (qrow < N) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + base + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2_t w;
        w[0] = Elem<0>::pack2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
        w[1] = Elem<0>::pack2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2_t*>(orow + db * 32 + 8 * g + 4 * hl) = w;
      }
    }
    if (hl == 0 && a.lse != nullptr)
      a.lse[(int64_t)bh * N + qrow] = m_run * kLn2 + __logf(l_tot);
  }
}

template <int D, int NW, bool CAUSAL>
hipError_t launch_one(const Fp8Args& a0, int BH, hipStream_t s) {
  constexpr int BM = 32 * NW;
  Fp8Args a = a0;
  a.n_qtiles = (a.N + BM - 1) / BM;
  const int64_t grid = (int64_t)a.n_qtiles * BH;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, 64, NW, CAUSAL>), dim3((unsigned)grid), dim3(NW * 64), 0,
                     s, a);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_d(const Fp8Args& a, int BH, bool causal, hipStream_t s) {
  return causal ? launch_one<D, NW, true>(a, BH, s) : launch_one<D, NW, false>(a, BH, s);
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Args& a, int B, int H, int d, bool causal, hipStream_t stream) {
  const int BH = B * H;
  switch (d) {
    case 64: return launch_d<64, 4>(a, BH, causal, stream);
    case 128: return launch_d<128, 8>(a, BH, causal, stream);
    case 256: return launch_d<256, 4>(a, BH, causal, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
