// Attention forward for gfx950: exact softmax attention computed tile by tile
// with an online softmax ("FlashAttention: Fast and Memory-Efficient Exact
// Attention with IO-Awareness", abstract: tiling between HBM and on-chip
// memory; FlashAttention-4 related-papers page, online-softmax snippet:
// running row maximum and normaliser; FlashAttention-3 review page, Appendix B
// fragment: exp2, row sum and output rescaling between the two products).
//
// Work unit: one workgroup = NW waves = 32*NW query rows of one (b, h).  Each
// wave keeps its 32 query rows in registers for the whole key loop.
//
// Data movement: key and value tiles of BN rows are copied from HBM straight
// into LDS by the asynchronous global->LDS DMA (no staging registers), into a
// ring of NS = 4 stages per tensor, three tiles ahead of the tile being
// consumed; the producers are the computing waves themselves (the pages'
// asynchronous copies overlapped with compute, FlashAttention-3 abstract).
// At the end of each tile a wave waits only for the copies the next tile
// needs, then the workgroup barrier publishes them.  LDS rows are unpadded; the 16-byte
// chunk index of row r is XOR-ed with swz<D>(r), which keeps both LDS read
// patterns below free of bank conflicts.
//
// Per tile and wave:
//   S^T = K_j Q^T on 32x32x16 matrix cores (keys are accumulator rows, the
//     wave's 32 queries columns: one lane owns one query row, so row
//     reductions are in-lane plus one exchange with the lane 32 away);
//   online softmax in the exp2 domain (scores times scale*log2(e)), with the
//     exp2 reference raised lazily; probabilities rounded to the input type;
//   O^T += V_j^T P^T on matrix cores, V read from LDS by transposed 16-bit
//     reads; O^T has one query per lane, so the rescale is a per-lane multiply.
#include <type_traits>

#include "common.h"
#include "kernels.h"

#ifndef FA_FWD128_NW
#define FA_FWD128_NW 8  // waves per workgroup of the d = 128 forward
#endif

namespace fa {

namespace {

// XOR applied to the 16-byte chunk index of row r of a K or V tile in LDS.
// Rows are 2*D bytes.  With it, (a) sixteen lanes reading the same chunk of
// sixteen consecutive rows, and (b) the 4 rows x 4 chunks of a transposed
// read by one half-wave, each hit all 64 banks once.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D >= 128)
    return 4 * (r & 3) + ((r >> 2) & 3);
  else
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// OCC = waves per SIMD the register budget is sized for (2: 256 registers).
template <int D, int BN, int NW, int OCC, bool CAUSAL, int DT>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
fwd_kernel(FwdArgs a) {
  using E = Elem<DT>;
  using v8 = typename E::v8;
  constexpr int BM = 32 * NW;
  constexpr int NS = 4;              // LDS stages per tensor
  constexpr int ROWB = 2 * D;        // bytes per LDS row
  constexpr int TILEB = BN * ROWB;   // bytes per tile per tensor
  constexpr int CH_ROW = D / 8;      // 16-byte chunks per row
  static_assert(TILEB % (1024 * NW) == 0, "a tile must split into whole 1 KiB copies per wave");
  constexpr int IPW = TILEB / 1024 / NW;  // copies per wave per tensor per tile
  constexpr int LPT = 2 * IPW;            // vector-memory ops per wave per tile
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;
  constexpr int NDC = D / 16;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * NS * TILEB];
  FA_LDS uint8_t* lds = (FA_LDS uint8_t*)smem;  // K stage s at s*TILEB, V at (NS+s)*TILEB

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int hl = lane >> 5;  // which half of K slots / accumulator rows
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
  const float c = a.scale_log2;

  // ---- DMA producer: copy j of this wave fills LDS chunk
  // (wave*IPW + j)*64 + lane of the tile, i.e. row dma_row[j], and must read
  // the logical chunk that the swizzle maps there.
  int dma_row[IPW], dma_col[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int p = (wave * IPW + j) * 64 + lane;
    dma_row[j] = p / CH_ROW;
    dma_col[j] = ((p % CH_ROW) ^ swz<D>(p / CH_ROW)) * 8;
  }
  auto issue = [&](int t) {
    const int stage = t % NS;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int key = min(t * BN + dma_row[j], N - 1);  // rows past N are masked later
      const int64_t off = (int64_t)key * D + dma_col[j];
      dma16(K + off, lds + stage * TILEB + (wave * IPW + j) * 1024);
      dma16(V + off, lds + (NS + stage) * TILEB + (wave * IPW + j) * 1024);
    }
  };
  // Q^T operand: lane holds query qrow, head-dim slots dc*16 + 8*hl + [0, 8).
  v8 qf[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
    u32x4_t raw = {0u, 0u, 0u, 0u};
    if (qrow < N) raw = ld_global16(Q + (int64_t)qrow * D + dc * 16 + 8 * hl);
    qf[dc] = __builtin_bit_cast(v8, raw);
  }

  f32x16_t oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_run = -INFINITY;  // exp2 reference of this lane's row, log2 units
  float l_run = 0.f;        // this lane's share of the normaliser

  // ---- LDS read offsets (bytes within a stage).
  // K operand of S^T: lane reads row kb*32 + l32, head-dim chunk 2*dc + hl.
  int koff[NDC];
  {
    const int f = swz<D>(l32);  // equals swz of row kb*32 + l32
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) koff[dc] = l32 * ROWB + 16 * ((2 * dc + hl) ^ f);
  }
  // V operand of O^T (transposed reads): supplier lane 4e + c4 of each 16-lane
  // group addresses row 16*cc + 4*hl + e (+8 for the second read) and column
  // group 16*g2 + 4*c4 of the 32-column block db.
  int voff[NDB][2];
  {
    const int e = (lane & 15) >> 2, c4 = lane & 3, g2 = (lane >> 4) & 1;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 4 * hl + e + 8 * hi;  // row within a 16-key chunk; cc adds 16 rows
      const int f = swz<D>(r);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        voff[db][hi] = r * ROWB + 16 * ((4 * db + 2 * g2 + (c4 >> 1)) ^ f) + 8 * (c4 & 1);
    }
  }

  // ---- S: raw scores of tile t (S^T block kb: key rows, query columns);
  // invisible keys are set to -inf.  MASKED tiles (the ragged last tile, the
  // causal diagonal) are a separate instantiation so that the common path
  // carries no masking work.
  auto phase_s = [&](int t, f32x16_t (&sacc)[NKB], auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const FA_LDS uint8_t* ks = lds + (t % NS) * TILEB;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const v8 kf = __builtin_bit_cast(v8, ld_lds16(ks + kb * 32 * ROWB + koff[dc]));
        sacc[kb] = E::mfma(kf, qf[dc], sacc[kb]);
      }
    }
    if constexpr (MASKED) {
      // Register r of block kb holds key t*BN + 4*hl + (kb*32 + 8*(r/4) + r%4);
      // it is visible iff that constant offset is below `lim`.
      int lim = N - t * BN - 4 * hl;
      if (CAUSAL) lim = min(lim, qrow + 1 - t * BN - 4 * hl);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) sacc[kb][r] = -INFINITY;
    }
  };

  // ---- SM: online softmax of one tile's scores into packed probabilities.
  // The exp2 reference m_run is raised only when the tile's maximum exceeds
  // it by kLazyMax, so the probabilities are computed against the current
  // reference before the maximum is known and recomputed in the rare raise
  // branch; the exponentials therefore do not wait for the row reduction.
  auto phase_sm = [&](f32x16_t (&sacc)[NKB], uint32_t (&pw)[NKB][8]) {
    auto probs = [&](float m_neg) {
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p0 = fast_exp2(fmaf(sacc[kb][2 * j], c, m_neg));
          const float p1 = fast_exp2(fmaf(sacc[kb][2 * j + 1], c, m_neg));
          pw[kb][j] = E::pack2(p0, p1);
          ps0 += p0;
          ps1 += p1;
        }
      return ps0 + ps1;  // fp32 sum of the unrounded values
    };
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    float psum = probs(m_run == -INFINITY ? 0.f : -m_run);
    // Empty uses pin the speculative results before the branch below;
    // otherwise the compiler sinks them past it, away from the matrix-core
    // work they are meant to overlap.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(pw[kb][j]));
    asm volatile("" ::"v"(psum));
    mx = max_halves(mx) * c;  // scale > 0, so max and scaling commute
    const bool raise = mx > m_run + kLazyMax;
    if (wave_any(raise)) {
      // Keeps the compiler from turning this rarely taken branch into
      // unconditional work on every tile.
      asm volatile("" ::: "memory");
      // mx is finite whenever raise holds; alpha = 0 on a row's first tile.
      const float alpha = raise ? fast_exp2(m_run - mx) : 1.0f;
      m_run = raise ? mx : m_run;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      psum = probs(m_run == -INFINITY ? 0.f : -m_run);
    }
    l_run += psum;
  };

  // ---- PV: O^T += V^T P^T, 16 keys per instruction.  Chunk cc of the tile
  // uses accumulator registers 8*(cc%2)..+7 of block cc/2, i.e. keys
  // 16cc + 8*(s/4) + 4*hl + s%4 for slot s; the V operand is read for the
  // same keys.
  auto phase_pv = [&](int t, const uint32_t (&pw)[NKB][8]) {
    const FA_LDS uint8_t* vs = lds + (NS + t % NS) * TILEB;
#pragma unroll
    for (int cc = 0; cc < BN / 16; ++cc) {
      const int j0 = 4 * (cc & 1);
      const v8 pf = __builtin_bit_cast(
          v8, u32x4_t{pw[cc >> 1][j0], pw[cc >> 1][j0 + 1], pw[cc >> 1][j0 + 2], pw[cc >> 1][j0 + 3]});
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const s16x4_t lo = ld_lds_tr16(vs + cc * 16 * ROWB + voff[db][0]);
        const s16x4_t hi = ld_lds_tr16(vs + cc * 16 * ROWB + voff[db][1]);
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        const v8 vf = __builtin_bit_cast(v8, u32x4_t{l2[0], l2[1], h2[0], h2[1]});
        oacc[db] = E::mfma(vf, pf, oacc[db]);
      }
    }
  };

  // Software pipeline (two stages, the pages' intra-group pipelining): at the
  // start of iteration j the scores S(j) are in registers and tiles up to j+1
  // are in LDS.  The iteration issues the copy of tile j+NS-1, computes
  // S(j+1) on the matrix cores while the softmax of tile j runs on the vector
  // ALUs (same basic block, so the hardware overlaps them), then O += P(j) V(j).
  // Tiles [0, t_mask) need no mask and every wave takes part in them, so the
  // main loop has no branches besides the rare reference raise.
  int t_mask = (N % BN) ? N / BN : ntiles;
  if (CAUSAL) t_mask = min(t_mask, (q0 + 1) / BN);
  t_mask = min(t_mask, ntiles);
  auto active = [&](int t) { return (qw0 < N) && (!CAUSAL || t * BN <= qw0 + 31); };

  f32x16_t scur[NKB], snxt[NKB];
  uint32_t pw[NKB][8];

  // Prologue: tiles 0 .. NS-2 in flight; wait for tiles 0 and 1; S(0).
  for (int t = 0; t < NS - 1 && t < ntiles; ++t) issue(t);
  if (ntiles > 2)
    dma_sync<LPT * (NS - 3)>();  // tiles 2 .. NS-2 may stay in flight
  else
    dma_sync<0>();
  if (active(0)) {
    if (t_mask > 0)
      phase_s(0, scur, std::false_type{});
    else
      phase_s(0, scur, std::true_type{});
  }

  int j = 0;
  // Main loop: tiles j and j+1 unmasked, all waves active.
  for (; j + 1 < t_mask; ++j) {
    const bool ahead = j + NS - 1 < ntiles;
    if (ahead) issue(j + NS - 1);  // its stage was last read before the previous barrier
    phase_s(j + 1, snxt, std::false_type{});
    phase_sm(scur, pw);
    phase_pv(j, pw);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) scur[kb] = snxt[kb];
    // Tile j+2 must be complete for the next iteration.
    if (j + NS - 1 < ntiles)
      dma_sync<LPT * (NS - 3)>();
    else
      dma_sync<0>();
  }
  // Tail: masked tiles and per-wave activity checks.
  for (; j < ntiles; ++j) {
    const bool ahead = j + NS - 1 < ntiles;
    if (ahead) issue(j + NS - 1);
    if (j + 1 < ntiles && active(j + 1)) phase_s(j + 1, snxt, std::true_type{});
    if (active(j)) {
      phase_sm(scur, pw);
      phase_pv(j, pw);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) scur[kb] = snxt[kb];
    if (ahead)
      dma_sync<LPT * (NS - 3)>();
    else
      dma_sync<0>();
  }

  // Epilogue: normalise, round, store; LSE in natural log.
  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + base + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
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

template <int D, int BN, int NW, int OCC, bool CAUSAL, int DT>
hipError_t launch_one(const FwdArgs& a, int BH, hipStream_t stream) {
  constexpr int BM = 32 * NW;
  FwdArgs args = a;
  args.n_qtiles = (a.N + BM - 1) / BM;
  const int64_t grid = (int64_t)args.n_qtiles * BH;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_kernel<D, BN, NW, OCC, CAUSAL, DT>), dim3((unsigned)grid),
                     dim3(NW * 64), 0, stream, args);
  return hipGetLastError();
}

template <int D, int BN, int NW, int OCC, int DT>
hipError_t launch_causal(const FwdArgs& a, int BH, bool causal, hipStream_t s) {
  return causal ? launch_one<D, BN, NW, OCC, true, DT>(a, BH, s)
                : launch_one<D, BN, NW, OCC, false, DT>(a, BH, s);
}

template <int DT>
hipError_t launch_dtype(const FwdArgs& a, int BH, int d, bool causal, hipStream_t s) {
  switch (d) {
    case 64: return launch_causal<64, 64, 8, 2, DT>(a, BH, causal, s);
    case 128: return launch_causal<128, 64, FA_FWD128_NW, 2, DT>(a, BH, causal, s);
    case 256: return launch_causal<256, 32, 4, 1, DT>(a, BH, causal, s);
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
