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
//   bwd_pre_kernel  per query row: (-LSE / scale, -D) into the workspace.
//   bwd_kv_kernel   one workgroup per (b, h, tile of BKV = 32*NW keys); wave w
//                   owns keys [32 w, 32 w + 32) of the tile and keeps their K
//                   and V rows, and their dK, dV accumulators, in registers.
//                   Query tiles of BQ rows (Q, dO and the row statistics)
//                   stream through a three-stage LDS ring filled by buffer
//                   loads with an LDS destination.  Per query tile:
//     A  S - LSE/scale and dP - D on 32x32x16 matrix cores (the accumulators
//        start from the row statistics), keys as accumulator columns (one key
//        per lane), Q and dO read from LDS;
//     V  P = exp2((S - LSE/scale) * scale * log2 e), dS' = P o (dP - D) in
//        fp32, rounded to the input type (dK = scale * dS'^T Q is scaled
//        once at the end);
//     B  dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T read from LDS by
//        transposed 16-bit reads.
//   bwd_dq_kernel   one workgroup per (b, h, tile of 32*NW queries), built like
//                   the forward: Q and dO rows stay in registers, K and V tiles
//                   stream through a three-stage LDS ring; per key tile it
//                   recomputes S^T = K Q^T and dP^T = V dO^T, forms dS^T and
//                   accumulates dQ^T += K^T dS^T in registers, written once at
//                   the end.  Recomputing two products costs 2/5 more matrix
//                   work than accumulating dQ with atomics from bwd_kv_kernel,
//                   whose fp32 atomic traffic (every key tile adds a full dQ
//                   tile) is bound by the L2 atomic units.
//   Rows past N (queries or keys) arrive as zeros; every product they enter
//   is then exactly zero or never stored, so only the causal mask is applied.
#include <type_traits>

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

// Per row: stat[row] = (-LSE / scale, -sum_c dO[row][c] * O[row][c]), the
// starting values of the S and dP accumulators of the backward kernels.  D/8
// threads per row.
template <int D, int DT>
__global__ void __launch_bounds__(256)
bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
               const float* __restrict__ lse, f32x2_t* __restrict__ stat, int64_t rows,
               float inv_scale) {
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
  if (row < rows && c == 0) stat[row] = f32x2_t{-lse[row] * inv_scale, -acc};
}

// Same chunk swizzle as the forward's K/V tiles (rows of 2*D bytes): both
// the 16-byte row reads and the transposed reads are free of bank conflicts.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D >= 128)
    return 4 * (r & 3) + ((r >> 2) & 3);
  else
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

template <int D, int NW, int BQ, bool CAUSAL, int DT>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_kv_kernel(BwdArgs a) {
  using E = Elem<DT>;
  using v8 = typename E::v8;
  constexpr int BKV = 32 * NW;       // keys per workgroup
  constexpr int ROWB = 2 * D;        // bytes per Q / dO / K row
  constexpr int QTB = BQ * ROWB;     // bytes per Q (or dO) tile
  constexpr int RSB = 1024 * NW;     // row-statistics area per stage (one 1 KiB copy per wave)
  constexpr int STAGEB = 2 * QTB + RSB;
  constexpr int NSTG = 3;
  constexpr int CH_ROW = D / 8;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NQB = BQ / 32;
  static_assert(QTB % (1024 * NW) == 0, "a Q tile must split into whole 1 KiB copies per wave");
  constexpr int IPW = QTB / 1024 / NW;           // copies per wave per tensor per tile
  constexpr int DMA_OPS = 2 * IPW + 1;           // per wave per tile (Q, dO, row stats)
  static_assert(BQ % 32 == 0, "query tile");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTG * STAGEB];
  FA_LDS uint8_t* lds = (FA_LDS uint8_t*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int N = a.N;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / a.n_ktiles;
  const int kt = logical % a.n_ktiles;
  const int64_t base = (int64_t)bh * N * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.q) + base;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + base;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v) + base;
  const uint16_t* dOg = static_cast<const uint16_t*>(a.dout) + base;
  const f32x2_t* statg = reinterpret_cast<const f32x2_t*>(a.dsum) + (int64_t)bh * N;

  const int k0 = kt * BKV;
  const int key = k0 + wave * 32 + l32;  // this lane's key (S accumulator column)
  const float c = a.scale_log2;

  // ---- Copies (buffer loads with an LDS destination; rows past N arrive as
  // zeros).  Copy jj of this wave fills LDS chunk (wave*IPW + jj)*64 + lane
  // of a tile: row p / CH_ROW, swizzled chunk.
  uint32_t dma_voff[IPW];
#pragma unroll
  for (int jj = 0; jj < IPW; ++jj) {
    const int p = (wave * IPW + jj) * 64 + lane;
    dma_voff[jj] = (uint32_t)((p / CH_ROW) * ROWB + ((p % CH_ROW) ^ swz<D>(p / CH_ROW)) * 16);
  }
  auto copy_rows = [&](const uint16_t* src, int r0, int nrows, FA_LDS uint8_t* dst) {
    const int rows = r0 >= N ? 0 : min(N - r0, nrows);
    const u32x4_t r = make_rsrc(src + (int64_t)max(r0, 0) * D, rows * ROWB);
#pragma unroll
    for (int jj = 0; jj < IPW; ++jj) dma16_buf(r, dma_voff[jj], dst + (wave * IPW + jj) * 1024);
  };
  // Query tile i into stage st: Q, dO, and the row statistics of the rows
  // [BQ/NW * wave, +BQ/NW) into this wave's 1 KiB block of the stage.
  auto issue_tile = [&](int i, int st) {
    FA_LDS uint8_t* sb = lds + st * STAGEB;
    const int q0 = i * BQ;
    copy_rows(Qg, q0, BQ, sb);
    copy_rows(dOg, q0, BQ, sb + QTB);
    constexpr int RPW = BQ / NW;
    const int r0 = q0 + wave * RPW;
    const int rows = r0 >= N ? 0 : min(N - r0, RPW);
    const u32x4_t r = make_rsrc(statg + max(r0, 0), rows * 8);
    dma16_buf(r, (uint32_t)lane * 16, sb + 2 * QTB + wave * 1024);
  };
  // Row statistics of query row q of the tile in stage sb: 4 consecutive rows
  // (q % 4 == 0) as {-LSE/scale, -D, -LSE/scale, -D, ...}.
  auto ld_stat4 = [&](const FA_LDS uint8_t* sb, int q, f32x4_t& lo, f32x4_t& hi) {
    constexpr int RPW = BQ / NW;
    const FA_LDS uint8_t* p = sb + 2 * QTB + (q / RPW) * 1024 + (q % RPW) * 8;
    lo = *(const FA_LDS f32x4_t*)p;
    hi = *(const FA_LDS f32x4_t*)(p + 16);
  };

  // ---- LDS read offsets within a Q / dO tile (or the staged K tile).
  // Row reads (A operand, rows = queries): row qb*32 + l32, chunk 2*dc + hl.
  int roff[NDC];
  {
    const int f = swz<D>(l32);
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) roff[dc] = l32 * ROWB + 16 * ((2 * dc + hl) ^ f);
  }
  // Transposed reads (A operand with rows = head dims, or B operand with
  // columns = head dims; K slots = 16 consecutive rows of the tile): supplier
  // lane 4e + c4 of each 16-lane group addresses row 16*cc + 4*hl + e (+8) and
  // column group 16*g2 + 4*c4 of head-dim block db.
  int toff[NDB][2];
  {
    const int e = (lane & 15) >> 2, c4 = lane & 3, g2 = (lane >> 4) & 1;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 4 * hl + e + 8 * hi;
      const int f = swz<D>(r);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        toff[db][hi] = r * ROWB + 16 * ((4 * db + 2 * g2 + (c4 >> 1)) ^ f) + 8 * (c4 & 1);
    }
  }
  auto ld_row = [&](const FA_LDS uint8_t* t, int qb, int dc) {
    return __builtin_bit_cast(v8, ld_lds16(t + qb * 32 * ROWB + roff[dc]));
  };
  auto ld_tr = [&](const FA_LDS uint8_t* t, int cc, int db) {
    const s16x4_t lo = ld_lds_tr16(t + cc * 16 * ROWB + toff[db][0]);
    const s16x4_t hi = ld_lds_tr16(t + cc * 16 * ROWB + toff[db][1]);
    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    return __builtin_bit_cast(v8, u32x4_t{l2[0], l2[1], h2[0], h2[1]});
  };
  // ---- Stationary operands.  K and V rows of this lane's key as B operands
  // of S and dP (head-dim slots dc*16 + 8*hl + [0, 8)).
  v8 kf[NDC], vf[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
    u32x4_t rk = {0u, 0u, 0u, 0u}, rv = {0u, 0u, 0u, 0u};
    if (key < N) {
      rk = ld_global16(Kg + (int64_t)key * D + dc * 16 + 8 * hl);
      rv = ld_global16(Vg + (int64_t)key * D + dc * 16 + 8 * hl);
    }
    kf[dc] = __builtin_bit_cast(v8, rk);
    vf[dc] = __builtin_bit_cast(v8, rv);
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
  const int i0 = CAUSAL ? k0 / BQ : 0;
  // Causal: query tile i needs the mask while some of its queries precede
  // some key of the tile.
  const int i_unmask = CAUSAL ? min(nq, (k0 + BKV + BQ - 2) / BQ) : i0;
  uint32_t pw[NQB][2][4], dw[NQB][2][4];  // P and dS packed as B operands (chunk c of block qb)

  // One query tile; MASKED applies the causal mask.
  auto iteration = [&](auto m_tag, int i, int st) {
    constexpr bool MASKED = decltype(m_tag)::value;
    const FA_LDS uint8_t* sb = lds + st * STAGEB;
    const FA_LDS uint8_t* qs = sb;
    const FA_LDS uint8_t* os = sb + QTB;
    const int q0 = i * BQ;

    // A: S - LSE/scale and dP - D for every query block (keys as accumulator
    // columns).  Register r of block qb is query row qb*32 + 8*(r/4) + 4*hl +
    // r%4; the accumulators start from that row's statistics.
    f32x16_t sacc[NQB], dpacc[NQB];
    {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4_t st_lo, st_hi;
          ld_stat4(sb, qb * 32 + 8 * g + 4 * hl, st_lo, st_hi);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            sacc[qb][4 * g + t] = t < 2 ? st_lo[2 * t] : st_hi[2 * (t - 2)];
            dpacc[qb][4 * g + t] = t < 2 ? st_lo[2 * t + 1] : st_hi[2 * (t - 2) + 1];
          }
        }
      constexpr int PF = 2, NST = NQB * NDC;
      v8 qr[PF + 1], orr[PF + 1];
      auto load = [&](int s) {
        qr[s % (PF + 1)] = ld_row(qs, s / NDC, s % NDC);
        orr[s % (PF + 1)] = ld_row(os, s / NDC, s % NDC);
      };
#pragma unroll
      for (int s = 0; s < PF; ++s) load(s);
#pragma unroll
      for (int s = 0; s < NST; ++s) {
        if (s + PF < NST) load(s + PF);
        const int qb = s / NDC, dc = s % NDC;
        sacc[qb] = E::mfma(qr[s % (PF + 1)], kf[dc], sacc[qb]);
        dpacc[qb] = E::mfma(orr[s % (PF + 1)], vf[dc], dpacc[qb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // V: probabilities and dS' of this tile, fp32, packed as B operands.
#pragma unroll
    for (int vg = 0; vg < NQB * 4; ++vg) {
      const int qb = vg / 4, g = vg % 4;
      const int qo = qb * 32 + 8 * g + 4 * hl;  // first of this lane's 4 query rows
      float p[4], ds[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 4 * g + t;
        float pv = fast_exp2(sacc[qb][r] * c);
        if constexpr (MASKED) {
          if (key > q0 + qo + t) pv = 0.f;
        }
        p[t] = pv;
        ds[t] = pv * dpacc[qb][r];
      }
      // Registers 4g..4g+3 are B-operand words (g%2)*2, +1 of chunk g/2.
      pw[qb][g >> 1][2 * (g & 1)] = E::pack2(p[0], p[1]);
      pw[qb][g >> 1][2 * (g & 1) + 1] = E::pack2(p[2], p[3]);
      dw[qb][g >> 1][2 * (g & 1)] = E::pack2(ds[0], ds[1]);
      dw[qb][g >> 1][2 * (g & 1) + 1] = E::pack2(ds[2], ds[3]);
    }

    // Refill: tile i+2 into the stage last read in the previous iteration.
    issue_tile(i + 2, st == 0 ? 2 : st - 1);

    {
      // B: dV^T += dO^T P and dK^T += Q^T dS, 16 queries per instruction.
      constexpr int PF = 2, NST = NDB * (BQ / 16);
      v8 otr[PF + 1], qtr[PF + 1];
      auto load = [&](int s) {
        otr[s % (PF + 1)] = ld_tr(os, s / NDB, s % NDB);
        qtr[s % (PF + 1)] = ld_tr(qs, s / NDB, s % NDB);
      };
#pragma unroll
      for (int s = 0; s < PF; ++s) load(s);
#pragma unroll
      for (int s = 0; s < NST; ++s) {
        if (s + PF < NST) load(s + PF);
        const int cc = s / NDB, db = s % NDB;  // chunk cc = query block cc/2, half cc%2
        const v8 pf = __builtin_bit_cast(v8, u32x4_t{pw[cc >> 1][cc & 1][0], pw[cc >> 1][cc & 1][1],
                                                     pw[cc >> 1][cc & 1][2], pw[cc >> 1][cc & 1][3]});
        const v8 df = __builtin_bit_cast(v8, u32x4_t{dw[cc >> 1][cc & 1][0], dw[cc >> 1][cc & 1][1],
                                                     dw[cc >> 1][cc & 1][2], dw[cc >> 1][cc & 1][3]});
        dvacc[db] = E::mfma(otr[s % (PF + 1)], pf, dvacc[db]);
        dkacc[db] = E::mfma(qtr[s % (PF + 1)], df, dkacc[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Tile i+1 must have landed; this iteration's copies may stay in flight.
    dma_sync<DMA_OPS>();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  if (i0 < nq) {
    issue_tile(i0, 0);
    issue_tile(i0 + 1, 1);
    dma_sync<DMA_OPS>();
    int st = 0, i = i0;
    for (; i < i_unmask; ++i) {
      iteration(T_{}, i, st);
      st = st == 2 ? 0 : st + 1;
    }
    for (; i < nq; ++i) {
      iteration(F_{}, i, st);
      st = st == 2 ? 0 : st + 1;
    }
  }
  wait_vmcnt<0>();  // copies past the last tile must land before LDS is released

  // dK = scale * dS'^T Q and dV for this lane's key: register r
  // of head-dim block db is head dim db*32 + 8*(r/4) + 4*hl + r%4.
  if (key < N) {
    uint16_t* dkrow = static_cast<uint16_t*>(a.dk) + base + (int64_t)key * D;
    uint16_t* dvrow = static_cast<uint16_t*>(a.dv) + base + (int64_t)key * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hl;
        u32x2_t w;
        w[0] = E::pack2(dkacc[db][4 * g + 0] * a.scale, dkacc[db][4 * g + 1] * a.scale);
        w[1] = E::pack2(dkacc[db][4 * g + 2] * a.scale, dkacc[db][4 * g + 3] * a.scale);
        *reinterpret_cast<u32x2_t*>(dkrow + d0) = w;
        w[0] = E::pack2(dvacc[db][4 * g + 0], dvacc[db][4 * g + 1]);
        w[1] = E::pack2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
        *reinterpret_cast<u32x2_t*>(dvrow + d0) = w;
      }
    }
  }
}


// dQ by recomputation, query-stationary: one workgroup per (b, h, tile of
// BM = 32*NW queries), wave w owns queries [32 w, 32 w + 32).  Like the
// forward, keys are accumulator rows and the wave's queries are columns (one
// query per lane), so the row statistics are per-lane scalars.  Per key tile
// t of BN keys:
//   S^T = K_t Q^T and dP^T = V_t dO^T on matrix cores (K and V read from LDS
//     as rows),
//   P^T = exp2((S^T - LSE/scale) * scale * log2 e),
//   dS'^T = P^T o (dP^T - D), rounded to the input type,
//   dQ^T += K_t^T dS'^T (K read from LDS by transposed reads); dQ = scale *
//     dQ^T^T is scaled once at the end.
// K and V tiles stream through a three-stage ring filled by buffer loads with
// an LDS destination; two waves share each SIMD, so one wave's vector work
// overlaps the other's matrix work.
template <int D, int BN, int NW, bool CAUSAL, int DT>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_kernel(BwdArgs a) {
  using E = Elem<DT>;
  using v8 = typename E::v8;
  constexpr int BM = 32 * NW;
  constexpr int NSTG = 3;
  constexpr int ROWB = 2 * D;
  constexpr int TILEB = BN * ROWB;
  constexpr int CH_ROW = D / 8;
  static_assert(TILEB % (1024 * NW) == 0, "a tile must split into whole 1 KiB copies per wave");
  constexpr int IPW = TILEB / 1024 / NW;
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;
  constexpr int NDC = D / 16;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * NSTG * TILEB];
  FA_LDS uint8_t* lds = (FA_LDS uint8_t*)smem;  // K stage s at s*TILEB, V at (NSTG+s)*TILEB

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int N = a.N;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / a.n_ktiles;  // n_ktiles holds the query-tile count here
  int qt = logical % a.n_ktiles;
  if (CAUSAL) qt = a.n_ktiles - 1 - qt;  // longest key ranges first
  const int64_t base = (int64_t)bh * N * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.q) + base;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + base;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v) + base;
  const uint16_t* dOg = static_cast<const uint16_t*>(a.dout) + base;
  const f32x2_t* statg = reinterpret_cast<const f32x2_t*>(a.dsum) + (int64_t)bh * N;

  const int q0 = qt * BM;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;
  const float c = a.scale_log2;

  // Copies: as in the forward (rows past N arrive as zeros).
  uint32_t dma_voff[IPW];
#pragma unroll
  for (int jj = 0; jj < IPW; ++jj) {
    const int p = (wave * IPW + jj) * 64 + lane;
    dma_voff[jj] = (uint32_t)((p / CH_ROW) * ROWB + ((p % CH_ROW) ^ swz<D>(p / CH_ROW)) * 16);
  }
  auto issue = [&](int t, int st) {
    const int rows = min(max(N - t * BN, 0), BN);
    const u32x4_t rk = make_rsrc(Kg + (int64_t)t * BN * D, rows * ROWB);
    const u32x4_t rv = make_rsrc(Vg + (int64_t)t * BN * D, rows * ROWB);
#pragma unroll
    for (int jj = 0; jj < IPW; ++jj) {
      dma16_buf(rk, dma_voff[jj], lds + st * TILEB + (wave * IPW + jj) * 1024);
      dma16_buf(rv, dma_voff[jj], lds + (NSTG + st) * TILEB + (wave * IPW + jj) * 1024);
    }
  };

  // Q and dO rows of this lane's query as B operands (head-dim slots
  // dc*16 + 8*hl + [0, 8)); row statistics as scalars.
  v8 qf[NDC], of[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
    u32x4_t rq = {0u, 0u, 0u, 0u}, ro = {0u, 0u, 0u, 0u};
    if (qrow < N) {
      rq = ld_global16(Qg + (int64_t)qrow * D + dc * 16 + 8 * hl);
      ro = ld_global16(dOg + (int64_t)qrow * D + dc * 16 + 8 * hl);
    }
    qf[dc] = __builtin_bit_cast(v8, rq);
    of[dc] = __builtin_bit_cast(v8, ro);
  }
  f32x2_t stat = {0.f, 0.f};
  if (qrow < N) stat = statg[qrow];  // (-LSE/scale, -D)
  const float pbias = stat[0] * c;    // -LSE * log2 e

  f32x16_t dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[i][r] = 0.f;

  // LDS read offsets: rows (K, V as A operands of S^T, dP^T) and transposed
  // reads (K^T as A operand of dQ^T), exactly as the forward's K and V reads.
  int koff[NDC];
  {
    const int f = swz<D>(l32);
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) koff[dc] = l32 * ROWB + 16 * ((2 * dc + hl) ^ f);
  }
  int toff[NDB][2];
  {
    const int e = (lane & 15) >> 2, c4 = lane & 3, g2 = (lane >> 4) & 1;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 4 * hl + e + 8 * hi;
      const int f = swz<D>(r);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        toff[db][hi] = r * ROWB + 16 * ((4 * db + 2 * g2 + (c4 >> 1)) ^ f) + 8 * (c4 & 1);
    }
  }
  auto ld_row = [&](const FA_LDS uint8_t* t, int kb, int dc) {
    return __builtin_bit_cast(v8, ld_lds16(t + kb * 32 * ROWB + koff[dc]));
  };
  auto ld_tr = [&](const FA_LDS uint8_t* t, int cc, int db) {
    const s16x4_t lo = ld_lds_tr16(t + cc * 16 * ROWB + toff[db][0]);
    const s16x4_t hi = ld_lds_tr16(t + cc * 16 * ROWB + toff[db][1]);
    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    return __builtin_bit_cast(v8, u32x4_t{l2[0], l2[1], h2[0], h2[1]});
  };

  int t_mask = ntiles;
  if (CAUSAL) t_mask = min(t_mask, (q0 + 1) / BN);

  // One key tile from stage st.
  auto tile = [&](auto m_tag, int t, int st) {
    constexpr bool MASKED = decltype(m_tag)::value;
    const FA_LDS uint8_t* ks = lds + st * TILEB;
    const FA_LDS uint8_t* vs = lds + (NSTG + st) * TILEB;
    issue(t + NSTG - 1, st == 0 ? NSTG - 1 : st - 1);  // refill the stage read last iteration
    f32x16_t sacc[NKB], dpacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[kb][r] = 0.f;
        dpacc[kb][r] = 0.f;
      }
    {
      constexpr int PF = 2, NST = NKB * NDC;
      v8 kr[PF + 1], vr[PF + 1];
      auto load = [&](int s) {
        kr[s % (PF + 1)] = ld_row(ks, s / NDC, s % NDC);
        vr[s % (PF + 1)] = ld_row(vs, s / NDC, s % NDC);
      };
#pragma unroll
      for (int s = 0; s < PF; ++s) load(s);
#pragma unroll
      for (int s = 0; s < NST; ++s) {
        if (s + PF < NST) load(s + PF);
        const int kb = s / NDC, dc = s % NDC;
        sacc[kb] = E::mfma(kr[s % (PF + 1)], qf[dc], sacc[kb]);
        dpacc[kb] = E::mfma(vr[s % (PF + 1)], of[dc], dpacc[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Register r of block kb holds key t*BN + kb*32 + 8*(r/4) + 4*hl + r%4.
    uint32_t dw[NKB][8];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float ds2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 2 * w + u;
          float pv = fast_exp2(fmaf(sacc[kb][r], c, pbias));
          if constexpr (MASKED) {
            const int key = t * BN + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (key > qrow) pv = 0.f;
          }
          ds2[u] = pv * (dpacc[kb][r] + stat[1]);
        }
        dw[kb][w] = E::pack2(ds2[0], ds2[1]);
      }
    {
      // dQ^T += K^T dS^T, 16 keys per instruction (chunk cc: registers
      // 8*(cc%2)..+7 of block cc/2, the same key order as the K^T read).
      constexpr int PF = 2, NST = (BN / 16) * NDB;
      v8 ktr[PF + 1];
      auto load = [&](int s) { ktr[s % (PF + 1)] = ld_tr(ks, s / NDB, s % NDB); };
#pragma unroll
      for (int s = 0; s < PF; ++s) load(s);
#pragma unroll
      for (int s = 0; s < NST; ++s) {
        if (s + PF < NST) load(s + PF);
        const int cc = s / NDB, db = s % NDB;
        const int j0 = 4 * (cc & 1);
        const v8 df = __builtin_bit_cast(v8, u32x4_t{dw[cc >> 1][j0], dw[cc >> 1][j0 + 1],
                                                     dw[cc >> 1][j0 + 2], dw[cc >> 1][j0 + 3]});
        dqacc[db] = E::mfma(ktr[s % (PF + 1)], df, dqacc[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    dma_sync<2 * IPW * (NSTG - 2)>();  // tile t+1 has landed; tile t+2 may be in flight
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  issue(0, 0);
  issue(1, 1);
  dma_sync<2 * IPW>();
  int t = 0, st = 0;
  for (; t < t_mask; ++t) {
    tile(F_{}, t, st);
    st = st == NSTG - 1 ? 0 : st + 1;
  }
  for (; t < ntiles; ++t) {
    tile(T_{}, t, st);
    st = st == NSTG - 1 ? 0 : st + 1;
  }
  wait_vmcnt<0>();  // copies past the last tile must land before LDS is released

  // dQ^T register r of block db is head dim db*32 + 8*(r/4) + 4*hl + r%4 of
  // this lane's query.
  if (qrow < N) {
    float* dqrow = a.dq + base + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4_t*>(dqrow + db * 32 + 8 * g + 4 * hl) =
            f32x4_t{dqacc[db][4 * g], dqacc[db][4 * g + 1], dqacc[db][4 * g + 2], dqacc[db][4 * g + 3]} *
            a.scale;
  }
}

template <int D, int NW, int BQ, int DQ_BN, int DQ_NW, int DT>
hipError_t launch_d(const BwdArgs& a0, int BH, bool causal, hipStream_t s) {
  BwdArgs a = a0;
  const int64_t rows = (int64_t)BH * a.N;
  constexpr int TPR = D / 8;
  const int64_t pre_blocks = (rows * TPR + 255) / 256;
  if (pre_blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_pre_kernel<D, DT>), dim3((unsigned)pre_blocks), dim3(256), 0, s,
                     static_cast<const uint16_t*>(a.o), static_cast<const uint16_t*>(a.dout),
                     a.lse, reinterpret_cast<f32x2_t*>(a.dsum), rows, 1.0f / a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int BKV = 32 * NW;
  a.n_ktiles = (a.N + BKV - 1) / BKV;
  int64_t grid = (int64_t)a.n_ktiles * BH;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (causal)
    hipLaunchKernelGGL((bwd_kv_kernel<D, NW, BQ, true, DT>), dim3((unsigned)grid), dim3(NW * 64),
                       0, s, a);
  else
    hipLaunchKernelGGL((bwd_kv_kernel<D, NW, BQ, false, DT>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int BM = 32 * DQ_NW;
  a.n_ktiles = (a.N + BM - 1) / BM;  // query tiles for the dQ kernel
  grid = (int64_t)a.n_ktiles * BH;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (causal)
    hipLaunchKernelGGL((bwd_dq_kernel<D, DQ_BN, DQ_NW, true, DT>), dim3((unsigned)grid),
                       dim3(DQ_NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, DQ_BN, DQ_NW, false, DT>), dim3((unsigned)grid),
                       dim3(DQ_NW * 64), 0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dtype(const BwdArgs& a, int BH, int d, bool causal, hipStream_t s) {
  switch (d) {
    case 64: return launch_d<64, 4, 64, 64, 8, DT>(a, BH, causal, s);
    case 128: return launch_d<128, 4, 64, 64, 8, DT>(a, BH, causal, s);
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
