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
// Kernels, in launch order (bwd_dq_kernel first: it also forms the row
// statistics, which bwd_kv3_kernel reads):
//   bwd_dq_kernel   one workgroup per (b, h, tile of 32*NW queries), built like
//                   the forward: Q and dO rows stay in registers, K and V tiles
//                   stream through a four-stage LDS ring (one workgroup
//                   barrier per pair of key tiles); per key tile it
//                   recomputes S^T = K Q^T and dP^T = V dO^T, forms dS^T and
//                   accumulates dQ^T += K^T dS^T in registers, written once at
//                   the end.  Recomputing two products costs 2/5 more matrix
//                   work than accumulating dQ with atomics from the dK/dV pass,
//                   whose fp32 atomic traffic (every key tile adds a full dQ
//                   tile) is bound by the L2 atomic units.  At its start it
//                   writes each of its query rows' -LSE / scale and -D into
//                   two planes of the workspace (all rows of one, then all
//                   rows of the other).
//   bwd_kv3_kernel  one workgroup of 8 waves per (b, h, tile of 128 keys); the
//                   four 32-key blocks each get two waves that share a SIMD:
//                   one keeps the block's K rows and dV accumulator (S, P,
//                   dV^T += dO^T P), the other its V rows and dK accumulator
//                   (dP, dS = P o (dP - D), dK^T += Q^T dS, one tile late); P
//                   passes between them through two LDS buffers in the input
//                   type.  Query tiles of 64 rows (Q, dO, row statistics)
//                   stream through a three-stage LDS ring filled by buffer
//                   loads with an LDS destination; one barrier per tile.  Keys
//                   are accumulator columns (one key per lane); Q and dO are
//                   read from LDS as rows (S, dP) and by transposed 16-bit
//                   reads (dV, dK).  The S and dP accumulators start from the
//                   row statistics, and dK = scale * dS^T Q is scaled once at
//                   the end.
//   Rows past N (queries or keys) arrive as zeros; every product they enter
//   is then exactly zero or never stored, so only the causal mask is applied.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

// LDS fragments read ahead of the matrix products in bwd_kv3_kernel (row
// and transposed reads alike).
#ifndef FA_KV_PF
#define FA_KV_PF 2
#endif

namespace fa {

namespace {

template <int DT> __device__ __forceinline__ float to_f32(uint16_t x);
template <> __device__ __forceinline__ float to_f32<0>(uint16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}
template <> __device__ __forceinline__ float to_f32<1>(uint16_t x) {
  return (float)__builtin_bit_cast(_Float16, x);
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



// Key-stationary dK/dV with two wave roles per 32-key block, so that two
// waves share each SIMD and one's vector work overlaps the other's matrix
// work.  One workgroup = 8 waves = 128 keys; wave w takes key block w % 4
// (waves w and w + 4 share a SIMD) and role w / 4.  Each wave keeps only its
// side's stationary operand (K or V rows of its 32 keys) and accumulator (dV
// or dK): half of what one wave holding both would need, so two waves fit per
// SIMD.  One barrier per query tile, and the same matrix work in both roles:
//   role 0 (S side):  S(i), P(i) = exp2(..) (causal mask), P(i) to LDS in the
//                     input type, dV^T += dO(i)^T P(i)          (32 products)
//   role 1 (dP side): dS'(i-1) = P(i-1) o (dP(i-1) - D) with P(i-1) from LDS
//                     and dP(i-1) - D kept in registers since the previous
//                     tile, dK^T += Q(i-1)^T dS'(i-1), then dP(i) - D
//                                                               (32 products)
//   barrier: P(i) published, tile i+1 landed.
// P passes through two LDS buffers (tile parity), so the single barrier per
// tile orders both its writes and its reads.  P is exchanged in the input
// type (the same rounding that feeds dV^T += dO^T P), which keeps both
// buffers inside LDS next to three query-tile stages; dS' is formed from it
// in fp32.  Tile i+1 is copied at the start of tile i into the stage of tile
// i-2, free since the previous barrier.
template <int D, int BQ, bool CAUSAL, int DT, bool PERSIST>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_kv3_kernel(BwdArgs a) {
  using E = Elem<DT>;
  using v8 = typename E::v8;
  constexpr int NW = 8;
  constexpr int BKV = 128;
  constexpr int ROWB = 2 * D;
  constexpr int QTB = BQ * ROWB;
  constexpr int RSB = 2048;          // row statistics of a tile: -LSE/scale, -D (1 KiB each)
  constexpr int STAGEB = 2 * QTB + RSB;
  constexpr int NSTG = 3;
  constexpr int NQB = BQ / 32;
  constexpr int PBUF = 4 * 64 * NQB * 2 * 16;  // P of the four key blocks, one tile
  constexpr int CH_ROW = D / 8;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  static_assert(QTB % (1024 * NW) == 0, "a Q tile must split into whole 1 KiB copies per wave");
  static_assert(BQ == 64, "four 16-byte P chunks per lane");
  constexpr int IPW = QTB / 1024 / NW;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTG * STAGEB + 2 * PBUF];
  FA_LDS uint8_t* lds = (FA_LDS uint8_t*)smem;
  FA_LDS uint8_t* p_lds = lds + NSTG * STAGEB;

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int kb = wave & 3;
  const int N = a.N;

  // One work unit: key tile kt of head bh.
  auto unit = [&](const int bh, const int kt) {
  // The lane index passes through an empty asm so that nothing derived from
  // it is hoisted out of a loop over units (it would stay live across units
  // and spill at the register limit).
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int64_t base = (int64_t)bh * N * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.q) + base;
  const uint16_t* dOg = static_cast<const uint16_t*>(a.dout) + base;
  const float* stat_lse = a.dsum + (int64_t)bh * N;
  const float* stat_d = a.dsum + a.plane + (int64_t)bh * N;

  const int k0 = kt * BKV;
  const int key = k0 + kb * 32 + l32;  // this lane's key (accumulator column)

  // ---- Copies (rows outside [0, N) arrive as zeros).
  uint32_t dma_voff[IPW];
#pragma unroll
  for (int jj = 0; jj < IPW; ++jj) {
    const int p = (wave * IPW + jj) * 64 + lane;
    dma_voff[jj] = (uint32_t)((p / CH_ROW) * ROWB + ((p % CH_ROW) ^ swz<D>(p / CH_ROW)) * 16);
  }
  auto tile_rows = [&](int r0) { return (r0 < 0 || r0 >= N) ? 0 : min(N - r0, BQ); };
  auto copy_rows = [&](const uint16_t* src, int r0, FA_LDS uint8_t* dst) {
    const u32x4_t r = make_rsrc(src + (int64_t)max(r0, 0) * D, tile_rows(r0) * ROWB);
#pragma unroll
    for (int jj = 0; jj < IPW; ++jj) {
      if (jj == 0) dma16_buf<4>(r, dma_voff[jj], dst + (wave * IPW + jj) * 1024);
      else dma16_buf<0>(r, dma_voff[jj], dst + (wave * IPW + jj) * 1024);
    }
  };
  auto issue_tile = [&](int i, int st) {
    FA_LDS uint8_t* sb = lds + st * STAGEB;
    const int q0 = i * BQ;
    copy_rows(Qg, q0, sb);
    copy_rows(dOg, q0, sb + QTB);
    if (wave < 2) {  // wave 0: -LSE/scale, wave 1: -D (64 rows = 256 bytes)
      const u32x4_t r = make_rsrc((wave == 0 ? stat_lse : stat_d) + max(q0, 0), tile_rows(q0) * 4);
      dma16_buf(r, (uint32_t)lane * 16, sb + 2 * QTB + wave * 1024);
    }
  };
  // Every copy issued so far has landed, this wave's LDS writes are
  // complete, then the workgroup barrier.
  auto tile_sync = [&]() {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt, expcnt untouched
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  int roff[NDC];
  {
    const int f = swz<D>(l32);
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) roff[dc] = l32 * ROWB + 16 * ((2 * dc + hl) ^ f);
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
  auto ld_row = [&](const FA_LDS uint8_t* t, int qb, int dc) {
    return __builtin_bit_cast(v8, ld_lds16(t + qb * 32 * ROWB + roff[dc]));
  };
  auto ld_tr = [&](const FA_LDS uint8_t* t, int cc, int db) {
    const s16x4_t lo = ld_lds_tr16(t + cc * 16 * ROWB + toff[db][0]);
    const s16x4_t hi = ld_lds_tr16(t + cc * 16 * ROWB + toff[db][1]);
    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    return __builtin_bit_cast(v8, u32x4_t{l2[0], l2[1], h2[0], h2[1]});
  };
  // P exchange: per key block, 64 lanes x 64 bytes (chunk m = the packed
  // words pw[m/2][m%2], queries 16 m .. 16 m + 15), chunk index XOR-swizzled
  // by a function of lane bits 1-3 such that any 8 consecutive lanes hit 8
  // different 16-byte units of a 128-byte window and any 16 consecutive lanes
  // 16 different units of a 256-byte window: 16-byte LDS accesses are served
  // eight lanes at a time (a swizzle by (lane / 4) % 4, distinct only over 16
  // lanes, measured 8.7 % of the kernel's LDS cycles in bank conflicts; this
  // one none).
  const int pswz = (((lane >> 1) & 1) | (((lane >> 2) & 1) << 1)) ^ (((lane >> 3) & 1) * 3);
  auto pchunk = [&](int buf, int m) {
    return p_lds + buf * PBUF + kb * (64 * 64) + lane * 64 + 16 * (m ^ pswz);
  };

  const int nq = (N + BQ - 1) / BQ;
  const int i0 = CAUSAL ? k0 / BQ : 0;
  const int i_unmask = CAUSAL ? min(nq, (k0 + BKV + BQ - 2) / BQ) : i0;

  auto run = [&](auto role_tag) {
    constexpr int ROLE = decltype(role_tag)::value;
    v8 kvf[NDC];
    {
      const uint16_t* src = static_cast<const uint16_t*>(ROLE == 0 ? a.k : a.v) + base;
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        u32x4_t rk = {0u, 0u, 0u, 0u};
        if (key < N) rk = ld_global16(src + (int64_t)key * D + dc * 16 + 8 * hl);
        kvf[dc] = __builtin_bit_cast(v8, rk);
      }
    }
    // Completing these loads before the first copy is issued tells the
    // compiler that no load of its own is outstanding inside the loop.
    wait_vmcnt<0>();
    f32x16_t acc[NDB];  // dV^T (role 0) or dK^T / scale (role 1)
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    // sacc: S - LSE/scale (role 0, this tile) or dP - D (role 1, kept one
    // tile); register r of block qb is query row qb*32 + 8*(r/4) + 4*hl + r%4.
    f32x16_t sacc[NQB];
    uint32_t pw[NQB][2][4];  // P (role 0) or dS' (role 1) as B operands

    auto load_stats = [&](const FA_LDS uint8_t* sb) {
      const FA_LDS uint8_t* ps = sb + 2 * QTB + ROLE * 1024 + 16 * hl;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4_t v = *(const FA_LDS f32x4_t*)(ps + (qb * 32 + 8 * g) * 4);
#pragma unroll
          for (int t = 0; t < 4; ++t) sacc[qb][4 * g + t] = v[t];
        }
    };
    // A tile's matrix work is a stream of row products (sacc += T K^T or
    // T V^T over rows T, block qb = k / NDC) and transposed products (acc +=
    // T^T W over 16-query chunks cc = k / NDB), NH of each, in the order of
    // the role (HALVES = 1: the first kind only).  Fragments are read PF
    // instructions ahead, across the two halves.  After the product of step
    // m comes vec(m), a share of the vector work, so that a wave forms its
    // probabilities or dS' words under its own products rather than between
    // them.
    constexpr int NH = NQB * NDC;
    static_assert(NH == NDB * (BQ / 16), "both halves have the same length");
    auto stream = [&](auto rows_first_tag, auto halves_tag, const FA_LDS uint8_t* rsrc,
                      const FA_LDS uint8_t* tsrc, auto&& vec) {
      constexpr bool ROWS_FIRST = decltype(rows_first_tag)::value;
      constexpr int NM = decltype(halves_tag)::value * NH;
      constexpr int PF = FA_KV_PF;
      auto is_row = [](int m) { return ROWS_FIRST ? m < NH : m >= NH; };
      auto frag = [&](int m) {
        const int k = m % NH;
        return is_row(m) ? ld_row(rsrc, k / NDC, k % NDC) : ld_tr(tsrc, k / NDB, k % NDB);
      };
      v8 fr[PF + 1];
#pragma unroll
      for (int m = 0; m < PF; ++m) fr[m] = frag(m);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (m + PF < NM) fr[(m + PF) % (PF + 1)] = frag(m + PF);
        const int k = m % NH;
        if (is_row(m)) {
          sacc[k / NDC] = E::mfma(fr[m % (PF + 1)], kvf[k % NDC], sacc[k / NDC]);
        } else {
          const int cc = k / NDB, db = k % NDB;
          const uint32_t* w = pw[cc >> 1][cc & 1];
          acc[db] = E::mfma(fr[m % (PF + 1)], __builtin_bit_cast(v8, u32x4_t{w[0], w[1], w[2], w[3]}),
                            acc[db]);
        }
        vec(m);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    static_assert(NQB == 2, "two query blocks per tile");
    // Role 1: dS' of the previous tile from its P (buffer pb) and the kept
    // dP - D, dK^T += Q^T dS' over that tile's rows qprev, then (DP) dP - D
    // of the current tile over its dO rows (stage sb).  Block 0's first four
    // words are formed before the first product (chunk 0 uses them), its
    // other four under chunk 0's products, block 1's under chunk 1's; then
    // sacc is free and the row statistics are read, well ahead of the dP
    // products.  The dS' + dK phase is the critical path of a tile: it runs
    // at raised priority, so the S side's products fill in around it (2-4 %
    // faster than equal priorities; raising either role for the whole tile
    // was slower at d = 128).
    auto dk_tile = [&](int pb, const FA_LDS uint8_t* qprev, auto dp_tag, const FA_LDS uint8_t* sb) {
      constexpr bool DP = decltype(dp_tag)::value;
      u32x4_t pp[NQB][2];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int h = 0; h < 2; ++h) pp[qb][h] = *(const FA_LDS u32x4_t*)pchunk(pb, qb * 2 + h);
      auto dsword = [&](int qb, int x) {
        // Word x = 4h + w holds registers 8h + 2w, 8h + 2w + 1 of block qb.
        const int h = x >> 2, w = x & 3, r = 8 * h + 2 * w;
        const uint32_t word = pp[qb][h][w];
        const float lo = to_f32<DT>((uint16_t)(word & 0xffffu));
        const float hi = to_f32<DT>((uint16_t)(word >> 16));
        pw[qb][h][w] = E::pack2(lo * sacc[qb][r], hi * sacc[qb][r + 1]);
      };
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int x = 0; x < 4; ++x) dsword(0, x);
      stream(std::false_type{}, std::integral_constant<int, DP ? 2 : 1>{}, sb + QTB, qprev,
             [&](int m) {
#pragma unroll
               for (int y = 0; y < 4; ++y)
                 if (m == (y * NDB) / 4) dsword(0, 4 + y);
#pragma unroll
               for (int x = 0; x < 8; ++x)
                 if (m == NDB + (x * NDB) / 8) dsword(1, x);
               if constexpr (DP) {
                 if (m == 2 * NDB - 1) load_stats(sb);
                 if (m == NH - 1) __builtin_amdgcn_s_setprio(0);
               }
             });
      if constexpr (!DP) __builtin_amdgcn_s_setprio(0);
    };

    auto iteration = [&](auto m_tag, auto first_tag, int i, int st) {
      constexpr bool MASKED = decltype(m_tag)::value;
      constexpr bool FIRST = decltype(first_tag)::value;
      const FA_LDS uint8_t* sb = lds + st * STAGEB;
      const int q0 = i * BQ;
      issue_tile(i + 1, st == 2 ? 0 : st + 1);  // the stage of tile i-2
      if constexpr (ROLE == 0) {
        // S(i) over Q rows (block 0, then block 1), then dV^T += dO(i)^T P(i)
        // (chunks 0-1 use block 0's P, 2-3 block 1's).  Block 0's P words
        // are formed under block 1's S products, block 1's under the first
        // half of the dV products; each 16-byte P chunk goes to LDS once
        // complete.
        const float c = a.scale_log2;
        auto pword = [&](int qb, int x) {
          const int h = x >> 2, w = x & 3, r = 8 * h + 2 * w;
          float p0 = fast_exp2(sacc[qb][r] * c), p1 = fast_exp2(sacc[qb][r + 1] * c);
          if constexpr (MASKED) {
            const int q = q0 + qb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (key > q) p0 = 0.f;
            if (key > q + 1) p1 = 0.f;
          }
          pw[qb][h][w] = E::pack2(p0, p1);
          if (w == 3)
            *(FA_LDS u32x4_t*)pchunk(i & 1, qb * 2 + h) =
                u32x4_t{pw[qb][h][0], pw[qb][h][1], pw[qb][h][2], pw[qb][h][3]};
        };
        load_stats(sb);
        stream(std::true_type{}, std::integral_constant<int, 2>{}, sb, sb + QTB, [&](int m) {
          constexpr int H2 = NH / 2;
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            if (m == H2 + (x * H2) / 8) pword(0, x);
            if (m == NH + (x * H2) / 8) pword(1, x);
          }
        });
      } else if constexpr (FIRST) {
        // dP(i) - D only.
        load_stats(sb);
        stream(std::true_type{}, std::integral_constant<int, 1>{}, sb + QTB, sb, [](int) {});
      } else {
        dk_tile((i - 1) & 1, lds + (st == 0 ? 2 : st - 1) * STAGEB, std::true_type{}, sb);
      }
      tile_sync();  // P(i) published; tile i+1 landed
    };
    using T_ = std::true_type;
    using F_ = std::false_type;

    if (i0 < nq) {
      issue_tile(i0, 0);
      tile_sync();
      int st = 0, i = i0;
      if (i < i_unmask)
        iteration(T_{}, T_{}, i, st);
      else
        iteration(F_{}, T_{}, i, st);
      st = 1;
      ++i;
      for (; i < i_unmask; ++i) {
        iteration(T_{}, F_{}, i, st);
        st = st == 2 ? 0 : st + 1;
      }
      for (; i < nq; ++i) {
        iteration(F_{}, F_{}, i, st);
        st = st == 2 ? 0 : st + 1;
      }
      // Role 1: dK of the last tile (its P was published by the last barrier).
      if constexpr (ROLE == 1)
        dk_tile((nq - 1) & 1, lds + (st == 0 ? 2 : st - 1) * STAGEB, std::false_type{}, lds);
    }
    wait_vmcnt<0>();  // copies past the last tile must land before LDS is released

    // A lane holds its key's row in 8-byte pieces, so stores straight from
    // the accumulators would scatter each instruction over 32 rows.  Once
    // every wave is done with the ring, each writes its 32 rows into it
    // (padded by 8 bytes, so the 8-byte writes of one half-wave hit distinct
    // banks) and stores whole rows, 16 bytes per lane.
    constexpr int OROWB = 2 * D + 8;
    static_assert(NW * 32 * OROWB <= NSTG * STAGEB, "the dK / dV blocks fit in the ring");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    FA_LDS uint8_t* ost = lds + wave * 32 * OROWB;
    const float f = ROLE == 0 ? 1.0f : a.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2_t w;
        w[0] = E::pack2(acc[db][4 * g + 0] * f, acc[db][4 * g + 1] * f);
        w[1] = E::pack2(acc[db][4 * g + 2] * f, acc[db][4 * g + 3] * f);
        *reinterpret_cast<FA_LDS u32x2_t*>(ost + l32 * OROWB + 2 * (db * 32 + 8 * g + 4 * hl)) = w;
      }
    }
    asm volatile("" ::: "memory");
    {
      constexpr int LPR = D / 8;     // lanes per row, 16 bytes each
      constexpr int RPI = 64 / LPR;  // rows per store instruction
      const int r0 = lane / LPR, cb = (lane % LPR) * 16;
      const int key0 = k0 + kb * 32;
      uint8_t* dst = static_cast<uint8_t*>(ROLE == 0 ? a.dv : a.dk) + 2 * (base + (int64_t)key0 * D);
#pragma unroll
      for (int k = 0; k < 32 / RPI; ++k) {
        const int r = r0 + RPI * k;
        const u32x4_t v = ld_lds16(ost + r * OROWB + cb);
        if (key0 + r < N) *reinterpret_cast<u32x4_t*>(dst + 2 * (int64_t)r * D + cb) = v;
      }
    }
  };
  if (wave < 4)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});
  };  // unit

  if constexpr (PERSIST) {
    // Causal: key tile kt meets the query tiles from its diagonal on, so
    // rank 0 (the heaviest) is key tile 0.
    lpt_units(a.n_ktiles, a.bh, a.pin != 0, [&](int bh, int rank, int, int) {
      unit(bh, rank);
      // The next unit's first copies reuse the ring and the P buffers.
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    });
  } else {
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    unit(logical / a.n_ktiles, logical % a.n_ktiles);
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
// K and V tiles stream through a four-stage ring filled by buffer loads with
// an LDS destination, two tiles per workgroup barrier; two waves share each
// SIMD, so one wave's vector work overlaps the other's matrix work.
template <int D, int BN, int NW, bool CAUSAL, int DT, bool PERSIST>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_kernel(BwdArgs a) {
  using E = Elem<DT>;
  using v8 = typename E::v8;
  constexpr int BM = 32 * NW;
  // Four stages, tiles in pairs with one barrier per pair (measured 3-7 %
  // faster for the whole backward than three stages and a barrier per tile,
  // which the code below also supports with NSTG = 3).
  constexpr int NSTG = 4;
  constexpr bool PAIR = NSTG == 4;
  constexpr int ROWB = 2 * D;
  constexpr int TILEB = BN * ROWB;
  constexpr int CH_ROW = D / 8;
  static_assert(TILEB % (1024 * NW) == 0, "a tile must split into whole 1 KiB copies per wave");
  constexpr int IPW = TILEB / 1024 / NW;
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;
  constexpr int NDC = D / 16;

  // dQ leaves through LDS in fp32 rows padded by 16 bytes: at d = 128 the
  // eight waves' blocks (132 KiB) exceed the ring, which is sized up.
  constexpr int OROWB = 4 * D + 16;
  constexpr int SMEM = 2 * NSTG * TILEB > NW * 32 * OROWB ? 2 * NSTG * TILEB : NW * 32 * OROWB;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
  FA_LDS uint8_t* lds = (FA_LDS uint8_t*)smem;  // K stage s at s*TILEB, V at (NSTG+s)*TILEB

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int N = a.N;

  // One work unit: query tile qt of head bh.
  auto unit = [&](const int bh, const int qt) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // as in the dK/dV kernel: nothing hoisted
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int64_t base = (int64_t)bh * N * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.q) + base;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + base;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v) + base;
  const uint16_t* dOg = static_cast<const uint16_t*>(a.dout) + base;
  float* stat_lse = a.dsum + (int64_t)bh * N;
  float* stat_d = a.dsum + a.plane + (int64_t)bh * N;

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
      if (jj == 0) {
        dma16_buf<4>(rk, dma_voff[jj], lds + st * TILEB + (wave * IPW + jj) * 1024);
        dma16_buf<4>(rv, dma_voff[jj], lds + (NSTG + st) * TILEB + (wave * IPW + jj) * 1024);
      } else {
        dma16_buf<0>(rk, dma_voff[jj], lds + st * TILEB + (wave * IPW + jj) * 1024);
        dma16_buf<0>(rv, dma_voff[jj], lds + (NSTG + st) * TILEB + (wave * IPW + jj) * 1024);
      }
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
  // The row statistics (-LSE/scale, -D) of this lane's query, D =
  // rowsum(dO o O): the lane holds half of the head dimension of dO already
  // and reads the same half of O; the other half is on lane l ^ 32.  This
  // kernel runs first and leaves them in the workspace for the dK/dV kernel.
  float dpart = 0.f;
  if (qrow < N) {
    const uint16_t* Og = static_cast<const uint16_t*>(a.o) + base + (int64_t)qrow * D;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      const u32x4_t o = ld_global16(Og + dc * 16 + 8 * hl);
      const u32x4_t g = __builtin_bit_cast(u32x4_t, of[dc]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dpart += to_f32<DT>((uint16_t)(o[i] & 0xffff)) * to_f32<DT>((uint16_t)(g[i] & 0xffff));
        dpart += to_f32<DT>((uint16_t)(o[i] >> 16)) * to_f32<DT>((uint16_t)(g[i] >> 16));
      }
    }
  }
  const float dsum = sum_halves(dpart);
  f32x2_t stat = {0.f, 0.f};
  if (qrow < N) {
    stat = f32x2_t{-a.lse[(int64_t)bh * N + qrow] * a.inv_scale, -dsum};
    if (hl == 0) {
      stat_lse[qrow] = stat[0];
      stat_d[qrow] = stat[1];
    }
  }
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
  auto tile = [&](auto m_tag, auto second_tag, int t, int st) {
    constexpr bool MASKED = decltype(m_tag)::value;
    constexpr bool SECOND = decltype(second_tag)::value;
    if constexpr (PAIR) st = t & 3;
    const FA_LDS uint8_t* ks = lds + st * TILEB;
    const FA_LDS uint8_t* vs = lds + (NSTG + st) * TILEB;
    if constexpr (!PAIR) {
      issue(t + NSTG - 1, st == 0 ? NSTG - 1 : st - 1);  // refill the stage read last iteration
    } else if constexpr (!SECOND) {
      // Tiles in pairs (t even, t + 1), one barrier per pair: the first
      // copies the next pair's tiles into the stages the previous pair read.
      issue(t + 2, (t + 2) & 3);
      issue(t + 3, (t + 3) & 3);
    }
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
        // Two waves share each SIMD: hand the issue lead over within a tile.
        if (s == 0) __builtin_amdgcn_s_setprio(1);
        if (s == NST - 1) __builtin_amdgcn_s_setprio(0);
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
          // (The masked body also runs for a pair whose first tile needs no
          // mask, and in the non-causal kernel for the tail pair.)
          if constexpr (MASKED && CAUSAL) {
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
    if constexpr (!PAIR)
      dma_sync<2 * IPW * (NSTG - 2)>();  // tile t+1 has landed; tile t+2 may be in flight
    else if constexpr (SECOND)
      dma_sync<0>();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  issue(0, 0);
  issue(1, 1);
  dma_sync<PAIR ? 0 : 2 * IPW>();
  int t = 0, st = 0;
  if constexpr (PAIR) {
    for (; t + 1 < t_mask; t += 2) {
      tile(F_{}, F_{}, t, 0);
      tile(F_{}, T_{}, t + 1, 0);
    }
    for (; t < ntiles; t += 2) {
      tile(T_{}, F_{}, t, 0);
      if (t + 1 >= ntiles) break;
      tile(T_{}, T_{}, t + 1, 0);
    }
  } else {
    for (; t < t_mask; ++t) {
      tile(F_{}, F_{}, t, st);
      st = st == NSTG - 1 ? 0 : st + 1;
    }
    for (; t < ntiles; ++t) {
      tile(T_{}, F_{}, t, st);
      st = st == NSTG - 1 ? 0 : st + 1;
    }
  }
  wait_vmcnt<0>();  // copies past the last tile must land before LDS is released

  // dQ^T register r of block db is head dim db*32 + 8*(r/4) + 4*hl + r%4 of
  // this lane's query.  Stored straight from the accumulators, each 16-byte
  // store would scatter over 32 rows; once every wave is done with the ring,
  // each writes its 32 rows into LDS and stores whole rows, 16 bytes per
  // lane.
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  FA_LDS uint8_t* ost = lds + wave * 32 * OROWB;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<FA_LDS f32x4_t*>(ost + l32 * OROWB + 4 * (db * 32 + 8 * g + 4 * hl)) =
          f32x4_t{dqacc[db][4 * g], dqacc[db][4 * g + 1], dqacc[db][4 * g + 2], dqacc[db][4 * g + 3]} *
          a.scale;
  asm volatile("" ::: "memory");
  {
    constexpr int LPR = D / 4;     // lanes per row, 16 bytes (four fp32) each
    constexpr int RPI = 64 / LPR;  // rows per store instruction
    const int r0 = lane / LPR, cb = (lane % LPR) * 16;
    uint8_t* dst = reinterpret_cast<uint8_t*>(a.dq + base + (int64_t)qw0 * D);
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int r = r0 + RPI * k;
      const u32x4_t v = ld_lds16(ost + r * OROWB + cb);
      if (qw0 + r < N) *reinterpret_cast<u32x4_t*>(dst + 4 * (int64_t)r * D + cb) = v;
    }
  }
  };  // unit

  // n_ktiles holds the query-tile count in this kernel.
  if constexpr (PERSIST) {
    // Causal: query tile qt meets the key tiles up to its diagonal, so rank
    // 0 (the heaviest) is the last query tile.
    lpt_units(a.n_ktiles, a.bh, a.pin != 0, [&](int bh, int rank, int, int) {
      unit(bh, a.n_ktiles - 1 - rank);
      // The next unit's first copies reuse the ring.
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    });
  } else {
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    int qt = logical % a.n_ktiles;
    if (CAUSAL) qt = a.n_ktiles - 1 - qt;  // longest key ranges first
    unit(logical / a.n_ktiles, qt);
  }
}

// Launches one of the two main kernels over a.n_ktiles tiles of each of BH
// heads: non-causal, one workgroup per tile (all tiles cost the same);
// causal, the persistent heaviest-first schedule with one workgroup per
// resident slot.
template <auto KPlain, auto KPersist>
hipError_t launch_grid(BwdArgs a, int BH, bool causal, int threads, hipStream_t s) {
  const int64_t units = (int64_t)a.n_ktiles * BH;
  if (units > 0x7fffffff) return hipErrorInvalidValue;
  if (!causal) {
    hipLaunchKernelGGL(KPlain, dim3((unsigned)units), dim3(threads), 0, s, a);
    return hipGetLastError();
  }
  const int slots = resident_slots<KPersist>(threads);
  if (slots <= 0) return hipErrorInvalidValue;
  const int64_t grid = std::min<int64_t>(units, slots);
  a.pin = (BH % 8 == 0 && grid % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(KPersist, dim3((unsigned)grid), dim3(threads), 0, s, a);
  return hipGetLastError();
}

template <int D, int NW, int BQ, int DQ_BN, int DQ_NW, int DT>
hipError_t launch_d(const BwdArgs& a0, int BH, bool causal, hipStream_t s) {
  BwdArgs a = a0;
  a.plane = (int64_t)BH * a.N;
  a.bh = BH;
  a.inv_scale = 1.0f / a.scale;
  // The dQ kernel first: it forms the row statistics the dK/dV kernel reads.
  constexpr int BM = 32 * DQ_NW;
  a.n_ktiles = (a.N + BM - 1) / BM;  // query tiles for the dQ kernel
  hipError_t e = launch_grid<bwd_dq_kernel<D, DQ_BN, DQ_NW, false, DT, false>,
                             bwd_dq_kernel<D, DQ_BN, DQ_NW, true, DT, true>>(a, BH, causal,
                                                                             DQ_NW * 64, s);
  if (e != hipSuccess) return e;
  constexpr int BKV = 128;
  a.n_ktiles = (a.N + BKV - 1) / BKV;
  return launch_grid<bwd_kv3_kernel<D, BQ, false, DT, false>,
                     bwd_kv3_kernel<D, BQ, true, DT, true>>(a, BH, causal, 512, s);
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

// ---------------------------------------------------------------- no-alloc

// Fixed device scratch of the allocation-free backward (fa_bwd_noalloc): it
// holds the two per-row planes that fa_bwd keeps in the caller's workspace.
// Each device holds its own copy, at its own address, for the life of the
// process.  In host code `scratch` names a host-side stand-in, never the
// device memory: kernels and copies only ever get the address that
// hipGetSymbolAddress returns for the current device (cached below).
static __device__ __align__(256) uint8_t scratch[kBwdScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

// Device address of `scratch` on the current device, looked up on the first
// call on that device; null if the lookup fails.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
      return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

hipError_t launch_bwd_noalloc(const BwdArgs& a0, int B, int H, int d, int dtype, bool causal,
                              hipStream_t stream) {
  void* p = scratch_on_current_device();
  if (p == nullptr) return hipErrorInvalidSymbol;
  BwdArgs a = a0;
  a.dsum = static_cast<float*>(p);
  return launch_bwd(a, B, H, d, dtype, causal, stream);
}

}  // namespace fa
