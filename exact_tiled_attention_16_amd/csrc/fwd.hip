// Attention forward for gfx950: exact softmax attention computed tile by tile
// with an online softmax ("FlashAttention: Fast and Memory-Efficient Exact
// Attention with IO-Awareness", abstract: tiling between HBM and on-chip
// memory; FlashAttention-4 related-papers page, online-softmax snippet:
// running row maximum and normaliser; FlashAttention-3 review page, Appendix B
// fragment: exp2, row sum and output rescaling between the two products).
//
// Work unit: one workgroup = NW waves = 32*QB*NW query rows of one (b, h).
// Each wave keeps QB blocks of 32 query rows in registers for the whole key
// loop; every K or V fragment read from LDS feeds QB matrix instructions.
//
// Data movement: key and value tiles of BN rows are copied from HBM straight
// into LDS by buffer loads with an LDS destination (no staging registers),
// into rings of two to four stages per tensor, two iterations ahead of their
// use; the producers are the computing waves themselves (the pages'
// asynchronous copies overlapped with compute, FlashAttention-3 abstract).
// At the end of each iteration (of each pair of iterations, with four stages)
// a wave waits only for the copies the next one needs, then the workgroup
// barrier publishes them.  LDS rows are unpadded; the
// 16-byte chunk index of row r is XOR-ed with swz<D>(r), which keeps both LDS
// read patterns below free of bank conflicts.
//
// Per tile and query block:
//   S^T = K_j Q^T on 32x32x16 matrix cores (keys are accumulator rows, the
//     block's 32 queries columns: one lane owns one query row, so row
//     reductions are in-lane plus one exchange with the lane 32 away);
//   online softmax in the exp2 domain (scores times scale*log2(e)), with the
//     exp2 reference raised lazily; probabilities rounded to the input type;
//   O^T += V_j^T P^T on matrix cores, V read from LDS by transposed 16-bit
//     reads; O^T has one query per lane, so the rescale is a per-lane multiply.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

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

// Explicit instruction order inside the fused steps (see `fused`).
#ifndef FA_FWD_SGB
#define FA_FWD_SGB 1
#endif
#ifndef FA_FWD_INTERLEAVE
#define FA_FWD_INTERLEAVE 1  // hand-placed instruction order in the main loop
#endif

// QB = query blocks of 32 rows per wave; OCC = waves per SIMD the register
// budget is sized for (1: 512 registers, 2: 256); NSTG = LDS stages per
// tensor (2 or 3, see the pipeline description below).
// PERSIST: the grid holds one workgroup per resident slot, and each loops
// over work units (b, h, query tile): causal, those of the heaviest-first
// schedule (lpt_units); non-causal, every G-th of the one-unit grid's order.
// Each unit's epilogue fetches the next unit's Q rows and first K tiles.
// Otherwise each workgroup takes one unit.
// PARTIAL: split-KV mode.  Unit (b, h, query tile, split s) attends to keys
// [s k_chunk, (s+1) k_chunk) only and writes O normalised over those keys in
// fp32 and their log-sum-exp to slot s of the partial outputs; a merge kernel
// combines the slots.
// SPARSE: block-sparse mode.  bs_list holds, per (mask head, query tile), the
// number of live key tiles and their list (see bs_index_kernel); the tile
// loop walks that list instead of every key tile, and a wave masks a listed
// tile out entirely when its own 128-row query block does not attend to it.
template <int D, int BN, int NW, int QB, int OCC, int NSTG, bool CAUSAL, int DT, bool PERSIST,
          bool PARTIAL, bool SPARSE>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
fwd_kernel(FwdArgs a, const int* __restrict__ bs_list) {
  using E = Elem<DT>;
  using v8 = typename E::v8;
  constexpr int WQ = 32 * QB;        // query rows per wave
  constexpr int BM = WQ * NW;        // query rows per workgroup
  constexpr int ROWB = 2 * D;        // bytes per row (LDS and HBM)
  constexpr int TILEB = BN * ROWB;   // bytes per tile per tensor
  constexpr int CH_ROW = D / 8;      // 16-byte chunks per row
  static_assert(TILEB % (1024 * NW) == 0, "a tile must split into whole 1 KiB copies per wave");
  constexpr int IPW = TILEB / 1024 / NW;  // copies per wave per tensor per tile
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(NSTG >= 2 && NSTG <= 4, "stage count");
  constexpr bool PAIR = NSTG == 4;  // iterations in pairs, one barrier per pair
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;
  constexpr int NDC = D / 16;

  // The persistent grids copy the next unit's first two K tiles into stages
  // 0 and 1 while the current unit's O passes through LDS: O is then staged
  // above them (not the causal grid at d = 256, where it measured 0.6 %
  // slower).
  constexpr bool PREFETCH = PERSIST && (!CAUSAL || D <= 128);
  constexpr int OROWB = 2 * D + 8;  // bytes per staged O row (8 bytes of padding)
  constexpr int OSTB = PREFETCH ? 2 * TILEB : 0;
  constexpr int SMEM = 2 * NSTG * TILEB > OSTB + NW * WQ * OROWB ? 2 * NSTG * TILEB
                                                                 : OSTB + NW * WQ * OROWB;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
  FA_LDS uint8_t* lds = (FA_LDS uint8_t*)smem;  // K stage s at s*TILEB, V at (NSTG+s)*TILEB

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave-uniform (scalar)
  const int N = a.N;

  // Q^T operand of block qb: lane holds query qw0 + 32 qb + l32, head-dim
  // slots dc*16 + 8*hl + [0, 8).  Declared outside the unit: the persistent
  // grids load the next unit's rows here during the current unit's epilogue.
  v8 qf[QB][NDC];

  // One work unit: query tile qt of head bh against the keys of split s.
  // nxt: the next unit of this workgroup (persistent grids; head *
  // n_qtiles + query tile), else -1; pre: this unit's Q rows and first two K
  // tiles were fetched by the previous unit's epilogue.
  auto unit = [&](const int bh, const int qt, const int s, const int nxt, const bool pre) {
  // The lane index passes through an empty asm so that nothing derived from
  // it is hoisted out of a loop over units (it would stay live across units
  // and spill at the register limit).
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int hl = lane >> 5;  // which half of K slots / accumulator rows
  const int l32 = lane & 31;
  // Keys of this unit: [kb0, kb0 + kn) of the head's Nk.  Causal: query row
  // i sees local key j iff j <= i + coff (coff = 0 for the plain forward).
  const int kb0 = s * a.k_chunk;
  const int kn = max(min(a.Nk - kb0, a.k_chunk), 0);
  const int coff = a.c_off - kb0;
  const int64_t base = (int64_t)bh * N * D;
  const int64_t kvbase = ((int64_t)bh * a.Nk + kb0) * D;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q) + base;
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + kvbase;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + kvbase;

  const int q0 = qt * BM;
  const int qw0 = q0 + wave * WQ;  // first query row of this wave
  const int kend = CAUSAL ? max(min(kn, q0 + BM + coff), 0) : kn;
  // Block-sparse: entry e of the list is key tile (e & 0xffffff), with bit
  // 24 + b set when query block b of the tile (rows q0 + 128 b ...) attends
  // to it.  The list is followed by padding entries that name a tile past the
  // last key (zeros, fully masked) with no bits, so that the reads below,
  // which run up to a few positions past the end, need no bounds check (a
  // branch there would break the straight-line schedule of the loop).
  const int* lst = nullptr;
  int nlist = 0, nfull = 0;
  if constexpr (SPARSE) {
    const int mh = a.bs_per_batch ? bh : bh % a.heads;
    lst = bs_list + ((int64_t)mh * a.n_qtiles + qt) * a.bs_stride;
    nlist = lst[0];
    nfull = lst[1];  // leading live tiles that need no mask
    lst += 1;        // entries at lst[1 + j]
  }
  auto tile_of = [&](int j) { return lst[1 + j] & 0xffffff; };
  const int ntiles = SPARSE ? nlist : (kend + BN - 1) / BN;
  const float c = a.scale_log2;

  // ---- Copies.  Copy jj of this wave fills LDS chunk (wave*IPW + jj)*64 + lane
  // of the tile, i.e. row p / CH_ROW, and reads the logical chunk that the
  // swizzle maps there.  Tile t is addressed through a buffer resource that
  // ends at key N, so rows past the end (the ragged tile, tiles past the last)
  // arrive as zeros without any clamping.
  uint32_t dma_voff[IPW];
#pragma unroll
  for (int jj = 0; jj < IPW; ++jj) {
    const int p = (wave * IPW + jj) * 64 + lane;
    dma_voff[jj] = (uint32_t)((p / CH_ROW) * ROWB + ((p % CH_ROW) ^ swz<D>(p / CH_ROW)) * 16);
  }
  auto issue = [&](const uint16_t* src, int t, FA_LDS uint8_t* stage) {
    if constexpr (SPARSE) {
      const int tt = tile_of(max(t, 0));
      t = t < 0 ? t : tt;
    }
    const int rows = t < 0 ? 0 : min(max(kn - t * BN, 0), BN);
    const u32x4_t r = make_rsrc(src + (int64_t)t * BN * D, rows * ROWB);
#pragma unroll
    for (int jj = 0; jj < IPW; ++jj) {
      if (jj == 0) dma16_buf<4>(r, dma_voff[jj], stage + (wave * IPW + jj) * 1024);
      else dma16_buf<0>(r, dma_voff[jj], stage + (wave * IPW + jj) * 1024);
    }
  };
  // Tile t lives in stage t % NSTG of each ring.  Iteration j reads K(j+1)
  // and V(j-1) and copies K(j+KAHEAD) and V(j+VAHEAD) into the stages they
  // replace (see the pipeline description below).
  constexpr int KAHEAD = NSTG == 3 ? 3 : 2;
  constexpr int VAHEAD = NSTG == 3 ? 1 : 0;
  constexpr int PENDING = NSTG == 3 ? 2 * IPW : 0;  // copies left in flight at an iteration's end
  // Stage arithmetic on st = j % NSTG, carried by the loops.
  auto snext = [](int x) { return x == NSTG - 1 ? 0 : x + 1; };
  auto sprev = [](int x) { return x == 0 ? NSTG - 1 : x - 1; };
  auto issue_iter = [&](int j, int st) {
    // (j + KAHEAD) % NSTG == st; (j + VAHEAD) % NSTG == st + 1 or st.
    issue(K, j + KAHEAD, lds + st * TILEB);
    issue(V, j + VAHEAD, lds + (NSTG + (NSTG == 3 ? snext(st) : st)) * TILEB);
  };
  // Four stages (tile t in stage t & 3): iterations run in pairs (j odd,
  // j + 1) with one workgroup barrier per pair.  The pair reads K(j+1),
  // K(j+2), V(j-1) and V(j); its first iteration copies K(j+3), K(j+4),
  // V(j+1) and V(j+2), which the next pair reads, into the stages the
  // previous pair read (free since its barrier); the second iteration waits
  // for those copies and ends with the barrier that publishes them.  Each
  // copy still has two iterations to land.
  auto issue_pair = [&](int j) {
    issue(K, j + 3, lds + ((j + 3) & 3) * TILEB);
    issue(K, j + 4, lds + ((j + 4) & 3) * TILEB);
    issue(V, j + 1, lds + (NSTG + ((j + 1) & 3)) * TILEB);
    issue(V, j + 2, lds + (NSTG + ((j + 2) & 3)) * TILEB);
  };

  auto load_q = [&](const uint16_t* Qh, int qw) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = qw + 32 * qb + l32;
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        u32x4_t raw = {0u, 0u, 0u, 0u};
        if (qrow < N) raw = ld_global16(Qh + (int64_t)qrow * D + dc * 16 + 8 * hl);
        qf[qb][dc] = __builtin_bit_cast(v8, raw);
      }
    }
  };
  if (!pre) load_q(Q, qw0);

  f32x16_t oacc[QB][NDB];
  float m_run[QB], l_run[QB];  // exp2 reference (log2 units), this lane's share of l
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][i][r] = 0.f;
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

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
  // group 16*g2 + 4*c4 of the 32-column block db.  The offsets include the
  // base of the V stages (NSTG * TILEB), hidden from the compiler so that it
  // is not folded into the reads' 16-bit immediates: with a stage known at
  // compile time, each read is then a lane offset plus an immediate.
  int voff[NDB][2];
  {
    const int e = (lane & 15) >> 2, c4 = lane & 3, g2 = (lane >> 4) & 1;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 4 * hl + e + 8 * hi;  // row within a 16-key chunk; cc adds 16 rows
      const int f = swz<D>(r);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        voff[db][hi] = NSTG * TILEB + r * ROWB + 16 * ((4 * db + 2 * g2 + (c4 >> 1)) ^ f) + 8 * (c4 & 1);
        asm volatile("" : "+v"(voff[db][hi]));
      }
    }
  }
  auto ld_k = [&](const FA_LDS uint8_t* ks, int kb, int dc) {
    return __builtin_bit_cast(v8, ld_lds16(ks + kb * 32 * ROWB + koff[dc]));
  };
  auto ld_v = [&](const FA_LDS uint8_t* vs, int cc, int db) {
    const s16x4_t lo = ld_lds_tr16(vs + cc * 16 * ROWB + voff[db][0]);
    const s16x4_t hi = ld_lds_tr16(vs + cc * 16 * ROWB + voff[db][1]);
    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    return __builtin_bit_cast(v8, u32x4_t{l2[0], l2[1], h2[0], h2[1]});
  };
  // P operand of chunk cc (16 keys): accumulator registers 8*(cc%2)..+7 of
  // score block cc/2, i.e. keys 16cc + 8*(s/4) + 4*hl + s%4 for slot s; the V
  // operand is read for the same keys.
  auto p_frag = [&](const uint32_t (&pw)[NKB][8], int cc) {
    const int j0 = 4 * (cc & 1);
    return __builtin_bit_cast(
        v8, u32x4_t{pw[cc >> 1][j0], pw[cc >> 1][j0 + 1], pw[cc >> 1][j0 + 2], pw[cc >> 1][j0 + 3]});
  };

  typedef f32x16_t Scores[QB][NKB];
  typedef uint32_t Probs[QB][NKB][8];

  // ---- One probability pair: keys (2w, 2w+1) of score block kb against the
  // exp2 reference -m_neg, rounded and packed; adds the unrounded values to
  // the lane's fp32 partial sums.
  auto prob_pair = [&](const f32x16_t& s, int w, float m_neg, float& ps0, float& ps1) {
    const float p0 = fast_exp2(fmaf(s[2 * w], c, m_neg));
    const float p1 = fast_exp2(fmaf(s[2 * w + 1], c, m_neg));
    ps0 += p0;
    ps1 += p1;
    return E::pack2(p0, p1);
  };
  auto phase_p = [&](const f32x16_t (&sacc)[NKB], uint32_t (&pw)[NKB][8], float m_neg) {
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int w = 0; w < 8; ++w) pw[kb][w] = prob_pair(sacc[kb], w, m_neg, ps0, ps1);
    return ps0 + ps1;
  };

  // ---- Reference raise (rare): block qb's probabilities were computed
  // against the current reference and some lane's partial sum left
  // [0, kLazySum] (or the row had no reference yet).  Raise every row's
  // reference to the maximum seen so far, rescale O (which already holds all
  // earlier tiles) and l, and recompute the tile's probabilities.
  const uint32_t opaque_zero = (uint32_t)(N >> 31);  // 0; unknown to the compiler
  auto raise_ref = [&](int qb, const f32x16_t (&sacc)[NKB], uint32_t (&pw)[NKB][8], float& psum) {
    asm volatile("" ::: "memory");  // keep this path a branch
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = max_halves(mx) * c;  // scale > 0, so max and scaling commute
    const float m_new = fmaxf(m_run[qb], mx);
    const float alpha = (m_new == m_run[qb]) ? 1.0f : fast_exp2(m_run[qb] - m_new);  // 0 on a first tile
    m_run[qb] = m_new;
    l_run[qb] *= alpha;
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (OCC == 1) {
          // With a 512-register budget O belongs in the accumulator
          // registers; a plain multiply here would pull it into the vector
          // registers for the whole kernel.
          float t;
          asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(t) : "a"(oacc[qb][i][r]));
          t *= alpha;
          asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(oacc[qb][i][r]) : "v"(t));
        } else {
          oacc[qb][i][r] *= alpha;
        }
      }
    uint32_t fresh[NKB][8];
    psum = phase_p(sacc, fresh, m_new == -INFINITY ? 0.f : -m_new);
    // Reading the speculative words here keeps the compiler from moving
    // their computation past the branch.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int w = 0; w < 8; ++w) pw[kb][w] = fresh[kb][w] | (pw[kb][w] & opaque_zero);
  };
  auto finish_tile = [&](const Scores& s_cur, Probs& p_cur, float (&psum)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (wave_any(!(psum[qb] <= kLazySum))) raise_ref(qb, s_cur[qb], p_cur[qb], psum[qb]);
      l_run[qb] += psum[qb];
    }
  };

  // Software pipeline over three tiles (the pages' intra-group pipelining,
  // one tile deeper than their two-stage listing).  Iteration j
  //   copies K(j+KAHEAD) and V(j+VAHEAD) into the stages they replace,
  //   computes S(j+1) = K_{j+1} Q^T          (matrix cores),
  //   turns S(j) into probabilities P(j)      (vector ALUs),
  //   accumulates O += P(j-1) V_{j-1}         (matrix cores),
  // three mutually independent streams, which the hardware overlaps.  A raise
  // of the reference found on P(j) rescales O after P(j-1) V_{j-1} has been
  // added: O and l then share the new reference.  At the end of iteration j,
  // K(j+2) and V(j) must have landed for iteration j+1.  With three stages
  // they were issued one iteration earlier and this iteration's copies stay
  // in flight; with two stages (half the LDS, so two workgroups fit on a CU)
  // they were issued at the start of this iteration and the wait drains all.
  int t_mask = (kn % BN) ? kn / BN : ntiles;
  if (CAUSAL) t_mask = min(t_mask, max(q0 + coff + 1, 0) / BN);
  t_mask = min(t_mask, ntiles);
  // Block-sparse: tiles dead for some wave of a multi-block workgroup need
  // the masked body; with one query block per workgroup only the trailing
  // diagonal / ragged tiles do.
  if constexpr (SPARSE) t_mask = BM > kSparseBlock ? 0 : nfull;

  Scores sA, sB;
  Probs pA, pB;

  // One iteration as NSTEP fused steps, each with QB S(j+1) and QB P(j-1) V
  // matrix instructions sharing one K and one V fragment, and a share of the
  // probability pairs of P(j); LDS fragments are read PF steps ahead.  A
  // scheduling barrier after each step keeps the vector work spread evenly
  // under the matrix work.  DS / DP / DPV select which of the three streams
  // run (the ragged end and the causal diagonal drop some for some waves);
  // MS masks S(j) before P(j).  S(j) is in s_cur, P(j-1) in p_prev; S(j+1) goes to
  // s_nxt and P(j) to p_cur.
  constexpr int NSTEP = NKB * NDC;  // == (BN / 16) * NDB
  constexpr int NPAIR = NKB * 8;    // probability pairs per lane, tile and block
  // Fragment prefetch distance in steps: 2 (1 at d = 256, and in the masked
  // iterations, which hold the mask's bounds as well).
  constexpr int PF0 = D >= 256 ? 1 : 2;
  // SECOND: the second iteration of a pair (j even), else the first.
  auto fused = [&](auto ds_tag, auto ms_tag, auto dp_tag, auto dpv_tag, auto second_tag, int j,
                   int st, Scores& s_cur, Scores& s_nxt, Probs& p_cur, const Probs& p_prev) {
    constexpr bool DS = decltype(ds_tag)::value, MS = decltype(ms_tag)::value;
    constexpr bool DP = decltype(dp_tag)::value, DPV = decltype(dpv_tag)::value;
    constexpr bool SECOND = decltype(second_tag)::value;
    if constexpr (!PAIR)
      issue_iter(j, st);
    else if constexpr (!SECOND)
      issue_pair(j);
    // st = j % NSTG (a constant in the unrolled main loops).
    const FA_LDS uint8_t* ks = lds + (PAIR ? (st + 1) & 3 : snext(st)) * TILEB;
    const FA_LDS uint8_t* vs = lds + (PAIR ? (st + 3) & 3 : sprev(st)) * TILEB;  // + NSTG * TILEB in voff
    if constexpr (DP && MS) {
      // The mask goes on S(j) here, before its probabilities are formed:
      // its products completed in the previous iteration, and nothing sits
      // between the steps and the tile's end (a mask on S(j+1) after the
      // steps waited for their products, and the compiler sank the
      // exponentials past its branch, out of the steps).  Register r of
      // block kb holds key t*BN + 4*hl + (kb*32 + 8*(r/4) + r%4) with t = j;
      // it is visible iff that constant offset is below `lim`.
      const int t = SPARSE ? tile_of(j) : j;
      // Block-sparse: the wave's query block does not attend to this tile.
      bool dead = false;
      if constexpr (SPARSE && BM > kSparseBlock)
        dead = !((lst[1 + j] >> (24 + (wave * WQ) / kSparseBlock)) & 1);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        int lim = kn - t * BN - 4 * hl;
        if (CAUSAL) lim = min(lim, qw0 + 32 * qb + l32 + 1 + coff - t * BN - 4 * hl);
        if (dead) lim = -BN;
        // Tiles of the masked tail that need no mask in any lane skip it.
        constexpr int kMaxOff = (NKB - 1) * 32 + 27;  // largest key offset of a register
        if (wave_any(lim <= kMaxOff)) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) s_cur[qb][kb][r] = -INFINITY;
        }
      }
    }
    constexpr int PF = MS ? 1 : PF0;
    v8 kfr[PF + 1], vfr[PF + 1];
    // S(j+1) runs key block by key block (kb-major) and P(j) consumes S(j)
    // in the same order, so only about half of each score set is live at once.
    auto load = [&](int step) {
      if constexpr (DS) kfr[step % (PF + 1)] = ld_k(ks, step / NDC, step % NDC);
      if constexpr (DPV) vfr[step % (PF + 1)] = ld_v(vs, step / NDB, step % NDB);
    };
    if constexpr (DS) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s_nxt[qb][kb][r] = 0.f;
    }
#pragma unroll
    for (int step = 0; step < PF; ++step) load(step);
    float m_neg[QB], ps0[QB], ps1[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m_neg[qb] = -m_run[qb];
      ps0[qb] = 0.f;
      ps1[qb] = 0.f;
    }
#pragma unroll
    for (int step = 0; step < NSTEP; ++step) {
      if (step + PF < NSTEP) load(step + PF);
      const int slot = step % (PF + 1);
      const int kb = step / NDC, dc = step % NDC;
      const int cc = step / NDB, db = step % NDB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if constexpr (DS) s_nxt[qb][kb] = E::mfma(kfr[slot], qf[qb][dc], s_nxt[qb][kb]);
        if constexpr (DPV) oacc[qb][db] = E::mfma(vfr[slot], p_frag(p_prev[qb], cc), oacc[qb][db]);
      }
      if constexpr (DP) {
#pragma unroll
        for (int pr = step * NPAIR / NSTEP; pr < (step + 1) * NPAIR / NSTEP; ++pr)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            p_cur[qb][pr / 8][pr % 8] =
                prob_pair(s_cur[qb][pr / 8], pr % 8, m_neg[qb], ps0[qb], ps1[qb]);
      }
      // Two waves share each SIMD and the older one wins issue ties, so it
      // would finish its tile first and idle at the barrier while the other
      // runs alone.  Raising the priority for the first half of the steps
      // and dropping it for the second hands the lead to the wave that is
      // behind once the leader passes the midpoint (measured +5-8%).
      if constexpr (DS && DP && DPV && OCC > 1) {
        if (step == 0) __builtin_amdgcn_s_setprio(1);
        if (step == NSTEP / 2) __builtin_amdgcn_s_setprio(0);
      }
      // Order inside a full step.  d <= 128 (two waves per SIMD): the score
      // product, four vector instructions, the P V product, the step's
      // fragment reads, the rest of the vector work; the compiler's own
      // order measured 1.6-2.0 % slower at d = 128 and 0.4 % at d = 64
      // (nine orders were timed).  d = 256 (one wave per SIMD, half a
      // probability pair per step): the score product, the reads, the P V
      // product, the vector work (1.1 % faster; the d <= 128 order was 7 %
      // slower there).
      if constexpr (DS && DP && DPV && QB == 1 && FA_FWD_SGB) {
        if constexpr (D <= 128) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // matrix
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // vector
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // matrix
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // LDS reads
          __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // vector
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // matrix
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // matrix
          __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // vector
        }
      }
#if FA_FWD_INTERLEAVE
      __builtin_amdgcn_sched_barrier(0);
#endif
    }
    if constexpr (DP) {
      float psum[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) psum[qb] = ps0[qb] + ps1[qb];
      finish_tile(s_cur, p_cur, psum);
    }
    if constexpr (!PAIR)
      dma_sync<PENDING>();
    else if constexpr (SECOND)
      dma_sync<0>();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  // Iterations run uniformly to j = ntiles, with no per-wave branches: a
  // tile past the last one, or past a wave's causal diagonal, arrives as
  // zeros (or is masked) so its scores are all -inf, its probabilities
  // exactly 0 and its P V product exactly 0.
  //
  // Prologue: K(0) and K(1) in flight, wait for K(0); iteration -1 computes
  // S(0) only and issues K(2) and V(0) like any iteration; its closing wait
  // leaves exactly those in flight, so K(1) has landed for iteration 0.
  // Four stages: the prologue pair (-1, 0) reads K(0) and K(1), copied and
  // published first.
  if (!pre) {
    issue(K, 0, lds);
    if constexpr (NSTG >= 3) issue(K, 1, lds + TILEB);
  }
  if constexpr (NSTG >= 3) {
    if (pre)
      dma_sync<0>();
    else
      dma_sync<PAIR ? 0 : IPW>();
  } else {
    dma_sync<0>();
  }
  fused(T_{}, T_{}, F_{}, F_{}, F_{}, -1, NSTG - 1, sB, sA, pB, pA);  // S(0) -> sA
  fused(T_{}, T_{}, T_{}, F_{}, T_{}, 0, 0, sA, sB, pA, pB);          // S(1) -> sB, P(0) -> pA
  // Unmasked iterations an even number per trip (six or four with the
  // stages as constants, else two), so that the score and probability
  // register sets swap roles instead of being copied; then the masked rest.
  // j is odd in the first iteration of a trip.
  int j = 1, st = 1 % NSTG;
  if constexpr (NSTG == 3 && !SPARSE) {
    // Six iterations per trip: iteration j uses stage j % 3, here a
    // compile-time constant, so that the LDS reads need no address
    // arithmetic.  The trip ends with j = 1 (mod 6) and st = 1 again.
    for (; j + 6 < t_mask; j += 6) {
      fused(T_{}, F_{}, T_{}, T_{}, F_{}, j, 1, sB, sA, pB, pA);
      fused(T_{}, F_{}, T_{}, T_{}, T_{}, j + 1, 2, sA, sB, pA, pB);
      fused(T_{}, F_{}, T_{}, T_{}, F_{}, j + 2, 0, sB, sA, pB, pA);
      fused(T_{}, F_{}, T_{}, T_{}, T_{}, j + 3, 1, sA, sB, pA, pB);
      fused(T_{}, F_{}, T_{}, T_{}, F_{}, j + 4, 2, sB, sA, pB, pA);
      fused(T_{}, F_{}, T_{}, T_{}, T_{}, j + 5, 0, sA, sB, pA, pB);
    }
  } else if constexpr (NSTG == 4 && !SPARSE) {
    // Four stages: four iterations (two pairs) per trip, stages 1, 2, 3, 0.
    for (; j + 4 < t_mask; j += 4) {
      fused(T_{}, F_{}, T_{}, T_{}, F_{}, j, 1, sB, sA, pB, pA);
      fused(T_{}, F_{}, T_{}, T_{}, T_{}, j + 1, 2, sA, sB, pA, pB);
      fused(T_{}, F_{}, T_{}, T_{}, F_{}, j + 2, 3, sB, sA, pB, pA);
      fused(T_{}, F_{}, T_{}, T_{}, T_{}, j + 3, 0, sA, sB, pA, pB);
    }
  } else {
    for (; j + 2 < t_mask; j += 2) {
      const int stb = snext(st);
      fused(T_{}, F_{}, T_{}, T_{}, F_{}, j, st, sB, sA, pB, pA);
      fused(T_{}, F_{}, T_{}, T_{}, T_{}, j + 1, stb, sA, sB, pA, pB);
      st = snext(stb);
    }
  }
  for (; j <= ntiles; j += 2) {
    const int stb = snext(st);
    fused(T_{}, T_{}, T_{}, T_{}, F_{}, j, st, sB, sA, pB, pA);
    if (j + 1 > ntiles) break;
    fused(T_{}, T_{}, T_{}, T_{}, T_{}, j + 1, stb, sA, sB, pA, pB);
    st = snext(stb);
  }
  wait_vmcnt<0>();  // copies past the last tile must land before LDS is released

  // Epilogue: normalise, round, store; LSE in natural log.
  if constexpr (PARTIAL) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = qw0 + 32 * qb + l32;
      const float l_tot = sum_halves(l_run[qb]);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if (qrow < N) {
        const int64_t slot = ((int64_t)s * a.bh + bh) * N + qrow;
        float* orow = a.o32 + slot * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4_t*>(orow + db * 32 + 8 * g + 4 * hl) =
                f32x4_t{oacc[qb][db][4 * g + 0], oacc[qb][db][4 * g + 1], oacc[qb][db][4 * g + 2],
                        oacc[qb][db][4 * g + 3]} * inv;
        }
        // No visible key: l = 0, O = 0 and the log-sum-exp is -inf.
        if (hl == 0) a.lse32[slot] = m_run[qb] * kLn2 + __logf(l_tot);
      }
    }
  } else {
    // A lane holds its query row in 8-byte pieces, so stores straight from
    // the accumulators would scatter each instruction over 32 rows.  Each
    // wave writes its rows into LDS instead (rows padded by 8 bytes, so the
    // 8-byte writes of one half-wave hit distinct banks) and stores whole
    // rows, 16 bytes per lane.  The K/V ring is free once every wave has
    // left the loop (each wave's own copies have landed, see above).
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (PREFETCH) {
      // The next unit's Q rows (this unit's are dead) and its first two K
      // tiles, into the stages below the O blocks, in flight while O leaves.
      if (nxt >= 0) {
        const int nbh = nxt / a.n_qtiles, nqt = nxt % a.n_qtiles;
        load_q(static_cast<const uint16_t*>(a.q) + (int64_t)nbh * N * D, nqt * BM + wave * WQ);
        const uint16_t* Kn = static_cast<const uint16_t*>(a.k) + ((int64_t)nbh * a.Nk + kb0) * D;
        issue(Kn, 0, lds);
        issue(Kn, 1, lds + TILEB);
      }
    }
    FA_LDS uint8_t* ost = lds + OSTB + wave * WQ * OROWB;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l_tot = sum_halves(l_run[qb]);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2_t w;
          w[0] = E::pack2(oacc[qb][db][4 * g + 0] * inv, oacc[qb][db][4 * g + 1] * inv);
          w[1] = E::pack2(oacc[qb][db][4 * g + 2] * inv, oacc[qb][db][4 * g + 3] * inv);
          *reinterpret_cast<FA_LDS u32x2_t*>(ost + (32 * qb + l32) * OROWB +
                                             2 * (db * 32 + 8 * g + 4 * hl)) = w;
        }
      }
      const int qrow = qw0 + 32 * qb + l32;
      if (qrow < N && hl == 0 && a.lse != nullptr)
        a.lse[(int64_t)bh * N + qrow] = m_run[qb] * kLn2 + __logf(l_tot);
    }
    asm volatile("" ::: "memory");
    constexpr int LPR = D / 8;     // lanes per row, 16 bytes each
    constexpr int RPI = 64 / LPR;  // rows per store instruction
    const int r0 = lane / LPR, cb = (lane % LPR) * 16;
#pragma unroll
    for (int k = 0; k < WQ / RPI; ++k) {
      const int r = r0 + RPI * k;
      const u32x4_t v = ld_lds16(ost + r * OROWB + cb);
      if (qw0 + r < N)
        *reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(a.o) + 2 * (base + (int64_t)(qw0 + r) * D) +
                                    cb) = v;
    }
  }
  };  // unit

  if constexpr (PERSIST && CAUSAL) {
    // A causal query tile qt costs qt + 1 key tiles: rank 0 is the last one.
    bool pre = false;
    lpt_units(a.n_qtiles, a.bh, a.pin != 0, [&](int bh, int rank, int nbh, int nrank) {
      unit(bh, a.n_qtiles - 1 - rank, 0,
           PREFETCH && nbh >= 0 ? nbh * a.n_qtiles + a.n_qtiles - 1 - nrank : -1, pre);
      pre = PREFETCH;
      // The next unit's first copies reuse the ring: every wave must be done
      // reading it (this wave's own copies have all landed already).
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    });
  } else if constexpr (PERSIST) {
    // Non-causal, all units alike: workgroup w takes units w, w + G, ... of
    // the (head, query tile) order under the XCD remap of the one-unit grid
    // below (when G is a multiple of 8, as the full grid of one workgroup per
    // CU is, each unit stays on the XCD it had there), and fetches each next
    // unit's Q rows and first K tiles during the current unit's epilogue.
    static_assert(!PARTIAL && !SPARSE && NSTG >= 3, "plain non-causal forward");
    const int total = a.n_qtiles * a.bh;
    for (int u = blockIdx.x; u < total; u += gridDim.x) {
      const int logical = xcd_remap(u, total);
      const int nu = u + (int)gridDim.x;
      unit(logical / a.n_qtiles, logical % a.n_qtiles, 0, nu < total ? xcd_remap(nu, total) : -1,
           u != (int)blockIdx.x);
      // The next unit's copies and O blocks reuse the ring: every wave must
      // be done reading it.
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
  } else {
    // Units in (head, split, query tile) order: the query tiles of one split
    // read the same keys, and the XCD remap keeps them on one L2.
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int hs = logical / a.n_qtiles;
    int qt = logical % a.n_qtiles;
    if (CAUSAL) qt = a.n_qtiles - 1 - qt;  // longest key ranges first
    unit(hs / a.n_split, qt, hs % a.n_split, -1, false);
  }
}

// Per head dimension: keys per tile, waves per workgroup, query blocks per
// wave, waves per SIMD, LDS stages per tensor.
template <int D> struct FwdCfg;
// d = 64 runs its iterations in pairs with one barrier per pair (four
// stages, 64 KiB of LDS): 1.3 % faster than a barrier per tile; at d = 128
// (128 KiB) that was 1 % slower than three stages.  Four-wave workgroups at
// d = 128 (two per CU, or one wave per SIMD with 64 query rows per wave)
// measured slower than eight waves with two per SIMD.
template <> struct FwdCfg<64> { static constexpr int BN = 64, NW = 8, QB = 1, OCC = 2, NSTG = 4; };
template <> struct FwdCfg<128> { static constexpr int BN = 64, NW = 8, QB = 1, OCC = 2, NSTG = 3; };
template <> struct FwdCfg<256> { static constexpr int BN = 32, NW = 4, QB = 1, OCC = 1, NSTG = 3; };

// Partial (split-KV) calls with at most kNarrowRows query rows -- decoding --
// use one wave per workgroup (32 query rows instead of 256, so far less of
// the matrix work is padding), 32-key tiles and a two-stage ring (32 KiB of
// LDS at d = 128), so that several workgroups share a CU: with so little
// compute per key the kernel is bound by HBM, and independent workgroups keep
// more K/V bytes in flight per CU than one workgroup's ring can.
constexpr int kNarrowRows = 32;
template <int D> struct FwdNarrowCfg {
  static constexpr int BN = 32, NW = 1, QB = 1, OCC = D == 256 ? 1 : 2, NSTG = 2;
};

// Block-sparse list geometry per head dimension: query tiles per head and
// ints per list (count, unmasked count, one entry per key tile, kSparsePad
// padding entries: the pipeline reads up to four positions past the last
// live tile).
constexpr int kSparsePad = 6;
// Block-sparse launches use workgroups of one 128-row query block (four
// waves), so a workgroup computes exactly its block's live key tiles, and a
// two-stage ring at d <= 128 so that two workgroups share a CU (a sparse
// workgroup has few tiles; its prologue and epilogue overlap the other's).
template <int D> struct FwdSparseCfg {
  static constexpr int BN = D == 256 ? 32 : 64, NW = 4, QB = 1, OCC = D == 256 ? 1 : 2,
                       NSTG = D == 256 ? 3 : 2;
};

template <int D>
int sparse_qtiles(int N) {
  constexpr int BM = 32 * FwdSparseCfg<D>::QB * FwdSparseCfg<D>::NW;
  return (N + BM - 1) / BM;
}
template <int D>
int sparse_list_stride(int N) {
  return (N + FwdSparseCfg<D>::BN - 1) / FwdSparseCfg<D>::BN + 2 + kSparsePad;
}

template <int D, bool CAUSAL, bool PERSIST, bool PARTIAL, int DT, bool SPARSE = false,
          class C = FwdCfg<D>>
hipError_t launch_one(const FwdArgs& a, int BH, hipStream_t stream,
                      const int* bs_list = nullptr) {
  constexpr int BM = 32 * C::QB * C::NW;
  FwdArgs args = a;
  args.n_qtiles = (a.N + BM - 1) / BM;
  args.bh = BH;
  const int64_t units = (int64_t)args.n_qtiles * BH * args.n_split;
  if (units > 0x7fffffff) return hipErrorInvalidValue;
  constexpr auto kernel =
      fwd_kernel<D, C::BN, C::NW, C::QB, C::OCC, C::NSTG, CAUSAL, DT, PERSIST, PARTIAL, SPARSE>;
  int64_t grid = units;
  if constexpr (PERSIST) {
    const int slots = resident_slots<kernel>(C::NW * 64);
    if (slots <= 0) return hipErrorInvalidValue;
    grid = std::min<int64_t>(units, slots);
    args.pin = (BH % 8 == 0 && grid % 8 == 0) ? 1 : 0;
  }
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(C::NW * 64), 0, stream, args, bs_list);
  return hipGetLastError();
}

// Causal schedule: the persistent heaviest-first grid, or (per_tile) one
// workgroup per query tile in dispatch order, heaviest tile of each head
// first.  Both produce bit-identical outputs.
template <int D, int DT>
hipError_t launch_causal(const FwdArgs& a, int BH, bool causal, bool per_tile, hipStream_t s) {
  if (!causal) return launch_one<D, false, true, false, DT>(a, BH, s);
  if (per_tile) return launch_one<D, true, false, false, DT>(a, BH, s);
  return launch_one<D, true, true, false, DT>(a, BH, s);
}

template <int DT>
hipError_t launch_dtype(const FwdArgs& a, int BH, int d, bool causal, bool per_tile,
                        hipStream_t s) {
  switch (d) {
    case 64: return launch_causal<64, DT>(a, BH, causal, per_tile, s);
    case 128: return launch_causal<128, DT>(a, BH, causal, per_tile, s);
    case 256: return launch_causal<256, DT>(a, BH, causal, per_tile, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int DT>
hipError_t launch_partial_d(const FwdArgs& a, int BH, bool causal, hipStream_t s) {
  if (a.N <= kNarrowRows) {
    using C = FwdNarrowCfg<D>;
    return causal ? launch_one<D, true, false, true, DT, false, C>(a, BH, s)
                  : launch_one<D, false, false, true, DT, false, C>(a, BH, s);
  }
  return causal ? launch_one<D, true, false, true, DT>(a, BH, s)
                : launch_one<D, false, false, true, DT>(a, BH, s);
}

template <int DT>
hipError_t launch_partial_dtype(const FwdArgs& a, int BH, int d, bool causal, hipStream_t s) {
  switch (d) {
    case 64: return launch_partial_d<64, DT>(a, BH, causal, s);
    case 128: return launch_partial_d<128, DT>(a, BH, causal, s);
    case 256: return launch_partial_d<256, DT>(a, BH, causal, s);
    default: return hipErrorInvalidValue;
  }
}

// Live key tiles of each (mask head, query tile) of the block-sparse forward:
// out[0] = count, out[1] = how many leading entries need no mask (full tiles
// below the causal diagonal of every row of the tile), out[2 + i] = key tile |
// (query-block bits << 24), in increasing tile order, then kSparsePad
// entries naming the first tile past the last key with no bits.  A key tile is live when some 128-row query block of
// the workgroup's tile attends to its 128-key block (and, when causal, the
// tile is not wholly above the diagonal).  One thread per list.
template <int D>
__global__ void __launch_bounds__(256)
bs_index_kernel(const uint8_t* __restrict__ mask, int* __restrict__ out, int n_lists,
                int n_qtiles, int N, int stride, int causal) {
  using C = FwdSparseCfg<D>;
  constexpr int BM = 32 * C::QB * C::NW;
  constexpr int BN = C::BN;
  constexpr int QBW = BM / kSparseBlock;  // query blocks per workgroup tile
  static_assert(BM % kSparseBlock == 0 && kSparseBlock % BN == 0, "sparse block sizes");
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= n_lists) return;
  const int mh = (int)(gid / n_qtiles);
  const int qt = (int)(gid % n_qtiles);
  const int nb = (N + kSparseBlock - 1) / kSparseBlock;
  const int nkt = (N + BN - 1) / BN;
  const int q0 = qt * BM;
  const int qlast = min(q0 + BM, N) - 1;
  const uint8_t* mrow = mask + (int64_t)mh * nb * nb;
  int* o = out + gid * stride + 1;
  int count = 0, full = 0;
  // Tiles below this need no mask: every key of the tile exists and is at or
  // before every query row of the workgroup tile.
  const int t_nomask = min(N / BN, causal ? (q0 + 1) / BN : N / BN);
  for (int t = 0; t < nkt; ++t) {
    if (causal && t * BN > qlast) break;
    const int kb = t * BN / kSparseBlock;
    int bits = 0;
#pragma unroll
    for (int b = 0; b < QBW; ++b) {
      const int qblk = q0 / kSparseBlock + b;
      if (qblk < nb && mrow[(int64_t)qblk * nb + kb] != 0) bits |= 1 << b;
    }
    if (bits) {
      if (full == count && t < t_nomask && bits == (1 << QBW) - 1) full = count + 1;
      o[1 + count++] = t | (bits << 24);
    }
  }
  for (int i = 0; i < kSparsePad; ++i) o[1 + count + i] = nkt;
  out[gid * stride] = count;
  o[0] = full;
}

template <int D, int DT>
hipError_t launch_sparse_d(const FwdArgs& a, int BH, bool causal, const uint8_t* mask,
                           int* list, hipStream_t s) {
  using C = FwdSparseCfg<D>;
  constexpr int BM = 32 * C::QB * C::NW;
  FwdArgs args = a;
  const int n_qtiles = (a.N + BM - 1) / BM;
  args.bs_stride = sparse_list_stride<D>(a.N);
  const int64_t n_lists = (int64_t)(a.bs_per_batch ? BH : a.heads) * n_qtiles;
  const int64_t blocks = (n_lists + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bs_index_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, s, mask, list,
                     (int)n_lists, n_qtiles, a.N, args.bs_stride, causal ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return causal ? launch_one<D, true, false, false, DT, true, C>(args, BH, s, list)
                : launch_one<D, false, false, false, DT, true, C>(args, BH, s, list);
}

template <int DT>
hipError_t launch_sparse_dtype(const FwdArgs& a, int BH, int d, bool causal, const uint8_t* mask,
                               int* list, hipStream_t s) {
  switch (d) {
    case 64: return launch_sparse_d<64, DT>(a, BH, causal, mask, list, s);
    case 128: return launch_sparse_d<128, DT>(a, BH, causal, mask, list, s);
    case 256: return launch_sparse_d<256, DT>(a, BH, causal, mask, list, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t sparse_list_bytes(int n_mask_heads, int N, int d) {
  int stride = 0, n_qtiles = 0;
  switch (d) {
    case 64: stride = sparse_list_stride<64>(N); n_qtiles = sparse_qtiles<64>(N); break;
    case 128: stride = sparse_list_stride<128>(N); n_qtiles = sparse_qtiles<128>(N); break;
    case 256: stride = sparse_list_stride<256>(N); n_qtiles = sparse_qtiles<256>(N); break;
    default: return 0;
  }
  return (size_t)n_mask_heads * n_qtiles * stride * sizeof(int);
}

hipError_t launch_fwd_sparse(const FwdArgs& a0, int B, int H, int d, int dtype, bool causal,
                             const uint8_t* mask, int* list, hipStream_t stream) {
  FwdArgs a = a0;
  a.Nk = a.N;
  a.c_off = 0;
  a.k_chunk = a.N;
  a.n_split = 1;
  a.heads = H;
  const int BH = B * H;
  return dtype == 0 ? launch_sparse_dtype<0>(a, BH, d, causal, mask, list, stream)
                    : launch_sparse_dtype<1>(a, BH, d, causal, mask, list, stream);
}

hipError_t launch_fwd(const FwdArgs& a0, int B, int H, int d, int dtype, bool causal,
                      hipStream_t stream, bool per_tile) {
  FwdArgs a = a0;
  a.Nk = a.N;  // every key, one split, top-left diagonal
  a.c_off = 0;
  a.k_chunk = a.N;
  a.n_split = 1;
  const int BH = B * H;
  return dtype == 0 ? launch_dtype<0>(a, BH, d, causal, per_tile, stream)
                    : launch_dtype<1>(a, BH, d, causal, per_tile, stream);
}

hipError_t launch_fwd_partial(const FwdArgs& a, int B, int H, int d, int dtype, bool causal,
                              hipStream_t stream) {
  const int BH = B * H;
  return dtype == 0 ? launch_partial_dtype<0>(a, BH, d, causal, stream)
                    : launch_partial_dtype<1>(a, BH, d, causal, stream);
}

}  // namespace fa
