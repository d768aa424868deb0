// FP8 (e4m3) attention forward for gfx950 ("FlashAttention-3: Fast and
// Accurate Attention with Asynchrony and Low-precision", abstract: FP8 with
// block quantization and incoherent processing).  Operands come from
// fa_quant_fp8: Q and K rotated by the same signed Hadamard transform (1/d
// folded into Q's scales), V unrotated, one fp32 scale per 128-row block.
//
// Same structure as the 16-bit forward (query rows in registers, K/V tiles
// copied from HBM into an LDS ring by buffer loads with an LDS destination
// (eight stages and one barrier per four tiles, or three and one per tile),
// three-stage fused pipeline S(j+1) | softmax(j) | PV(j-1), S^T layout with
// one query per lane, lazy exp2 reference), with:
//   * S^T = K8 Q8^T on v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, fp32 acc);
//     the product of the query block's and key block's scales, the softmax
//     scale and log2(e) is one fp32 multiplier per tile (a key tile lies in
//     one 128-row scale block, a wave's 32 queries likewise);
//   * probabilities P~ = exp2(s - m_ref) are rounded to e4m3 (round to
//     nearest even) for O += P V; the reference m_ref never exceeds the
//     running maximum and is raised when some lane's partial row sum of a
//     tile exceeds kLazySum8 = 448, so every P~ stays at most 448 (the e4m3
//     maximum: no saturation); the row normaliser is summed from the fp32
//     P~;
//   * the output accumulator is kept in units of one value block's scale
//     vs_acc; a later block whose scale differs from vs_acc by a power of two
//     (power-of-two block scales, or one scale per tensor) has that factor
//     applied as the e4m3 operand's block-scale exponent of its P V products
//     (the scaled matrix instruction's E8M0 scale: exact, no vector work);
//     any other block scale re-expresses O by vs_acc / vs_new at the end of
//     the tile before the block's first P V product, where a reference raise
//     also rescales O;
//   * V8 stays row-major in LDS and is read transposed with ds_read_b64_tr_b8
//     (inside a 16-lane group, lane j's byte e is byte j%8 of the chunk
//     addressed by lane 2e + j/8); 16-byte chunks of a V row are XOR-swizzled
//     so that the eight rows those reads touch fall in distinct LDS banks, and
//     K rows so that sixteen rows read at one column do.
#include <algorithm>

#include "common.h"
#include "kernels.h"

// Operand fragments read ahead of the fp8 matrix instructions.
#ifndef FA_FP8_PF
#define FA_FP8_PF 2
#endif
// Explicit instruction order inside the fused steps (see `fused`).
#ifndef FA_FP8_SGB
#define FA_FP8_SGB 1
#endif

namespace fa {

namespace {

typedef int i32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16_t mfma_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
  // Format code 0 = e4m3 for both operands; no per-block hardware scaling.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same product with A's elements multiplied by 2^(ea - 127): an E8M0
// block scale (lane l's value covers row l % 32 over its 32 K slots; here the
// same value in every lane), B's scale 127 = 1.
__device__ __forceinline__ f32x16_t mfma_fp8_scale_a(i32x8_t a, i32x8_t b, f32x16_t c, int ea) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, 127);
}

__device__ __forceinline__ i32x2_t ld_lds_tr8(const FA_LDS void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      reinterpret_cast<FA_LDS i32x2_t*>(const_cast<FA_LDS void*>(p)));
}

// Probabilities are at most this: the e4m3 maximum, so rounding P~ never
// saturates (a threshold of 256 raised the reference more often: 1-4 % slower
// on inputs with outliers).
constexpr float kLazySum8 = 448.0f;

// XOR applied to the 8-byte unit index of V row `row` (a multiple of 2, i.e.
// whole 16-byte chunks).
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  const int g = ((row >> 1) & 1) | (((row >> 3) & 1) << 1);
  return (4 * g) & (D / 8 - 4);
}
// XOR applied to the 16-byte chunk index of K row `row`: rows sharing a
// 256-byte bank window get distinct chunks.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return (row / (256 / D)) & (D / 16 - 1);
}

// The key and value scales are separate read-only, non-aliased arguments so
// that their per-tile reads can be scalar loads.
// NSTG = LDS stages per tensor: 8 runs the iterations in groups of four with
// one workgroup barrier per group, 3 has one barrier per iteration (see
// below).
template <int D, int BN, int NW, int OCC, int NSTG, bool CAUSAL, bool PERSIST>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
fwd_fp8_kernel(Fp8Args a, const float* __restrict__ k_scale, const float* __restrict__ v_scale) {
  constexpr int BM = 32 * NW;
  static_assert(NSTG == 3 || NSTG == 8, "stage count");
  constexpr bool GROUPED = NSTG == 8;  // tile t in stage t % NSTG; groups of G iterations
  constexpr int G = NSTG / 2;       // iterations per barrier
  constexpr int MSK = NSTG - 1;
  constexpr int ROWB = D;            // bytes per row
  constexpr int TILEB = BN * ROWB;
  constexpr int CH_ROW = D / 16;
  static_assert(TILEB % (1024 * NW) == 0, "a tile must split into whole 1 KiB copies per wave");
  constexpr int IPW = TILEB / 1024 / NW;
  static_assert(BN == 64, "one 32x32x64 product per pair of 32-key blocks");
  static_assert(128 % BN == 0, "tiles inside one scale block");
  constexpr int NKB = BN / 32;
  constexpr int NDC = D / 64;        // 64-wide head-dim chunks of S
  constexpr int NDB = D / 32;

  // The persistent grids at d = 128 copy the next unit's first two K tiles
  // into stages 0 and 1 while the current unit's O passes through LDS: O is
  // then staged above them.
  constexpr bool PREFETCH = PERSIST && D == 128;
  constexpr int OROWB = 2 * D + 8;  // bytes per staged O row (8 bytes of padding)
  constexpr int OSTB = PREFETCH ? 2 * TILEB : 0;
  constexpr int SMEM = 2 * NSTG * TILEB > OSTB + NW * 32 * OROWB ? 2 * NSTG * TILEB
                                                                 : OSTB + NW * 32 * OROWB;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
  FA_LDS uint8_t* lds = (FA_LDS uint8_t*)smem;  // K stage s at s*TILEB, V at (NSTG+s)*TILEB

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int N = a.N;

  // Q8^T operand: lane holds query qrow, head-dim bytes dc*64 + 32*hl +
  // [0, 32).  Declared outside the unit: the persistent grids load the next
  // unit's rows here during the current unit's epilogue.
  i32x8_t qf[NDC];

  // One work unit: query tile qt of head bh.  nxt: the next unit of this
  // workgroup (persistent grids at d = 128; head * n_qtiles + query tile),
  // else -1; pre: this unit's Q rows and first two K tiles were fetched by
  // the previous unit's epilogue.
  auto unit = [&](const int bh_in, const int qt_in, const int nxt, const bool pre)
                  __attribute__((always_inline)) {
  // The unit's indices come out of runtime divisions, which the compiler
  // does on the vector ALU; taken to scalar registers here, every address
  // and tile bound derived from them stays on the scalar unit instead of
  // costing vector instructions (and v_readfirstlane) in every iteration.
  const int bh = __builtin_amdgcn_readfirstlane(bh_in);
  const int qt = __builtin_amdgcn_readfirstlane(qt_in);
  // In the persistent loop the lane index passes through an empty asm so
  // that nothing derived from it is hoisted out of the loop over units (it
  // would stay live across units and spill at the register limit).
  int tid = threadIdx.x;
  if constexpr (PERSIST) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int64_t base = (int64_t)bh * N * D;
  const uint8_t* Q = static_cast<const uint8_t*>(a.q8) + base;
  const uint8_t* K = static_cast<const uint8_t*>(a.k8) + base;
  const uint8_t* V = static_cast<const uint8_t*>(a.v8) + base;
  const float* qsc = a.q_scale + (int64_t)bh * a.nblk;
  const float* ksc = k_scale + (int64_t)bh * a.nblk;
  const float* vsc = v_scale + (int64_t)bh * a.nblk;

  const int q0 = qt * BM;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;
  const float q_scale = qsc[min(qw0, N - 1) / 128];
  const float qmul = q_scale * a.scale_log2;
  // Scales of tile t (clamped past the last block: such tiles are all zero).
  // These must be scalar loads: a vector load here would be followed by a
  // wait on the vector-memory counter, which also waits for every tile copy
  // in flight.
  const int nblk = a.nblk;
  auto blk = [&](int t) { return __builtin_amdgcn_readfirstlane(min(max(t, 0) * BN / 128, nblk - 1)); };
  auto kscale = [&](int t) { return ksc[blk(t)]; };
  auto vscale = [&](int t) { return vsc[blk(t)]; };

  // ---- Copies.  Copy jj of this wave fills LDS chunk (wave*IPW + jj)*64 +
  // lane of a tile: row p / CH_ROW; K and V swizzle differently.
  uint32_t koff_dma[IPW], voff_dma[IPW];
#pragma unroll
  for (int jj = 0; jj < IPW; ++jj) {
    const int p = (wave * IPW + jj) * 64 + lane;
    const int r = p / CH_ROW, pc = p % CH_ROW;
    koff_dma[jj] = (uint32_t)(r * ROWB + (pc ^ k_swz<D>(r)) * 16);
    voff_dma[jj] = (uint32_t)(r * ROWB + (pc ^ (v_swz<D>(r) >> 1)) * 16);
  }
  // Rows of tile t: BN up to the last full tile, the remainder on the
  // partial one, none before the first tile or past the end.  Written as
  // comparisons and selects, which stay on the scalar unit (a clamp becomes
  // a vector med3 and a readfirstlane per copy).
  const int nfull = N / BN, nrem = N % BN;
  auto issue = [&](const uint8_t* src, int t, FA_LDS uint8_t* stage, const uint32_t (&voff)[IPW]) {
    const int rows = (uint32_t)t < (uint32_t)nfull ? BN : (t == nfull ? nrem : 0);
    const u32x4_t r = make_rsrc(src + (int64_t)max(t, 0) * BN * D, rows * ROWB);
#pragma unroll
    for (int jj = 0; jj < IPW; ++jj) {
      if (jj == 0) dma16_buf<4>(r, voff[jj], stage + (wave * IPW + jj) * 1024);
      else dma16_buf<0>(r, voff[jj], stage + (wave * IPW + jj) * 1024);
    }
  };
  // Tile t lives in stage t % NSTG; st = the stage of tile j, carried by the
  // loops.  Iteration j reads K(j+1) and V(j-1).
  auto snext = [](int x) { return x == NSTG - 1 ? 0 : x + 1; };
  auto sprev = [](int x) { return x == 0 ? NSTG - 1 : x - 1; };
  // Eight stages: iterations run in groups of G = 4 (j odd .. j + 3) with one
  // workgroup barrier per group.  A group reads K(j+1 .. j+G) and
  // V(j-1 .. j+G-2); its first iteration copies K(j+G+1 .. j+2G) and
  // V(j+G-1 .. j+2G-2), which the next group reads, into the stages the
  // previous group read (free since its barrier); its last iteration waits
  // for those copies and ends with the barrier that publishes them.  The
  // prologue pair (-1, 0) reads K(0) and K(1) and copies K(2 .. G+1) and
  // V(0 .. G-1).  The stage of tile t >= -2 is computed from t directly
  // (measured faster than carrying it).  Fewer barriers shorten the time the
  // leading wave of a SIMD waits for the other: one barrier per two tiles was
  // 3-4 % faster than one per tile, one per four another 2-4 %.
  // Three stages: iteration j copies K(j+3) and V(j+1) into the stages of K(j)
  // and V(j-2) and ends with a barrier after waiting for K(j+2) and V(j).
  auto issue_range = [&](int k0, int v0) {
#pragma unroll
    for (int i = 0; i < G; ++i) issue(K, k0 + i, lds + ((k0 + i) & MSK) * TILEB, koff_dma);
#pragma unroll
    for (int i = 0; i < G; ++i) issue(V, v0 + i, lds + (NSTG + ((v0 + i) & MSK)) * TILEB, voff_dma);
  };

  auto load_q = [&](const uint8_t* Qh, int row) {
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      u32x4_t lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (row < N) {
        const uint8_t* p = Qh + (int64_t)row * D + dc * 64 + 32 * hl;
        lo = ld_global16(p);
        hi = ld_global16(p + 16);
      }
      qf[dc] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  };
  if (!pre) load_q(Q, qrow);

  f32x16_t oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_run = -INFINITY;  // exp2 reference, log2 units
  float l_run = 0.f;
  // V scale the accumulator is expressed in, as its fp32 bit pattern: the
  // comparisons with a new block's scale are integer work on the scalar unit.
  uint32_t vs_acc = __float_as_uint(vscale(0));

  // ---- LDS read offsets.  K rows (A operand of S^T): lane reads row
  // kb*32 + l32, logical chunks 4*dc + 2*hl + {0, 1}.
  int koff[NDC][2];
  {
    const int f = k_swz<D>(l32);  // equals k_swz of row kb*32 + l32
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
      for (int u = 0; u < 2; ++u) koff[dc][u] = l32 * ROWB + 16 * ((4 * dc + 2 * hl + u) ^ f);
  }
  // V^T (A operand of O^T): supplier lane 2e + c of each 16-lane group reads
  // row 16 rd + tr_row of the tile and 8-byte unit db*4 + tr_unit.  The
  // swizzle depends on row bits 1 and 3 only, so the four reads rd of one
  // block sit 16 rows apart at one lane-dependent offset: one address per
  // block, the rest in the instructions' immediate offsets.  The offsets
  // include the base of the V stages (NSTG * TILEB), hidden from the
  // compiler so that it cannot fold it into the immediates: the immediate
  // field holds 16 bits, enough for a stage offset inside one region but
  // not for the V region's base on top of it.
  const int tr_e = (lane & 15) >> 1;
  const int tr_unit = ((lane >> 4) & 1) * 2 + (lane & 1);
  int voff[NDB];
  {
    const int row = 8 * (tr_e >> 2) + 4 * hl + (tr_e & 3);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      voff[db] = NSTG * TILEB + row * ROWB + (((db * 4 + tr_unit) ^ v_swz<D>(row)) * 8);
      asm volatile("" : "+v"(voff[db]));
    }
  }
  auto ld_k = [&](const FA_LDS uint8_t* ks, int kb, int dc) {
    const FA_LDS uint8_t* p = ks + kb * 32 * ROWB;
    const u32x4_t lo = ld_lds16(p + koff[dc][0]), hi = ld_lds16(p + koff[dc][1]);
    return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto ld_v = [&](const FA_LDS uint8_t* vs, int db) {
    i32x8_t vf;
    const FA_LDS uint8_t* vb = vs + voff[db];
#pragma unroll
    for (int rd = 0; rd < 4; ++rd) {
      const i32x2_t v2 = ld_lds_tr8(vb + rd * 16 * ROWB);
      vf[2 * rd] = v2[0];
      vf[2 * rd + 1] = v2[1];
    }
    return vf;
  };

  typedef f32x16_t Scores[NKB];
  typedef int Probs[8];  // P^T operand: byte s = 16*kb + r holds key 32*kb + 8*(r/4) + 4*hl + r%4

  // ---- Probabilities of one tile (scores already multiplied to log2 units
  // by mul) against the reference -m_neg, packed as e4m3; returns the lane's
  // fp32 sum of the unrounded values.
  // Partial sums start at -0, the additive identity, so that the first
  // addition folds away.  The packing of four probabilities writes the low
  // half of a word, then the high half; the word's old content is passed for
  // the untouched half of the first write (it is overwritten by the second),
  // which saves materialising a zero.
  auto pack4 = [](float p0, float p1, float p2, float p3, int old) {
    const int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, old, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
  };
  auto phase_p = [&](const Scores& s, Probs& pw, float mul, float m_neg) {
    float ps0 = -0.f, ps1 = -0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const f32x16_t& sb = s[w >> 2];
      const int r0 = 4 * (w & 3);
      float p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) p[u] = fast_exp2(fmaf(sb[r0 + u], mul, m_neg));
      ps0 += p[0] + p[2];
      ps1 += p[1] + p[3];
      pw[w] = pack4(p[0], p[1], p[2], p[3], pw[w]);
    }
    return ps0 + ps1;
  };

  // Ratio of two value-block scales (fp32 bit patterns), exactly 1 for
  // equal scales, otherwise by a hardware reciprocal (within 1 ulp; far below
  // the e4m3 rounding of P and V).
  auto vscale_ratio = [](uint32_t from, uint32_t to) {
    return from == to ? 1.0f : __uint_as_float(from) * __builtin_amdgcn_rcpf(__uint_as_float(to));
  };
  // E8M0 exponent that carries scale `b` relative to scale `a` (fp32 bit
  // patterns; 127 + the exponent difference) when both are normal values
  // with equal mantissas and the difference fits the E8M0 range; -1
  // otherwise.
  auto vscale_exponent = [](uint32_t a, uint32_t b) {
    const int ea = (int)((a >> 23) & 0xffu), eb = (int)((b >> 23) & 0xffu);
    const int x = 127 + eb - ea;
    const bool ok = ((a ^ b) & 0x807fffffu) == 0 && ea != 0 && eb != 0 && x >= 0 && x <= 254;
    return ok ? x : -1;
  };

  // ---- End of a tile: raise the reference if the tile's probabilities left
  // [0, kLazySum8] (or the row had none), rescaling O (which already holds
  // P(j-1) V(j-1)) and l to the new reference.
  const uint32_t opaque_zero = (uint32_t)(N >> 31);
  // `vchange`: the tile starts a value block whose scale `vto` is not a
  // power of two times the accumulator's `vfrom` (fp32 bit patterns); O is
  // then re-expressed by vfrom / vto.  The ratio is formed only on that
  // rare path.
  auto finish_tile = [&](const Scores& s, Probs& pw, float mul, float psum, bool vchange,
                         uint32_t vfrom, uint32_t vto) {
    float alpha = 1.0f;
    if (wave_any(!(psum <= kLazySum8))) {
      asm volatile("" ::: "memory");
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = max_halves(mx) * mul;  // mul > 0
      const float m_new = fmaxf(m_run, mx);
      alpha = (m_new == m_run) ? 1.0f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      Probs fresh;
#pragma unroll
      for (int w = 0; w < 8; ++w) fresh[w] = pw[w];
      psum = phase_p(s, fresh, mul, m_new == -INFINITY ? 0.f : -m_new);
#pragma unroll
      for (int w = 0; w < 8; ++w) pw[w] = (int)((uint32_t)fresh[w] | ((uint32_t)pw[w] & opaque_zero));
    }
    l_run += psum;
    float f = alpha;
    if (vchange) {  // wave-uniform; rare
      asm volatile("" ::: "memory");
      f *= vscale_ratio(vfrom, vto);
    }
    if (f != 1.0f) {  // rare
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (OCC == 1) {
            float t;
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(t) : "a"(oacc[i][r]));
            t *= f;
            asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(oacc[i][r]) : "v"(t));
          } else {
            oacc[i][r] *= f;
          }
        }
    }
  };

  // Fused iteration (see the 16-bit forward): NSTEP steps, each with one
  // S(j+1) and one P(j-1) V matrix instruction and a share of the
  // probability words of P(j).
  constexpr int NS_S = NKB * NDC, NS_PV = NDB;
  constexpr int NSTEP = (NS_S + NS_PV) / 2;
  static_assert((NS_S + NS_PV) % 2 == 0, "two matrix instructions per step");
  // The K and V scales of tile j are loaded one iteration ahead: a scalar
  // load shares its wait counter with the LDS reads, so waiting for it inside
  // the steps would also wait for every fragment read in flight.
  float ks_pre = kscale(-1), vs_pre = vscale(-1);
  // VB: tile j starts a value block (j even: 128-row blocks of two 64-key
  // tiles).  Its scale vs_j is carried either by the E8M0 exponent ea_cur of
  // the P V products of the block (when vs_j = 2^k vs_acc), or by
  // re-expressing O in vs_j at the end of the iteration, once P(j-1) V(j-1)
  // is in O and before P(j) V(j) is added in the next one: O times
  // vs_acc / vs_j on the rare path of the tile's end, so that the steps
  // themselves hold no branch (a branch there lets the compiler move the
  // products and the softmax apart).
  int ea_cur = 127;  // E8M0 exponent of the value block of the P V products
  i32x8_t pre_fr[FA_FP8_PF];  // first fragments of the next iteration, read ahead
  auto issue_iter = [&](int j, int st) {
    issue(K, j + 3, lds + st * TILEB, koff_dma);
    issue(V, j + 1, lds + (NSTG + snext(st)) * TILEB, voff_dma);
  };
  auto fused = [&](auto ds_tag, auto ms_tag, auto dp_tag, auto dpv_tag, auto vb_tag, auto pos_tag,
                   auto ph_tag, int j, int st, Scores& s_cur, Scores& s_nxt, Probs& p_cur,
                   const Probs& p_prev) {
    constexpr bool DS = decltype(ds_tag)::value, MS = decltype(ms_tag)::value;
    constexpr bool DP = decltype(dp_tag)::value, DPV = decltype(dpv_tag)::value;
    constexpr bool VB = decltype(vb_tag)::value && DP && DPV;
    // POS: -2 / -1 = first / second iteration of the prologue, else the
    // position in a group (0 .. G-1; 0 and 1 with three stages).
    constexpr int POS = decltype(pos_tag)::value;
    // PH: with eight stages, the parity of the group (j = 1 + G * PH + POS
    // modulo NSTG) when the caller knows it, else -1.  A known phase makes
    // the stages of the tiles read compile-time constants, so that every
    // LDS read address is a lane offset plus an immediate.
    constexpr int PH = decltype(ph_tag)::value;
    constexpr bool KNOWN = GROUPED && PH >= 0 && POS >= 0;
    // Inside a group the next iteration's value tile is already published:
    // the last step reads its first fragments (PRE: this iteration's were
    // read so), which the next iteration's first products would otherwise
    // wait for at its start.
    constexpr bool PRE = KNOWN && POS > 0 && DPV;
    constexpr bool NXT = KNOWN && POS < G - 1;
    const float ks_j = ks_pre, vs_j = vs_pre;
    if constexpr (!GROUPED) {  // d = 256: loaded ahead of the steps (fewer live registers)
      ks_pre = kscale(j + 1);
      vs_pre = vscale(j + 1);
    }
    if constexpr (!GROUPED)
      issue_iter(j, st);
    else if constexpr (POS == -2)
      issue_range(2, 0);
    else if constexpr (POS == 0)
      issue_range(j + G + 1, j + G - 1);
    const int kst = KNOWN ? (2 + G * PH + POS) & MSK : GROUPED ? (j + 1) & MSK : snext(st);
    const int vst = KNOWN ? (G * PH + POS) & MSK : GROUPED ? (j - 1) & MSK : sprev(st);
    const FA_LDS uint8_t* ks = lds + kst * TILEB;
    const FA_LDS uint8_t* vs = lds + vst * TILEB;  // voff holds the V region's base
    const float mul = qmul * ks_j;  // tile j's scores to log2 units
    const float m_neg = -m_run;
    const int ea_pv = ea_cur;  // P(j-1) V(j-1): the previous tile's block
    bool vchange = false;
    const uint32_t vfrom = vs_acc;
    if constexpr (VB) {
      const uint32_t vb = __float_as_uint(vs_j);
      const int x = vscale_exponent(vs_acc, vb);
      vchange = x < 0;
      ea_cur = vchange ? 127 : x;
      vs_acc = vchange ? vb : vs_acc;
    }
    if constexpr (DS) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s_nxt[kb][r] = 0.f;
    }
    if constexpr (DP && MS) {
      // The mask goes on S(j) before its probabilities are formed (its
      // products completed in the previous iteration): a mask on S(j+1)
      // after the steps waited for their products.  Register r of block kb
      // holds key j*BN + 4*hl + (kb*32 + 8*(r/4) + r%4).
      int lim = N - j * BN - 4 * hl;
      if (CAUSAL) lim = min(lim, qrow + 1 - j * BN - 4 * hl);
      // Tiles of the masked tail that need no mask in any lane skip it.
      constexpr int kMaxOff = (NKB - 1) * 32 + 27;  // largest key offset of a register
      if (wave_any(lim <= kMaxOff)) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) s_cur[kb][r] = -INFINITY;
      }
    }
    float ps0 = -0.f, ps1 = -0.f;
    // The P(j-1) V products come first and the S(j+1) products last, so O is
    // complete when the end of the tile may rescale it, while S(j+1) is not
    // needed before the next iteration.
    const i32x8_t pf = {p_prev[0], p_prev[1], p_prev[2], p_prev[3],
                        p_prev[4], p_prev[5], p_prev[6], p_prev[7]};
    // Matrix instructions m = M0 .. M1-1 of this iteration (PV first, then
    // S); the operand fragment of instruction m is read PF instructions
    // ahead, into a ring of PF + 1 fragments.
    constexpr int M0 = DPV ? 0 : NS_PV, M1 = DS ? NS_PV + NS_S : NS_PV;
    constexpr int PF = FA_FP8_PF;
    static_assert(!NXT || PF <= NS_PV, "the fragments read ahead are value fragments");
    auto frag = [&](int m) {
      if (m < NS_PV) return ld_v(vs, m);
      return ld_k(ks, (m - NS_PV) % NKB, (m - NS_PV) / NKB);
    };
    i32x8_t fr[PF + 1];
#pragma unroll
    for (int m = M0; m < M1 && m < M0 + PF; ++m)
      fr[(m - M0) % (PF + 1)] = PRE ? pre_fr[m - M0] : frag(m);
#pragma unroll
    for (int step = 0; step < NSTEP; ++step) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int m = 2 * step + u;  // matrix instruction index: PV first, then S
        if (m >= M0 && m < M1) {
          if (m + PF < M1) fr[(m + PF - M0) % (PF + 1)] = frag(m + PF);
          const i32x8_t& f = fr[(m - M0) % (PF + 1)];
          if (m < NS_PV) {
            oacc[m] = mfma_fp8_scale_a(f, pf, oacc[m], ea_pv);
          } else {
            const int kb = (m - NS_PV) % NKB, dc = (m - NS_PV) / NKB;
            s_nxt[kb] = mfma_fp8(f, qf[dc], s_nxt[kb]);
          }
        }
      }
      if constexpr (DP) {
#pragma unroll
        for (int w = step * 8 / NSTEP; w < (step + 1) * 8 / NSTEP; ++w) {
          const f32x16_t& sb = s_cur[w >> 2];
          const int r0 = 4 * (w & 3);
          float p[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) p[u] = fast_exp2(fmaf(sb[r0 + u], mul, m_neg));
          ps0 += p[0] + p[2];
          ps1 += p[1] + p[3];
          p_cur[w] = pack4(p[0], p[1], p[2], p[3], p_cur[w]);
        }
      }
      if constexpr (DS && DP && DPV && OCC > 1) {
        if (step == 0) __builtin_amdgcn_s_setprio(1);
        if (step == NSTEP / 2) __builtin_amdgcn_s_setprio(0);
      }
      // Order inside a full step: the first product, the step's fragment
      // reads, a few vector instructions (four at d <= 128, two at d = 256),
      // the second product, the rest of the vector work.  Left to itself the
      // compiler issues the two products nearly back to back, and the wave
      // then waits for the matrix unit before its vector work; this order
      // measured 1.2-1.7 % faster at d = 128 (other splits, 0-28 vector
      // instructions before the second product, in between) and 5-6 % at
      // d = 256.
      if constexpr (DS && DP && DPV && FA_FP8_SGB) {
        constexpr int kBefore = D == 256 ? 2 : 4;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // matrix
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);        // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, kBefore, 0);  // vector
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // matrix
        __builtin_amdgcn_sched_group_barrier(0x002, 28 - kBefore, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NXT) {
      const FA_LDS uint8_t* vs_n = lds + ((G * PH + POS + 1) & MSK) * TILEB;
#pragma unroll
      for (int m = 0; m < PF; ++m) pre_fr[m] = ld_v(vs_n, m);
    }
    // The scales of tile j + 1, for the next iteration.  Issued here, after
    // the last fragment wait: a scalar load in flight turns every wait for
    // an LDS read into a wait for everything.
    if constexpr (GROUPED) {
      ks_pre = kscale(j + 1);
      vs_pre = vscale(j + 1);
    }
    if constexpr (DP) finish_tile(s_cur, p_cur, mul, ps0 + ps1, vchange, vfrom, vs_acc);
    if constexpr (!GROUPED)
      dma_sync<2 * IPW>();
    else if constexpr (POS == -1 || POS == G - 1)
      dma_sync<0>();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  int t_mask = (N % BN) ? N / BN : ntiles;
  if (CAUSAL) t_mask = min(t_mask, (q0 + 1) / BN);
  t_mask = min(t_mask, ntiles);

  Scores sA, sB;
  Probs pA, pB;

  // Prologue and iterations as in the 16-bit forward: tiles past the last one
  // (or past a wave's causal diagonal) come out fully masked, so their
  // probabilities and P V products are exactly zero.
  // The prologue pair (-1, 0) reads K(0) and K(1), copied and published
  // first.
  if (!pre) {
    issue(K, 0, lds, koff_dma);
    issue(K, 1, lds + TILEB, koff_dma);
  }
  if (GROUPED || pre)
    dma_sync<0>();
  else
    dma_sync<IPW>();
  using PM2 = std::integral_constant<int, -2>;
  using PM1 = std::integral_constant<int, -1>;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  using PHR = std::integral_constant<int, -1>;  // group phase known at run time only
  using PH0 = std::integral_constant<int, 0>;
  using PH1 = std::integral_constant<int, 1>;
  fused(T_{}, T_{}, F_{}, F_{}, F_{}, PM2{}, PHR{}, -1, NSTG - 1, sB, sA, pB, pA);  // S(0) -> sA
  fused(T_{}, T_{}, T_{}, F_{}, F_{}, PM1{}, PHR{}, 0, 0, sA, sB, pA, pB);  // S(1) -> sB, P(0) -> pA
  int j = 1, st = 1;
  // j is odd at the start of a trip; even iterations start a value block.
  if constexpr (NSTG == 3) {
    for (; j + 2 < t_mask; j += 2) {
      const int stb = snext(st);
      fused(T_{}, F_{}, T_{}, T_{}, F_{}, P0{}, PHR{}, j, st, sB, sA, pB, pA);
      fused(T_{}, F_{}, T_{}, T_{}, T_{}, P1{}, PHR{}, j + 1, stb, sA, sB, pA, pB);
      st = snext(stb);
    }
    for (; j <= ntiles; j += 2) {
      const int stb = snext(st);
      fused(T_{}, T_{}, T_{}, T_{}, F_{}, P0{}, PHR{}, j, st, sB, sA, pB, pA);
      if (j + 1 > ntiles) break;
      fused(T_{}, T_{}, T_{}, T_{}, T_{}, P1{}, PHR{}, j + 1, stb, sA, sB, pA, pB);
      st = snext(stb);
    }
  } else {
    // Two groups per trip: the first starts at j = 1 modulo NSTG, so both
    // groups' stages are compile-time constants.  What is left (at most a
    // group without masks, then the masked tail) takes the stages from j.
    static_assert(G == 4 && NSTG == 2 * G, "four iterations per group, two groups per ring");
    auto group = [&](auto ph, int jg) __attribute__((always_inline)) {
      fused(T_{}, F_{}, T_{}, T_{}, F_{}, P0{}, ph, jg, 0, sB, sA, pB, pA);
      fused(T_{}, F_{}, T_{}, T_{}, T_{}, P1{}, ph, jg + 1, 0, sA, sB, pA, pB);
      fused(T_{}, F_{}, T_{}, T_{}, F_{}, P2{}, ph, jg + 2, 0, sB, sA, pB, pA);
      fused(T_{}, F_{}, T_{}, T_{}, T_{}, P3{}, ph, jg + 3, 0, sA, sB, pA, pB);
    };
    for (; j + 2 * G < t_mask; j += 2 * G) {
      group(PH0{}, j);
      group(PH1{}, j + G);
    }
    for (; j <= ntiles; j += 4) {
      fused(T_{}, T_{}, T_{}, T_{}, F_{}, P0{}, PHR{}, j, 0, sB, sA, pB, pA);
      if (j + 1 > ntiles) break;
      fused(T_{}, T_{}, T_{}, T_{}, T_{}, P1{}, PHR{}, j + 1, 0, sA, sB, pA, pB);
      if (j + 2 > ntiles) break;
      fused(T_{}, T_{}, T_{}, T_{}, F_{}, P2{}, PHR{}, j + 2, 0, sB, sA, pB, pA);
      if (j + 3 > ntiles) break;
      fused(T_{}, T_{}, T_{}, T_{}, T_{}, P3{}, PHR{}, j + 3, 0, sA, sB, pA, pB);
    }
  }
  wait_vmcnt<0>();

  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.f ? __uint_as_float(vs_acc) / l_tot : 0.f;
  // O leaves through LDS: each lane holds one query row in 8-byte pieces, so
  // storing from the accumulators would scatter every store instruction over
  // 32 rows (measured ~6,000 cycles per wave).  The wave writes its 32 x D
  // block into LDS (rows padded by 8 bytes, so the 8-byte writes of one
  // half-wave hit distinct banks), then stores whole rows, 16 bytes per lane.
  // The K/V ring is free once every wave has left the loop.
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if constexpr (PREFETCH) {
    // The next unit's Q rows (this unit's are dead) and its first two K
    // tiles, into the stages below the O blocks, in flight while O leaves.
    if (nxt >= 0) {
      const int nbh = nxt / a.n_qtiles, nqt = nxt % a.n_qtiles;
      const int64_t nbase = (int64_t)nbh * N * D;
      load_q(static_cast<const uint8_t*>(a.q8) + nbase, nqt * BM + wave * 32 + l32);
      const uint8_t* Kn = static_cast<const uint8_t*>(a.k8) + nbase;
      issue(Kn, 0, lds, koff_dma);
      issue(Kn, 1, lds + TILEB, koff_dma);
    }
  }
  FA_LDS uint8_t* ost = lds + OSTB + wave * 32 * OROWB;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2_t w;
      w[0] = Elem<0>::pack2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
      w[1] = Elem<0>::pack2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      *reinterpret_cast<FA_LDS u32x2_t*>(ost + l32 * OROWB + 2 * (db * 32 + 8 * g + 4 * hl)) = w;
    }
  }
  asm volatile("" ::: "memory");
  {
    constexpr int LPR = D / 8;          // lanes per row, 16 bytes each
    constexpr int RPI = 64 / LPR;       // rows per store instruction
    const int r0 = lane / LPR, cb = (lane % LPR) * 16;
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int r = r0 + RPI * k;
      const u32x4_t v = ld_lds16(ost + r * OROWB + cb);
      if (qw0 + r < N)
        *reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(a.o) + 2 * (base + (int64_t)(qw0 + r) * D) +
                                    cb) = v;
    }
  }
  if (qrow < N && hl == 0 && a.lse != nullptr)
    a.lse[(int64_t)bh * N + qrow] = m_run * kLn2 + __logf(l_tot);
  };  // unit

  if constexpr (PERSIST && CAUSAL) {
    // Causal: query tile qt costs qt + 1 key tiles; rank 0 is the last one.
    bool pre = false;
    lpt_units(a.n_qtiles, a.bh, a.pin != 0, [&](int bh, int rank, int nbh, int nrank) {
      unit(bh, a.n_qtiles - 1 - rank,
           PREFETCH && nbh >= 0 ? nbh * a.n_qtiles + a.n_qtiles - 1 - nrank : -1, pre);
      pre = PREFETCH;
      // The next unit's first copies reuse the ring.
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    });
  } else if constexpr (PERSIST) {
    // Non-causal, all units alike: workgroup w takes units w, w + G, ... of
    // the (head, query tile) order under the XCD remap of the one-unit grid
    // below (when G is a multiple of 8, as the full grid of one workgroup per
    // CU is, each unit stays on the XCD it had there), and fetches each next
    // unit's Q rows and first K tiles during the current unit's epilogue.
    const int total = a.n_qtiles * a.bh;
    for (int u = blockIdx.x; u < total; u += gridDim.x) {
      const int logical = xcd_remap(u, total);
      const int nu = u + (int)gridDim.x;
      unit(logical / a.n_qtiles, logical % a.n_qtiles, nu < total ? xcd_remap(nu, total) : -1,
           u != (int)blockIdx.x);
      // The next unit's copies and O blocks reuse the ring.
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
  } else {
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    int qt = logical % a.n_qtiles;
    if (CAUSAL) qt = a.n_qtiles - 1 - qt;  // longest key ranges first
    unit(logical / a.n_qtiles, qt, -1, false);
  }
}

// Causal launches walk the units on a persistent heaviest-first grid at
// d = 128 and 256 (+4 to +21 % over one workgroup per tile); at d = 64 that
// measured 35 % slower (two 128-row workgroups per CU: 64 concurrent units
// of an XCD spread over eight heads' keys and values instead of one head's,
// at the lowest arithmetic intensity), so d = 64 keeps one workgroup per
// tile in dispatch order.
template <int D, int NW, int OCC, int NSTG, bool CAUSAL>
hipError_t launch_one(const Fp8Args& a0, int BH, hipStream_t s) {
  constexpr int BM = 32 * NW;
  // Non-causal launches at d = 128 also run persistent, prefetching each
  // next unit (+0.4-1.8 % in the 16-bit forward); d = 64 fits two
  // workgroups per CU, which overlap each other's prologues already, and at
  // d = 256 the prefetching unit spills registers.
  constexpr bool PERSIST = CAUSAL ? D >= 128 : D == 128;
  Fp8Args a = a0;
  a.n_qtiles = (a.N + BM - 1) / BM;
  a.bh = BH;
  const int64_t units = (int64_t)a.n_qtiles * BH;
  if (units > 0x7fffffff) return hipErrorInvalidValue;
  if constexpr (!PERSIST) {
    hipLaunchKernelGGL((fwd_fp8_kernel<D, 64, NW, OCC, NSTG, CAUSAL, false>),
                       dim3((unsigned)units), dim3(NW * 64), 0, s, a, a.k_scale, a.v_scale);
  } else {
    constexpr auto kernel = fwd_fp8_kernel<D, 64, NW, OCC, NSTG, CAUSAL, true>;
    const int slots = resident_slots<kernel>(NW * 64);
    if (slots <= 0) return hipErrorInvalidValue;
    const int64_t grid = std::min<int64_t>(units, slots);
    a.pin = (BH % 8 == 0 && grid % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(NW * 64), 0, s, a, a.k_scale,
                       a.v_scale);
  }
  return hipGetLastError();
}

template <int D, int NW, int OCC, int NSTG>
hipError_t launch_d(const Fp8Args& a, int BH, bool causal, hipStream_t s) {
  return causal ? launch_one<D, NW, OCC, NSTG, true>(a, BH, s)
                : launch_one<D, NW, OCC, NSTG, false>(a, BH, s);
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Args& a, int B, int H, int d, bool causal, hipStream_t stream) {
  const int BH = B * H;
  switch (d) {
    // One barrier per four tiles where two waves share a SIMD (d = 64, 128);
    // d = 256 has one wave per SIMD and measured 3 % faster with a barrier
    // per tile than with one per pair.
    case 64: return launch_d<64, 4, 2, 8>(a, BH, causal, stream);
    case 128: return launch_d<128, 8, 2, 8>(a, BH, causal, stream);
    case 256: return launch_d<256, 4, 1, 3>(a, BH, causal, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
