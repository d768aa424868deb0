// Instruction-rate probe for gfx950 -- a measurement aid, built as its own
// program (isa_probe), not part of the attention library.
//
// Each kernel runs a fixed loop of register-only work (or LDS reads of a
// 64 KiB block it filled itself) and every wave records the shader-cycle
// counter around the loop.  Cycles per loop trip, taken as the median over
// waves, give the issue cost of the instructions the attention kernels are
// built from, independently of the clock (which on this device depends on
// power, hence on the data and the mix):
//   * vector instructions of the softmax (exp2, fma, add/mul, the e4m3 and
//     bf16 pair conversions) with one and two waves per SIMD;
//   * the bf16 and fp8 matrix instructions, alone, as one dependent chain
//     and as independent accumulators;
//   * one 64-key tile's matrix and softmax work per wave, mixed, for the bf16
//     and the fp8 forward;
//   * LDS read bandwidth of the 16-byte row reads and the transposing 8-byte
//     reads, with the bf16 forward's own swizzled address patterns.
// Every loop has a fixed trip count and every access stays inside the
// kernel's own buffers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <vector>

namespace {

#define LDS_AS __attribute__((address_space(3)))
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((vector_size(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

enum Mode {
  kExp,        // 32 v_exp_f32
  kFma,        // 32 v_fma_f32
  kAddMul,     // 32 v_add_f32 + 32 v_mul_f32
  kPackE4m3,   // 16 v_cvt_pk_fp8_f32
  kPackBf16,   // 16 bf16 pair conversions (+ 16 xor, 16 add to keep them live)
  kFp8Mma,     // 8 fp8 32x32x64 products into 4 accumulators
  kFp8Chain,   // 8 fp8 32x32x64 products into 1 accumulator
  kBf16Mma,    // 32 bf16 32x32x16 products into 4 accumulators
  kBf16Chain,  // 32 bf16 32x32x16 products into 1 accumulator
  kFp8Tile,    // 8 fp8 products + 32 fma, 32 exp2, 32 add, 16 e4m3 packs
  kBf16Tile,   // 32 bf16 products + 32 fma, 32 exp2, 32 add, 16 bf16 packs
};

template <int MODE>
__global__ void __launch_bounds__(512) alu_kernel(float* out, long long* cyc, int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  float f[32];
  for (int i = 0; i < 32; ++i) f[i] = -1.0f - 0.001f * (i + lane);
  int w[16];
  for (int i = 0; i < 16; ++i) w[i] = lane + i;
  i32x8 a8, b8;
  bf16x8 ab, bb;
  for (int i = 0; i < 8; ++i) {
    a8[i] = 0x38383838 + lane + i;
    b8[i] = 0x30303030 + lane * 3 + i;
    ab[i] = (__bf16)(0.001f * (lane + i));
    bb[i] = (__bf16)(0.002f * (lane - i));
  }
  f32x16 acc[4];
  for (int m = 0; m < 4; ++m)
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  const float c1 = 0.5f, c2 = -3.0f;
  const long long t0 = __builtin_readcyclecounter();
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == kExp) {
      for (int i = 0; i < 32; ++i) f[i] = __builtin_amdgcn_exp2f(f[i]);
    } else if constexpr (MODE == kFma) {
      for (int i = 0; i < 32; ++i) f[i] = fmaf(f[i], c1, c2);
    } else if constexpr (MODE == kAddMul) {
      for (int i = 0; i < 32; i += 4) {
        s0 += f[i]; s1 += f[i + 1]; s2 += f[i + 2]; s3 += f[i + 3];
        for (int u = 0; u < 4; ++u) f[i + u] *= c1;
      }
    } else if constexpr (MODE == kPackE4m3) {
      for (int i = 0; i < 16; i += 2) {
        w[i] = __builtin_amdgcn_cvt_pk_fp8_f32(f[2 * i], f[2 * i + 1], w[i], false);
        w[i + 1] = __builtin_amdgcn_cvt_pk_fp8_f32(f[2 * i + 2], f[2 * i + 3], w[i + 1], true);
      }
    } else if constexpr (MODE == kPackBf16) {
      for (int i = 0; i < 16; ++i) {
        w[i] ^= __builtin_bit_cast(int, __builtin_convertvector((f32x2){f[2 * i], f[2 * i + 1]}, bf16x2));
        f[2 * i] += c1;
      }
    } else if constexpr (MODE == kFp8Mma || MODE == kFp8Chain) {
      for (int m = 0; m < 8; ++m) {
        const int slot = MODE == kFp8Mma ? (m & 3) : 0;
        acc[slot] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[slot], 0, 0, 0, 127, 0, 127);
      }
    } else if constexpr (MODE == kBf16Mma || MODE == kBf16Chain) {
      for (int m = 0; m < 32; ++m) {
        const int slot = MODE == kBf16Mma ? (m & 3) : 0;
        acc[slot] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, acc[slot], 0, 0, 0);
      }
    } else if constexpr (MODE == kFp8Tile) {
      for (int m = 0; m < 8; ++m)
        acc[m & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[m & 3], 0, 0, 0, 127, 0, 127);
      for (int i = 0; i < 32; ++i) f[i] = __builtin_amdgcn_exp2f(fmaf(f[i], c1, c2));
      for (int i = 0; i < 32; i += 4) { s0 += f[i]; s1 += f[i + 1]; s2 += f[i + 2]; s3 += f[i + 3]; }
      for (int i = 0; i < 16; i += 2) {
        w[i] = __builtin_amdgcn_cvt_pk_fp8_f32(f[2 * i], f[2 * i + 1], w[i], false);
        w[i + 1] = __builtin_amdgcn_cvt_pk_fp8_f32(f[2 * i + 2], f[2 * i + 3], w[i + 1], true);
      }
    } else if constexpr (MODE == kBf16Tile) {
      for (int m = 0; m < 32; ++m) {
        acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, acc[m & 3], 0, 0, 0);
        f[m] = __builtin_amdgcn_exp2f(fmaf(f[m], c1, c2));
        if (m & 1) {
          w[m >> 1] ^= __builtin_bit_cast(int, __builtin_convertvector((f32x2){f[m - 1], f[m]}, bf16x2));
          s0 += f[m - 1];
          s1 += f[m];
        }
      }
    }
  }
  const long long t1 = __builtin_readcyclecounter();
  float sink = s0 + s1 + s2 + s3;
  for (int i = 0; i < 32; ++i) sink += f[i];
  for (int i = 0; i < 16; ++i) sink += (float)w[i];
  for (int m = 0; m < 4; ++m)
    for (int r = 0; r < 16; ++r) sink += acc[m][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = sink;
  if (lane == 0) cyc[blockIdx.x * nw + wave] = t1 - t0;
}

enum LdsMode { kB128, kTr16, kTr8, kB128Fwd, kTr16Fwd };

// 16 LDS reads per trip per wave into a 64 KiB block; each read's data is
// folded into one register by one or two xors, so that the vector work per
// read stays far below the read's own cost.
template <int MODE>
__global__ void __launch_bounds__(1024) lds_kernel(unsigned* out, long long* cyc, int iters) {
  __shared__ __attribute__((aligned(16))) unsigned smem[16384];
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) smem[i] = i * 2654435761u;
  __syncthreads();
  LDS_AS unsigned char* l = (LDS_AS unsigned char*)smem;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  unsigned acc = 0;
  const long long t0 = __builtin_readcyclecounter();
  for (int it = 0; it < iters; ++it) {
    asm volatile("" ::: "memory");  // re-read every trip
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if constexpr (MODE == kB128) {  // consecutive 16-byte rows per lane
        const u32x4 v = *(const LDS_AS u32x4*)(l + (((wave * 16 + k) * 1024 + lane * 16) & 65535));
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      } else if constexpr (MODE == kTr16 || MODE == kTr8) {  // consecutive 8-byte units
        LDS_AS unsigned char* p = l + (((wave * 16 + k) * 512 + lane * 8) & 65535);
        u32x2 v;
        if constexpr (MODE == kTr16)
          v = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p));
        else
          v = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)p));
        acc ^= v[0] ^ v[1];
      } else if constexpr (MODE == kB128Fwd) {  // the bf16 forward's K reads (d = 128)
        const int kb = k >> 3, dc = k & 7;
        const int f = 4 * (l32 & 3) + ((l32 >> 2) & 3);
        const int off = kb * 32 * 256 + l32 * 256 + 16 * ((2 * dc + hl) ^ f);
        const u32x4 v = *(const LDS_AS u32x4*)(l + off);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      } else {  // the bf16 forward's transposed V reads (d = 128)
        const int e = (lane & 15) >> 2, c4 = lane & 3, g2 = (lane >> 4) & 1;
        const int hi = k & 1, db = (k >> 1) & 3, cc = k >> 3;
        const int r = 4 * hl + e + 8 * hi;
        const int f = 4 * (r & 3) + ((r >> 2) & 3);
        const int off = cc * 16 * 256 + r * 256 + 16 * ((4 * db + 2 * g2 + (c4 >> 1)) ^ f) + 8 * (c4 & 1);
        const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(l + off)));
        acc ^= v[0] ^ v[1];
      }
    }
  }
  const long long t1 = __builtin_readcyclecounter();
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
  if (lane == 0) cyc[blockIdx.x * nw + wave] = t1 - t0;
}

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return false;                                                               \
    }                                                                             \
  } while (0)

constexpr int kGrid = 256;  // one workgroup per compute unit
constexpr int kIters = 2000;

// Median over all waves of the cycles per trip.
bool median_cycles(const long long* dcyc, int nwaves, double* med) {
  std::vector<long long> h(nwaves);
  CHECK(hipMemcpy(h.data(), dcyc, h.size() * sizeof(long long), hipMemcpyDeviceToHost));
  std::sort(h.begin(), h.end());
  *med = (double)h[h.size() / 2] / kIters;
  return true;
}

template <int MODE>
bool run_alu(const char* what, double per, float* out, long long* cyc) {
  double c[2];
  for (int i = 0; i < 2; ++i) {
    const int nw = 4 * (i + 1);  // one, then two waves per SIMD
    hipLaunchKernelGGL(alu_kernel<MODE>, dim3(kGrid), dim3(64 * nw), 0, 0, out, cyc, kIters);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    if (!median_cycles(cyc, kGrid * nw, &c[i])) return false;
  }
  // With two waves per SIMD both run the same trips side by side: the SIMD
  // spends c[1] cycles on two trips.
  std::printf("| %-44s | %8.1f | %8.1f | %8.2f |\n", what, c[0], c[1] / 2, c[1] / 2 / per);
  std::fflush(stdout);
  return true;
}

template <int MODE>
bool run_lds(const char* what, int bytes, unsigned* out, long long* cyc) {
  double bw[2];
  for (int i = 0; i < 2; ++i) {
    const int nw = 8 * (i + 1);
    hipLaunchKernelGGL(lds_kernel<MODE>, dim3(kGrid), dim3(64 * nw), 0, 0, out, cyc, kIters);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    double c;
    if (!median_cycles(cyc, kGrid * nw, &c)) return false;
    bw[i] = (double)nw * 16 * bytes / c;  // bytes per cycle per compute unit
  }
  std::printf("| %-44s | %8.0f | %8.0f |\n", what, bw[0], bw[1]);
  std::fflush(stdout);
  return true;
}

bool run_all() {
  float* out = nullptr;
  long long* cyc = nullptr;
  unsigned* uout = nullptr;
  CHECK(hipMalloc(&out, kGrid * 1024 * sizeof(float)));
  CHECK(hipMalloc(&uout, kGrid * 1024 * sizeof(unsigned)));
  CHECK(hipMalloc(&cyc, kGrid * 16 * sizeof(long long)));
  std::printf("Cycles per loop trip per wave (median over waves); last column: SIMD cycles\n"
              "per instruction with two waves per SIMD.\n\n");
  std::printf("| %-44s | %8s | %8s | %8s |\n", "loop body", "1 wave", "2 waves", "per inst");
  std::printf("|---|---|---|---|\n");
  bool ok = run_alu<kExp>("32 v_exp_f32", 32, out, cyc) &&
            run_alu<kFma>("32 v_fma_f32", 32, out, cyc) &&
            run_alu<kAddMul>("32 v_add_f32 + 32 v_mul_f32", 64, out, cyc) &&
            run_alu<kPackE4m3>("16 v_cvt_pk_fp8_f32", 16, out, cyc) &&
            run_alu<kPackBf16>("16 bf16 pair packs (+ 32 xor/add)", 16, out, cyc) &&
            run_alu<kFp8Mma>("8 fp8 32x32x64 products, 4 accumulators", 8, out, cyc) &&
            run_alu<kFp8Chain>("8 fp8 32x32x64 products, 1 accumulator", 8, out, cyc) &&
            run_alu<kBf16Mma>("32 bf16 32x32x16 products, 4 accumulators", 32, out, cyc) &&
            run_alu<kBf16Chain>("32 bf16 32x32x16 products, 1 accumulator", 32, out, cyc) &&
            run_alu<kFp8Tile>("fp8 tile: 8 products + softmax of 32 scores", 8, out, cyc) &&
            run_alu<kBf16Tile>("bf16 tile: 32 products + softmax of 32 scores", 32, out, cyc);
  if (ok) {
    std::printf("\nLDS reads: bytes per cycle per compute unit\n\n");
    std::printf("| %-44s | %8s | %8s |\n", "read", "8 waves", "16 waves");
    std::printf("|---|---|---|\n");
    ok = run_lds<kB128>("ds_read_b128, consecutive", 1024, uout, cyc) &&
         run_lds<kTr16>("ds_read_b64_tr_b16, consecutive", 512, uout, cyc) &&
         run_lds<kTr8>("ds_read_b64_tr_b8, consecutive", 512, uout, cyc) &&
         run_lds<kB128Fwd>("ds_read_b128, bf16 forward K pattern", 1024, uout, cyc) &&
         run_lds<kTr16Fwd>("ds_read_b64_tr_b16, bf16 forward V pattern", 512, uout, cyc);
  }
  CHECK(hipFree(out));
  CHECK(hipFree(uout));
  CHECK(hipFree(cyc));
  return ok;
}

}  // namespace

int main() {
  const bool ok = run_all();
  std::printf(ok ? "done\n" : "failed\n");
  return ok ? 0 : 1;
}
