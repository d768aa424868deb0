// Internal launcher interface between the C ABI (fa_api.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;     // [B][H][N][d]
  const void* k;     // [B][H][Nk][d]
  const void* v;     // [B][H][Nk][d]
  void* o;           // [B][H][N][d] (plain forward)
  float* lse;        // [B][H][N] or null (plain forward)
  int N;             // query rows per head
  int n_qtiles;      // filled in by the launcher
  float scale_log2;  // softmax scale * log2(e)
  int bh;            // B * H (launcher)
  int pin;           // persistent schedule keeps each head on one XCD (launcher)
  // Split-KV (launch_fwd_partial; launch_fwd sets one split over all keys):
  int Nk;            // key rows per head
  int c_off;         // causal: query row i sees key j iff j <= i + c_off
  int k_chunk;       // keys per split
  int n_split;       // splits: split s covers keys [s k_chunk, (s+1) k_chunk)
  float* o32;        // [n_split][B][H][N][d] fp32, O normalised within the split
  float* lse32;      // [n_split][B][H][N], log-sum-exp within the split (-inf if empty)
  // Block-sparse (launch_fwd_sparse):
  int heads;         // H
  int bs_per_batch;  // mask is [B][H][nb][nb] (1) or [H][nb][nb] (0)
  int bs_stride;     // ints per live-tile list (launcher)
};

// Rows and keys per block of the block-sparse mask.
constexpr int kSparseBlock = 128;

// Enqueue the 16-bit forward.  Arguments are validated by the caller.
// per_tile selects, for causal calls, one workgroup per query tile in
// dispatch order instead of the persistent schedule (same outputs bit for
// bit; a comparison aid).
hipError_t launch_fwd(const FwdArgs& a, int B, int H, int d, int dtype, bool causal,
                      hipStream_t stream, bool per_tile = false);

// Enqueue the split-KV partial forward (fp32 partial outputs per split).
hipError_t launch_fwd_partial(const FwdArgs& a, int B, int H, int d, int dtype, bool causal,
                              hipStream_t stream);

// Enqueue the block-sparse forward: builds the live-tile lists in `list`
// (sparse_list_bytes bytes) from the block mask, then the forward over them.
hipError_t launch_fwd_sparse(const FwdArgs& a, int B, int H, int d, int dtype, bool causal,
                             const uint8_t* mask, int* list, hipStream_t stream);
size_t sparse_list_bytes(int n_mask_heads, int N, int d);

struct MergeArgs {
  const float* o_parts;    // [S][rows][d] fp32
  const float* lse_parts;  // [S][rows]
  void* o;                 // [rows][d], 16-bit type
  float* lse;              // [rows] or null
  int64_t rows;            // B * H * N
  int n_parts;             // S
};

// Enqueue the log-sum-exp merge of S partial results.
hipError_t launch_merge(const MergeArgs& a, int d, int dtype, hipStream_t stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* dsum;       // workspace: two planes of B*H*N floats, -LSE/scale then -rowsum(dO o O)
  int64_t plane;     // B*H*N, filled in by the launcher
  float* dq;         // fp32 [B][H][N][d], written once per row by the dQ kernel
  void* dk;
  void* dv;
  int N;
  int n_ktiles;      // filled in by the launcher
  int bh;            // B * H (launcher)
  int pin;           // persistent schedule keeps each head on one XCD (launcher)
  float scale;
  float scale_log2;
  float inv_scale;   // 1 / scale (launcher)
};

struct QuantArgs {
  const void* x;       // [B][H][N][d] bf16 / fp16
  void* x8;            // [B][H][N][d] e4m3 codes
  float* scales;       // [B][H][nblk]
  const float* signs;  // d entries of +-1, or null (no rotation)
  float scale_mul;
  int N;
  int nblk;            // ceil(N / 128)
};

// mode: 0 block scales, 1 one scale per tensor, 2 block scales rounded up
// to a power of two.
hipError_t launch_quant_fp8(const QuantArgs& a, int B, int H, int d, int dtype, int mode,
                            hipStream_t stream);

struct Fp8Args {
  const void* q8;
  const void* k8;
  const void* v8;
  const float* q_scale;  // [B][H][nblk], 1/d already folded in for rotated Q
  const float* k_scale;
  const float* v_scale;
  void* o;               // bf16
  float* lse;
  int N;
  int nblk;
  int n_qtiles;          // filled in by the launcher
  int bh;                // B * H (launcher)
  int pin;               // persistent schedule keeps each head on one XCD (launcher)
  float scale_log2;
};

hipError_t launch_fwd_fp8(const Fp8Args& a, int B, int H, int d, bool causal, hipStream_t stream);

// Head dimensions the backward is built for.
bool bwd_supported(int d);

// Enqueue the backward kernels (dQ with the row statistics, then dK/dV).
// Arguments are validated by the caller.
hipError_t launch_bwd(const BwdArgs& a, int B, int H, int d, int dtype, bool causal,
                      hipStream_t stream);

// Size of the fixed device scratch of the allocation-free backward: the
// backward's per-row workspace for up to kBwdScratchBytes / 8 rows (B*H*N).
constexpr size_t kBwdScratchBytes = size_t(16) << 20;

// launch_bwd with the workspace in the fixed device scratch (a.dsum is
// ignored); the caller checks the size against kBwdScratchBytes.
hipError_t launch_bwd_noalloc(const BwdArgs& a, int B, int H, int d, int dtype, bool causal,
                              hipStream_t stream);

}  // namespace fa
