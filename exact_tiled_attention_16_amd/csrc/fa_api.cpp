// C ABI of libfa.so (declared in include/fa.h): argument validation and
// dispatch to the kernel launchers.  Nothing here allocates, frees or
// synchronises; every check happens before anything is enqueued.
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "kernels.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool valid_dims(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0) return false;
  // Workgroup counts and per-(b,h) row indices are 32-bit inside the kernels.
  const int64_t bh = (int64_t)B * H;
  return bh <= 0x7fffffff && (int64_t)N <= 0x7fffffff / 2;
}

bool supported_d(int d) { return d == 64 || d == 128 || d == 256; }

// Longest sequence and largest position of the split-KV calls (keeps the
// kernels' 32-bit position arithmetic far from overflow).
constexpr int kMaxLen = 1 << 29;

bool valid_scale(float s) { return isfinite(s) && s > 0.f; }

int launch_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID: return "invalid argument (null or misaligned pointer, bad size, dtype or scale)";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration (head dimension must be 64, 128 or 256)";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_TOO_LARGE:
      return "problem too large for the fixed scratch of fa_bwd_noalloc "
             "(B*H*N above FA_BWD_NOALLOC_MAX_ROWS)";
    default: return "unknown status";
  }
}

namespace {

int fwd_entry(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int N, int d, int dtype, float scale, int causal, void* stream, bool per_tile) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_INVALID;
  if (!aligned4(lse)) return FA_ERR_INVALID;
  if (!valid_dims(B, H, N) || (dtype != FA_BF16 && dtype != FA_FP16)) return FA_ERR_INVALID;
  if (!valid_scale(scale) || (causal != 0 && causal != 1)) return FA_ERR_INVALID;
  if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.N = N;
  a.scale_log2 = scale * 1.4426950408889634f;
  return launch_status(fa::launch_fwd(a, B, H, d, dtype, causal != 0,
                                      static_cast<hipStream_t>(stream), per_tile));
}

}  // namespace

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, int dtype, float scale, int causal, void* stream) {
  return fwd_entry(q, k, v, o, lse, B, H, N, d, dtype, scale, causal, stream, false);
}

// Not part of the ABI (no declaration in include/): fa_fwd with the causal
// work dispatched as one workgroup per query tile instead of the persistent
// schedule.  The outputs are bit-identical to fa_fwd's; the parity tests use
// it to check that, and the benchmark to time the two schedules side by side.
int fa_testing_fwd_per_tile(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int N, int d, int dtype, float scale, int causal,
                            void* stream) {
  return fwd_entry(q, k, v, o, lse, B, H, N, d, dtype, scale, causal, stream, true);
}

int fa_fwd_partial(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                   int H, int Nq, int Nk, int d, int dtype, float scale, int causal, int q_pos0,
                   int k_pos0, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID;
  if (!valid_dims(B, H, Nq) || !valid_dims(B, H, Nk)) return FA_ERR_INVALID;
  if (Nq > kMaxLen || Nk > kMaxLen || (dtype != FA_BF16 && dtype != FA_FP16))
    return FA_ERR_INVALID;
  if (q_pos0 < 0 || k_pos0 < 0 || q_pos0 > kMaxLen || k_pos0 > kMaxLen) return FA_ERR_INVALID;
  if (!valid_scale(scale) || (causal != 0 && causal != 1)) return FA_ERR_INVALID;
  if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.N = Nq;
  a.Nk = Nk;
  a.c_off = q_pos0 - k_pos0;
  a.k_chunk = Nk;
  a.n_split = 1;
  a.o32 = o;
  a.lse32 = lse;
  a.scale_log2 = scale * 1.4426950408889634f;
  return launch_status(
      fa::launch_fwd_partial(a, B, H, d, dtype, causal != 0, static_cast<hipStream_t>(stream)));
}

int fa_merge(const float* o_parts, const float* lse_parts, int n_parts, void* o, float* lse,
             int B, int H, int N, int d, int dtype, void* stream) {
  if (!o_parts || !lse_parts || !o) return FA_ERR_INVALID;
  if (!aligned16(o_parts) || !aligned4(lse_parts) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID;
  if (!valid_dims(B, H, N) || n_parts < 1 || (dtype != FA_BF16 && dtype != FA_FP16))
    return FA_ERR_INVALID;
  if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
  fa::MergeArgs a{};
  a.o_parts = o_parts;
  a.lse_parts = lse_parts;
  a.o = o;
  a.lse = lse;
  a.rows = (int64_t)B * H * N;
  a.n_parts = n_parts;
  return launch_status(fa::launch_merge(a, d, dtype, static_cast<hipStream_t>(stream)));
}

size_t fa_splitkv_workspace_size(int B, int H, int Nq, int d, int n_splits) {
  if (B <= 0 || H <= 0 || Nq <= 0 || n_splits <= 0 || !supported_d(d)) return 0;
  const size_t rows = (size_t)B * H * Nq * n_splits;
  return rows * (size_t)(d + 1) * sizeof(float);  // partial O, then partial LSE
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, int B, int H, int Nq, int Nk, int d, int dtype, float scale,
                   int causal, int n_splits, void* stream) {
  if (!q || !k || !v || !o || !workspace) return FA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse) ||
      !aligned16(workspace))
    return FA_ERR_INVALID;
  if (!valid_dims(B, H, Nq) || !valid_dims(B, H, Nk) || n_splits < 1) return FA_ERR_INVALID;
  if (Nq > kMaxLen || Nk > kMaxLen || (dtype != FA_BF16 && dtype != FA_FP16))
    return FA_ERR_INVALID;
  if (!valid_scale(scale) || (causal != 0 && causal != 1)) return FA_ERR_INVALID;
  if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
  // Parts of a whole number of 64-key tiles; the last may be shorter.
  const int per = (Nk + n_splits - 1) / n_splits;
  const int chunk = (per + 63) / 64 * 64;
  const int parts = (Nk + chunk - 1) / chunk;
  const int64_t rows = (int64_t)B * H * Nq;
  float* o32 = static_cast<float*>(workspace);
  float* lse32 = o32 + rows * parts * d;
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.N = Nq;
  a.Nk = Nk;
  a.c_off = Nk - Nq;
  a.k_chunk = chunk;
  a.n_split = parts;
  a.o32 = o32;
  a.lse32 = lse32;
  a.scale_log2 = scale * 1.4426950408889634f;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = fa::launch_fwd_partial(a, B, H, d, dtype, causal != 0, s);
  if (e != hipSuccess) return FA_ERR_LAUNCH;
  fa::MergeArgs m{};
  m.o_parts = o32;
  m.lse_parts = lse32;
  m.o = o;
  m.lse = lse;
  m.rows = rows;
  m.n_parts = parts;
  return launch_status(fa::launch_merge(m, d, dtype, s));
}

size_t fa_blocksparse_workspace_size(int B, int H, int N, int d, int mask_per_batch) {
  if (!valid_dims(B, H, N) || !supported_d(d) || (mask_per_batch != 0 && mask_per_batch != 1))
    return 0;
  return fa::sparse_list_bytes(mask_per_batch ? B * H : H, N, d);
}

int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                       const void* block_mask, int mask_per_batch, void* workspace, int B, int H,
                       int N, int d, int dtype, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !block_mask || !workspace) return FA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse) ||
      !aligned4(workspace))
    return FA_ERR_INVALID;
  if (!valid_dims(B, H, N) || (dtype != FA_BF16 && dtype != FA_FP16)) return FA_ERR_INVALID;
  if (mask_per_batch != 0 && mask_per_batch != 1) return FA_ERR_INVALID;
  if (!valid_scale(scale) || (causal != 0 && causal != 1)) return FA_ERR_INVALID;
  if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.N = N;
  a.bs_per_batch = mask_per_batch;
  a.scale_log2 = scale * 1.4426950408889634f;
  return launch_status(fa::launch_fwd_sparse(a, B, H, d, dtype, causal != 0,
                                             static_cast<const uint8_t*>(block_mask),
                                             static_cast<int*>(workspace),
                                             static_cast<hipStream_t>(stream)));
}

int fa_quant_fp8(const void* x, int dtype, void* x8, float* scales, const float* signs,
                 float scale_mul, int mode, int B, int H, int N, int d, void* stream) {
  if (!x || !x8 || !scales) return FA_ERR_INVALID;
  if (!aligned16(x) || !aligned16(x8) || !aligned4(scales) || !aligned4(signs))
    return FA_ERR_INVALID;
  if (!valid_scale(scale_mul)) return FA_ERR_INVALID;
  if (!valid_dims(B, H, N) || (dtype != FA_BF16 && dtype != FA_FP16)) return FA_ERR_INVALID;
  if (mode != FA_FP8_BLOCK_SCALES && mode != FA_FP8_TENSOR_SCALE && mode != FA_FP8_BLOCK_POW2)
    return FA_ERR_INVALID;
  if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
  fa::QuantArgs a{};
  a.x = x;
  a.x8 = x8;
  a.scales = scales;
  a.signs = signs;
  a.scale_mul = scale_mul;
  a.N = N;
  a.nblk = (N + FA_FP8_BLOCK - 1) / FA_FP8_BLOCK;
  if ((int64_t)B * H * a.nblk > 0x7fffffff) return FA_ERR_INVALID;
  return launch_status(
      fa::launch_quant_fp8(a, B, H, d, dtype, mode, static_cast<hipStream_t>(stream)));
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_scale,
               const float* k_scale, const float* v_scale, void* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, void* stream) {
  if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale || !o) return FA_ERR_INVALID;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o)) return FA_ERR_INVALID;
  if (!aligned4(q_scale) || !aligned4(k_scale) || !aligned4(v_scale) || !aligned4(lse))
    return FA_ERR_INVALID;
  if (!valid_dims(B, H, N) || !valid_scale(scale) || (causal != 0 && causal != 1))
    return FA_ERR_INVALID;
  if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
  fa::Fp8Args a{};
  a.q8 = q8;
  a.k8 = k8;
  a.v8 = v8;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.o = o;
  a.lse = lse;
  a.N = N;
  a.nblk = (N + FA_FP8_BLOCK - 1) / FA_FP8_BLOCK;
  a.scale_log2 = scale * 1.4426950408889634f;
  return launch_status(
      fa::launch_fwd_fp8(a, B, H, d, causal != 0, static_cast<hipStream_t>(stream)));
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  if (!valid_dims(B, H, N) || !supported_d(d) || !fa::bwd_supported(d)) return 0;
  return (size_t)B * H * N * 2 * sizeof(float);  // per row: LSE * log2 e, rowsum(dO o O)
}

namespace {

// Argument checks shared by fa_bwd and fa_bwd_noalloc (everything but the
// workspace pointer).
int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, float* dq, void* dk, void* dv, int B, int H, int N, int d,
              int dtype, float scale, int causal) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned4(lse))
    return FA_ERR_INVALID;
  if (!valid_dims(B, H, N) || (dtype != FA_BF16 && dtype != FA_FP16)) return FA_ERR_INVALID;
  if (!valid_scale(scale) || (causal != 0 && causal != 1)) return FA_ERR_INVALID;
  if (!supported_d(d) || !fa::bwd_supported(d)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

fa::BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, float* dq, void* dk, void* dv,
                     void* workspace, int N, float scale) {
  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dsum = static_cast<float*>(workspace);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.N = N;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  return a;
}

}  // namespace

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, float* dq, void* dk, void* dv, void* workspace, int B, int H,
           int N, int d, int dtype, float scale, int causal, void* stream) {
  if (!workspace || !aligned16(workspace)) return FA_ERR_INVALID;
  const int rc = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, dtype, scale, causal);
  if (rc != FA_OK) return rc;
  const fa::BwdArgs a = bwd_args(q, k, v, o, dout, lse, dq, dk, dv, workspace, N, scale);
  return launch_status(
      fa::launch_bwd(a, B, H, d, dtype, causal != 0, static_cast<hipStream_t>(stream)));
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, float* dq, void* dk, void* dv, int B, int H, int N, int d,
                   int dtype, float scale, int causal, void* stream) {
  const int rc = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, dtype, scale, causal);
  if (rc != FA_OK) return rc;
  static_assert((size_t)FA_BWD_NOALLOC_MAX_ROWS * 2 * sizeof(float) == fa::kBwdScratchBytes,
                "scratch size and the documented row limit agree");
  if ((int64_t)B * H * N > FA_BWD_NOALLOC_MAX_ROWS) return FA_ERR_TOO_LARGE;
  if (fa_bwd_workspace_size(B, H, N, d) > fa::kBwdScratchBytes) return FA_ERR_TOO_LARGE;
  const fa::BwdArgs a = bwd_args(q, k, v, o, dout, lse, dq, dk, dv, nullptr, N, scale);
  return launch_status(
      fa::launch_bwd_noalloc(a, B, H, d, dtype, causal != 0, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
