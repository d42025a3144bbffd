// C ABI of the osattn library: argument validation and dispatch to the kernels.
// See include/osattn.h for the contract.  Nothing here allocates, synchronises
// or keeps state; every check happens before the first launch.
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/osattn.h"
#include "launch.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int validate_sizes(int B, int H, int Hkv, int N, int d, int dtype) {
  if (B < 1 || H < 1 || Hkv < 1 || N < 1) return ATTN_ERR_SHAPE;
  // Row indices (b * H + h) * N + i must fit comfortably in 32-bit arithmetic.
  if ((long long)B * H * N >= (1LL << 31) || (long long)B * Hkv * N >= (1LL << 31))
    return ATTN_ERR_SHAPE;
  // One head's rows are addressed with 32-bit byte offsets.
  if ((long long)N * d * 4 >= (1LL << 31)) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (H % Hkv != 0) return ATTN_ERR_GQA;
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  return ATTN_OK;
}

int validate_scale(float scale) {
  if (!isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_SCALE;
  return ATTN_OK;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int Hkv, int N, int d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  int st = validate_sizes(B, H, Hkv, N, d, dtype);
  if (st != ATTN_OK) return st;
  st = validate_scale(scale);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_ALIGN;
  osattn::FwdArgs a{q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, dtype, stream};
  const hipError_t e = dtype == ATTN_F32 ? osattn::launch_fwd_f32(a) : osattn::launch_fwd_mfma(a);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_bwd_workspace_bytes(int B, int H, int Hkv, int N, int d, int dtype) {
  if (validate_sizes(B, H, Hkv, N, d, dtype) != ATTN_OK) return 0;
  // D and LSE * log2(e), one float32 per query row each.
  return 2 * round256((size_t)B * H * N * sizeof(float));
}

namespace {

bool aligned_all(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned16(p)) return false;
  return true;
}

// Checks shared by every backward entry point (pointers are checked by the caller).
int validate_bwd(int B, int H, int Hkv, int N, int d, float scale, int causal, int dtype,
                 const void* workspace, size_t workspace_bytes) {
  int st = validate_sizes(B, H, Hkv, N, d, dtype);
  if (st != ATTN_OK) return st;
  st = validate_scale(scale);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_SHAPE;
  if (!workspace || workspace_bytes < attn_bwd_workspace_bytes(B, H, Hkv, N, d, dtype))
    return ATTN_ERR_WORKSPACE;
  return ATTN_OK;
}

osattn::BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dO, void* dq, void* dk, void* dv, int B,
                         int H, int Hkv, int N, int d, float scale, int causal, int dtype,
                         const void* workspace, void* stream, int stages) {
  float* dvec = (float*)workspace;
  float* lse2 = (float*)((char*)workspace + round256((size_t)B * H * N * sizeof(float)));
  return osattn::BwdArgs{q,   k,   v, o, lse,   dO,     dq,    dk,     dv,     dvec, lse2, B,
                         H, Hkv, N, d, scale, causal, dtype, stream, stages};
}

int run_bwd_kernels(const osattn::BwdArgs& a) {
  const hipError_t e = a.dtype == ATTN_F32 ? osattn::launch_bwd_f32(a) : osattn::launch_bwd_mfma(a);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
             float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
             void* stream) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return ATTN_ERR_NULL;
  const int st = validate_bwd(B, H, Hkv, N, d, scale, causal, dtype, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  if (!aligned_all({q, k, v, o, lse, dO, dq, dk, dv, workspace})) return ATTN_ERR_ALIGN;
  const osattn::BwdArgs a = bwd_args(q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, N, d, scale,
                                     causal, dtype, workspace, stream,
                                     osattn::kStageDkdv | osattn::kStageDq);
  if (osattn::launch_bwd_preprocess(a) != hipSuccess) return ATTN_ERR_LAUNCH;
  return run_bwd_kernels(a);
}

int attn_bwd_preprocess(const void* o, const float* lse, const void* dO, int B, int H, int Hkv,
                        int N, int d, int dtype, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!o || !lse || !dO) return ATTN_ERR_NULL;
  const int st = validate_bwd(B, H, Hkv, N, d, 1.f, 0, dtype, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  if (!aligned_all({o, lse, dO, workspace})) return ATTN_ERR_ALIGN;
  const osattn::BwdArgs a = bwd_args(nullptr, nullptr, nullptr, o, lse, dO, nullptr, nullptr,
                                     nullptr, B, H, Hkv, N, d, 1.f, 0, dtype, workspace, stream, 0);
  return osattn::launch_bwd_preprocess(a) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                  void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale,
                  int causal, int dtype, const void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (!q || !k || !v || !lse || !dO || !dk || !dv) return ATTN_ERR_NULL;
  const int st = validate_bwd(B, H, Hkv, N, d, scale, causal, dtype, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  if (!aligned_all({q, k, v, lse, dO, dk, dv, workspace})) return ATTN_ERR_ALIGN;
  return run_bwd_kernels(bwd_args(q, k, v, nullptr, lse, dO, nullptr, dk, dv, B, H, Hkv, N, d,
                                  scale, causal, dtype, workspace, stream, osattn::kStageDkdv));
}

int attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                void* dq, int B, int H, int Hkv, int N, int d, float scale, int causal, int dtype,
                const void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !lse || !dO || !dq) return ATTN_ERR_NULL;
  const int st = validate_bwd(B, H, Hkv, N, d, scale, causal, dtype, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  if (!aligned_all({q, k, v, lse, dO, dq, workspace})) return ATTN_ERR_ALIGN;
  return run_bwd_kernels(bwd_args(q, k, v, nullptr, lse, dO, dq, nullptr, nullptr, B, H, Hkv, N,
                                  d, scale, causal, dtype, workspace, stream, osattn::kStageDq));
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer argument";
    case ATTN_ERR_SHAPE: return "invalid shape (B, H, Hkv, N must be >= 1 and fit 32-bit row indices; causal must be 0 or 1)";
    case ATTN_ERR_HEAD_DIM: return "unsupported head dimension (d must be 64 or 128)";
    case ATTN_ERR_GQA: return "H is not a multiple of Hkv";
    case ATTN_ERR_DTYPE: return "unsupported dtype";
    case ATTN_ERR_SCALE: return "scale must be finite and > 0";
    case ATTN_ERR_ALIGN: return "tensor base address not 16-byte aligned";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
