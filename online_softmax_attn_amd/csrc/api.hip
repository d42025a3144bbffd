// C ABI of the osattn library: argument validation and dispatch to the kernels.
// See include/osattn.h for the contract.  Nothing here allocates, synchronises
// or keeps state; every check happens before the first launch.
#include <math.h>
#include <stdint.h>

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

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
             float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
             void* stream) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return ATTN_ERR_NULL;
  int st = validate_sizes(B, H, Hkv, N, d, dtype);
  if (st != ATTN_OK) return st;
  st = validate_scale(scale);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_SHAPE;
  if (!workspace || workspace_bytes < attn_bwd_workspace_bytes(B, H, Hkv, N, d, dtype))
    return ATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dO) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(workspace))
    return ATTN_ERR_ALIGN;
  float* dvec = (float*)workspace;
  float* lse2 = (float*)((char*)workspace + round256((size_t)B * H * N * sizeof(float)));
  osattn::BwdArgs a{q, k,   v, o, lse,   dO,     dq,    dk,    dv, dvec, lse2,
                    B, H, Hkv, N, d, scale, causal, dtype, stream};
  hipError_t e = osattn::launch_bwd_preprocess(a);
  if (e == hipSuccess) e = dtype == ATTN_F32 ? osattn::launch_bwd_f32(a) : osattn::launch_bwd_mfma(a);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
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
