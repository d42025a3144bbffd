// C ABI of the osattn library: argument validation and dispatch to the kernels.
// See include/osattn.h for the contract.  Nothing here allocates, synchronises
// or keeps state; every check happens before the first launch.
#include <math.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

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

namespace {

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Sizes of the interval-masked calls: the attn_fwd limits for Nq and for Nk.
int validate_masked_sizes(int B, int H, int Hkv, int Nq, int Nk, int d, int dtype) {
  int st = validate_sizes(B, H, Hkv, Nq, d, dtype);
  if (st != ATTN_OK) return st;
  return validate_sizes(B, H, Hkv, Nk, d, dtype);
}

}  // namespace

int attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                    int Hkv, int Nq, int Nk, int d, float scale, const int* kv_lo,
                    const int* kv_hi, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !kv_lo || !kv_hi) return ATTN_ERR_NULL;
  int st = validate_masked_sizes(B, H, Hkv, Nq, Nk, d, dtype);
  if (st != ATTN_OK) return st;
  st = validate_scale(scale);
  if (st != ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned4(kv_lo) || !aligned4(kv_hi))
    return ATTN_ERR_ALIGN;
  osattn::FwdArgs a{q, k, v, o, lse, B, H, Hkv, Nq, d, scale, 0, dtype, stream, Nk, kv_lo, kv_hi};
  const hipError_t e = dtype == ATTN_F32 ? osattn::launch_fwd_f32(a) : osattn::launch_fwd_mfma(a);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_bwd_workspace_bytes(int B, int H, int Hkv, int N, int d, int dtype) {
  if (validate_sizes(B, H, Hkv, N, d, dtype) != ATTN_OK) return 0;
  // D and LSE * log2(e), one float32 per query row each.
  return 2 * round256((size_t)B * H * N * sizeof(float));
}

// Helpers with C++ types (inside the extern "C" block, they need C++ linkage).
extern "C++" {
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
}  // extern "C++"

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

// ---- allocation-free backward ---------------------------------------------------
// The workspace of attn_bwd_noalloc lives in this fixed device array; every GPU that
// loads the library holds its own copy until the process ends.  Host code never
// passes the array's name to a kernel or a copy (on the host it is only a stand-in
// for the symbol): it uses the device address looked up per device below.
extern "C++" {
namespace {

static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first call
// made with that device current and kept for the process's lifetime.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_ERR_LAUNCH;
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return ATTN_OK;
}

}  // namespace
}  // extern "C++"

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dO, void* dq, void* dk, void* dv, int B,
                     int H, int Hkv, int N, int d, float scale, int causal, int dtype,
                     void* stream) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return ATTN_ERR_NULL;
  int st = validate_sizes(B, H, Hkv, N, d, dtype);
  if (st != ATTN_OK) return st;
  st = validate_scale(scale);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_SHAPE;
  if (attn_bwd_workspace_bytes(B, H, Hkv, N, d, dtype) > ATTN_NOALLOC_SCRATCH_BYTES)
    return ATTN_ERR_SCRATCH;
  if (!aligned_all({q, k, v, o, lse, dO, dq, dk, dv})) return ATTN_ERR_ALIGN;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != ATTN_OK) return st;
  return attn_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, N, d, scale, causal, dtype, ws,
                  ATTN_NOALLOC_SCRATCH_BYTES, stream);
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

namespace {

struct SplitPlan {
  int n_splits;    // non-empty chunks
  int split_keys;  // keys per chunk (multiple of 32)
};

// Workgroups of the split-KV chunk kernel that fit on the current device at once:
// CUs times how many workgroups one CU's 160 KB of LDS (gfx950) holds, capped.  The
// runtime's shared-memory attribute reports the per-workgroup limit, not the CU's
// capacity, so only the CU count is asked for (256 if the runtime cannot say).
long long split_slots(int d) {
  constexpr int kLdsPerCu = 160 * 1024;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  // At most four per CU: a grid that needs every last LDS slot (five 32 KB
  // workgroups per CU at d = 64) is not packed perfectly by the dispatcher, and the
  // stragglers form a second round (measured: 10 chunks 45% slower than 8 there).
  int per_cu = kLdsPerCu / osattn::splitkv_lds_bytes(d);
  per_cu = per_cu > 4 ? 4 : (per_cu < 1 ? 1 : per_cu);
  return (long long)cus * per_cu;
}

// Chunking of the key axis.  Requested n_splits >= 1 is honoured up to one chunk
// per 32-key tile.  n_splits = 0 picks enough chunks for one full round of
// resident workgroups (the measured best: fewer leaves CUs idle, more adds a
// second partial round), keeping at least four tiles per chunk.
SplitPlan split_plan(int B, int Hkv, int n_rep, int Nq, int Nk, int d, int n_splits) {
  const long long tiles = (Nk + 31) / 32;
  const int rows = n_rep * Nq;
  const int nw = osattn::splitkv_waves(rows);
  const long long rowblocks = (rows + 32LL * nw - 1) / (32LL * nw);
  long long want = n_splits;
  if (want <= 0) {
    const long long base = (long long)B * Hkv * rowblocks;
    const long long slots = split_slots(d);
    want = (slots + base - 1) / base;
    want = want > tiles / 4 ? tiles / 4 : want;
  }
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const long long per_tiles = (tiles + want - 1) / want;
  SplitPlan p;
  p.split_keys = (int)(per_tiles * 32);
  p.n_splits = (int)((Nk + p.split_keys - 1) / p.split_keys);
  return p;
}

int validate_split(int B, int H, int Hkv, int Nq, int Nk, int d, int causal, int dtype,
                   int n_splits) {
  if (B < 1 || H < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || n_splits < 0) return ATTN_ERR_SHAPE;
  if (causal != 0 && causal != 1) return ATTN_ERR_SHAPE;
  if (causal && Nk < Nq) return ATTN_ERR_SHAPE;  // every query must see key 0
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (H % Hkv != 0) return ATTN_ERR_GQA;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  // 32-bit row indices and byte offsets inside one head / one query group.
  if ((long long)B * H * Nq >= (1LL << 31) || (long long)B * Hkv * Nk >= (1LL << 31))
    return ATTN_ERR_SHAPE;
  if ((long long)Nk * d * 4 >= (1LL << 31) || (long long)(H / Hkv) * Nq * d * 4 >= (1LL << 31))
    return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// Both launches count their work-items in 32 bits: the chunk kernel runs
// B * Hkv * n_splits row blocks of up to four waves, the merge one wave per row.
bool split_grid_fits(int B, int H, int Hkv, int Nq, const SplitPlan& p) {
  const int rows = (H / Hkv) * Nq;
  const int nw = osattn::splitkv_waves(rows);
  const long long n_rb = (rows + 32LL * nw - 1) / (32LL * nw);
  return (long long)B * Hkv * p.n_splits * n_rb * nw * 64 < (1LL << 32) &&
         (long long)B * H * Nq * 64 < (1LL << 32);
}

size_t split_workspace(int B, int H, int Nq, int d, const SplitPlan& p) {
  const size_t rows = (size_t)B * H * Nq;
  return round256((size_t)p.n_splits * rows * d * sizeof(float)) +
         round256((size_t)p.n_splits * rows * sizeof(float));
}

}  // namespace

size_t attn_fwd_splitkv_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d,
                                        int causal, int dtype, int n_splits) {
  if (validate_split(B, H, Hkv, Nq, Nk, d, causal, dtype, n_splits) != ATTN_OK) return 0;
  const SplitPlan p = split_plan(B, Hkv, H / Hkv, Nq, Nk, d, n_splits);
  if (!split_grid_fits(B, H, Hkv, Nq, p)) return 0;
  return split_workspace(B, H, Nq, d, p);
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype,
                     int n_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  int st = validate_split(B, H, Hkv, Nq, Nk, d, causal, dtype, n_splits);
  if (st != ATTN_OK) return st;
  st = validate_scale(scale);
  if (st != ATTN_OK) return st;
  const SplitPlan p = split_plan(B, Hkv, H / Hkv, Nq, Nk, d, n_splits);
  if (!split_grid_fits(B, H, Hkv, Nq, p)) return ATTN_ERR_SHAPE;
  if (!workspace || workspace_bytes < split_workspace(B, H, Nq, d, p)) return ATTN_ERR_WORKSPACE;
  if (!aligned_all({q, k, v, o, lse, workspace})) return ATTN_ERR_ALIGN;
  const size_t rows = (size_t)B * H * Nq;
  float* o_part = (float*)workspace;
  float* lse_part = (float*)((char*)workspace + round256((size_t)p.n_splits * rows * d * sizeof(float)));
  osattn::SplitArgs a{q,  k, v,  o,     lse,    o_part, lse_part,   B,          H,
                      Hkv, Nq, Nk, d, scale, causal, dtype, p.n_splits, p.split_keys, stream};
  return osattn::launch_splitkv(a) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t attn_bwd_masked_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d, int dtype) {
  if (validate_masked_sizes(B, H, Hkv, Nq, Nk, d, dtype) != ATTN_OK) return 0;
  // D and LSE * log2(e) per query row, then 4 int32 per (batch, 64-row query tile).
  const size_t rows = round256((size_t)B * H * Nq * sizeof(float));
  const size_t tiles = round256((size_t)B * ((Nq + 63) / 64) * 4 * sizeof(int));
  return 2 * rows + tiles;
}

int attn_bwd_masked(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dO, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq,
                    int Nk, int d, float scale, const int* kv_lo, const int* kv_hi, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !kv_lo || !kv_hi)
    return ATTN_ERR_NULL;
  int st = validate_masked_sizes(B, H, Hkv, Nq, Nk, d, dtype);
  if (st != ATTN_OK) return st;
  st = validate_scale(scale);
  if (st != ATTN_OK) return st;
  if (!workspace ||
      workspace_bytes < attn_bwd_masked_workspace_bytes(B, H, Hkv, Nq, Nk, d, dtype))
    return ATTN_ERR_WORKSPACE;
  if (!aligned_all({q, k, v, o, lse, dO, dq, dk, dv, workspace}) || !aligned4(kv_lo) ||
      !aligned4(kv_hi))
    return ATTN_ERR_ALIGN;
  const size_t rows = round256((size_t)B * H * Nq * sizeof(float));
  osattn::BwdArgs a{q,      k,         v,      o,  lse,
                    dO,     dq,        dk,     dv, (float*)workspace,
                    (float*)((char*)workspace + rows),
                    B,      H,         Hkv,    Nq, d,
                    scale,  0,         dtype,  stream,
                    osattn::kStageDkdv | osattn::kStageDq,
                    Nk,     kv_lo,     kv_hi,  (char*)workspace + 2 * rows};
  if (osattn::launch_bwd_preprocess(a) != hipSuccess) return ATTN_ERR_LAUNCH;
  return run_bwd_kernels(a);
}

namespace {

int validate_rows(long long rows, int cols, int dtype) {
  // Element indices inside a row are 32-bit with headroom for a few strides.
  if (rows < 1 || cols < 1 || rows >= (1LL << 31) || cols > (1 << 30)) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  return ATTN_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

}  // namespace

int rowsoftmax_fwd(const void* x, void* y, long long rows, int cols, int log_softmax, int dtype,
                   void* stream) {
  if (!x || !y) return ATTN_ERR_NULL;
  const int st = validate_rows(rows, cols, dtype);
  if (st != ATTN_OK) return st;
  if (log_softmax != 0 && log_softmax != 1) return ATTN_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(y)) return ATTN_ERR_ALIGN;
  osattn::RowArgs a;
  a.x = x;
  a.y = y;
  a.rows = rows;
  a.cols = cols;
  a.log = log_softmax;
  a.dtype = dtype;
  a.stream = stream;
  return launched(osattn::launch_rowsoftmax(a, false));
}

int rowsoftmax_bwd(const void* y, const void* dy, void* dx, long long rows, int cols,
                   int log_softmax, int dtype, void* stream) {
  if (!y || !dy || !dx) return ATTN_ERR_NULL;
  const int st = validate_rows(rows, cols, dtype);
  if (st != ATTN_OK) return st;
  if (log_softmax != 0 && log_softmax != 1) return ATTN_ERR_SHAPE;
  if (!aligned16(y) || !aligned16(dy) || !aligned16(dx)) return ATTN_ERR_ALIGN;
  osattn::RowArgs a;
  a.y = (void*)y;
  a.dy = dy;
  a.dx = dx;
  a.rows = rows;
  a.cols = cols;
  a.log = log_softmax;
  a.dtype = dtype;
  a.stream = stream;
  return launched(osattn::launch_rowsoftmax(a, true));
}

int rowxent_fwd(const void* logits, const int* targets, float* loss, float* lse, long long rows,
                int cols, int dtype, void* stream) {
  if (!logits || !targets || !loss || !lse) return ATTN_ERR_NULL;
  const int st = validate_rows(rows, cols, dtype);
  if (st != ATTN_OK) return st;
  if (!aligned16(logits) || !aligned4(targets) || !aligned4(loss) || !aligned4(lse))
    return ATTN_ERR_ALIGN;
  osattn::RowArgs a;
  a.x = logits;
  a.targets = targets;
  a.loss = loss;
  a.lse_out = lse;
  a.rows = rows;
  a.cols = cols;
  a.dtype = dtype;
  a.stream = stream;
  return launched(osattn::launch_rowxent(a, false));
}

int rowxent_bwd(const void* logits, const int* targets, const float* lse, const float* dloss,
                void* dlogits, long long rows, int cols, int dtype, void* stream) {
  if (!logits || !targets || !lse || !dloss || !dlogits) return ATTN_ERR_NULL;
  const int st = validate_rows(rows, cols, dtype);
  if (st != ATTN_OK) return st;
  if (!aligned16(logits) || !aligned16(dlogits) || !aligned4(targets) || !aligned4(lse) ||
      !aligned4(dloss))
    return ATTN_ERR_ALIGN;
  osattn::RowArgs a;
  a.x = logits;
  a.targets = targets;
  a.lse = lse;
  a.dloss = dloss;
  a.dx = dlogits;
  a.rows = rows;
  a.cols = cols;
  a.dtype = dtype;
  a.stream = stream;
  return launched(osattn::launch_rowxent(a, true));
}

size_t attn_fwd_fp8_workspace_bytes(int B, int Hkv, int N, int d) {
  if (B < 1 || Hkv < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  return round256(osattn::fp8_vt_bytes(B, Hkv, N, d));
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int Hkv, int N, int d, float scale, float descale_q, float descale_k,
                 float descale_v, int causal, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return ATTN_ERR_NULL;
  int st = validate_sizes(B, H, Hkv, N, d, ATTN_BF16);  // output dtype
  if (st != ATTN_OK) return st;
  // (d in {64, 128} is checked by validate_sizes.)  V^T holds one head's d dims x N
  // rounded up to 128 keys, with 32-bit offsets.
  if ((long long)d * (N + 127) >= (1LL << 31)) return ATTN_ERR_SHAPE;
  if (causal != 0 && causal != 1) return ATTN_ERR_SHAPE;
  st = validate_scale(scale);
  if (st == ATTN_OK) st = validate_scale(descale_q);
  if (st == ATTN_OK) st = validate_scale(descale_k);
  if (st == ATTN_OK) st = validate_scale(descale_v);
  if (st != ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(workspace))
    return ATTN_ERR_ALIGN;
  if (workspace_bytes < attn_fwd_fp8_workspace_bytes(B, Hkv, N, d)) return ATTN_ERR_WORKSPACE;
  osattn::Fp8Args a{q, k, v, o, lse, B, H, Hkv, N, d, scale, descale_q, descale_k, descale_v,
                    causal, workspace, stream};
  return osattn::launch_fwd_fp8(a) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer argument";
    case ATTN_ERR_SHAPE: return "invalid shape (sizes must be >= 1 and fit 32-bit row indices; flags must be 0 or 1)";
    case ATTN_ERR_HEAD_DIM: return "unsupported head dimension (d must be 64 or 128)";
    case ATTN_ERR_GQA: return "H is not a multiple of Hkv";
    case ATTN_ERR_DTYPE: return "unsupported dtype";
    case ATTN_ERR_SCALE: return "scale must be finite and > 0";
    case ATTN_ERR_ALIGN: return "tensor base address not 16-byte aligned";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_SCRATCH: return "problem too large for the allocation-free backward's fixed scratch (B*H*N > 4194304)";
    default: return "unknown status";
  }
}

}  // extern "C"
