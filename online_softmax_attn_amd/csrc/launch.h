// Internal launcher interface between the C ABI (api.cpp) and the kernel files.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#ifndef OSATTN_SPLIT_NBUF
#define OSATTN_SPLIT_NBUF 4  // K/V tiles staged per split-KV workgroup (3 or 4)
#endif

namespace osattn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, N, d;
  float scale;
  int causal;
  int dtype;  // 0 fp32, 1 fp16, 2 bf16
  void* stream;
  // Interval masks (attn_fwd_masked): N is then the query count, Nk the key count,
  // and query row i of batch b sees keys kv_lo[b*N + i] .. kv_hi[b*N + i].
  int Nk = 0;                  // 0: same as N
  const int* kv_lo = nullptr;  // nullptr: no interval mask
  const int* kv_hi = nullptr;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dO;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;  // workspace: D = rowsum(dO * O), [B][H][N] float32
  float* lse2;  // workspace: LSE * log2(e), [B][H][N] float32
  int B, H, Hkv, N, d;
  float scale;
  int causal;
  int dtype;
  void* stream;
  int stages;  // bit set of kStageDkdv and kStageDq: which backward kernels to launch
  // Interval masks (attn_bwd_masked): N is the query count, Nk the key count.
  int Nk = 0;                  // 0: same as N
  const int* kv_lo = nullptr;  // nullptr: no interval mask
  const int* kv_hi = nullptr;
  void* tile_sum = nullptr;    // workspace: per 64-row query tile, 4 int32 (see bwd kernels)
};

struct SplitArgs {
  const void* q;  // [B][H][Nq][d]
  const void* k;  // [B][Hkv][Nk][d]
  const void* v;
  void* o;        // [B][H][Nq][d]
  float* lse;     // [B][H][Nq]
  float* o_part;  // workspace: [n_splits][B*H*Nq][d] chunk outputs
  float* lse_part;  // workspace: [n_splits][B*H*Nq] chunk logsumexps
  int B, H, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  int dtype;       // 1 fp16, 2 bf16
  int n_splits;    // chunks actually launched (each non-empty)
  int split_keys;  // keys per chunk, a multiple of 32
  void* stream;
};

// Compute units of the current device (256 on MI355X if the runtime cannot say).
inline int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return cus;
}

// Workgroups of `kernel` that one CU holds at once (1 if the runtime cannot say).
template <typename K>
inline int resident_per_cu(K kernel, int threads) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  return per_cu;
}

// Workgroups of a persistent grid for `jobs` tiles: one per resident slot of the device,
// or fewer if there are fewer tiles.
inline long long persistent_grid(int per_cu, long long jobs) {
  const long long slots = (long long)device_cus() * per_cu;
  return jobs < slots ? jobs : slots;
}

// Waves per split-KV workgroup (32 query rows each) for a query group of `rows`
// rows: one per 32 rows, up to four.
inline int splitkv_waves(int rows) {
  const int rb32 = (rows + 31) / 32;
  return rb32 >= 4 ? 4 : (rb32 >= 2 ? 2 : 1);
}
// LDS bytes of one split-KV workgroup: staged K and V tiles of 32 rows.
inline int splitkv_lds_bytes(int d) { return OSATTN_SPLIT_NBUF * 2 * 32 * d * 2; }

constexpr int kStageDkdv = 1;
constexpr int kStageDq = 2;

hipError_t launch_fwd_mfma(const FwdArgs& a);

// fp8 (e4m3) forward, d = 64 or 128: codes q [B][H][N][d], k, v [B][Hkv][N][d];
// o bf16, lse fp32; workspace >= fp8_vt_bytes(B, Hkv, N, d) bytes (V transposed).
struct Fp8Args {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, N, d;
  float scale, descale_q, descale_k, descale_v;
  int causal;
  void* workspace;
  void* stream;
};
size_t fp8_vt_bytes(int B, int Hkv, int N, int d);
hipError_t launch_fwd_fp8(const Fp8Args& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_bwd_preprocess(const BwdArgs& a);
hipError_t launch_bwd_mfma(const BwdArgs& a);
hipError_t launch_bwd_f32(const BwdArgs& a);
hipError_t launch_splitkv(const SplitArgs& a);

// Row softmax / log-softmax / cross-entropy (rows of `cols` elements, row-major).
struct RowArgs {
  const void* x = nullptr;    // forward input (softmax) or logits (cross-entropy)
  void* y = nullptr;          // softmax / log-softmax output
  const void* dy = nullptr;   // upstream gradient of y
  void* dx = nullptr;         // gradient of the input
  const int* targets = nullptr;
  float* loss = nullptr;
  float* lse_out = nullptr;   // cross-entropy forward: row logsumexp
  const float* lse = nullptr; // cross-entropy backward: the saved row logsumexp
  const float* dloss = nullptr;
  long long rows = 0;
  int cols = 0;
  int log = 0;                // 1: log-softmax
  int dtype = 0;
  void* stream = nullptr;
};
hipError_t launch_rowsoftmax(const RowArgs& a, bool backward);
hipError_t launch_rowxent(const RowArgs& a, bool backward);

}  // namespace osattn
