// Row softmax, log-softmax and cross-entropy with logits, forward and backward
// (softmax-backward page on shreyansh26.github.io: the row softmax with its shared
// denominator, the backward as the row Jacobian-vector product
// y * (dy - <y, dy>), the log-softmax backward dy - softmax * rowsum(dy), and the
// cross-entropy logits gradient softmax - onehot(target)).
//
// All of these are HBM-bound (a few flops per element), so the design goal is to
// touch every input and output element of HBM exactly once:
//  * register kernels (softmax / log-softmax, both passes): the whole row stays in
//    registers as raw 16-byte chunks between its reductions and its output.  One
//    wave per row for rows of up to 4 chunks per lane, one 256- or 1024-thread
//    workgroup per row above that (up to 16 chunks per thread);
//  * streaming kernels (longer or unaligned rows): each thread keeps an online
//    (max, sum) over its strided elements and the workgroup merges them by rescaling
//    to the common max (the same exact merge as the attention forward); the output
//    pass re-reads the row;
//  * cross-entropy: the forward needs only the row logsumexp and the target logit,
//    one pass; the backward rebuilds softmax from the saved logsumexp, one pass.
// Statistics are fp32; exponentials are exp2 with log2(e) folded in.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace osattn {

namespace {

// ---- element access ------------------------------------------------------------
template <typename E> struct Elem;
template <> struct Elem<float> {
  static constexpr int kV = 4;  // elements per 16-byte chunk
  static __device__ __forceinline__ float get(const u32x4& c, int j) { return __builtin_bit_cast(f32x4, c)[j]; }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
  static __device__ __forceinline__ void store1(float* p, float v) { *p = v; }
  static __device__ __forceinline__ u32x4 pack(const float* v) {
    const f32x4 f = {v[0], v[1], v[2], v[3]};
    return __builtin_bit_cast(u32x4, f);
  }
};
template <typename T16> struct Elem16 {
  static constexpr int kV = 8;
  static __device__ __forceinline__ float get(const u32x4& c, int j) {
    const uint32_t w = c[j >> 1];
    return from_bits<T16>((uint16_t)((j & 1) ? (w >> 16) : (w & 0xffff)));
  }
  static __device__ __forceinline__ float load1(const T16* p) { return (float)*p; }
  static __device__ __forceinline__ void store1(T16* p, float v) { *p = (T16)v; }
  static __device__ __forceinline__ u32x4 pack(const float* v) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      r[k] = (uint32_t)to_bits<T16>(v[2 * k]) | ((uint32_t)to_bits<T16>(v[2 * k + 1]) << 16);
    return r;
  }
};
template <> struct Elem<__bf16> : Elem16<__bf16> {};
template <> struct Elem<_Float16> : Elem16<_Float16> {};

// ---- reductions over the TPR threads of one row ------------------------------------
// TPR = 64: the row is one wave; otherwise the row is TPR / 64 waves of the workgroup
// whose per-wave results meet in LDS (`sh` points at the row's TPR / 64 slots).  The
// barriers are workgroup-wide, so every row of a workgroup must take them together.
template <int TPR>
__device__ __forceinline__ float row_max(float v, float* sh) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if constexpr (TPR > 64) {
    const int wave = (threadIdx.x % TPR) >> 6;
    if ((threadIdx.x & 63) == 0) sh[wave] = v;
    __syncthreads();
    v = sh[0];
#pragma unroll
    for (int w = 1; w < TPR / 64; ++w) v = fmaxf(v, sh[w]);
    __syncthreads();
  }
  return v;
}
template <int TPR>
__device__ __forceinline__ float row_sum(float v, float* sh) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if constexpr (TPR > 64) {
    const int wave = (threadIdx.x % TPR) >> 6;
    if ((threadIdx.x & 63) == 0) sh[wave] = v;
    __syncthreads();
    v = 0.f;
#pragma unroll
    for (int w = 0; w < TPR / 64; ++w) v += sh[w];
    __syncthreads();
  }
  return v;
}
// Exact merge of per-thread online-softmax states (m, s): rescale each s to the
// common max.  A thread that saw no element has m = -inf, s = 0.
template <int TPR>
__device__ __forceinline__ void row_merge(float& m, float& s, float* sh) {
  const float mm = row_max<TPR>(m, sh);
  s = row_sum<TPR>(m == -INFINITY ? 0.f : s * fast_exp2((m - mm) * kLog2e), sh);
  m = mm;
}

// One element into a thread's online (m, s).  An element of -inf (a masked class)
// adds nothing; it must not meet a running max of -inf, where the rescale would be
// exp(-inf + inf).
__device__ __forceinline__ void online_add(float& m, float& s, float v) {
  if (v > m) {
    s = (m == -INFINITY ? 0.f : s * fast_exp2((m - v) * kLog2e)) + 1.f;
    m = v;
  } else if (v != -INFINITY) {
    s += fast_exp2((v - m) * kLog2e);
  }
}

// ---- register kernels: softmax / log-softmax forward -------------------------------
// Block = max(TPR, 256) threads holding 256 / TPR rows (TPR < 256) or one row.
// Row r's chunk c of thread i is elements (c * TPR + i) * V .. + V - 1.  A row past
// the end (last workgroup) has no elements but still takes the barriers.
template <typename E, int TPR, int CPT, bool LOG>
__global__ __launch_bounds__(TPR > 256 ? TPR : 256) void rs_fwd_reg(const E* __restrict__ X,
                                                                    E* __restrict__ Y,
                                                                    long long rows, int cols) {
  using L = Elem<E>;
  constexpr int V = L::kV;
  constexpr int kRowsPerBlock = TPR >= 256 ? 1 : 256 / TPR;
  constexpr int kWaves = (TPR > 256 ? TPR : 256) / 64;
  __shared__ float sh_all[kWaves];
  float* sh = sh_all + (threadIdx.x / TPR) * (TPR / 64);
  const int t = threadIdx.x % TPR;
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / TPR;
  if (TPR == 64 && row >= rows) return;  // one-wave rows take no barrier
  const int cols_r = row < rows ? cols : 0;
  const E* x = X + row * cols;
  E* y = Y + row * cols;
  u32x4 buf[CPT];
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int idx = (c * TPR + t) * V;
    if (idx < cols_r) {
      buf[c] = *(const u32x4*)(x + idx);
#pragma unroll
      for (int j = 0; j < V; ++j) m = fmaxf(m, L::get(buf[c], j));
    }
  }
  m = row_max<TPR>(m, sh);
  const float mb = m * kLog2e;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
    if ((c * TPR + t) * V < cols_r)
#pragma unroll
      for (int j = 0; j < V; ++j) s += fast_exp2(fmaf(L::get(buf[c], j), kLog2e, -mb));
  s = row_sum<TPR>(s, sh);
  const float inv = 1.0f / s;
  const float shift = m + __logf(s);  // log-softmax: x - m - ln s
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int idx = (c * TPR + t) * V;
    if (idx < cols_r) {
      float o[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const float v = L::get(buf[c], j);
        o[j] = LOG ? v - shift : fast_exp2(fmaf(v, kLog2e, -mb)) * inv;
      }
      *(u32x4*)(y + idx) = L::pack(o);
    }
  }
}

// ---- register kernels: backward ---------------------------------------------------
// softmax:     dx = y * (dy - <y, dy>)
// log-softmax: dx = dy - exp(y) * rowsum(dy)      (y is the log-softmax output)
template <typename E, int TPR, int CPT, bool LOG>
__global__ __launch_bounds__(TPR > 256 ? TPR : 256) void rs_bwd_reg(const E* __restrict__ Yv,
                                                                    const E* __restrict__ dY,
                                                                    E* __restrict__ dX,
                                                                    long long rows, int cols) {
  using L = Elem<E>;
  constexpr int V = L::kV;
  constexpr int kRowsPerBlock = TPR >= 256 ? 1 : 256 / TPR;
  constexpr int kWaves = (TPR > 256 ? TPR : 256) / 64;
  __shared__ float sh_all[kWaves];
  float* sh = sh_all + (threadIdx.x / TPR) * (TPR / 64);
  const int t = threadIdx.x % TPR;
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / TPR;
  if (TPR == 64 && row >= rows) return;
  const int cols_r = row < rows ? cols : 0;
  const E* y = Yv + row * cols;
  const E* dy = dY + row * cols;
  E* dx = dX + row * cols;
  u32x4 by[CPT], bg[CPT];
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int idx = (c * TPR + t) * V;
    if (idx < cols_r) {
      by[c] = *(const u32x4*)(y + idx);
      bg[c] = *(const u32x4*)(dy + idx);
#pragma unroll
      for (int j = 0; j < V; ++j)
        acc += LOG ? L::get(bg[c], j) : L::get(by[c], j) * L::get(bg[c], j);
    }
  }
  acc = row_sum<TPR>(acc, sh);
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int idx = (c * TPR + t) * V;
    if (idx < cols_r) {
      float o[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const float yv = L::get(by[c], j), g = L::get(bg[c], j);
        o[j] = LOG ? g - fast_exp2(yv * kLog2e) * acc : yv * (g - acc);
      }
      *(u32x4*)(dx + idx) = L::pack(o);
    }
  }
}

// ---- streaming kernels (any row length and alignment) -----------------------------
// Thread i of the row's workgroup handles elements i, i + T, i + 2T, ... (coalesced).
template <typename E, int T, bool LOG>
__global__ __launch_bounds__(T) void rs_fwd_stream(const E* __restrict__ X, E* __restrict__ Y,
                                                   int cols) {
  using L = Elem<E>;
  __shared__ float sh[T / 64];
  const long long row = blockIdx.x;
  const E* x = X + row * cols;
  E* y = Y + row * cols;
  float m = -INFINITY, s = 0.f;
  for (int j = threadIdx.x; j < cols; j += T) online_add(m, s, L::load1(x + j));
  row_merge<T>(m, s, sh);
  const float mb = m * kLog2e, inv = 1.0f / s, shift = m + __logf(s);
  for (int j = threadIdx.x; j < cols; j += T) {
    const float v = L::load1(x + j);
    L::store1(y + j, LOG ? v - shift : fast_exp2(fmaf(v, kLog2e, -mb)) * inv);
  }
}

template <typename E, int T, bool LOG>
__global__ __launch_bounds__(T) void rs_bwd_stream(const E* __restrict__ Yv,
                                                   const E* __restrict__ dY, E* __restrict__ dX,
                                                   int cols) {
  using L = Elem<E>;
  __shared__ float sh[T / 64];
  const long long row = blockIdx.x;
  const E* y = Yv + row * cols;
  const E* dy = dY + row * cols;
  E* dx = dX + row * cols;
  float acc = 0.f;
  for (int j = threadIdx.x; j < cols; j += T)
    acc += LOG ? L::load1(dy + j) : L::load1(y + j) * L::load1(dy + j);
  acc = row_sum<T>(acc, sh);
  for (int j = threadIdx.x; j < cols; j += T) {
    const float yv = L::load1(y + j), g = L::load1(dy + j);
    L::store1(dx + j, LOG ? g - fast_exp2(yv * kLog2e) * acc : yv * (g - acc));
  }
}

// ---- cross-entropy with logits ------------------------------------------------------
// Forward: loss = lse - x_t (0 for an ignored row, t outside 0 .. cols-1), lse saved.
// VEC: the row is read in 16-byte chunks (row starts 16-byte aligned).
template <typename E, int T, bool VEC>
__global__ __launch_bounds__(T) void xent_fwd_kernel(const E* __restrict__ X,
                                                     const int* __restrict__ tgt,
                                                     float* __restrict__ loss,
                                                     float* __restrict__ lse_out, int cols) {
  using L = Elem<E>;
  constexpr int V = L::kV;
  __shared__ float sh[T / 64];
  const long long row = blockIdx.x;
  const E* x = X + row * cols;
  float m = -INFINITY, s = 0.f;
  if constexpr (VEC) {
    // The chunk's max first, then one rescale per chunk: fewer exponentials per element.
    for (int idx = threadIdx.x * V; idx < cols; idx += T * V) {
      const u32x4 c = *(const u32x4*)(x + idx);
      float cm = L::get(c, 0);
#pragma unroll
      for (int j = 1; j < V; ++j) cm = fmaxf(cm, L::get(c, j));
      const float mn = fmaxf(m, cm);
      if (mn == -INFINITY) continue;  // nothing but masked classes so far
      s = (m == -INFINITY ? 0.f : s * fast_exp2((m - mn) * kLog2e));
      const float mb = mn * kLog2e;
#pragma unroll
      for (int j = 0; j < V; ++j) s += fast_exp2(fmaf(L::get(c, j), kLog2e, -mb));
      m = mn;
    }
  } else {
    for (int j = threadIdx.x; j < cols; j += T) online_add(m, s, L::load1(x + j));
  }
  row_merge<T>(m, s, sh);
  if (threadIdx.x == 0) {
    const float l = m + __logf(s);
    const int t = tgt[row];
    lse_out[row] = l;
    loss[row] = (t >= 0 && t < cols) ? l - L::load1(x + t) : 0.f;
  }
}

// Backward: dx_j = dloss * (exp(x_j - lse) - [j == t]); zero for an ignored row.
// Once the row's lse, target and dloss are known the gradient is elementwise, so for
// rows of whole 16-byte chunks the launch is flat over the chunks of all its rows, one
// chunk per thread in address order (no loop: measured faster than a workgroup
// walking its row); `cpr` is chunks per row.
template <typename E>
__global__ __launch_bounds__(256) void xent_bwd_flat(const E* __restrict__ X,
                                                     const int* __restrict__ tgt,
                                                     const float* __restrict__ lse,
                                                     const float* __restrict__ dloss,
                                                     E* __restrict__ dX, unsigned n_chunks,
                                                     unsigned cpr) {
  using L = Elem<E>;
  constexpr int V = L::kV;
  const unsigned ci = blockIdx.x * 256u + threadIdx.x;
  if (ci >= n_chunks) return;
  const unsigned row = ci / cpr;
  const int j0 = (int)(ci - row * cpr) * V;
  const int cols = (int)cpr * V;
  const int t = tgt[row];
  const bool live = t >= 0 && t < cols;
  const float g = live ? dloss[row] : 0.f;
  const float lb = lse[row] * kLog2e;
  const u32x4 c = ((const u32x4*)X)[ci];
  float o[V];
#pragma unroll
  for (int j = 0; j < V; ++j)
    o[j] = g * (fast_exp2(fmaf(L::get(c, j), kLog2e, -lb)) - (j0 + j == t ? 1.f : 0.f));
  ((u32x4*)dX)[ci] = L::pack(o);
}

// Rows of any length: a workgroup per row, one element per thread and step.
template <typename E, int T>
__global__ __launch_bounds__(T) void xent_bwd_kernel(const E* __restrict__ X,
                                                     const int* __restrict__ tgt,
                                                     const float* __restrict__ lse,
                                                     const float* __restrict__ dloss,
                                                     E* __restrict__ dX, int cols) {
  using L = Elem<E>;
  const long long row = blockIdx.x;
  const E* x = X + row * cols;
  E* dx = dX + row * cols;
  const int t = tgt[row];
  const bool live = t >= 0 && t < cols;
  const float g = live ? dloss[row] : 0.f;
  const float lb = lse[row] * kLog2e;
  for (int j = threadIdx.x; j < cols; j += T)
    L::store1(dx + j, g * (fast_exp2(fmaf(L::load1(x + j), kLog2e, -lb)) - (j == t ? 1.f : 0.f)));
}

// ---- dispatch -----------------------------------------------------------------------
constexpr int kStreamT = 1024;

// A launch's work-item count must fit 32 bits, so rows go out in launches of at
// most 2^20 workgroups; each launch gets its rows' base pointers.
constexpr long long kMaxGrid = 1LL << 20;

// Calls launch(first_row, n_rows, n_blocks) for consecutive row ranges.
template <typename F>
hipError_t for_row_ranges(long long rows, long long rows_per_block, F launch) {
  const long long step = kMaxGrid * rows_per_block;
  for (long long r0 = 0; r0 < rows; r0 += step) {
    const long long n = rows - r0 < step ? rows - r0 : step;
    launch(r0, n, (unsigned)((n + rows_per_block - 1) / rows_per_block));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename E>
bool row_aligned(int cols) {
  return ((long long)cols * sizeof(E)) % 16 == 0;
}

// Register-kernel shape for a row of `chunks` 16-byte chunks: threads per row and
// chunks per thread; false if the row is too long to hold.  Measured on the MI355X
// over rows of 64 .. 8192 chunks: the forward is fastest with two chunks per thread
// (more threads per row and one chunk each, or fewer threads and more chunks, lost
// up to 20%), the backward with one chunk of y and dy per thread, both up to 1024
// threads per row.  The backward holds two rows (y and dy), so it stops at 8 chunks
// per thread: 16 would not fit the 128 registers a lane has at 1024 threads.
bool reg_shape(long long chunks, bool backward, int& tpr, int& cpt) {
  static const int fwd_tpr[] = {64, 64, 128, 256, 512, 1024, 1024, 1024, 1024};
  static const int fwd_cpt[] = {1, 2, 2, 2, 2, 2, 4, 8, 16};
  static const int bwd_tpr[] = {64, 128, 256, 512, 1024, 1024, 1024, 1024};
  static const int bwd_cpt[] = {1, 1, 1, 1, 1, 2, 4, 8};
  const int* tp = backward ? bwd_tpr : fwd_tpr;
  const int* cp = backward ? bwd_cpt : fwd_cpt;
  const int n = backward ? 8 : 9;
  for (int i = 0; i < n; ++i)
    if (chunks <= (long long)tp[i] * cp[i]) {
      tpr = tp[i];
      cpt = cp[i];
      return true;
    }
  return false;
}

template <typename E, int TPR, int CPT, bool LOG>
hipError_t fwd_reg_t(const RowArgs& a) {
  constexpr int kRPB = TPR >= 256 ? 1 : 256 / TPR;
  return for_row_ranges(a.rows, kRPB, [&](long long r0, long long n, unsigned blocks) {
    hipLaunchKernelGGL((rs_fwd_reg<E, TPR, CPT, LOG>), dim3(blocks), dim3(TPR > 256 ? TPR : 256),
                       0, (hipStream_t)a.stream, (const E*)a.x + r0 * a.cols,
                       (E*)a.y + r0 * a.cols, n, a.cols);
  });
}
template <typename E, int TPR, int CPT, bool LOG>
hipError_t bwd_reg_t(const RowArgs& a) {
  constexpr int kRPB = TPR >= 256 ? 1 : 256 / TPR;
  return for_row_ranges(a.rows, kRPB, [&](long long r0, long long n, unsigned blocks) {
    hipLaunchKernelGGL((rs_bwd_reg<E, TPR, CPT, LOG>), dim3(blocks), dim3(TPR > 256 ? TPR : 256),
                       0, (hipStream_t)a.stream, (const E*)a.y + r0 * a.cols,
                       (const E*)a.dy + r0 * a.cols, (E*)a.dx + r0 * a.cols, n, a.cols);
  });
}

template <typename E, bool LOG, bool BWD>
hipError_t softmax_dispatch(const RowArgs& a) {
  const long long chunks = ((long long)a.cols + Elem<E>::kV - 1) / Elem<E>::kV;
  int tpr = 0, cpt = 0;
  if (row_aligned<E>(a.cols) && reg_shape(chunks, BWD, tpr, cpt)) {
#define OSATTN_REG_CASE(TP, CP)                                                           \
  if (tpr == TP && cpt == CP) {                                                           \
    if constexpr (BWD) return bwd_reg_t<E, TP, CP, LOG>(a);                               \
    else return fwd_reg_t<E, TP, CP, LOG>(a);                                             \
  }
    OSATTN_REG_CASE(64, 1)
    OSATTN_REG_CASE(1024, 2)
    OSATTN_REG_CASE(1024, 4)
    OSATTN_REG_CASE(1024, 8)
    if constexpr (BWD) {
      OSATTN_REG_CASE(128, 1)
      OSATTN_REG_CASE(256, 1)
      OSATTN_REG_CASE(512, 1)
      OSATTN_REG_CASE(1024, 1)
    } else {
      OSATTN_REG_CASE(64, 2)
      OSATTN_REG_CASE(128, 2)
      OSATTN_REG_CASE(256, 2)
      OSATTN_REG_CASE(512, 2)
      OSATTN_REG_CASE(1024, 16)
    }
#undef OSATTN_REG_CASE
  }
  return for_row_ranges(a.rows, 1, [&](long long r0, long long, unsigned blocks) {
    const long long off = r0 * a.cols;
    if constexpr (BWD)
      hipLaunchKernelGGL((rs_bwd_stream<E, kStreamT, LOG>), dim3(blocks), dim3(kStreamT), 0,
                         (hipStream_t)a.stream, (const E*)a.y + off, (const E*)a.dy + off,
                         (E*)a.dx + off, a.cols);
    else
      hipLaunchKernelGGL((rs_fwd_stream<E, kStreamT, LOG>), dim3(blocks), dim3(kStreamT), 0,
                         (hipStream_t)a.stream, (const E*)a.x + off, (E*)a.y + off, a.cols);
  });
}

template <typename E, int T, bool VEC>
hipError_t xent_fwd_t(const RowArgs& a) {
  return for_row_ranges(a.rows, 1, [&](long long r0, long long, unsigned blocks) {
    hipLaunchKernelGGL((xent_fwd_kernel<E, T, VEC>), dim3(blocks), dim3(T), 0,
                       (hipStream_t)a.stream, (const E*)a.x + r0 * a.cols, a.targets + r0,
                       a.loss + r0, a.lse_out + r0, a.cols);
  });
}

template <typename E, int T>
hipError_t xent_bwd_rows_t(const RowArgs& a) {
  return for_row_ranges(a.rows, 1, [&](long long r0, long long, unsigned blocks) {
    hipLaunchKernelGGL((xent_bwd_kernel<E, T>), dim3(blocks), dim3(T), 0, (hipStream_t)a.stream,
                       (const E*)a.x + r0 * a.cols, a.targets + r0, a.lse + r0, a.dloss + r0,
                       (E*)a.dx + r0 * a.cols, a.cols);
  });
}

// Flat backward: whole rows per launch, at most 2^28 chunks (2^20 workgroups).
template <typename E>
hipError_t xent_bwd_flat_t(const RowArgs& a) {
  const long long cpr = a.cols / Elem<E>::kV;
  const long long rows_per_launch = ((1LL << 28) / cpr) > 0 ? (1LL << 28) / cpr : 1;
  for (long long r0 = 0; r0 < a.rows; r0 += rows_per_launch) {
    const long long n = a.rows - r0 < rows_per_launch ? a.rows - r0 : rows_per_launch;
    const long long n_chunks = n * cpr;
    hipLaunchKernelGGL((xent_bwd_flat<E>), dim3((unsigned)((n_chunks + 255) / 256)), dim3(256), 0,
                       (hipStream_t)a.stream, (const E*)a.x + r0 * a.cols, a.targets + r0,
                       a.lse + r0, a.dloss + r0, (E*)a.dx + r0 * a.cols, (unsigned)n_chunks,
                       (unsigned)cpr);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename E>
hipError_t xent_dispatch(const RowArgs& a, bool bwd) {
  // Forward: 256 threads per row for short rows, 1024 above 8192 elements.
  const bool vec = row_aligned<E>(a.cols);
  const bool big = a.cols > 8192;
  if (bwd) {
    if (vec) return xent_bwd_flat_t<E>(a);
    return big ? xent_bwd_rows_t<E, 1024>(a) : xent_bwd_rows_t<E, 256>(a);
  }
  if (big) return vec ? xent_fwd_t<E, 1024, true>(a) : xent_fwd_t<E, 1024, false>(a);
  return vec ? xent_fwd_t<E, 256, true>(a) : xent_fwd_t<E, 256, false>(a);
}

}  // namespace

hipError_t launch_rowsoftmax(const RowArgs& a, bool backward) {
  if (a.dtype == 0)
    return a.log ? (backward ? softmax_dispatch<float, true, true>(a) : softmax_dispatch<float, true, false>(a))
                 : (backward ? softmax_dispatch<float, false, true>(a) : softmax_dispatch<float, false, false>(a));
  if (a.dtype == 1)
    return a.log ? (backward ? softmax_dispatch<_Float16, true, true>(a) : softmax_dispatch<_Float16, true, false>(a))
                 : (backward ? softmax_dispatch<_Float16, false, true>(a) : softmax_dispatch<_Float16, false, false>(a));
  return a.log ? (backward ? softmax_dispatch<__bf16, true, true>(a) : softmax_dispatch<__bf16, true, false>(a))
               : (backward ? softmax_dispatch<__bf16, false, true>(a) : softmax_dispatch<__bf16, false, false>(a));
}

hipError_t launch_rowxent(const RowArgs& a, bool backward) {
  if (a.dtype == 0) return xent_dispatch<float>(a, backward);
  if (a.dtype == 1) return xent_dispatch<_Float16>(a, backward);
  return xent_dispatch<__bf16>(a, backward);
}

}  // namespace osattn
