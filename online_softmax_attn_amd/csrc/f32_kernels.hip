// float32 forward and backward kernels (vector FMA, no reduced-precision inputs).
//
// Same method as the MFMA path (FlashAttention-2 page: per query tile, a loop
// over key/value tiles with running max, running denominator and unnormalised
// output; the backward rebuilds P from the saved logsumexp), written for exact
// float32 products: every dot product is a chain of fp32 FMAs.  One wave owns 32
// rows; lane l handles row l % 32 and the column half l / 32 of the head
// dimension, and the two halves of each dot product meet with one lane exchange.
// Tiles of 32 key (or query) rows are staged in LDS and read as broadcasts.
#include "common.h"
#include "launch.h"

namespace osattn {

namespace {

constexpr int kRows = 32;  // rows per workgroup (one wave of 64 lanes)

template <int D>
__device__ __forceinline__ float half_dot(const float* a, const float* lds_row) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < D / 2; ++c) s = fmaf(a[c], lds_row[c], s);
  return s;
}

// Cooperative copy of `rows` rows of D floats (row-major, global) into LDS,
// zero-filling rows at or beyond `limit`.
template <int D>
__device__ __forceinline__ void stage_rows(float* lds, const float* g, int first, int limit) {
  for (int e = threadIdx.x; e < kRows * D; e += 64) {
    const int r = e / D;
    lds[e] = (first + r < limit) ? g[(size_t)(first + r) * D + (e % D)] : 0.f;
  }
}

// Interval mask of one query row (clamped; empty = lo > hi) and, over the 32 rows of a
// wave, the smallest lo and largest hi (both lane halves hold the same rows).
__device__ __forceinline__ void row_interval(const int* kv_lo, const int* kv_hi, int b, int Nq,
                                             int Nk, int row, int& lo, int& hi) {
  lo = Nk;
  hi = -1;
  if (row < Nq) {
    lo = max(kv_lo[(size_t)b * Nq + row], 0);
    hi = min(kv_hi[(size_t)b * Nq + row], Nk - 1);
  }
}
__device__ __forceinline__ void wave_span(int lo, int hi, int& w_lo, int& w_hi) {
  w_lo = lo <= hi ? lo : INT32_MAX;
  w_hi = lo <= hi ? hi : -1;
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    w_lo = min(w_lo, __shfl_xor(w_lo, off));
    w_hi = max(w_hi, __shfl_xor(w_hi, off));
  }
}

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ Q,
                                                     const float* __restrict__ K,
                                                     const float* __restrict__ V,
                                                     float* __restrict__ O,
                                                     float* __restrict__ LSE, int H, int Hkv,
                                                     int Nq, int Nk, float scale,
                                                     const int* __restrict__ kv_lo,
                                                     const int* __restrict__ kv_hi) {
  __shared__ float ks[kRows * D];
  __shared__ float vs[kRows * D];
  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int bh = blockIdx.y;
  const int h = bh % H, b = bh / H;
  const int kvh = h / (H / Hkv);
  const int row = blockIdx.x * kRows + (lane & 31);
  const float* Qp = Q + (size_t)bh * Nq * D;
  const float* Kp = K + (size_t)(b * Hkv + kvh) * Nk * D;
  const float* Vp = V + (size_t)(b * Hkv + kvh) * Nk * D;

  float q[D / 2], o[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) {
    q[c] = row < Nq ? Qp[(size_t)row * D + half * (D / 2) + c] : 0.f;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  int k_begin = 0, k_end = Nk;
  if (CAUSAL) k_end = min(Nk, blockIdx.x * kRows + kRows);
  int lo = 0, hi = Nk - 1;
  if constexpr (MASK) {
    row_interval(kv_lo, kv_hi, b, Nq, Nk, row, lo, hi);
    int w_lo, w_hi;
    wave_span(lo, hi, w_lo, w_hi);
    k_begin = w_hi >= 0 ? (w_lo / kRows) * kRows : 0;
    k_end = w_hi >= 0 ? w_hi + 1 : 0;
  }
  for (int k0 = k_begin; k0 < k_end; k0 += kRows) {
    __syncthreads();
    stage_rows<D>(ks, Kp, k0, Nk);
    stage_rows<D>(vs, Vp, k0, Nk);
    __syncthreads();
    float s[kRows];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      float x = half_dot<D>(q, ks + j * D + half * (D / 2));
      x = (x + __shfl_xor(x, 32)) * scale;
      const int key = k0 + j;
      if (key >= Nk || (CAUSAL && key > row) || (MASK && (key < lo || key > hi))) x = -INFINITY;
      s[j] = x;
      mt = fmaxf(mt, x);
    }
    const float mn = fmaxf(m, mt);
    // A row with every key masked so far keeps m = -inf; its weights stay zero.
    const float alpha = (mn == -INFINITY) ? 1.f : expf(m - mn);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D / 2; ++c) o[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      const float p = (s[j] == -INFINITY) ? 0.f : expf(s[j] - mn);
      l += p;
      const float* vr = vs + j * D + half * (D / 2);
#pragma unroll
      for (int c = 0; c < D / 2; ++c) o[c] = fmaf(p, vr[c], o[c]);
    }
    m = mn;
  }
  if (row < Nq) {
    // A row that sees no key (interval masks only): O = 0, LSE = -inf.
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
#pragma unroll
    for (int c = 0; c < D / 2; ++c) O[((size_t)bh * Nq + row) * D + half * (D / 2) + c] = o[c] * inv;
    if (half == 0) LSE[(size_t)bh * Nq + row] = empty ? -INFINITY : m + logf(l);
  }
}

// dK, dV for 32 key rows of one key/value head, looping over every query row of
// every query head in its group (single writer per key row).
template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    float* __restrict__ dK, float* __restrict__ dV, int H, int Hkv, int Nq, int Nk, float scale,
    const int* __restrict__ kv_lo, const int* __restrict__ kv_hi) {
  __shared__ float qs[kRows * D];
  __shared__ float dos[kRows * D];
  __shared__ float lse_s[kRows];
  __shared__ float d_s[kRows];
  __shared__ int lo_s[kRows], hi_s[kRows];
  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int bg = blockIdx.y;  // b * Hkv + kvh
  const int kvh = bg % Hkv, b = bg / Hkv;
  const int n_rep = H / Hkv;
  const int key0 = blockIdx.x * kRows;
  const int key = key0 + (lane & 31);
  const float* Kp = K + (size_t)bg * Nk * D;
  const float* Vp = V + (size_t)bg * Nk * D;

  float kr[D / 2], vr[D / 2], dk[D / 2], dv[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) {
    kr[c] = key < Nk ? Kp[(size_t)key * D + half * (D / 2) + c] : 0.f;
    vr[c] = key < Nk ? Vp[(size_t)key * D + half * (D / 2) + c] : 0.f;
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  const int first_q = CAUSAL ? blockIdx.x * kRows : 0;
  for (int r = 0; r < n_rep; ++r) {
    const int bh = b * H + kvh * n_rep + r;
    const float* Qp = Q + (size_t)bh * Nq * D;
    const float* dOp = dO + (size_t)bh * Nq * D;
    for (int i0 = first_q; i0 < Nq; i0 += kRows) {
      if constexpr (MASK) {
        // Skip 32-row query tiles none of whose rows sees these 32 keys.
        int lo, hi, w_lo, w_hi;
        row_interval(kv_lo, kv_hi, b, Nq, Nk, i0 + (lane & 31), lo, hi);
        wave_span(lo, hi, w_lo, w_hi);
        if (w_hi < key0 || w_lo > key0 + kRows - 1) continue;
      }
      __syncthreads();
      stage_rows<D>(qs, Qp, i0, Nq);
      stage_rows<D>(dos, dOp, i0, Nq);
      if (lane < kRows) {
        const int i = i0 + lane;
        lse_s[lane] = i < Nq ? LSE[(size_t)bh * Nq + i] : INFINITY;
        d_s[lane] = i < Nq ? Dv[(size_t)bh * Nq + i] : 0.f;
        if constexpr (MASK) row_interval(kv_lo, kv_hi, b, Nq, Nk, i, lo_s[lane], hi_s[lane]);
      }
      __syncthreads();
      for (int ii = 0; ii < kRows; ++ii) {
        const int i = i0 + ii;
        float s = half_dot<D>(kr, qs + ii * D + half * (D / 2));
        s = (s + __shfl_xor(s, 32)) * scale;
        float dp = half_dot<D>(vr, dos + ii * D + half * (D / 2));
        dp = dp + __shfl_xor(dp, 32);
        const bool masked = (i >= Nq) || (CAUSAL && key > i) ||
                            (MASK && (key < lo_s[ii] || key > hi_s[ii]));
        const float p = masked ? 0.f : expf(s - lse_s[ii]);
        const float ds = p * (dp - d_s[ii]);
        const float* qrow = qs + ii * D + half * (D / 2);
        const float* dorow = dos + ii * D + half * (D / 2);
#pragma unroll
        for (int c = 0; c < D / 2; ++c) {
          dv[c] = fmaf(p, dorow[c], dv[c]);
          dk[c] = fmaf(ds, qrow[c], dk[c]);
        }
      }
    }
  }
  if (key < Nk) {
#pragma unroll
    for (int c = 0; c < D / 2; ++c) {
      dK[(size_t)bg * Nk * D + (size_t)key * D + half * (D / 2) + c] = dk[c] * scale;
      dV[(size_t)bg * Nk * D + (size_t)key * D + half * (D / 2) + c] = dv[c];
    }
  }
}

// dQ for 32 query rows, looping over the key/value tiles they see.
template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    float* __restrict__ dQ, int H, int Hkv, int Nq, int Nk, float scale,
    const int* __restrict__ kv_lo, const int* __restrict__ kv_hi) {
  __shared__ float ks[kRows * D];
  __shared__ float vs[kRows * D];
  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int bh = blockIdx.y;
  const int h = bh % H, b = bh / H;
  const int kvh = h / (H / Hkv);
  const int row = blockIdx.x * kRows + (lane & 31);
  const float* Kp = K + (size_t)(b * Hkv + kvh) * Nk * D;
  const float* Vp = V + (size_t)(b * Hkv + kvh) * Nk * D;

  float q[D / 2], dor[D / 2], dq[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) {
    q[c] = row < Nq ? Q[((size_t)bh * Nq + row) * D + half * (D / 2) + c] : 0.f;
    dor[c] = row < Nq ? dO[((size_t)bh * Nq + row) * D + half * (D / 2) + c] : 0.f;
    dq[c] = 0.f;
  }
  const float lse = row < Nq ? LSE[(size_t)bh * Nq + row] : INFINITY;
  const float dd = row < Nq ? Dv[(size_t)bh * Nq + row] : 0.f;
  int k_begin = 0, k_end = Nk;
  if (CAUSAL) k_end = min(Nk, blockIdx.x * kRows + kRows);
  int lo = 0, hi = Nk - 1;
  if constexpr (MASK) {
    row_interval(kv_lo, kv_hi, b, Nq, Nk, row, lo, hi);
    int w_lo, w_hi;
    wave_span(lo, hi, w_lo, w_hi);
    k_begin = w_hi >= 0 ? (w_lo / kRows) * kRows : 0;
    k_end = w_hi >= 0 ? w_hi + 1 : 0;
  }
  for (int k0 = k_begin; k0 < k_end; k0 += kRows) {
    __syncthreads();
    stage_rows<D>(ks, Kp, k0, Nk);
    stage_rows<D>(vs, Vp, k0, Nk);
    __syncthreads();
    for (int j = 0; j < kRows; ++j) {
      const int key = k0 + j;
      float s = half_dot<D>(q, ks + j * D + half * (D / 2));
      s = (s + __shfl_xor(s, 32)) * scale;
      float dp = half_dot<D>(dor, vs + j * D + half * (D / 2));
      dp = dp + __shfl_xor(dp, 32);
      const bool masked = (key >= Nk) || (row >= Nq) || (CAUSAL && key > row) ||
                          (MASK && (key < lo || key > hi));
      const float p = masked ? 0.f : expf(s - lse);
      const float ds = p * (dp - dd);
      const float* krow = ks + j * D + half * (D / 2);
#pragma unroll
      for (int c = 0; c < D / 2; ++c) dq[c] = fmaf(ds, krow[c], dq[c]);
    }
  }
  if (row < Nq) {
#pragma unroll
    for (int c = 0; c < D / 2; ++c) dQ[((size_t)bh * Nq + row) * D + half * (D / 2) + c] = dq[c] * scale;
  }
}

template <int D, bool CAUSAL, bool MASK>
hipError_t fwd_f32_t(const FwdArgs& a) {
  dim3 grid((a.N + kRows - 1) / kRows, a.B * a.H);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, MASK>), grid, dim3(64), 0, (hipStream_t)a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                     a.H, a.Hkv, a.N, a.Nk ? a.Nk : a.N, a.scale, a.kv_lo, a.kv_hi);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool MASK>
hipError_t bwd_f32_t(const BwdArgs& a) {
  const int Nk = a.Nk ? a.Nk : a.N;
  if (a.stages & kStageDkdv) {
    dim3 gk((Nk + kRows - 1) / kRows, a.B * a.Hkv);
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL, MASK>), gk, dim3(64), 0,
                       (hipStream_t)a.stream, (const float*)a.q, (const float*)a.k,
                       (const float*)a.v, (const float*)a.dO, a.lse, a.dvec, (float*)a.dk,
                       (float*)a.dv, a.H, a.Hkv, a.N, Nk, a.scale, a.kv_lo, a.kv_hi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.stages & kStageDq) {
    dim3 gq((a.N + kRows - 1) / kRows, a.B * a.H);
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL, MASK>), gq, dim3(64), 0,
                       (hipStream_t)a.stream, (const float*)a.q, (const float*)a.k,
                       (const float*)a.v, (const float*)a.dO, a.lse, a.dvec, (float*)a.dq, a.H,
                       a.Hkv, a.N, Nk, a.scale, a.kv_lo, a.kv_hi);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) {
  if (a.kv_lo) return a.d == 64 ? fwd_f32_t<64, false, true>(a) : fwd_f32_t<128, false, true>(a);
  if (a.d == 64) return a.causal ? fwd_f32_t<64, true, false>(a) : fwd_f32_t<64, false, false>(a);
  return a.causal ? fwd_f32_t<128, true, false>(a) : fwd_f32_t<128, false, false>(a);
}

hipError_t launch_bwd_f32(const BwdArgs& a) {
  if (a.kv_lo) return a.d == 64 ? bwd_f32_t<64, false, true>(a) : bwd_f32_t<128, false, true>(a);
  if (a.d == 64) return a.causal ? bwd_f32_t<64, true, false>(a) : bwd_f32_t<64, false, false>(a);
  return a.causal ? bwd_f32_t<128, true, false>(a) : bwd_f32_t<128, false, false>(a);
}

}  // namespace osattn
