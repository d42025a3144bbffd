// float32 forward and backward kernels (vector FMA, no reduced-precision inputs).
//
// Same method as the MFMA path (FlashAttention-2 page: per query tile, a loop
// over key/value tiles with running max, running denominator and unnormalised
// output; the backward rebuilds P from the saved logsumexp), written for float32
// inputs and outputs.
//
// Accuracy.  The products of two float32 numbers are exact in float64, so every
// score (and every dP = dO . V) is accumulated in float64 and rounded once: a
// score of magnitude |s| then carries at most half a float32 ulp of |s| into
// exp(s - m), instead of the sqrt(d) ulps a float32 FMA chain would (large scores,
// e.g. |s| ~ 50, otherwise cost ~1e-5 of relative weight error).  The outputs'
// own sums (P V, P^T dO, dS K, dS^T Q) stay float32 FMA chains, blocked per tile.
//
// Parallel layout.  A row of d values is spread over G = d/32 lanes (32 columns
// each), so a wave covers R = 64/G rows (32 at d = 64, 16 at d = 128): lane l holds
// row l % R and columns 32*(l / R) .. +31, and the G parts of a dot product meet
// by lane exchanges.  A workgroup is four waves over the same R rows; the loop over
// the other side (keys for the forward and dQ, query rows for dK/dV) is split over
// the four waves in tiles of 16, each wave staging its own tiles in its own LDS
// slice with 16-byte loads.  At the end the four partial results are merged
// through LDS (the forward exactly, by moving each wave's (m, l, o) to the common
// max) and written with 16-byte stores.
#include "common.h"
#include "launch.h"

namespace osattn {

namespace {

constexpr int kWaves = 4;   // waves per workgroup, splitting the inner loop
constexpr int kTile = 16;   // rows of the other side staged per wave and step
constexpr int kCols = 32;   // head-dimension columns per lane

template <int D>
struct F32Map {
  static constexpr int G = D / kCols;     // lanes per row
  static constexpr int R = 64 / G;        // rows per wave (and per workgroup)
  static constexpr int kSlice = 2 * kTile * D;     // LDS floats per wave (two tiles)
  static constexpr int kFloats = kWaves * kSlice;  // also holds [wave][row][D] partials
  static_assert(kFloats >= kWaves * R * D, "merge space");
  // Writer mapping of the merge: 256 threads cover R rows x D columns, 8 each.
  static constexpr int kThrPerRow = D / 8;
  static_assert(R * kThrPerRow == 64 * kWaves, "merge writers");
};

// Dot product of this lane's 32 columns `a` with a staged row's same columns, in
// float64 (exact products), four independent partial sums.
__device__ __forceinline__ double part_dot64(const float* a, const float* lds_cols) {
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
#pragma unroll
  for (int c = 0; c < kCols; c += 4) {
    const f32x4 b = *(const f32x4*)(lds_cols + c);
    s0 = fma((double)a[c + 0], (double)b[0], s0);
    s1 = fma((double)a[c + 1], (double)b[1], s1);
    s2 = fma((double)a[c + 2], (double)b[2], s2);
    s3 = fma((double)a[c + 3], (double)b[3], s3);
  }
  return (s0 + s1) + (s2 + s3);
}

// Sum of the G lane parts of a row's dot product (lanes l, l ^ R, ...), the same
// value, bit for bit, in every part.
template <int D>
__device__ __forceinline__ double row_sum(double x) {
  using Mp = F32Map<D>;
  if constexpr (Mp::G == 4) x = x + __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// One wave copies kTile rows of D floats (row-major, global) into its LDS slice
// with 16-byte loads; rows at or beyond `limit` read as zero.
template <int D>
__device__ __forceinline__ void stage_tile(float* lds, const float* g, int first, int limit,
                                           int lane) {
  constexpr int kVec = kTile * D / 4;  // float4 per tile
#pragma unroll
  for (int e = lane; e < kVec; e += 64) {
    const int r = (4 * e) / D;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (first + r < limit) x = *(const f32x4*)(g + (size_t)(first + r) * D + (4 * e) % D);
    *(f32x4*)(lds + 4 * e) = x;
  }
}

// Load this lane's 32 columns of a global row (zero if the row does not exist).
__device__ __forceinline__ void load_cols(float* dst, const float* src, bool ok) {
#pragma unroll
  for (int c = 0; c < kCols; c += 4) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (ok) x = *(const f32x4*)(src + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[c + e] = x[e];
  }
}

__device__ __forceinline__ void store_cols(float* lds, const float* src) {
#pragma unroll
  for (int c = 0; c < kCols; c += 4) *(f32x4*)(lds + c) = f32x4{src[c], src[c + 1], src[c + 2], src[c + 3]};
}

// Order this wave's LDS writes before its following reads (and earlier reads
// before later writes): LDS operations of one wave complete in issue order; the
// barrier keeps the compiler from moving accesses across.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Interval mask of one query row (clamped; empty = lo > hi) and, over the R rows,
// the smallest lo and largest hi (all lane parts hold the same rows).
__device__ __forceinline__ void row_interval(const int* kv_lo, const int* kv_hi, int b, int Nq,
                                             int Nk, int row, int& lo, int& hi) {
  lo = Nk;
  hi = -1;
  if (row < Nq) {
    lo = max(kv_lo[(size_t)b * Nq + row], 0);
    hi = min(kv_hi[(size_t)b * Nq + row], Nk - 1);
  }
}
__device__ __forceinline__ void rows_span(int lo, int hi, int& w_lo, int& w_hi) {
  w_lo = lo <= hi ? lo : INT32_MAX;
  w_hi = lo <= hi ? hi : -1;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    w_lo = min(w_lo, __shfl_xor(w_lo, off));
    w_hi = max(w_hi, __shfl_xor(w_hi, off));
  }
}

// Sum of the four waves' partial [row][D] arrays (in wave order) times `mul`, written
// to rows first .. first+R-1 (those < limit) of a [.][D] global array.
template <int D>
__device__ __forceinline__ void write_wave_sum(float* dst, const float* part, int first,
                                               int limit, float mul) {
  using Mp = F32Map<D>;
  const int t = threadIdx.x;
  const int r = t / Mp::kThrPerRow;
  const int c0 = (t % Mp::kThrPerRow) * 8;
  if (first + r >= limit) return;
#pragma unroll
  for (int c = 0; c < 8; c += 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const f32x4 x = *(const f32x4*)(part + (w * Mp::R + r) * D + c0 + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += x[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= mul;
    *(f32x4*)(dst + (size_t)(first + r) * D + c0 + c) = acc;
  }
}

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q,
                                                      const float* __restrict__ K,
                                                      const float* __restrict__ V,
                                                      float* __restrict__ O,
                                                      float* __restrict__ LSE, int H, int Hkv,
                                                      int Nq, int Nk, float scale,
                                                      const int* __restrict__ kv_lo,
                                                      const int* __restrict__ kv_hi) {
  using Mp = F32Map<D>;
  constexpr int R = Mp::R;
  __shared__ __attribute__((aligned(16))) float lds[Mp::kFloats];
  __shared__ double ml[kWaves * R * 2];  // each wave's (m, l) per row, for the merge
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col0 = (lane / R) * kCols;
  const int bh = blockIdx.y;
  const int h = bh % H, b = bh / H;
  const int kvh = h / (H / Hkv);
  const int row0 = blockIdx.x * R;
  const int row = row0 + lane % R;
  const float* Kp = K + (size_t)(b * Hkv + kvh) * Nk * D;
  const float* Vp = V + (size_t)(b * Hkv + kvh) * Nk * D;
  float* ks = lds + wave * Mp::kSlice;
  float* vs = ks + kTile * D;

  float q[kCols], o[kCols];
  load_cols(q, Q + ((size_t)bh * Nq + row) * D + col0, row < Nq);
#pragma unroll
  for (int c = 0; c < kCols; ++c) o[c] = 0.f;
  // Running max and denominator of this wave's keys.
  double m = -INFINITY, l = 0.0;
  int k_begin = 0, k_end = Nk;
  if (CAUSAL) k_end = min(Nk, row0 + R);
  int lo = 0, hi = Nk - 1;
  if constexpr (MASK) {
    row_interval(kv_lo, kv_hi, b, Nq, Nk, row, lo, hi);
    int w_lo, w_hi;
    rows_span(lo, hi, w_lo, w_hi);
    k_begin = w_hi >= 0 ? (w_lo / kTile) * kTile : 0;
    k_end = w_hi >= 0 ? w_hi + 1 : 0;
  }
  for (int k0 = k_begin + wave * kTile; k0 < k_end; k0 += kWaves * kTile) {
    wave_lds_sync();
    stage_tile<D>(ks, Kp, k0, Nk, lane);
    stage_tile<D>(vs, Vp, k0, Nk, lane);
    wave_lds_sync();
    double s[kTile];
    double mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      double x = row_sum<D>(part_dot64(q, ks + j * D + col0)) * (double)scale;
      const int key = k0 + j;
      if (key >= Nk || (CAUSAL && key > row) || (MASK && (key < lo || key > hi))) x = -INFINITY;
      s[j] = x;
      mt = fmax(mt, x);
    }
    const double mn = fmax(m, mt);
    // A row with every key masked so far keeps m = -inf; its weights stay zero.
    if (mn != -INFINITY) {
      const float alpha = expf((float)(m - mn));  // 0 on the first visible tile
      l *= alpha;
#pragma unroll
      for (int c = 0; c < kCols; ++c) o[c] *= alpha;
      m = mn;
    }
    float ot[kCols];
#pragma unroll
    for (int c = 0; c < kCols; ++c) ot[c] = 0.f;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const float p = (s[j] == -INFINITY) ? 0.f : expf((float)(s[j] - m));
      l += p;
      const float* vr = vs + j * D + col0;
#pragma unroll
      for (int c = 0; c < kCols; c += 4) {
        const f32x4 vv = *(const f32x4*)(vr + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) ot[c + e] = fmaf(p, vv[e], ot[c + e]);
      }
    }
#pragma unroll
    for (int c = 0; c < kCols; ++c) o[c] += ot[c];
  }

  // Merge the four waves' (m, l, o) exactly: move each to the common max.
  __syncthreads();
  float* mo = lds;  // [wave][row][D] partial outputs
  if (lane < R) {
    ml[2 * (wave * R + lane)] = m;
    ml[2 * (wave * R + lane) + 1] = l;
  }
  store_cols(mo + (wave * R + lane % R) * D + col0, o);
  __syncthreads();
  const int t = threadIdx.x;
  const int r = t / Mp::kThrPerRow;
  const int c0 = (t % Mp::kThrPerRow) * 8;
  const int orow = row0 + r;
  double mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mx = fmax(mx, ml[2 * (w * R + r)]);
  double wt[kWaves], lsum = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const double mw = ml[2 * (w * R + r)];
    wt[w] = mw == -INFINITY ? 0.0 : exp(mw - mx);
    lsum += wt[w] * ml[2 * (w * R + r) + 1];
  }
  // A row that sees no key (interval masks only): O = 0, LSE = -inf.
  const bool empty = !(lsum > 0.0);
  if (orow < Nq) {
#pragma unroll
    for (int c = 0; c < 8; c += 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (!empty) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          double x = 0.0;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) x += wt[w] * (double)mo[(w * R + r) * D + c0 + c + e];
          acc[e] = (float)(x / lsum);
        }
      }
      *(f32x4*)(O + ((size_t)bh * Nq + orow) * D + c0 + c) = acc;
    }
    if (c0 == 0) LSE[(size_t)bh * Nq + orow] = empty ? -INFINITY : (float)(mx + log(lsum));
  }
}

// dK, dV for R key rows of one key/value head; the loop over every query row of
// every query head in its group is split over the four waves (one writer per key
// row: the waves' partial sums are added through LDS at the end).
template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    float* __restrict__ dK, float* __restrict__ dV, int H, int Hkv, int Nq, int Nk, float scale,
    const int* __restrict__ kv_lo, const int* __restrict__ kv_hi) {
  using Mp = F32Map<D>;
  constexpr int R = Mp::R;
  __shared__ __attribute__((aligned(16))) float lds[Mp::kFloats];
  __shared__ float lse_s[kWaves][kTile], d_s[kWaves][kTile];
  __shared__ int lo_s[kWaves][kTile], hi_s[kWaves][kTile];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col0 = (lane / R) * kCols;
  const int bg = blockIdx.y;  // b * Hkv + kvh
  const int kvh = bg % Hkv, b = bg / Hkv;
  const int n_rep = H / Hkv;
  const int key0 = blockIdx.x * R;
  const int key = key0 + lane % R;
  const float* Kp = K + (size_t)bg * Nk * D;
  const float* Vp = V + (size_t)bg * Nk * D;
  float* qs = lds + wave * Mp::kSlice;
  float* dos = qs + kTile * D;

  float kr[kCols], vr[kCols], dk[kCols], dv[kCols];
  load_cols(kr, Kp + (size_t)key * D + col0, key < Nk);
  load_cols(vr, Vp + (size_t)key * D + col0, key < Nk);
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  // (Nq == Nk here: rectangular problems take the interval path.)
  const int first_q = CAUSAL ? (key0 / kTile) * kTile : 0;
  const int n_qt = (Nq - first_q + kTile - 1) / kTile;  // query tiles per head
  for (int t = wave; t < n_rep * n_qt; t += kWaves) {
    const int r = t / n_qt;
    const int i0 = first_q + (t % n_qt) * kTile;
    const int bh = b * H + kvh * n_rep + r;
    if constexpr (MASK) {
      // Skip query tiles none of whose rows sees these keys.
      int lo = Nk, hi = -1;
      if (lane < kTile) row_interval(kv_lo, kv_hi, b, Nq, Nk, i0 + lane, lo, hi);
      int w_lo, w_hi;
      rows_span(lo, hi, w_lo, w_hi);
      if (w_hi < key0 || w_lo > key0 + R - 1) continue;
    }
    wave_lds_sync();
    stage_tile<D>(qs, Q + (size_t)bh * Nq * D, i0, Nq, lane);
    stage_tile<D>(dos, dO + (size_t)bh * Nq * D, i0, Nq, lane);
    if (lane < kTile) {
      const int i = i0 + lane;
      lse_s[wave][lane] = i < Nq ? LSE[(size_t)bh * Nq + i] : INFINITY;
      d_s[wave][lane] = i < Nq ? Dv[(size_t)bh * Nq + i] : 0.f;
      if constexpr (MASK) row_interval(kv_lo, kv_hi, b, Nq, Nk, i, lo_s[wave][lane], hi_s[wave][lane]);
    }
    wave_lds_sync();
#pragma unroll 2
    for (int ii = 0; ii < kTile; ++ii) {
      const int i = i0 + ii;
      const float* qrow = qs + ii * D + col0;
      const float* dorow = dos + ii * D + col0;
      const double s = row_sum<D>(part_dot64(kr, qrow)) * (double)scale;
      const double dp = row_sum<D>(part_dot64(vr, dorow));
      const bool masked = (i >= Nq) || (CAUSAL && key > i) ||
                          (MASK && (key < lo_s[wave][ii] || key > hi_s[wave][ii]));
      const float p = masked ? 0.f : expf((float)(s - (double)lse_s[wave][ii]));
      const float ds = p * (float)(dp - (double)d_s[wave][ii]);
#pragma unroll
      for (int c = 0; c < kCols; c += 4) {
        const f32x4 qq = *(const f32x4*)(qrow + c);
        const f32x4 dd = *(const f32x4*)(dorow + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dv[c + e] = fmaf(p, dd[e], dv[c + e]);
          dk[c + e] = fmaf(ds, qq[e], dk[c + e]);
        }
      }
    }
  }
  // Add the four waves' partial dK, then dV (in wave order) through LDS.
  __syncthreads();
  store_cols(lds + (wave * R + lane % R) * D + col0, dk);
  __syncthreads();
  write_wave_sum<D>(dK + (size_t)bg * Nk * D, lds, key0, Nk, scale);
  __syncthreads();
  store_cols(lds + (wave * R + lane % R) * D + col0, dv);
  __syncthreads();
  write_wave_sum<D>(dV + (size_t)bg * Nk * D, lds, key0, Nk, 1.f);
}

// dQ for R query rows; the loop over the key/value tiles they see is split over
// the four waves and the partial sums are added through LDS at the end.
template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    float* __restrict__ dQ, int H, int Hkv, int Nq, int Nk, float scale,
    const int* __restrict__ kv_lo, const int* __restrict__ kv_hi) {
  using Mp = F32Map<D>;
  constexpr int R = Mp::R;
  __shared__ __attribute__((aligned(16))) float lds[Mp::kFloats];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col0 = (lane / R) * kCols;
  const int bh = blockIdx.y;
  const int h = bh % H, b = bh / H;
  const int kvh = h / (H / Hkv);
  const int row0 = blockIdx.x * R;
  const int row = row0 + lane % R;
  const float* Kp = K + (size_t)(b * Hkv + kvh) * Nk * D;
  const float* Vp = V + (size_t)(b * Hkv + kvh) * Nk * D;
  float* ks = lds + wave * Mp::kSlice;
  float* vs = ks + kTile * D;

  float q[kCols], dor[kCols], dq[kCols];
  load_cols(q, Q + ((size_t)bh * Nq + row) * D + col0, row < Nq);
  load_cols(dor, dO + ((size_t)bh * Nq + row) * D + col0, row < Nq);
#pragma unroll
  for (int c = 0; c < kCols; ++c) dq[c] = 0.f;
  const double lse = row < Nq ? (double)LSE[(size_t)bh * Nq + row] : INFINITY;
  const double dd = row < Nq ? (double)Dv[(size_t)bh * Nq + row] : 0.0;
  int k_begin = 0, k_end = Nk;
  if (CAUSAL) k_end = min(Nk, row0 + R);
  int lo = 0, hi = Nk - 1;
  if constexpr (MASK) {
    row_interval(kv_lo, kv_hi, b, Nq, Nk, row, lo, hi);
    int w_lo, w_hi;
    rows_span(lo, hi, w_lo, w_hi);
    k_begin = w_hi >= 0 ? (w_lo / kTile) * kTile : 0;
    k_end = w_hi >= 0 ? w_hi + 1 : 0;
  }
  for (int k0 = k_begin + wave * kTile; k0 < k_end; k0 += kWaves * kTile) {
    wave_lds_sync();
    stage_tile<D>(ks, Kp, k0, Nk, lane);
    stage_tile<D>(vs, Vp, k0, Nk, lane);
    wave_lds_sync();
#pragma unroll 1
    for (int j = 0; j < kTile; ++j) {
      const int key = k0 + j;
      const float* krow = ks + j * D + col0;
      const double s = row_sum<D>(part_dot64(q, krow)) * (double)scale;
      const double dp = row_sum<D>(part_dot64(dor, vs + j * D + col0));
      const bool masked = (key >= Nk) || (row >= Nq) || (CAUSAL && key > row) ||
                          (MASK && (key < lo || key > hi));
      const float p = masked ? 0.f : expf((float)(s - lse));
      const float ds = p * (float)(dp - dd);
#pragma unroll
      for (int c = 0; c < kCols; c += 4) {
        const f32x4 kk = *(const f32x4*)(krow + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) dq[c + e] = fmaf(ds, kk[e], dq[c + e]);
      }
    }
  }
  __syncthreads();
  store_cols(lds + (wave * R + lane % R) * D + col0, dq);
  __syncthreads();
  write_wave_sum<D>(dQ + (size_t)bh * Nq * D, lds, row0, Nq, scale);
}

template <int D, bool CAUSAL, bool MASK>
hipError_t fwd_f32_t(const FwdArgs& a) {
  constexpr int R = F32Map<D>::R;
  dim3 grid((a.N + R - 1) / R, a.B * a.H);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, MASK>), grid, dim3(64 * kWaves), 0,
                     (hipStream_t)a.stream, (const float*)a.q, (const float*)a.k,
                     (const float*)a.v, (float*)a.o, a.lse, a.H, a.Hkv, a.N, a.Nk ? a.Nk : a.N,
                     a.scale, a.kv_lo, a.kv_hi);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool MASK>
hipError_t bwd_f32_t(const BwdArgs& a) {
  constexpr int R = F32Map<D>::R;
  const int Nk = a.Nk ? a.Nk : a.N;
  if (a.stages & kStageDkdv) {
    dim3 gk((Nk + R - 1) / R, a.B * a.Hkv);
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL, MASK>), gk, dim3(64 * kWaves), 0,
                       (hipStream_t)a.stream, (const float*)a.q, (const float*)a.k,
                       (const float*)a.v, (const float*)a.dO, a.lse, a.dvec, (float*)a.dk,
                       (float*)a.dv, a.H, a.Hkv, a.N, Nk, a.scale, a.kv_lo, a.kv_hi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.stages & kStageDq) {
    dim3 gq((a.N + R - 1) / R, a.B * a.H);
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL, MASK>), gq, dim3(64 * kWaves), 0,
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
