// Backward pass of fused attention on bf16/fp16 MFMA (gfx950), plus the
// D = rowsum(dO * O) preprocess shared with the float32 path.
//
// The backward rebuilds P tile by tile from the saved logsumexp instead of
// storing it (FlashAttention-2 page, "Recomputation in backward pass"), and uses
// the softmax Jacobian-vector product per row, dS = P * (dP - D) with
// D_i = sum_j P_ij dP_ij = rowsum(dO * O)_i (softmax-backward page,
// "Backpropagating Through Softmax").  Then dV = P^T dO, dK = scale * dS^T Q and
// dQ = scale * dS K.
//
// Kernels:
//  1. preprocess: D (float32, into the caller's workspace).
//  2. dK/dV: one workgroup owns 128 keys of one key/value head (32 per wave, K and
//     V rows resident in registers) and loops over every query head of its GQA
//     group and every query tile that sees those keys; dK and dV have a single
//     writer.  S = Q K^T and dP = dO V^T put one key per lane, so P and dS feed
//     dV^T += dO^T P and dK^T += Q^T dS directly from registers; dO^T and Q^T are
//     read from LDS with the transpose read.
//  3. dQ: one workgroup owns 128 query rows and loops over key tiles, recomputing
//     S and dP (transposed, one query row per lane as in the forward) and forming
//     dQ^T += K^T dS^T.  No atomics; every output element has one writer.
#include "common.h"
#include "launch.h"

namespace osattn {

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O) in float32.
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const E* __restrict__ O,
                                                             const E* __restrict__ dO,
                                                             float* __restrict__ Dv,
                                                             long long rows) {
  constexpr int kEPT = 16 / sizeof(E);   // elements per 16-byte load
  constexpr int kTPR = D / kEPT;          // threads per row (8, 16 or 32)
  const long long row = (long long)blockIdx.x * (256 / kTPR) + threadIdx.x / kTPR;
  const int col = (threadIdx.x % kTPR) * kEPT;
  float acc = 0.f;
  if (row < rows) {
    if constexpr (sizeof(E) == 4) {
      // Loaded as float vectors: bit-casting an element of an integer vector
      // lvalue is miscompiled by this toolchain (every element reads lane 0).
      const f32x4 a = *(const f32x4*)(O + row * D + col);
      const f32x4 g = *(const f32x4*)(dO + row * D + col);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = fmaf(a[j], g[j], acc);
    } else {
      const u32x4 a = *(const u32x4*)(O + row * D + col);
      const u32x4 g = *(const u32x4*)(dO + row * D + col);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = fmaf(from_bits<E>((uint16_t)(a[j] & 0xffff)), from_bits<E>((uint16_t)(g[j] & 0xffff)), acc);
        acc = fmaf(from_bits<E>((uint16_t)(a[j] >> 16)), from_bits<E>((uint16_t)(g[j] >> 16)), acc);
      }
    }
  }
#pragma unroll
  for (int off = kTPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && (threadIdx.x % kTPR) == 0) Dv[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. dK / dV.
template <int D>
struct DkdvCfg {
  static constexpr int kKeys = 128;  // keys per workgroup (32 per wave)
  static constexpr int kQT = 64;     // query rows per staged tile
  static constexpr int kStride = D + 8;
  static constexpr int kTile = kQT * kStride;
  static constexpr int kChunksPerRow = D / 8;
  static constexpr int kRowsPerPass = 256 / kChunksPerRow;
  static constexpr int kPasses = kQT / kRowsPerPass;
};

template <typename T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
__attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                     const float* __restrict__ LSE, const float* __restrict__ Dv,
                     uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int H, int Hkv,
                     int N, int n_ktiles, float scale, float scale_log2) {
  using C = DkdvCfg<D>;
  using M = Mfma<T>;
  using vec8 = typename M::vec8;
  __shared__ __attribute__((aligned(16))) uint16_t lds_q[2][C::kTile];
  __shared__ __attribute__((aligned(16))) uint16_t lds_do[2][C::kTile];
  __shared__ __attribute__((aligned(16))) float lds_lse[2][C::kQT];
  __shared__ __attribute__((aligned(16))) float lds_d[2][C::kQT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = L % n_ktiles;
  const int bg = L / n_ktiles;  // b * Hkv + kvh
  const int kvh = bg % Hkv;
  const int b = bg / Hkv;
  const int n_rep = H / Hkv;
  const int k0 = kt * C::kKeys;
  const int kw = k0 + 32 * wave;  // first key of this wave

  const uint16_t* Kp = K + (size_t)bg * N * D;
  const uint16_t* Vp = V + (size_t)bg * N * D;

  // K and V rows of this wave (B operands of S = Q K^T and dP = dO V^T).
  vec8 kf[D / 16], vf[D / 16];
  {
    const int key = kw + l32;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
      if (key < N) {
        xk = *(const u32x4*)(Kp + (size_t)key * D + 16 * c + 8 * hi);
        xv = *(const u32x4*)(Vp + (size_t)key * D + 16 * c + 8 * hi);
      }
      kf[c] = as_vec8<T>(xk);
      vf[c] = as_vec8<T>(xv);
    }
  }

  f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk_acc[t][r] = 0.f;
      dv_acc[t][r] = 0.f;
    }

  // Query tiles that see these keys: all of them, or (causal) from the diagonal on.
  const int qt_first = CAUSAL ? (k0 / C::kQT) : 0;
  const int n_qt = (N + C::kQT - 1) / C::kQT;
  const int per_head = n_qt - qt_first;
  const int n_iter = per_head * n_rep;

  const int ld_row = tid / C::kChunksPerRow;
  const int ld_col = (tid % C::kChunksPerRow) * 8;
  u32x4 qst[C::kPasses], dst[C::kPasses];
  float lse_st = 0.f, d_st = 0.f;
  auto gload = [&](int it) {
    const int r = it / per_head;
    const int i0 = (qt_first + it % per_head) * C::kQT;
    const size_t bh = (size_t)b * H + kvh * n_rep + r;
    const uint16_t* Qp = Q + bh * N * D;
    const uint16_t* dOp = dO + bh * N * D;
#pragma unroll
    for (int p = 0; p < C::kPasses; ++p) {
      const int row = i0 + p * C::kRowsPerPass + ld_row;
      u32x4 zq = {0u, 0u, 0u, 0u}, zd = {0u, 0u, 0u, 0u};
      if (row < N) {
        zq = *(const u32x4*)(Qp + (size_t)row * D + ld_col);
        zd = *(const u32x4*)(dOp + (size_t)row * D + ld_col);
      }
      qst[p] = zq;
      dst[p] = zd;
    }
    if (tid < C::kQT) {
      const int row = i0 + tid;
      // Rows past the end get P = exp2(-inf) = 0 and D = 0.
      lse_st = row < N ? LSE[bh * N + row] * kLog2e : INFINITY;
      d_st = row < N ? Dv[bh * N + row] : 0.f;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < C::kPasses; ++p) {
      const int row = p * C::kRowsPerPass + ld_row;
      *(u32x4*)&lds_q[buf][row * C::kStride + ld_col] = qst[p];
      *(u32x4*)&lds_do[buf][row * C::kStride + ld_col] = dst[p];
    }
    if (tid < C::kQT) {
      lds_lse[buf][tid] = lse_st;
      lds_d[buf][tid] = d_st;
    }
  };

  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  if (n_iter > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    if (it + 1 < n_iter) gload(it + 1);
    const int i0 = (qt_first + it % per_head) * C::kQT;
#pragma unroll
    for (int qb = 0; qb < C::kQT / 32; ++qb) {
      const int qs = i0 + 32 * qb;
      if (CAUSAL && qs + 31 < kw) continue;  // every key of this wave is after every row
      // S = Q K^T and dP = dO V^T (result: lane = key, register = query row).
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const u32x4 aq = *(const u32x4*)&lds_q[buf][(32 * qb + l32) * C::kStride + 16 * c + 8 * hi];
        const u32x4 ad = *(const u32x4*)&lds_do[buf][(32 * qb + l32) * C::kStride + 16 * c + 8 * hi];
        s = M::mma32(as_vec8<T>(aq), kf[c], s);
        dp = M::mma32(as_vec8<T>(ad), vf[c], dp);
      }
      const int key = kw + l32;
      float p[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ql = 32 * qb + 8 * g + 4 * hi;  // local query row of register 4g
        const f32x4 lse4 = *(const f32x4*)&lds_lse[buf][ql];
        const f32x4 d4 = *(const f32x4*)&lds_d[buf][ql];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pv = fast_exp2(fmaf(s[r], scale_log2, -lse4[e]));
          if (CAUSAL && key > i0 + ql + e) pv = 0.f;
          p[r] = pv;
          ds[r] = pv * (dp[r] - d4[e]);
        }
      }
      // dV^T += dO^T P ; dK^T += Q^T dS  (reduction over the 32 query rows)
#pragma unroll
      for (int cq = 0; cq < 2; ++cq) {
        const vec8 pp = pack8<T>(p + 8 * cq);
        const vec8 ps = pack8<T>(ds + 8 * cq);
        const int row = 32 * qb + 16 * cq + tr_row;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const uint16_t* db = &lds_do[buf][row * C::kStride + 32 * t + tr_col];
          const uint16_t* qb_ = &lds_q[buf][row * C::kStride + 32 * t + tr_col];
          const vec8 adt = join8<T>(lds_read_tr4(db), lds_read_tr4(db + 8 * C::kStride));
          const vec8 aqt = join8<T>(lds_read_tr4(qb_), lds_read_tr4(qb_ + 8 * C::kStride));
          dv_acc[t] = M::mma32(adt, pp, dv_acc[t]);
          dk_acc[t] = M::mma32(aqt, ps, dk_acc[t]);
        }
      }
    }
    if (it + 1 < n_iter) lstore(buf ^ 1);
    __syncthreads();
  }

  // Store: lane = key, register r of tile t = column 32t + 8(r/4) + 4hi + r%4.
  const int key = kw + l32;
  if (key < N) {
    uint16_t* dkp = dK + ((size_t)bg * N + key) * D;
    uint16_t* dvp = dV + ((size_t)bg * N + key) * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 wk, wv;
        wk[0] = (uint32_t)to_bits<T>(dk_acc[t][4 * g + 0] * scale) |
                ((uint32_t)to_bits<T>(dk_acc[t][4 * g + 1] * scale) << 16);
        wk[1] = (uint32_t)to_bits<T>(dk_acc[t][4 * g + 2] * scale) |
                ((uint32_t)to_bits<T>(dk_acc[t][4 * g + 3] * scale) << 16);
        wv[0] = (uint32_t)to_bits<T>(dv_acc[t][4 * g + 0]) |
                ((uint32_t)to_bits<T>(dv_acc[t][4 * g + 1]) << 16);
        wv[1] = (uint32_t)to_bits<T>(dv_acc[t][4 * g + 2]) |
                ((uint32_t)to_bits<T>(dv_acc[t][4 * g + 3]) << 16);
        *(u32x2*)(dkp + 32 * t + 8 * g + 4 * hi) = wk;
        *(u32x2*)(dvp + 32 * t + 8 * g + 4 * hi) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ.
template <int D>
struct DqCfg {
  static constexpr int kRows = 128;  // query rows per workgroup (32 per wave)
  static constexpr int kBC = 64;     // keys per staged tile
  static constexpr int kStride = D + 8;
  static constexpr int kTile = kBC * kStride;
  static constexpr int kChunksPerRow = D / 8;
  static constexpr int kRowsPerPass = 256 / kChunksPerRow;
  static constexpr int kPasses = kBC / kRowsPerPass;
};

template <typename T, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
__attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                   const float* __restrict__ LSE, const float* __restrict__ Dv,
                   uint16_t* __restrict__ dQ, int H, int Hkv, int N, int n_qtiles, float scale,
                   float scale_log2) {
  using C = DqCfg<D>;
  using M = Mfma<T>;
  using vec8 = typename M::vec8;
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][C::kTile];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][C::kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  int qt = L % n_qtiles;
  const int bh = L / n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;
  const int h = bh % H;
  const int b = bh / H;
  const int kvh = h / (H / Hkv);
  const int q0 = qt * C::kRows;
  const int wrow0 = q0 + 32 * wave;
  const int row = wrow0 + l32;

  const uint16_t* Kp = K + (size_t)(b * Hkv + kvh) * N * D;
  const uint16_t* Vp = V + (size_t)(b * Hkv + kvh) * N * D;

  vec8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4 xq = {0u, 0u, 0u, 0u}, xd = {0u, 0u, 0u, 0u};
    if (row < N) {
      xq = *(const u32x4*)(Q + ((size_t)bh * N + row) * D + 16 * c + 8 * hi);
      xd = *(const u32x4*)(dO + ((size_t)bh * N + row) * D + 16 * c + 8 * hi);
    }
    qf[c] = as_vec8<T>(xq);
    df[c] = as_vec8<T>(xd);
  }
  const float lse2 = row < N ? LSE[(size_t)bh * N + row] * kLog2e : INFINITY;
  const float drow = row < N ? Dv[(size_t)bh * N + row] : 0.f;

  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;

  int n_kt = (N + C::kBC - 1) / C::kBC;
  if (CAUSAL) n_kt = min(n_kt, (q0 + C::kRows + C::kBC - 1) / C::kBC);

  const int ld_row = tid / C::kChunksPerRow;
  const int ld_col = (tid % C::kChunksPerRow) * 8;
  u32x4 kst[C::kPasses], vst[C::kPasses];
  auto gload = [&](int kt) {
#pragma unroll
    for (int p = 0; p < C::kPasses; ++p) {
      const int r = kt * C::kBC + p * C::kRowsPerPass + ld_row;
      u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
      if (r < N) {
        zk = *(const u32x4*)(Kp + (size_t)r * D + ld_col);
        zv = *(const u32x4*)(Vp + (size_t)r * D + ld_col);
      }
      kst[p] = zk;
      vst[p] = zv;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < C::kPasses; ++p) {
      const int r = p * C::kRowsPerPass + ld_row;
      *(u32x4*)&lds_k[buf][r * C::kStride + ld_col] = kst[p];
      *(u32x4*)&lds_v[buf][r * C::kStride + ld_col] = vst[p];
    }
  };

  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) gload(kt + 1);
    const int k0 = kt * C::kBC;
    const bool active = !CAUSAL || (k0 <= wrow0 + 31);
    if (active) {
      // S^T = K Q^T, dP^T = V dO^T (lane = query row, register = key)
      f32x16 s[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[kb][r] = 0.f;
          dp[kb][r] = 0.f;
        }
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 ak = *(const u32x4*)&lds_k[buf][(kb * 32 + l32) * C::kStride + 16 * c + 8 * hi];
          const u32x4 av = *(const u32x4*)&lds_v[buf][(kb * 32 + l32) * C::kStride + 16 * c + 8 * hi];
          s[kb] = M::mma32(as_vec8<T>(ak), qf[c], s[kb]);
          dp[kb] = M::mma32(as_vec8<T>(av), df[c], dp[kb]);
        }
      }
      const bool need_mask = (k0 + C::kBC > N) || (CAUSAL && k0 + C::kBC - 1 > wrow0);
      float dsv[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = fast_exp2(fmaf(s[kb][r], scale_log2, -lse2));
          if (need_mask) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key >= N || (CAUSAL && key > row)) pv = 0.f;
          }
          dsv[kb][r] = pv * (dp[kb][r] - drow);
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const vec8 ps = pack8<T>(&dsv[c4 >> 1][8 * (c4 & 1)]);
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const uint16_t* kb_ = &lds_k[buf][(16 * c4 + tr_row) * C::kStride + 32 * t + tr_col];
          const vec8 a = join8<T>(lds_read_tr4(kb_), lds_read_tr4(kb_ + 8 * C::kStride));
          acc[t] = M::mma32(a, ps, acc[t]);
        }
      }
    }
    if (kt + 1 < n_kt) lstore(buf ^ 1);
    __syncthreads();
  }

  if (row < N) {
    uint16_t* qp = dQ + ((size_t)bh * N + row) * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = (uint32_t)to_bits<T>(acc[t][4 * g + 0] * scale) |
               ((uint32_t)to_bits<T>(acc[t][4 * g + 1] * scale) << 16);
        w[1] = (uint32_t)to_bits<T>(acc[t][4 * g + 2] * scale) |
               ((uint32_t)to_bits<T>(acc[t][4 * g + 3] * scale) << 16);
        *(u32x2*)(qp + 32 * t + 8 * g + 4 * hi) = w;
      }
  }
}

// ---------------------------------------------------------------------------
template <typename E, int D>
static hipError_t preprocess_t(const BwdArgs& a) {
  constexpr int kTPR = D / (16 / sizeof(E));
  const long long rows = (long long)a.B * a.H * a.N;
  const long long blocks = (rows + (256 / kTPR) - 1) / (256 / kTPR);
  hipLaunchKernelGGL((bwd_preprocess_kernel<E, D>), dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)a.stream, (const E*)a.o, (const E*)a.dO, a.dvec, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_preprocess(const BwdArgs& a) {
  if (a.dtype == 0) return a.d == 64 ? preprocess_t<float, 64>(a) : preprocess_t<float, 128>(a);
  if (a.dtype == 1) return a.d == 64 ? preprocess_t<_Float16, 64>(a) : preprocess_t<_Float16, 128>(a);
  return a.d == 64 ? preprocess_t<__bf16, 64>(a) : preprocess_t<__bf16, 128>(a);
}

template <typename T, int D, bool CAUSAL>
static hipError_t bwd_t(const BwdArgs& a) {
  const float sl2 = a.scale * kLog2e;
  {
    using C = DkdvCfg<D>;
    const int n_kt = (a.N + C::kKeys - 1) / C::kKeys;
    const long long blocks = (long long)n_kt * a.B * a.Hkv;
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (const uint16_t*)a.dO, a.lse, a.dvec,
                       (uint16_t*)a.dk, (uint16_t*)a.dv, a.H, a.Hkv, a.N, n_kt, a.scale, sl2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    using C = DqCfg<D>;
    const int n_qt = (a.N + C::kRows - 1) / C::kRows;
    const long long blocks = (long long)n_qt * a.B * a.H;
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (const uint16_t*)a.dO, a.lse, a.dvec,
                       (uint16_t*)a.dq, a.H, a.Hkv, a.N, n_qt, a.scale, sl2);
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t bwd_dt(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? bwd_t<T, 64, true>(a) : bwd_t<T, 64, false>(a);
  return a.causal ? bwd_t<T, 128, true>(a) : bwd_t<T, 128, false>(a);
}

hipError_t launch_bwd_mfma(const BwdArgs& a) {
  return a.dtype == 2 ? bwd_dt<__bf16>(a) : bwd_dt<_Float16>(a);
}

}  // namespace osattn
