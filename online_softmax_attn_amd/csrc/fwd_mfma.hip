// Forward pass of fused attention on bf16/fp16 MFMA (gfx950).
//
// The algorithm is the FlashAttention-2 forward (FlashAttention-2 page, inner
// loop steps 1-5 and the final normalisation): one workgroup owns a tile of query
// rows and the whole loop over key/value tiles ("Work partitioning"), keeps the
// running row max m, running denominator l and unnormalised output Ot on chip,
// and writes O = Ot / l and the row logsumexp once.
//
// Mapping onto CDNA4:
//  * 4 waves per workgroup; each wave owns QB blocks of 32 query rows.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: the
//    result layout then gives every lane one query row (lane % 32) and 16 keys per
//    32-key block, so the row max and row sum are in-lane, plus one exchange with
//    lane ^ 32.  The Q tile stays in registers as the B operand for the whole loop.
//  * O^T = V^T P^T uses the probabilities straight from registers as the B operand
//    (the key order inside a 16-key chunk is permuted identically on both operands).
//    V stays row-major in LDS and is read transposed with ds_read_b64_tr_b16.
//  * K/V tiles of 64 keys are double-buffered in LDS: the next tile's global loads
//    are issued before the current tile's math and stored to LDS after it.
//  * exp2 with log2(e) * scale folded into one FMA per score.
//  * Rescaling of Ot and l is lazy: the reference max is only moved when a row's
//    new max exceeds it by more than 8 (log2 units), so exp2 arguments stay <= 8.
//    The result is exact for any reference value (the correction the pages
//    describe cancels in Ot / l); it only avoids rescaling work.
//  * Causal: key tiles wholly after a wave's last row are skipped (loop bound per
//    workgroup, skip per wave); only tiles that cross the diagonal are masked.
#include "common.h"
#include "launch.h"

namespace osattn {

template <int D, int QB>
struct FwdCfg {
  static constexpr int kWaves = 4;
  static constexpr int kBR = kWaves * 32 * QB;  // query rows per workgroup
  static constexpr int kBC = 64;                // keys per tile
  static constexpr int kKStride = D + 8;        // K row stride in LDS (elements): +16 B
  static constexpr int kVStride = D + 32;       // V row stride in LDS (elements): +64 B
  static constexpr int kKTile = kBC * kKStride;
  static constexpr int kVTile = kBC * kVStride;
  static constexpr int kChunksPerRow = D / 8;   // 16-byte chunks per row
  static constexpr int kRowsPerPass = 256 / kChunksPerRow;
  static constexpr int kPasses = kBC / kRowsPerPass;
};

template <typename T, int D, int QB, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
__attribute__((amdgpu_waves_per_eu(QB == 1 ? 2 : 1, QB == 1 ? 2 : 1)))
void fwd_mfma_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                     float* __restrict__ LSE, int H, int Hkv, int N, int n_qtiles,
                     float scale_log2) {
  using C = FwdCfg<D, QB>;
  using M = Mfma<T>;
  using vec8 = typename M::vec8;
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][C::kKTile];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][C::kVTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  int qt = L % n_qtiles;
  const int bh = L / n_qtiles;  // b * H + h
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // longest rows first
  const int h = bh % H;
  const int b = bh / H;
  const int kvh = h / (H / Hkv);
  const int q0 = qt * C::kBR;
  const int wrow0 = q0 + wave * 32 * QB;

  const uint16_t* Qp = Q + (size_t)bh * N * D;
  const uint16_t* Kp = K + (size_t)(b * Hkv + kvh) * N * D;
  const uint16_t* Vp = V + (size_t)(b * Hkv + kvh) * N * D;

  // Query fragments (B operand of S^T = K Q^T): lane holds row l32 of each block,
  // columns 16c + 8*hi .. +7 for every 16-column chunk c.
  vec8 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + 32 * qb + l32;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < N) x = *(const u32x4*)(Qp + (size_t)row * D + 16 * c + 8 * hi);
      qf[qb][c] = as_vec8<T>(x);
    }
  }

  int n_kt = (N + C::kBC - 1) / C::kBC;
  if (CAUSAL) n_kt = min(n_kt, (q0 + C::kBR + C::kBC - 1) / C::kBC);

  // Global -> register staging of one K/V tile, then register -> LDS.
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
      *(u32x4*)&lds_k[buf][r * C::kKStride + ld_col] = kst[p];
      *(u32x4*)&lds_v[buf][r * C::kVStride + ld_col] = vst[p];
    }
  };

  f32x16 acc[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][t][r] = 0.f;
  // Running statistics per query row, in log2 units of the scaled scores.  The
  // finite sentinel keeps exp2(m_old - m_new) free of inf - inf.
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -1e30f;
    l_run[qb] = 0.f;
  }

  // Transposed-read addressing of V (see common.h): lane group g = lane / 16,
  // index i = lane % 16 points at row 4*hi + i/4 (+8 for the second half) of the
  // 16-key chunk and columns 16*(g%2) + 4*(i%4) .. +3 of the 32-column tile.
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) gload(kt + 1);
    const int k0 = kt * C::kBC;
    const bool active = !CAUSAL || (k0 <= wrow0 + 32 * QB - 1);
    if (active) {
      // ---- step 1: S^T = K_j Q_i^T ---------------------------------------------
      f32x16 s[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 a =
              *(const u32x4*)&lds_k[buf][(kb * 32 + l32) * C::kKStride + 16 * c + 8 * hi];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb] = M::mma32(as_vec8<T>(a), qf[qb][c], s[qb][kb]);
        }
      }
      // ---- causal / ragged-tail mask ------------------------------------------
      const bool need_mask = (k0 + C::kBC > N) || (CAUSAL && k0 + C::kBC - 1 > wrow0);
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int row = wrow0 + 32 * qb + l32;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              if (key >= N || (CAUSAL && key > row)) s[qb][kb][r] = -INFINITY;
            }
        }
      }
      // ---- step 2/4: row max, lazy move of the reference max ---------------------
      float mt[QB];
      bool grow = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
        mt[qb] = wave_xor32_max(mx) * scale_log2;
        grow |= mt[qb] > m_run[qb] + 8.0f;
      }
      if (__any(grow)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float mn = fmaxf(m_run[qb], mt[qb]);
          const float alpha = fast_exp2(m_run[qb] - mn);
          m_run[qb] = mn;
          l_run[qb] *= alpha;
#pragma unroll
          for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qb][t][r] *= alpha;
        }
      }
      // ---- step 2/3: P = exp2(S*c - m), row sums of the rounded P ---------------
      vec8 pf[QB][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float part = 0.f;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          float pv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            pv[j] = fast_exp2(fmaf(s[qb][c4 >> 1][8 * (c4 & 1) + j], scale_log2, -m_run[qb]));
          pf[qb][c4] = pack8<T>(pv);
#pragma unroll
          for (int j = 0; j < 8; ++j) part += (float)pf[qb][c4][j];
        }
        l_run[qb] += part;
      }
      // ---- step 5: O^T += V_j^T P^T ---------------------------------------------
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const uint16_t* vb = &lds_v[buf][(16 * c4 + tr_row) * C::kVStride + 32 * t + tr_col];
          const i16x4 lo = lds_read_tr4(vb);
          const i16x4 up = lds_read_tr4(vb + 8 * C::kVStride);
          const vec8 a = join8<T>(lo, up);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc[qb][t] = M::mma32(a, pf[qb][c4], acc[qb][t]);
        }
      }
    }
    if (kt + 1 < n_kt) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- final normalisation: O = Ot / l, LSE = ln(2) * (m + log2 l) -------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + 32 * qb + l32;
    const float l = wave_xor32_sum(l_run[qb]);
    const float inv = 1.0f / l;
    if (row < N) {
      uint16_t* op = O + ((size_t)bh * N + row) * D;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = (uint32_t)to_bits<T>(acc[qb][t][4 * g + 0] * inv) |
                 ((uint32_t)to_bits<T>(acc[qb][t][4 * g + 1] * inv) << 16);
          w[1] = (uint32_t)to_bits<T>(acc[qb][t][4 * g + 2] * inv) |
                 ((uint32_t)to_bits<T>(acc[qb][t][4 * g + 3] * inv) << 16);
          *(u32x2*)(op + 32 * t + 8 * g + 4 * hi) = w;
        }
      if (hi == 0) LSE[(size_t)bh * N + row] = (m_run[qb] + __log2f(l)) * kLn2;
    }
  }
}

template <typename T, int D, int QB, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  using C = FwdCfg<D, QB>;
  const int n_qtiles = (a.N + C::kBR - 1) / C::kBR;
  const long long blocks = (long long)n_qtiles * a.B * a.H;
  hipLaunchKernelGGL((fwd_mfma_kernel<T, D, QB, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.H, a.Hkv, a.N, n_qtiles,
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_fwd_d(const FwdArgs& a) {
  // Two query blocks per wave double the reuse of every K/V operand read from LDS;
  // short problems keep one block per wave so that more workgroups fill the chip.
  const long long rows = (long long)a.B * a.H * a.N;
  const bool big = rows >= 256LL * 256 * 2;
  if (a.causal)
    return big ? launch_fwd_t<T, D, 2, true>(a) : launch_fwd_t<T, D, 1, true>(a);
  return big ? launch_fwd_t<T, D, 2, false>(a) : launch_fwd_t<T, D, 1, false>(a);
}

hipError_t launch_fwd_mfma(const FwdArgs& a) {
  if (a.dtype == 2) return a.d == 64 ? launch_fwd_d<__bf16, 64>(a) : launch_fwd_d<__bf16, 128>(a);
  return a.d == 64 ? launch_fwd_d<_Float16, 64>(a) : launch_fwd_d<_Float16, 128>(a);
}

}  // namespace osattn
