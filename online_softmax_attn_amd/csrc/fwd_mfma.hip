// Forward pass of fused attention on bf16/fp16 MFMA (gfx950).
//
// The algorithm is the FlashAttention-2 forward (FlashAttention-2 page, inner
// loop steps 1-5 and the final normalisation): one workgroup owns a tile of query
// rows and the whole loop over key/value tiles ("Work partitioning"), keeps the
// running row max m, running denominator l and unnormalised output Ot on chip,
// and writes O = Ot / l and the row logsumexp once.
//
// Mapping onto CDNA4:
//  * NW waves per workgroup (8: two per SIMD, so one wave's softmax arithmetic
//    overlaps another wave's matrix-core work); each wave owns QB blocks of 32
//    query rows.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: the
//    result layout then gives every lane one query row (lane % 32) and 16 keys per
//    32-key block, so the row max and row sum are in-lane, plus one exchange with
//    lane ^ 32.  The Q tile stays in registers as the B operand for the whole loop.
//  * O^T = V^T P^T uses the probabilities straight from registers as the B operand
//    (the key order inside a 16-key chunk is permuted identically on both operands).
//    V stays row-major in LDS and is read transposed with ds_read_b64_tr_b16.
//  * K/V tiles of 64 keys go from HBM/L2 straight into LDS (buffer_load ... lds,
//    16 bytes per lane, rows past the end read as zero), NBUF tiles in flight.
//    LDS rows are unpadded; 16-byte granules are XOR-swizzled by row so that the
//    128-bit K reads and the transposed V reads are free of bank conflicts.
//  * exp2 with log2(e) * scale folded into one FMA per score; row sums with
//    v_dot2 over the rounded probabilities the matrix core consumes.
//  * The reference max is lazy: P is formed against the current reference and the
//    exact tile max is taken (with the rescale of Ot and l) only on the first tile
//    and when a row's tile sum of P leaves [0, 2^30].  The result is exact for any
//    reference value (the correction the pages describe cancels in Ot / l); it only
//    avoids the per-tile max and rescaling work.
//  * Causal: key tiles wholly after the workgroup's last row are not loaded, tiles
//    wholly after a wave's last row are skipped by that wave, and only tiles that
//    cross the diagonal are masked.  Workgroups with the longest rows start first.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace osattn {

template <int D>
struct FwdSwizzle {
  // 16-byte granule index XOR applied to row `row` of a K tile / a V tile.
  static __device__ __forceinline__ int k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  static __device__ __forceinline__ int v(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
};

template <int D, int NW, int QB, int NBUF, int BC>
struct FwdCfg {
  static constexpr int kBR = NW * 32 * QB;     // query rows per workgroup
  static constexpr int kBC = BC;               // keys per tile (64 or 128)
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileElems = kBC * D;   // one K or V tile (16-bit elements)
  static constexpr int kChunks = kBC * kRowBytes / 1024;  // 1 KB LDS-DMA chunks per tile
  static constexpr int kCPW = kChunks / NW;    // chunks per wave per tensor
  static_assert(kCPW >= 1 && kChunks % NW == 0, "tile must split evenly over the waves");
};

// Persistent grid (StaticSchedule) for every forward without an interval mask: the
// causal query tiles differ in length, and with equal tiles it still saves the gap
// between one workgroup's end and the next one's dispatch on each CU (about 1.5% at
// B4 H16 N8192 d128).
#ifndef OSATTN_FWD_PERSIST
#define OSATTN_FWD_PERSIST 1
#endif

// Kernel arguments.
struct FwdKernelArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  float* LSE;
  int H, Hkv, Nq, Nk, n_qtiles;
  float scale_log2;
  const int* kv_lo;
  const int* kv_hi;
  int n_jobs;  // logical tiles (query tiles x heads)
  int pad_;
};

template <typename T, int D, int NW, int QB, int NBUF, int BC, bool CAUSAL, bool MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_mfma_kernel(const FwdKernelArgs args) {
  using C = FwdCfg<D, NW, QB, NBUF, BC>;
  using M = Mfma<T>;
  using vec8 = typename M::vec8;
  using Swz = FwdSwizzle<D>;
  constexpr bool PERSIST = OSATTN_FWD_PERSIST && !MASK;
  // One array per pipeline stage: with the stage known at compile time, the
  // compiler can tell that reads of one stage do not alias the DMA writes still in
  // flight into the others, and inserts no wait for them.
  static_assert(NBUF >= 2 && NBUF <= 4, "two to four stages");
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k0[C::kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v0[C::kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k1[C::kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v1[C::kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k2[NBUF > 2 ? C::kTileElems : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v2[NBUF > 2 ? C::kTileElems : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k3[NBUF > 3 ? C::kTileElems : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v3[NBUF > 3 ? C::kTileElems : 8];

  const int tid0 = threadIdx.x;

  // Logical tile L: query tile L % n_qtiles of head L / n_qtiles.  A persistent grid
  // (no interval mask) walks its schedule (see StaticSchedule), longest first within each
  // head when causal, as below; otherwise each workgroup runs one tile.
  StaticSchedule sched(args.n_jobs, blockIdx.x, gridDim.x);
  int L;
  if constexpr (PERSIST) {
    L = sched.next();
  } else {
    // Interval masks can give the K/V-head groups very different amounts of work (packed
    // documents differ per batch entry): deal the groups over the XCDs.
    L = (OSATTN_XCD_GROUPS && MASK)
            ? xcd_group_remap(blockIdx.x, gridDim.x, args.n_qtiles * (args.H / args.Hkv))
            : xcd_remap(blockIdx.x, gridDim.x);
  }
  while (L >= 0) {
    // A persistent grid reads its arguments afresh for each tile (see fresh_kernel_args).
    // At d = 64 it also hides the lane index from the compiler per tile, so that
    // lane-dependent offsets are computed per tile rather than held in registers from
    // the first (2% faster there, 2% slower at d = 128).
    int tid = tid0;
    if constexpr (PERSIST && D == 64) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: LDS-DMA addresses stay SALU
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const FwdKernelArgs a = PERSIST ? fresh_kernel_args<FwdKernelArgs>() : args;
    const uint16_t* __restrict__ Q = a.Q;
    const uint16_t* __restrict__ K = a.K;
    const uint16_t* __restrict__ V = a.V;
    uint16_t* __restrict__ O = a.O;
    float* __restrict__ LSE = a.LSE;
    const int H = a.H, Hkv = a.Hkv, Nq = a.Nq, Nk = a.Nk, n_qtiles = a.n_qtiles;
    const float scale_log2 = a.scale_log2;
    const int* __restrict__ kv_lo = a.kv_lo;
    const int* __restrict__ kv_hi = a.kv_hi;
    int qt = L % n_qtiles;
    const int bh = L / n_qtiles;  // b * H + h
    // Longest rows first: under a causal mask, and under interval masks, whose usual
    // forms (causal, windows, documents) give later rows at least as many keys.
    if (CAUSAL || (OSATTN_MASK_LONGEST_FIRST && MASK)) qt = n_qtiles - 1 - qt;
    const int h = bh % H;
    const int b = bh / H;
    const int kvh = h / (H / Hkv);
    const int q0 = qt * C::kBR;
    const int wrow0 = q0 + wave * 32 * QB;

    const auto rq = make_rsrc(Q + (size_t)bh * Nq * D, (uint32_t)Nq * C::kRowBytes);
    const uint32_t kv_bytes = (uint32_t)Nk * C::kRowBytes;
    const auto rk = make_rsrc(K + (size_t)(b * Hkv + kvh) * Nk * D, kv_bytes);
    const auto rv = make_rsrc(V + (size_t)(b * Hkv + kvh) * Nk * D, kv_bytes);

    // Query fragments (B operand of S^T = K Q^T): lane holds row l32 of each block,
    // columns 16c + 8*hi .. +7 for every 16-column chunk c.  Rows >= N read zero.
    vec8 qf[QB][D / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const uint32_t rowoff = (uint32_t)(wrow0 + 32 * qb + l32) * C::kRowBytes;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) qf[qb][c] = as_vec8<T>(buffer_load16(rq, rowoff + (16 * c + 8 * hi) * 2));
    }

    int kt0 = 0;  // first key tile of the loop
    int n_kt = (Nk + C::kBC - 1) / C::kBC;
    if (CAUSAL) n_kt = min(n_kt, (q0 + C::kBR + C::kBC - 1) / C::kBC);

    // Interval masks: row i sees keys lo_i .. hi_i (clamped to the sequence; an empty
    // interval, and any row past Nq, is lo = Nk, hi = -1).  A wave skips tiles outside
    // the union of its rows' intervals and masks only tiles not inside all of them;
    // the workgroup loads only the tiles some wave needs.
    int lo_r[QB], hi_r[QB];
    int w_lo = 0, w_hi = 0, w_maxlo = 0, w_minhi = 0;
    if constexpr (MASK) {
      __shared__ int wg_bounds[2 * NW];
      w_lo = Nk;
      w_hi = -1;
      w_maxlo = 0;
      w_minhi = Nk - 1;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int row = wrow0 + 32 * qb + l32;
        int lo = Nk, hi = -1;
        if (row < Nq) {
          lo = max(load_global<int>(kv_lo + (size_t)b * Nq + row), 0);
          hi = min(load_global<int>(kv_hi + (size_t)b * Nq + row), Nk - 1);
          if (lo > hi) {
            lo = Nk;
            hi = -1;
          }
        }
        lo_r[qb] = lo;
        hi_r[qb] = hi;
        w_lo = min(w_lo, lo);
        w_hi = max(w_hi, hi);
        w_maxlo = max(w_maxlo, lo);
        w_minhi = min(w_minhi, hi);
      }
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {  // over the 32 rows (both lane halves agree)
        w_lo = min(w_lo, __shfl_xor(w_lo, off));
        w_hi = max(w_hi, __shfl_xor(w_hi, off));
        w_maxlo = max(w_maxlo, __shfl_xor(w_maxlo, off));
        w_minhi = min(w_minhi, __shfl_xor(w_minhi, off));
      }
      if (lane == 0) {
        wg_bounds[2 * wave] = w_lo;
        wg_bounds[2 * wave + 1] = w_hi;
      }
      __syncthreads();
      int g_lo = Nk, g_hi = -1;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        g_lo = min(g_lo, wg_bounds[2 * w]);
        g_hi = max(g_hi, wg_bounds[2 * w + 1]);
      }
      kt0 = g_hi >= g_lo ? g_lo / C::kBC : 0;
      n_kt = g_hi >= g_lo ? g_hi / C::kBC + 1 - kt0 : 0;
    }

    // Global offsets of this lane's 16 bytes in each of its LDS-DMA chunks: chunk ch
    // covers LDS bytes [ch*1024, +1024) of the tile, i.e. tile row off / kRowBytes,
    // physical granule pg; the data there is logical granule pg ^ swizzle(row).
    uint32_t goff_k[C::kCPW], goff_v[C::kCPW];
#pragma unroll
    for (int i = 0; i < C::kCPW; ++i) {
      const int off = (wave * C::kCPW + i) * 1024 + lane * 16;
      const int row = off / C::kRowBytes;
      const int pg = (off % C::kRowBytes) / 16;
      goff_k[i] = row * C::kRowBytes + ((pg ^ Swz::k(row)) * 16);
      goff_v[i] = row * C::kRowBytes + ((pg ^ Swz::v(row)) * 16);
    }
    auto issue = [&](int kt, uint16_t* lk, uint16_t* lv) __attribute__((always_inline)) {
      const uint32_t base = (uint32_t)(kt0 + kt) * C::kBC * C::kRowBytes;
#pragma unroll
      for (int i = 0; i < C::kCPW; ++i) {
        const int ch = wave * C::kCPW + i;
        // Tile base in the scalar offset, loop-invariant lane offsets: no vector
        // address arithmetic per load.
        buffer_load16_lds(rk, lk + ch * 512, goff_k[i], base);
        buffer_load16_lds(rv, lv + ch * 512, goff_v[i], base);
      }
    };

    // LDS read offsets (bytes within a tile), loop-invariant per lane.
    //  K (A operand of S^T): row kb*32 + l32, logical granule 2c + hi.
    uint32_t koff[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) koff[c] = l32 * C::kRowBytes + (((2 * c + hi) ^ Swz::k(l32)) * 16);
    //  V (transposed reads, see common.h): group g = lane / 16 and index i = lane % 16
    //  read row 4*hi + i/4 (+8 for the upper half) of a 16-key chunk and columns
    //  32t + 16*(g%2) + 4*(i%4) .. +3.
    const int tr_row = 4 * hi + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    uint32_t voff[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const int col = 32 * t + tr_col;
      voff[t] = tr_row * C::kRowBytes + (((col >> 3) ^ Swz::v(tr_row)) * 16) + (col & 7) * 2;
    }

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

    auto compute = [&](int kt, const char* kbase, const char* vbase) __attribute__((always_inline)) {
      const int k0 = (kt0 + kt) * C::kBC;
      const bool active = (!CAUSAL || (k0 <= wrow0 + 32 * QB - 1)) &&
                          (!MASK || (k0 <= w_hi && k0 + C::kBC - 1 >= w_lo));
      if (!active) return;

      // ---- step 1: S^T = K_j Q_i^T -------------------------------------------------
      constexpr int KB = BC / 32;  // 32-key blocks per tile
      f32x16 s[QB][KB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const u32x4 a = *(const u32x4*)(kbase + kb * 32 * C::kRowBytes + koff[c]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb] = M::mma32(as_vec8<T>(a), qf[qb][c], s[qb][kb]);
        }
      }
      {  // Keep 8 K reads in flight ahead of the MFMAs that consume them (left alone, the
         // scheduler issues two and waits for them before every pair of MFMAs).
        constexpr int nR = D / 16 * KB, AH = 8;
        __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
#pragma unroll
        for (int i = 0; i < nR - AH; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x8, QB, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x8, AH * QB, 0);
      }
      // ---- causal / ragged-tail mask (only on tiles that need it) ------------------------
      const bool need_mask = (k0 + C::kBC > Nk) || (CAUSAL && k0 + C::kBC - 1 > wrow0) ||
                             (MASK && !(k0 >= w_maxlo && k0 + C::kBC - 1 <= w_minhi));
      if (need_mask) {
        // Element r of block kb holds key k0 + 4*hi + ko, ko a compile-time constant:
        // each test compares that constant with a limit taken once per tile.
        const int base = k0 + 4 * hi;
        const int lim_n = Nk - base;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int lim_c = wrow0 + 32 * qb + l32 - base;
          const int lim_lo = MASK ? lo_r[qb] - base : 0;
          const int lim_hi = MASK ? min(hi_r[qb] - base, lim_n - 1) : lim_n - 1;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int ko = kb * 32 + 8 * (r >> 2) + (r & 3);
              if ((CAUSAL && ko > lim_c) || (MASK && ko < lim_lo) || ko > lim_hi)
                s[qb][kb][r] = -INFINITY;
            }
        }
      }
      // ---- steps 2-4: probabilities against the running reference max -------------------
      // P = exp2(S*c - m) with the current reference m.  The reference only has to keep
      // the exponentials in a safe range: Ot / l and m + log2 l do not depend on it.  So
      // the exact tile max is computed only on a wave's first tile and when some row's
      // tile sum leaves [0, 2^30] (or is not finite); then Ot and l are rescaled by
      // exp2(m_old - m_new) (the correction of the pages' step 4) and P is recomputed.
      vec8 pf[QB][2 * KB];
      float part[QB];
      auto probs = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float neg_m = -m_run[qb];
          part[qb] = 0.f;
#pragma unroll
          for (int c4 = 0; c4 < 2 * KB; ++c4) {
            float pv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) pv[j] = fast_exp2(fmaf(s[qb][c4 >> 1][8 * (c4 & 1) + j], scale_log2, neg_m));
            pf[qb][c4] = pack8<T>(pv);
            part[qb] = sum8<T>(pf[qb][c4], part[qb]);
          }
        }
      };
      auto move_reference = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float mx = fmaxf(s[qb][0][0], s[qb][0][1]);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = (kb == 0 ? 2 : 0); r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[qb][kb][r], s[qb][kb][r + 1]));
          const float mn = fmaxf(m_run[qb], wave_xor32_max(mx) * scale_log2);
          const float alpha = fast_exp2(m_run[qb] - mn);
          m_run[qb] = mn;
          l_run[qb] *= alpha;
#pragma unroll
          for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qb][t][r] *= alpha;
        }
      };
      if (!MASK && kt == 0) move_reference();  // masked rows may start later: left to the range check
      probs();
      bool unsafe = false;
#pragma unroll
      // 2^30 per tile keeps l below 2^44 for any N <= 2^24, far from fp32 overflow.
      for (int qb = 0; qb < QB; ++qb) unsafe |= !(part[qb] <= 1073741824.0f);  // also catches NaN
      if (__any(unsafe)) {
        move_reference();
        probs();
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) l_run[qb] += part[qb];
      // ---- step 5: O^T += V_j^T P^T ---------------------------------------------------
#pragma unroll
      for (int c4 = 0; c4 < 2 * KB; ++c4) {
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const char* vb = vbase + 16 * c4 * C::kRowBytes + voff[t];
          const vec8 a = join8<T>(lds_read_tr4(vb), lds_read_tr4(vb + 8 * C::kRowBytes));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc[qb][t] = M::mma32(a, pf[qb][c4], acc[qb][t]);
        }
      }
      {  // the same for the transposed V reads: 4 MFMA operands (8 reads) ahead
        constexpr int nA = 2 * KB * (D / 32), AH = 4;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * AH, 0);
#pragma unroll
        for (int i = 0; i < nA - AH; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x8, QB, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x8, AH * QB, 0);
      }
    };

    auto stage_k = [&](auto sc) __attribute__((always_inline)) -> uint16_t* {
      constexpr int S = decltype(sc)::value;
      if constexpr (S == 0) return lds_k0;
      else if constexpr (S == 1) return lds_k1;
      else if constexpr (S == 2) return lds_k2;
      else return lds_k3;
    };
    auto stage_v = [&](auto sc) __attribute__((always_inline)) -> uint16_t* {
      constexpr int S = decltype(sc)::value;
      if constexpr (S == 0) return lds_v0;
      else if constexpr (S == 1) return lds_v1;
      else if constexpr (S == 2) return lds_v2;
      else return lds_v3;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (0 < n_kt) issue(0, lds_k0, lds_v0);
    if (NBUF > 2 && 1 < n_kt) issue(1, lds_k1, lds_v1);
    if (NBUF > 3 && 2 < n_kt) issue(2, lds_k2, lds_v2);

    // One pipeline step for tile kt held in stage S (compile-time).
    auto step = [&](auto stage_c, int kt) __attribute__((always_inline)) {
      constexpr int SN = (decltype(stage_c)::value + NBUF - 1) % NBUF;  // receives tile kt + NBUF - 1
      uint16_t* lk = stage_k(stage_c);
      uint16_t* lv = stage_v(stage_c);
      uint16_t* nk = stage_k(std::integral_constant<int, SN>{});
      uint16_t* nv = stage_v(std::integral_constant<int, SN>{});
      // Tile kt has landed once at most the loads of the (up to NBUF - 2) tiles
      // issued after it are outstanding.
      const int ahead = min(NBUF - 2, n_kt - 1 - kt);
      if (NBUF > 3 && ahead >= 2) wait_vmcnt<4 * C::kCPW>();
      else if (NBUF > 2 && ahead >= 1) wait_vmcnt<2 * C::kCPW>();
      else wait_vmcnt<0>();
      block_barrier();  // every wave's share of tile kt is in LDS; tile kt-1 is free
      if (kt + NBUF - 1 < n_kt) issue(kt + NBUF - 1, nk, nv);
      compute(kt, (const char*)lk, (const char*)lv);
    };
    for (int kt = 0; kt < n_kt; kt += NBUF) {
      step(I0{}, kt);
      if (kt + 1 < n_kt) step(I1{}, kt + 1);
      if constexpr (NBUF > 2)
        if (kt + 2 < n_kt) step(I2{}, kt + 2);
      if constexpr (NBUF > 3)
        if (kt + 3 < n_kt) step(std::integral_constant<int, 3>{}, kt + 3);
    }

    // ---- final normalisation: O = Ot / l, LSE = ln(2) * (m + log2 l) ---------------
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = wrow0 + 32 * qb + l32;
      const float l = wave_xor32_sum(l_run[qb]);
      const bool empty = MASK && !(l > 0.f);  // a row that sees no key: O = 0, LSE = -inf
      const float inv = empty ? 0.f : 1.0f / l;
      if (row < Nq) {
        uint16_t* op = O + ((size_t)bh * Nq + row) * D;
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u32x2 w;
            w[0] = (uint32_t)to_bits<T>(acc[qb][t][4 * g + 0] * inv) |
                   ((uint32_t)to_bits<T>(acc[qb][t][4 * g + 1] * inv) << 16);
            w[1] = (uint32_t)to_bits<T>(acc[qb][t][4 * g + 2] * inv) |
                   ((uint32_t)to_bits<T>(acc[qb][t][4 * g + 3] * inv) << 16);
            store_global(op + 32 * t + 8 * g + 4 * hi, w);
          }
        if (hi == 0)
          store_global(LSE + (size_t)bh * Nq + row, empty ? -INFINITY : (m_run[qb] + __log2f(l)) * kLn2);
      }
    }
    if constexpr (!PERSIST) break;
    __syncthreads();  // every wave is done with the staged tiles
    L = sched.next();
  }
}

template <typename T, int D, int NW, int QB, int NBUF, int BC, bool CAUSAL, bool MASK>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  using C = FwdCfg<D, NW, QB, NBUF, BC>;
  const int n_qtiles = (a.N + C::kBR - 1) / C::kBR;
  const long long jobs = (long long)n_qtiles * a.B * a.H;
  auto kernel = fwd_mfma_kernel<T, D, NW, QB, NBUF, BC, CAUSAL, MASK>;
  long long blocks = jobs;
  if (OSATTN_FWD_PERSIST && !MASK) {
    static const int per_cu = resident_per_cu(kernel, NW * 64);
    blocks = persistent_grid(per_cu, jobs);
  }
  const FwdKernelArgs ka{(const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                         (uint16_t*)a.o, a.lse, a.H, a.Hkv, a.N, a.Nk ? a.Nk : a.N, n_qtiles,
                         a.scale * kLog2e, a.kv_lo, a.kv_hi, (int)jobs, 0};
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(NW * 64), 0, (hipStream_t)a.stream, ka);
  return hipGetLastError();
}

// Tile configuration (waves per workgroup, 32-row query blocks per wave, K/V
// buffers); the defaults are the measured best on MI355X and can be overridden
// at build time for tuning sweeps.
#ifndef OSATTN_FWD_NW
#define OSATTN_FWD_NW 8
#endif
#ifndef OSATTN_FWD_QB
#define OSATTN_FWD_QB 1
#endif
#ifndef OSATTN_FWD_NBUF
#define OSATTN_FWD_NBUF 2
#endif
#ifndef OSATTN_FWD_BC
#define OSATTN_FWD_BC 128
#endif

// d = 64 has its own tile shapes: the smaller Q fragments and O accumulators leave
// room for two 32-row blocks per wave at two waves per SIMD (every shape here runs
// two waves per SIMD: one workgroup of 8 waves or two of 4 per CU).
#ifndef OSATTN_FWD64_NW
#define OSATTN_FWD64_NW 8
#endif
#ifndef OSATTN_FWD64C_NW
#define OSATTN_FWD64C_NW 8
#endif
#ifndef OSATTN_FWD64C_QB
#define OSATTN_FWD64C_QB 1
#endif
#ifndef OSATTN_FWD64C_NBUF
#define OSATTN_FWD64C_NBUF 2
#endif
#ifndef OSATTN_FWD64C_BC
#define OSATTN_FWD64C_BC 128
#endif
#ifndef OSATTN_FWD64_QB
#define OSATTN_FWD64_QB 2
#endif
#ifndef OSATTN_FWD64_NBUF
#define OSATTN_FWD64_NBUF 2
#endif
#ifndef OSATTN_FWD64_BC
#define OSATTN_FWD64_BC 64
#endif

template <typename T, int D>
static hipError_t launch_fwd_d(const FwdArgs& a) {
  constexpr int NW = OSATTN_FWD_NW, QB = OSATTN_FWD_QB, NB = OSATTN_FWD_NBUF, BC = OSATTN_FWD_BC;
  if (a.kv_lo) return launch_fwd_t<T, D, NW, QB, NB, BC, false, true>(a);
  if constexpr (D == 64) {
    if (a.causal)
      return launch_fwd_t<T, D, OSATTN_FWD64C_NW, OSATTN_FWD64C_QB, OSATTN_FWD64C_NBUF,
                          OSATTN_FWD64C_BC, true, false>(a);
    // Workgroups of 512 rows (two 32-row blocks per wave) halve the LDS bytes per MFMA,
    // but a grid of them smaller than the chip leaves CUs idle (N = 1024 at B*H = 64:
    // 128 workgroups, 0.039 ms, against 0.029 ms with 256-row workgroups): below one
    // workgroup per CU, the 256-row tiles.
    constexpr int kRows64 = OSATTN_FWD64_NW * 32 * OSATTN_FWD64_QB;
    const long long wide = (long long)((a.N + kRows64 - 1) / kRows64) * a.B * a.H;
    if (wide < device_cus()) return launch_fwd_t<T, D, NW, QB, NB, BC, false, false>(a);
    return launch_fwd_t<T, D, OSATTN_FWD64_NW, OSATTN_FWD64_QB, OSATTN_FWD64_NBUF,
                        OSATTN_FWD64_BC, false, false>(a);
  } else {
    if (a.causal) return launch_fwd_t<T, D, NW, QB, NB, BC, true, false>(a);
    return launch_fwd_t<T, D, NW, QB, NB, BC, false, false>(a);
  }
}

hipError_t launch_fwd_mfma(const FwdArgs& a) {
  if (a.dtype == 2) return a.d == 64 ? launch_fwd_d<__bf16, 64>(a) : launch_fwd_d<__bf16, 128>(a);
  return a.d == 64 ? launch_fwd_d<_Float16, 64>(a) : launch_fwd_d<_Float16, 128>(a);
}

}  // namespace osattn
