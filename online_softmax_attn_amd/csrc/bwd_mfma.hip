// Backward pass of fused attention on bf16/fp16 MFMA (gfx950), plus the
// per-row preprocess shared with the float32 path.
//
// The backward rebuilds P tile by tile from the saved logsumexp instead of
// storing it (FlashAttention-2 page, "Recomputation in backward pass"), and uses
// the softmax Jacobian-vector product per row, dS = P * (dP - D) with
// D_i = sum_j P_ij dP_ij = rowsum(dO * O)_i (softmax-backward page,
// "Backpropagating Through Softmax").  Then dV = P^T dO, dK = scale * dS^T Q and
// dQ = scale * dS K.
//
// Kernels:
//  1. preprocess: D = rowsum(dO * O) and LSE * log2(e), float32, into the
//     caller's workspace.
//  2. dK/dV: one workgroup (4 waves, one per SIMD) owns 128 (d = 128) or 256
//     (d = 64) keys of one key/value head; each wave keeps its 32 or 64 keys of K
//     and V in registers next to the dK, dV accumulators, and loops over every
//     query head of its GQA group and every query tile that sees those keys
//     (single writer).  S = Q K^T and dP = dO V^T put one key per lane, so P and
//     dS feed dV^T += dO^T P and dK^T += Q^T dS straight from registers.  With 64
//     keys per wave each Q or dO operand read from LDS feeds two MFMAs.
//  3. dQ: one workgroup (8 waves, two per SIMD) owns 256 query rows and loops over
//     key tiles, recomputing S and dP transposed (one query row per lane, as in
//     the forward) and forming dQ^T += K^T dS^T.  No atomics.
//
// Query/dO tiles (dK/dV kernel) and K/V tiles (dQ kernel) go from memory straight
// into LDS (buffer_load ... lds; rows past N read as zero) in compile-time
// pipeline stages.  Each tile is read both row-wise (128-bit reads) and
// transposed (ds_read_b64_tr_b16); one 16-byte-granule XOR swizzle keeps both
// access patterns free of bank conflicts.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace osattn {

// Granule XOR for row `row` of a [rows][D] 16-bit tile in LDS.  Row-wise reads
// touch one logical granule in 16 consecutive rows; transposed reads touch 4
// consecutive rows x 4 consecutive granules.  Bits 2-3 of the XOR separate the 4
// rows of a transposed read into different 64-byte bank groups, bits 0-1 make the
// XOR distinct over 16 consecutive rows.
template <int D>
__device__ __forceinline__ int bwd_swz(int row) {
  return D == 128 ? (4 * (row & 3) + ((row >> 2) & 3)) : (4 * ((row >> 1) & 1) + ((row >> 2) & 3));
}

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O) and LSE * log2(e), float32.
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const E* __restrict__ O,
                                                             const E* __restrict__ dO,
                                                             const float* __restrict__ LSE,
                                                             float* __restrict__ Dv,
                                                             float* __restrict__ lse2,
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
  if (row < rows && (threadIdx.x % kTPR) == 0) {
    Dv[row] = acc;
    // A row that sees no key (interval masks) has LSE = -inf: store +inf so that
    // exp2(S*c - LSE*log2e) is 0 for it rather than inf.
    if (lse2) lse2[row] = LSE[row] == -INFINITY ? INFINITY : LSE[row] * kLog2e;
  }
}

// Per 64-row query tile of each batch, the interval summary the dK/dV kernel uses
// to pick and classify tiles: (min lo, max hi) over rows that see some key, and
// (max lo, min hi) over all rows (an empty row, or a row past Nq, counts as
// lo = Nk, hi = -1, which forces masking of any tile holding it).
__global__ __launch_bounds__(64) void mask_tiles_kernel(const int* __restrict__ kv_lo,
                                                        const int* __restrict__ kv_hi,
                                                        i32x4* __restrict__ tile_sum, int Nq,
                                                        int Nk, int n_qt) {
  const int t = blockIdx.x, b = blockIdx.y;
  const int row = t * 64 + (int)threadIdx.x;
  int lo = Nk, hi = -1;
  if (row < Nq) {
    lo = max(kv_lo[(size_t)b * Nq + row], 0);
    hi = min(kv_hi[(size_t)b * Nq + row], Nk - 1);
    if (lo > hi) {
      lo = Nk;
      hi = -1;
    }
  }
  int mn_lo = lo, mx_hi = hi, mx_lo = lo, mn_hi = hi;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    mn_lo = min(mn_lo, __shfl_xor(mn_lo, off));
    mx_hi = max(mx_hi, __shfl_xor(mx_hi, off));
    mx_lo = max(mx_lo, __shfl_xor(mx_lo, off));
    mn_hi = min(mn_hi, __shfl_xor(mn_hi, off));
  }
  if (threadIdx.x == 0) tile_sum[(size_t)b * n_qt + t] = i32x4{mn_lo, mx_hi, mx_lo, mn_hi};
}

// ---------------------------------------------------------------------------
// 2. dK / dV.
#ifndef OSATTN_DKDV_PIPE
#define OSATTN_DKDV_PIPE 1
#endif
// Interleave of the pipelined d = 128 tile (per phase: LDS reads and vector instructions
// placed before the first MFMA, then per MFMA).  Measured on the headline shape and the
// causal GQA workload against the earlier 24 / 16 / 2 / 7 and 0 / 2 / 8: three reads per
// MFMA and a shorter lead (8 reads, 8 vector instructions) took dK/dV 4% and 7% faster.
#ifndef OSATTN_IL1_DS0
#define OSATTN_IL1_DS0 8
#endif
#ifndef OSATTN_IL1_V0
#define OSATTN_IL1_V0 8
#endif
#ifndef OSATTN_IL1_DS
#define OSATTN_IL1_DS 3
#endif
#ifndef OSATTN_IL1_V
#define OSATTN_IL1_V 7
#endif
#ifndef OSATTN_IL2_V0
#define OSATTN_IL2_V0 0
#endif
#ifndef OSATTN_IL2_DS
#define OSATTN_IL2_DS 3
#endif
#ifndef OSATTN_IL2_V
#define OSATTN_IL2_V 8
#endif

template <int D, int NBUF>
struct DkdvCfg {
  static constexpr int kNW = 4;                 // waves (one per SIMD)
  // 32-key blocks per wave: two at d = 64; at d = 128 the K/V fragments and the
  // dK/dV accumulators of two blocks would not fit in one wave's registers.
  static constexpr int kKB = D == 64 ? 2 : 1;
  static constexpr int kKeys = kNW * 32 * kKB;  // keys per workgroup
  static constexpr int kQT = 64;                // query rows per staged tile
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileElems = kQT * D;
  static constexpr int kChunks = kQT * kRowBytes / 1024;
  static constexpr int kCPW = kChunks / kNW;
  static_assert(kCPW >= 1 && kChunks % kNW == 0, "tile must split evenly over the waves");
};

// Persistent grid (StaticSchedule) for the causal dK/dV, whose key tiles differ in
// length.
#ifndef OSATTN_DKDV_PERSIST
#define OSATTN_DKDV_PERSIST 1
#endif

// dK/dV kernel arguments.
struct DkdvKernelArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* dO;
  const float* LSE2;
  const float* Dv;
  uint16_t* dK;
  uint16_t* dV;
  int H, Hkv, Nq, n_ktiles;
  float scale, scale_log2;
  const int* kv_lo;
  const int* kv_hi;
  const i32x4* tile_sum;
  int Nk;          // keys (interval masks; otherwise equal to Nq)
  int n_jobs;  // logical tiles (key tiles x K/V heads)
  int pad_;
};

template <typename T, int D, int NBUF, bool CAUSAL, bool IMASK>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
__attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(const DkdvKernelArgs args) {
  constexpr bool PERSIST = OSATTN_DKDV_PERSIST && CAUSAL && !IMASK;
  using C = DkdvCfg<D, NBUF>;
  using M = Mfma<T>;
  using vec8 = typename M::vec8;
  constexpr int KB = C::kKB;
  static_assert(NBUF >= 2 && NBUF <= 4, "two to four stages");
  __shared__ __attribute__((aligned(1024))) uint16_t lq0[C::kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t ld0[C::kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lq1[C::kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t ld1[C::kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lq2[NBUF > 2 ? C::kTileElems : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t ld2[NBUF > 2 ? C::kTileElems : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lq3[NBUF > 3 ? C::kTileElems : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t ld3[NBUF > 3 ? C::kTileElems : 8];
  __shared__ __attribute__((aligned(256))) float ll0[C::kQT], lD0[C::kQT];
  __shared__ __attribute__((aligned(256))) float ll1[C::kQT], lD1[C::kQT];
  __shared__ __attribute__((aligned(256))) float ll2[C::kQT], lD2[C::kQT];
  __shared__ __attribute__((aligned(256))) float ll3[NBUF > 3 ? C::kQT : 4], lD3[NBUF > 3 ? C::kQT : 4];
  // Interval masks: each staged tile's row intervals, lo in [0, kQT), hi in [kQT, 2kQT),
  // then the tile's summary (min lo, max hi, max lo, min hi) at 2kQT (the DMA brings 64
  // words: the summaries of this tile and the next 15, or zeros past the last tile).
  constexpr int kLM = IMASK ? 2 * C::kQT + 64 : 4;
  __shared__ __attribute__((aligned(256))) int lm0[kLM], lm1[kLM], lm2[kLM], lm3[kLM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Logical tile L: key tile L % n_ktiles of K/V head L / n_ktiles (the key tiles of a
  // head longest first).  A persistent grid (causal) walks its schedule (see
  // StaticSchedule); otherwise each workgroup runs one tile.
  StaticSchedule sched(args.n_jobs, blockIdx.x, gridDim.x);
  int L;
  if constexpr (PERSIST) {
    L = sched.next();
  } else {
    // Interval masks: K/V-head groups dealt over the XCDs (see the forward).
    L = (OSATTN_XCD_GROUPS && IMASK) ? xcd_group_remap(blockIdx.x, gridDim.x, args.n_ktiles)
                                     : xcd_remap(blockIdx.x, gridDim.x);
  }
  while (L >= 0) {
    // Arguments read afresh for each tile of a persistent grid (see the forward).
    const DkdvKernelArgs a = PERSIST ? fresh_kernel_args<DkdvKernelArgs>() : args;
    const uint16_t* __restrict__ Q = a.Q;
    const uint16_t* __restrict__ K = a.K;
    const uint16_t* __restrict__ V = a.V;
    const uint16_t* __restrict__ dO = a.dO;
    const float* __restrict__ LSE2 = a.LSE2;
    const float* __restrict__ Dv = a.Dv;
    uint16_t* __restrict__ dK = a.dK;
    uint16_t* __restrict__ dV = a.dV;
    const int H = a.H, Hkv = a.Hkv, Nq = a.Nq, n_ktiles = a.n_ktiles;
    const float scale = a.scale, scale_log2 = a.scale_log2;
    const int* __restrict__ kv_lo = a.kv_lo;
    const int* __restrict__ kv_hi = a.kv_hi;
    const i32x4* __restrict__ tile_sum = a.tile_sum;
    // Keys and queries differ in number only under interval masks.
    const int Nk = IMASK ? a.Nk : Nq;
    const int kt = L % n_ktiles;
    const int bg = L / n_ktiles;  // b * Hkv + kvh
    const int kvh = bg % Hkv;
    const int b = bg / Hkv;
    const int n_rep = H / Hkv;
    const int k0 = kt * C::kKeys;
    const int kw = k0 + 32 * KB * wave;  // first key of this wave

    const uint32_t q_bytes = (uint32_t)Nq * C::kRowBytes;
    const uint32_t kv_bytes = (uint32_t)Nk * C::kRowBytes;
    const auto rk = make_rsrc(K + (size_t)bg * Nk * D, kv_bytes);
    const auto rv = make_rsrc(V + (size_t)bg * Nk * D, kv_bytes);

    // K and V rows of this wave (B operands of S = Q K^T and dP = dO V^T).
    vec8 kf[KB][D / 16], vf[KB][D / 16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint32_t rowoff = (uint32_t)(kw + 32 * kb + l32) * C::kRowBytes;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        kf[kb][c] = as_vec8<T>(buffer_load16(rk, rowoff + (16 * c + 8 * hi) * 2));
        vf[kb][c] = as_vec8<T>(buffer_load16(rv, rowoff + (16 * c + 8 * hi) * 2));
      }
    }

    f32x16 dk_acc[KB][D / 32], dv_acc[KB][D / 32];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dk_acc[kb][t][r] = 0.f;
          dv_acc[kb][t][r] = 0.f;
        }

    // Query tiles that see these keys: all of them, or (causal) from the diagonal on,
    // or (interval masks) the first through the last tile whose rows' intervals meet
    // this workgroup's keys, from the per-tile summaries (min lo, max hi, max lo, min hi).
    const int n_qt = (Nq + C::kQT - 1) / C::kQT;
    int qt_first = CAUSAL ? (k0 / C::kQT) : 0;
    int per_head = n_qt - qt_first;
    if constexpr (IMASK) {
      const int key_hi = min(Nk, k0 + C::kKeys) - 1;
      int f = n_qt, l = -1;
      for (int t = lane; t < n_qt; t += 64) {
        const i32x4 sm = load_global<i32x4>(tile_sum + (size_t)b * n_qt + t);
        if (sm[0] <= key_hi && sm[1] >= k0) {
          f = min(f, t);
          l = max(l, t);
        }
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        f = min(f, __shfl_xor(f, off));
        l = max(l, __shfl_xor(l, off));
      }
      // (Equal in every lane after the reduction; read from lane 0 so that the loop's
      // trip count and its wait choices are scalar.)
      qt_first = __builtin_amdgcn_readfirstlane(l >= 0 ? f : 0);
      per_head = __builtin_amdgcn_readfirstlane(l >= 0 ? l - f + 1 : 0);
    }
    const int n_iter = per_head * n_rep;

    // LDS-DMA offsets: chunk ch of a tile holds tile row off / kRowBytes, physical
    // granule pg, i.e. logical granule pg ^ swizzle(row).
    uint32_t goff[C::kCPW];
#pragma unroll
    for (int i = 0; i < C::kCPW; ++i) {
      const int off = (wave * C::kCPW + i) * 1024 + lane * 16;
      const int row = off / C::kRowBytes;
      const int pg = (off % C::kRowBytes) / 16;
      goff[i] = row * C::kRowBytes + ((pg ^ bwd_swz<D>(row)) * 16);
    }
    const uint32_t lane4 = (uint32_t)lane * 4;  // per-lane offset of the 4-byte row loads
    auto issue = [&](int it, uint16_t* lq, uint16_t* ld, float* ll, float* lD, int* lm)
        __attribute__((always_inline)) {
      const int r = it / per_head;
      const uint32_t i0 = (uint32_t)(qt_first + it % per_head) * C::kQT;
      const size_t bh = (size_t)b * H + kvh * n_rep + r;
      const auto rq = make_rsrc(Q + bh * Nq * D, q_bytes);
      const auto rd = make_rsrc(dO + bh * Nq * D, q_bytes);
#pragma unroll
      for (int i = 0; i < C::kCPW; ++i) {
        const int ch = wave * C::kCPW + i;
        buffer_load16_lds(rq, lq + ch * 512, goff[i], i0 * C::kRowBytes);
        buffer_load16_lds(rd, ld + ch * 512, goff[i], i0 * C::kRowBytes);
      }
      if (wave == 0) {  // 64 rows x 4 bytes of LSE*log2(e) and D; rows >= Nq read zero
        const auto rl = make_rsrc(LSE2 + bh * Nq, (uint32_t)Nq * 4);
        const auto rD = make_rsrc(Dv + bh * Nq, (uint32_t)Nq * 4);
        buffer_load4_lds(rl, ll, lane4, i0 * 4);
        buffer_load4_lds(rD, lD, lane4, i0 * 4);
        if constexpr (IMASK) {  // and the rows' key intervals
          const auto rlo = make_rsrc(kv_lo + (size_t)b * Nq, (uint32_t)Nq * 4);
          const auto rhi = make_rsrc(kv_hi + (size_t)b * Nq, (uint32_t)Nq * 4);
          buffer_load4_lds(rlo, lm, lane4, i0 * 4);
          buffer_load4_lds(rhi, lm + C::kQT, lane4, i0 * 4);
          // The tile's summary comes through LDS too: read from global memory in the
          // loop, it would need a vmcnt wait that also drains the prefetches in flight.
          // (The tile offset goes into the per-lane offset, which the buffer's range check
          // always covers: lanes past the last summary read zero.)
          const auto rs = make_rsrc(tile_sum + (size_t)b * n_qt, (uint32_t)n_qt * 16);
          buffer_load4_lds(rs, lm + 2 * C::kQT, lane4 + (i0 / C::kQT) * 16, 0);
        }
      }
    };
    // Outstanding loads per staged tile: 2 * kCPW per wave, and wave 0 also loads LSE
    // and D (and the two interval arrays and the tile summary).
    constexpr int kW0 = IMASK ? 5 : 2;

    // LDS read offsets (bytes in a tile), loop-invariant per lane.
    //  row-wise (A operand of S and dP): row 32qb + l32, logical granule 2c + hi
    uint32_t roff[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) roff[c] = l32 * C::kRowBytes + (((2 * c + hi) ^ bwd_swz<D>(l32)) * 16);
    //  transposed (A operands of dV^T and dK^T): rows 16cq + tr_row (+8), columns
    //  32t + tr_col .. +3 (see common.h for the lane pattern of the transpose read)
    const int tr_row = 4 * hi + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    //  The upper half (rows +8) has swizzle bwd_swz(row) ^ 2: granule bit 1, i.e. byte
    //  bit 5 of the in-row offset, flips.
    uint32_t toff[D / 32], toff8[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const int col = 32 * t + tr_col;
      toff[t] = tr_row * C::kRowBytes + (((col >> 3) ^ bwd_swz<D>(tr_row)) * 16) + (col & 7) * 2;
      toff8[t] = (tr_row + 8) * C::kRowBytes + (((col >> 3) ^ bwd_swz<D>(tr_row + 8)) * 16) + (col & 7) * 2;
    }

    // One staged tile of 64 query rows = two 32-row blocks.  The scores and dP of
    // both blocks are issued first; the softmax-JVP arithmetic of block 0 then
    // overlaps the MFMAs of block 1 and the dV/dK MFMAs of block 0 overlap the
    // arithmetic of block 1.  Everything is one basic block (masking is a
    // compile-time variant chosen per tile) so the scheduler can interleave.
    // Variant for 32 keys per wave: one staged tile of 64 query rows, processed as
    // two 32-row blocks.  For each block every LDS operand is requested before the
    // instructions that consume it, with scheduling fences in between, so that LDS
    // latency overlaps other work of the same wave (one wave per SIMD has nothing
    // else to hide it):
    //   row-wise Q/dO reads + LSE/D   | S, dP MFMAs
    //   transposed Q/dO reads         | softmax-JVP arithmetic
    //                                 | dV, dK MFMAs
    auto compute_tile_fenced = [&](auto mask_c, int i0, const char* qb_, const char* db_, const float* ll,
                            const float* lD, const int* lm) __attribute__((always_inline)) {
      constexpr int MM = decltype(mask_c)::value;  // 0 none, 1 causal, 2 intervals
#pragma unroll
      for (int qb = 0; qb < C::kQT / 32; ++qb) {
        // -- operand requests for S and dP
        u32x4 aq[D / 16], ad[D / 16];
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          aq[c] = *(const u32x4*)(qb_ + 32 * qb * C::kRowBytes + roff[c]);
          ad[c] = *(const u32x4*)(db_ + 32 * qb * C::kRowBytes + roff[c]);
        }
        f32x4 lse4[4], d4[4];  // rows 32qb + 8g + 4hi + 0..3 for register group g
        i32x4 lo4[4], hi4[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          lse4[g] = *(const f32x4*)&ll[32 * qb + 8 * g + 4 * hi];
          d4[g] = *(const f32x4*)&lD[32 * qb + 8 * g + 4 * hi];
          if constexpr (MM == 2) {
            lo4[g] = *(const i32x4*)&lm[32 * qb + 8 * g + 4 * hi];
            hi4[g] = *(const i32x4*)&lm[C::kQT + 32 * qb + 8 * g + 4 * hi];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // -- S = Q K^T, dP = dO V^T (lane = key, register r = query row 8(r/4)+4hi+r%4)
        f32x16 s[KB], dp[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[kb][r] = 0.f;
            dp[kb][r] = 0.f;
          }
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            s[kb] = M::mma32(as_vec8<T>(aq[c]), kf[kb][c], s[kb]);
            dp[kb] = M::mma32(as_vec8<T>(ad[c]), vf[kb][c], dp[kb]);
          }
        // -- operand requests for dV^T and dK^T (transposed reads of the same tiles)
        vec8 adt[2][D / 32], aqt[2][D / 32];
#pragma unroll
        for (int cq = 0; cq < 2; ++cq) {
          const int rowb = (32 * qb + 16 * cq) * C::kRowBytes;
#pragma unroll
          for (int t = 0; t < D / 32; ++t) {
            adt[cq][t] = join8<T>(lds_read_tr4(db_ + rowb + toff[t]), lds_read_tr4(db_ + rowb + toff8[t]));
            aqt[cq][t] = join8<T>(lds_read_tr4(qb_ + rowb + toff[t]), lds_read_tr4(qb_ + rowb + toff8[t]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // -- P = exp2(S*c - LSE*log2e) (0 where masked), dS = P * (dP - D)
        vec8 pp[2][KB], ps[2][KB];
#pragma unroll
        for (int cq = 0; cq < 2; ++cq)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const int key = kw + 32 * kb + l32;
            float p8[8], d8[8];
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2) {
              const int g = 2 * cq + g2;
              const int ql = 32 * qb + 8 * g + 4 * hi;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                float pv = fast_exp2(fmaf(s[kb][r], scale_log2, -lse4[g][e]));
                if constexpr (MM == 1) {
                  if (key > i0 + ql + e) pv = 0.f;
                } else if constexpr (MM == 2) {
                  if (key < lo4[g][e] || key > hi4[g][e]) pv = 0.f;
                }
                p8[4 * g2 + e] = pv;
                d8[4 * g2 + e] = pv * (dp[kb][r] - d4[g][e]);
              }
            }
            pp[cq][kb] = pack8<T>(p8);
            ps[cq][kb] = pack8<T>(d8);
          }
        // -- dV^T += dO^T P ; dK^T += Q^T dS  (reduction over the 32 query rows)
#pragma unroll
        for (int cq = 0; cq < 2; ++cq)
#pragma unroll
          for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              dv_acc[kb][t] = M::mma32(adt[cq][t], pp[cq][kb], dv_acc[kb][t]);
              dk_acc[kb][t] = M::mma32(aqt[cq][t], ps[cq][kb], dk_acc[kb][t]);
            }
      }
    };
    auto compute_tile_wide = [&](auto mask_c, int i0, const char* qb_, const char* db_, const float* ll,
                            const float* lD, const int* lm) __attribute__((always_inline)) {
      constexpr int MM = decltype(mask_c)::value;  // 0 none, 1 causal, 2 intervals
      constexpr int NQB = C::kQT / 32;
      // S = Q K^T, dP = dO V^T (lane = key, register r = query row 8(r/4)+4hi+r%4)
      f32x16 s[NQB][KB], dp[NQB][KB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[qb][kb][r] = 0.f;
            dp[qb][kb][r] = 0.f;
          }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          const u32x4 aq = *(const u32x4*)(qb_ + 32 * qb * C::kRowBytes + roff[c]);
          const u32x4 ad = *(const u32x4*)(db_ + 32 * qb * C::kRowBytes + roff[c]);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            s[qb][kb] = M::mma32(as_vec8<T>(aq), kf[kb][c], s[qb][kb]);
            dp[qb][kb] = M::mma32(as_vec8<T>(ad), vf[kb][c], dp[qb][kb]);
          }
        }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        // P = exp2(S*c - LSE*log2e) (0 where masked), dS = P * (dP - D)
#pragma unroll
        for (int cq = 0; cq < 2; ++cq) {
          vec8 pp[KB], ps[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const int key = kw + 32 * kb + l32;
            float p8[8], d8[8];
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2) {
              const int ql = 32 * qb + 16 * cq + 8 * g2 + 4 * hi;  // local row of register 8cq+4g2
              const f32x4 lse4 = *(const f32x4*)&ll[ql];
              const f32x4 d4 = *(const f32x4*)&lD[ql];
              i32x4 lo4 = {}, hi4 = {};
              if constexpr (MM == 2) {
                lo4 = *(const i32x4*)&lm[ql];
                hi4 = *(const i32x4*)&lm[C::kQT + ql];
              }
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 8 * cq + 4 * g2 + e;
                float pv = fast_exp2(fmaf(s[qb][kb][r], scale_log2, -lse4[e]));
                if constexpr (MM == 1) {
                  if (key > i0 + ql + e) pv = 0.f;
                } else if constexpr (MM == 2) {
                  if (key < lo4[e] || key > hi4[e]) pv = 0.f;
                }
                p8[4 * g2 + e] = pv;
                d8[4 * g2 + e] = pv * (dp[qb][kb][r] - d4[e]);
              }
            }
            pp[kb] = pack8<T>(p8);
            ps[kb] = pack8<T>(d8);
          }
          // dV^T += dO^T P ; dK^T += Q^T dS  (reduction over these 16 query rows)
          const int rowb = (32 * qb + 16 * cq) * C::kRowBytes;
#pragma unroll
          for (int t = 0; t < D / 32; ++t) {
            const vec8 adt = join8<T>(lds_read_tr4(db_ + rowb + toff[t]), lds_read_tr4(db_ + rowb + toff8[t]));
            const vec8 aqt = join8<T>(lds_read_tr4(qb_ + rowb + toff[t]), lds_read_tr4(qb_ + rowb + toff8[t]));
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              dv_acc[kb][t] = M::mma32(adt, pp[kb], dv_acc[kb][t]);
              dk_acc[kb][t] = M::mma32(aqt, ps[kb], dk_acc[kb][t]);
            }
          }
        }
      }
    };
    // Software-pipelined variant for 32 keys per wave.  Per 32-row block qb the work
    // is G1 (S and dP: 16 MFMAs), J (the softmax-JVP arithmetic: about 130 VALU
    // instructions) and G2 (dV and dK: 16 MFMAs).  With one wave per SIMD nothing
    // else hides J, so the tile runs
    //   G1(0) | G1(1) with J(0) | G2(0) with J(1) | G2(1)
    // and scheduling groups interleave the VALU work between the MFMAs of the same
    // phase (MFMA and VALU of one wave overlap when they are independent).
    struct RowOps {
      u32x4 aq[D / 16], ad[D / 16];
      f32x4 lse4[4], d4[4];  // rows 32qb + 8g + 4hi + 0..3 for register group g
    };
    struct TrOps {
      vec8 adt[2][D / 32], aqt[2][D / 32];
    };
    auto read_rows = [&](RowOps& o, int qb, const char* qb_, const char* db_, const float* ll,
                         const float* lD) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        o.aq[c] = *(const u32x4*)(qb_ + 32 * qb * C::kRowBytes + roff[c]);
        o.ad[c] = *(const u32x4*)(db_ + 32 * qb * C::kRowBytes + roff[c]);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        o.lse4[g] = *(const f32x4*)&ll[32 * qb + 8 * g + 4 * hi];
        o.d4[g] = *(const f32x4*)&lD[32 * qb + 8 * g + 4 * hi];
      }
    };
    auto read_tr = [&](TrOps& o, int qb, const char* qb_, const char* db_)
        __attribute__((always_inline)) {
#pragma unroll
      for (int cq = 0; cq < 2; ++cq) {
        const int rowb = (32 * qb + 16 * cq) * C::kRowBytes;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          o.adt[cq][t] = join8<T>(lds_read_tr4(db_ + rowb + toff[t]), lds_read_tr4(db_ + rowb + toff8[t]));
          o.aqt[cq][t] = join8<T>(lds_read_tr4(qb_ + rowb + toff[t]), lds_read_tr4(qb_ + rowb + toff8[t]));
        }
      }
    };
    auto g1 = [&](const RowOps& o, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        s = M::mma32(as_vec8<T>(o.aq[c]), kf[0][c], s);
        dp = M::mma32(as_vec8<T>(o.ad[c]), vf[0][c], dp);
      }
    };
    auto jvp = [&](auto mask_c, int i0, int qb, const RowOps& o, const f32x16& s, const f32x16& dp,
                   vec8 (&pp)[2], vec8 (&ps)[2], const int* lm) __attribute__((always_inline)) {
      constexpr int MM = decltype(mask_c)::value;  // 0 none, 1 causal, 2 intervals
      const int key = kw + l32;
#pragma unroll
      for (int cq = 0; cq < 2; ++cq) {
        float p8[8], d8[8];
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const int g = 2 * cq + g2;
          const int ql = 32 * qb + 8 * g + 4 * hi;
          i32x4 lo4 = {}, hi4 = {};  // the rows' key intervals (interval masks only)
          if constexpr (MM == 2) {
            lo4 = *(const i32x4*)&lm[ql];
            hi4 = *(const i32x4*)&lm[C::kQT + ql];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float pv = fast_exp2(fmaf(s[r], scale_log2, -o.lse4[g][e]));
            if constexpr (MM == 1) {
              if (key > i0 + ql + e) pv = 0.f;
            } else if constexpr (MM == 2) {
              if (key < lo4[e] || key > hi4[e]) pv = 0.f;
            }
            p8[4 * g2 + e] = pv;
            d8[4 * g2 + e] = pv * (dp[r] - o.d4[g][e]);
          }
        }
        pp[cq] = pack8<T>(p8);
        ps[cq] = pack8<T>(d8);
      }
    };
    auto g2 = [&](const TrOps& o, const vec8 (&pp)[2], const vec8 (&ps)[2])
        __attribute__((always_inline)) {
#pragma unroll
      for (int cq = 0; cq < 2; ++cq)
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          dv_acc[0][t] = M::mma32(o.adt[cq][t], pp[cq], dv_acc[0][t]);
          dk_acc[0][t] = M::mma32(o.aqt[cq][t], ps[cq], dk_acc[0][t]);
        }
    };
    // One phase's interleave: n_ds LDS reads and n_v0 VALU first (to cover the first
    // MFMA's operand latency), then 16 times one MFMA, ds_per LDS reads, v_per VALU.
    auto interleave16 = [&](auto n_ds_c, auto n_v0_c, auto ds_per_c, auto v_per_c)
        __attribute__((always_inline)) {
      constexpr int kVALU = 0x2 | 0x400;  // VALU including transcendental
      __builtin_amdgcn_sched_group_barrier(0x100, decltype(n_ds_c)::value, 0);
      __builtin_amdgcn_sched_group_barrier(kVALU, decltype(n_v0_c)::value, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, decltype(ds_per_c)::value, 0);
        __builtin_amdgcn_sched_group_barrier(kVALU, decltype(v_per_c)::value, 0);
      }
    };
    auto compute_tile_pipe = [&](auto mask_c, int i0, const char* qb_, const char* db_,
                                 const float* ll, const float* lD, const int* lm)
        __attribute__((always_inline)) {
      using IC0 = std::integral_constant<int, 0>;
      RowOps r0, r1;
      TrOps t0, t1;
      f32x16 s0, dp0, s1, dp1;
      vec8 pp0[2], ps0[2], pp1[2], ps1[2];
      // G1(0)
      read_rows(r0, 0, qb_, db_, ll, lD);
      g1(r0, s0, dp0);
      __builtin_amdgcn_sched_barrier(0);
      // G1(1) with J(0); block 0's transposed operands are requested here too
      read_rows(r1, 1, qb_, db_, ll, lD);
      read_tr(t0, 0, qb_, db_);
      jvp(mask_c, i0, 0, r0, s0, dp0, pp0, ps0, lm);
      g1(r1, s1, dp1);
      interleave16(std::integral_constant<int, OSATTN_IL1_DS0>{}, std::integral_constant<int, OSATTN_IL1_V0>{},
                   std::integral_constant<int, OSATTN_IL1_DS>{}, std::integral_constant<int, OSATTN_IL1_V>{});
      __builtin_amdgcn_sched_barrier(0);
      // G2(0) with J(1); block 1's transposed operands
      read_tr(t1, 1, qb_, db_);
      jvp(mask_c, i0, 1, r1, s1, dp1, pp1, ps1, lm);
      g2(t0, pp0, ps0);
      interleave16(std::integral_constant<int, 0>{}, std::integral_constant<int, OSATTN_IL2_V0>{},
                   std::integral_constant<int, OSATTN_IL2_DS>{}, std::integral_constant<int, OSATTN_IL2_V>{});
      __builtin_amdgcn_sched_barrier(0);
      // G2(1)
      g2(t1, pp1, ps1);
      (void)IC0{};
    };
    auto compute_tile = [&](auto mask_c, int i0, const char* qb_, const char* db_, const float* ll,
                            const float* lD, const int* lm) __attribute__((always_inline)) {
      if constexpr (KB == 1) {
        if constexpr (OSATTN_DKDV_PIPE) compute_tile_pipe(mask_c, i0, qb_, db_, ll, lD, lm);
        else compute_tile_fenced(mask_c, i0, qb_, db_, ll, lD, lm);
      } else {
        compute_tile_wide(mask_c, i0, qb_, db_, ll, lD, lm);
      }
    };
    using M0 = std::integral_constant<int, 0>;
    using M1 = std::integral_constant<int, 1>;
    using M2 = std::integral_constant<int, 2>;
    auto compute = [&](int it, const char* qb_, const char* db_, const float* ll, const float* lD,
                       const int* lm) __attribute__((always_inline)) {
      const int tq = qt_first + it % per_head;
      const int i0 = tq * C::kQT;
      if constexpr (IMASK) {
        // Skip the tile if no row's interval meets this wave's keys; mask it unless every
        // row sees all of them.
        const i32x4 smv = *(const i32x4*)(lm + 2 * C::kQT);
        const int sm[4] = {__builtin_amdgcn_readfirstlane(smv[0]), __builtin_amdgcn_readfirstlane(smv[1]),
                           __builtin_amdgcn_readfirstlane(smv[2]), __builtin_amdgcn_readfirstlane(smv[3])};
        const int kw_last = kw + 32 * KB - 1;
        if (sm[0] > kw_last || sm[1] < kw) return;
        if (sm[2] <= kw && sm[3] >= kw_last) compute_tile(M0{}, i0, qb_, db_, ll, lD, lm);
        else compute_tile(M2{}, i0, qb_, db_, ll, lD, lm);
        return;
      }
      if (CAUSAL && i0 + C::kQT - 1 < kw) return;  // every key of this wave is after every row
      // Causal: only tiles whose first row precedes this wave's last key need the mask.
      if (CAUSAL && i0 < kw + 32 * KB - 1)
        compute_tile(M1{}, i0, qb_, db_, ll, lD, lm);
      else
        compute_tile(M0{}, i0, qb_, db_, ll, lD, lm);
    };

    auto stage = [&](auto sc, auto fn) __attribute__((always_inline)) {
      constexpr int S = decltype(sc)::value;
      // The interval arrays only exist for interval masks (elsewhere they must not be
      // referenced at all, or the compiler stops telling the stages' LDS apart).
      int* const m0 = IMASK ? lm0 : nullptr;
      int* const m1 = IMASK ? lm1 : nullptr;
      int* const m2 = IMASK ? lm2 : nullptr;
      int* const m3 = IMASK ? lm3 : nullptr;
      if constexpr (S == 0) fn(lq0, ld0, ll0, lD0, m0);
      else if constexpr (S == 1) fn(lq1, ld1, ll1, lD1, m1);
      else if constexpr (S == 2) fn(lq2, ld2, ll2, lD2, m2);
      else fn(lq3, ld3, ll3, lD3, m3);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (0 < n_iter)
      stage(I0{}, [&](uint16_t* a, uint16_t* d, float* l, float* dd, int* mm) { issue(0, a, d, l, dd, mm); });
    if (NBUF > 2 && 1 < n_iter)
      stage(I1{}, [&](uint16_t* a, uint16_t* d, float* l, float* dd, int* mm) { issue(1, a, d, l, dd, mm); });
    if (NBUF > 3 && 2 < n_iter)
      stage(I2{}, [&](uint16_t* a, uint16_t* d, float* l, float* dd, int* mm) { issue(2, a, d, l, dd, mm); });

    auto step = [&](auto sc, int it) __attribute__((always_inline)) {
      constexpr int S = decltype(sc)::value;
      constexpr int SN = (S + NBUF - 1) % NBUF;  // receives tile it + NBUF - 1
      // Tile `it` has landed once at most the loads of the tiles issued after it
      // (up to NBUF - 2 of them) are outstanding.
      constexpr int kPer = 2 * C::kCPW;  // loads per tile and wave (+kW0 on wave 0)
      const int ahead = min(NBUF - 2, n_iter - 1 - it);
      if (NBUF > 3 && ahead >= 2) {
        if (wave == 0) wait_vmcnt<2 * (kPer + kW0)>();
        else wait_vmcnt<2 * kPer>();
      } else if (NBUF > 2 && ahead >= 1) {
        if (wave == 0) wait_vmcnt<kPer + kW0>();
        else wait_vmcnt<kPer>();
      } else {
        wait_vmcnt<0>();
      }
      block_barrier();
      if (it + NBUF - 1 < n_iter)
        stage(std::integral_constant<int, SN>{},
              [&](uint16_t* a, uint16_t* d, float* l, float* dd, int* mm) {
                issue(it + NBUF - 1, a, d, l, dd, mm);
              });
      stage(sc, [&](uint16_t* a, uint16_t* d, float* l, float* dd, int* mm) {
        compute(it, (const char*)a, (const char*)d, l, dd, mm);
      });
    };
    for (int it = 0; it < n_iter; it += NBUF) {
      step(I0{}, it);
      if (it + 1 < n_iter) step(I1{}, it + 1);
      if constexpr (NBUF > 2)
        if (it + 2 < n_iter) step(I2{}, it + 2);
      if constexpr (NBUF > 3)
        if (it + 3 < n_iter) step(std::integral_constant<int, 3>{}, it + 3);
    }

    // Store: lane = key, register r of tile t = column 32t + 8(r/4) + 4hi + r%4.
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int key = kw + 32 * kb + l32;
      if (key < Nk) {
        uint16_t* dkp = dK + ((size_t)bg * Nk + key) * D;
        uint16_t* dvp = dV + ((size_t)bg * Nk + key) * D;
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u32x2 wk, wv;
            wk[0] = (uint32_t)to_bits<T>(dk_acc[kb][t][4 * g + 0] * scale) |
                    ((uint32_t)to_bits<T>(dk_acc[kb][t][4 * g + 1] * scale) << 16);
            wk[1] = (uint32_t)to_bits<T>(dk_acc[kb][t][4 * g + 2] * scale) |
                    ((uint32_t)to_bits<T>(dk_acc[kb][t][4 * g + 3] * scale) << 16);
            wv[0] = (uint32_t)to_bits<T>(dv_acc[kb][t][4 * g + 0]) |
                    ((uint32_t)to_bits<T>(dv_acc[kb][t][4 * g + 1]) << 16);
            wv[1] = (uint32_t)to_bits<T>(dv_acc[kb][t][4 * g + 2]) |
                    ((uint32_t)to_bits<T>(dv_acc[kb][t][4 * g + 3]) << 16);
            store_global(dkp + 32 * t + 8 * g + 4 * hi, wk);
            store_global(dvp + 32 * t + 8 * g + 4 * hi, wv);
          }
      }
    }
    if constexpr (!PERSIST) break;
    __syncthreads();  // every wave is done with the staged tiles
    L = sched.next();
  }
}

// ---------------------------------------------------------------------------
// 3. dQ.
#ifndef OSATTN_DQ_BC
#define OSATTN_DQ_BC 64
#endif

template <int D, int NBUF, int QB>
struct DqCfg {
  static constexpr int kNW = 8;              // waves (two per SIMD)
  static constexpr int kRows = kNW * 32 * QB;  // query rows per workgroup (QB 32-row blocks per wave)
  static constexpr int kBC = OSATTN_DQ_BC;   // keys per staged tile
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileElems = kBC * D;
  static constexpr int kChunks = kBC * kRowBytes / 1024;
  static constexpr int kCPW = kChunks / kNW;
  static_assert(kCPW >= 1 && kChunks % kNW == 0, "tile must split evenly over the waves");
};

template <typename T, int D, int NBUF, int QB, bool CAUSAL, bool IMASK>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512)))
__attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                   const float* __restrict__ LSE2, const float* __restrict__ Dv,
                   uint16_t* __restrict__ dQ, int H, int Hkv, int Nq, int n_qtiles,
                   float scale, float scale_log2, const int* __restrict__ kv_lo,
                   const int* __restrict__ kv_hi, int Nk_arg) {
  const int Nk = IMASK ? Nk_arg : Nq;  // keys differ from queries only under interval masks
  using C = DqCfg<D, NBUF, QB>;
  using M = Mfma<T>;
  using vec8 = typename M::vec8;
  static_assert(NBUF >= 2 && NBUF <= 4, "two to four stages");
  __shared__ __attribute__((aligned(1024))) uint16_t lk0[C::kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lv0[C::kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lk1[C::kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lv1[C::kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lk2[NBUF > 2 ? C::kTileElems : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lv2[NBUF > 2 ? C::kTileElems : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lk3[NBUF > 3 ? C::kTileElems : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lv3[NBUF > 3 ? C::kTileElems : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int L = (OSATTN_XCD_GROUPS && IMASK)
                    ? xcd_group_remap(blockIdx.x, gridDim.x, n_qtiles * (H / Hkv))
                    : xcd_remap(blockIdx.x, gridDim.x);
  int qt = L % n_qtiles;
  const int bh = L / n_qtiles;
  // Longest rows first (causal, and the usual interval masks: see the forward).
  if (CAUSAL || (OSATTN_MASK_LONGEST_FIRST && IMASK)) qt = n_qtiles - 1 - qt;
  const int h = bh % H;
  const int b = bh / H;
  const int kvh = h / (H / Hkv);
  const int q0 = qt * C::kRows;
  const int wrow0 = q0 + 32 * QB * wave;  // the wave's rows: QB blocks of 32 from here

  const uint32_t q_bytes = (uint32_t)Nq * C::kRowBytes;
  const uint32_t kv_bytes = (uint32_t)Nk * C::kRowBytes;
  const auto rq = make_rsrc(Q + (size_t)bh * Nq * D, q_bytes);
  const auto rdo = make_rsrc(dO + (size_t)bh * Nq * D, q_bytes);
  const auto rk = make_rsrc(K + (size_t)(b * Hkv + kvh) * Nk * D, kv_bytes);
  const auto rv = make_rsrc(V + (size_t)(b * Hkv + kvh) * Nk * D, kv_bytes);

  // Q and dO rows of this lane, one per row block (B operands of S^T = K Q^T and
  // dP^T = V dO^T), with their LSE*log2(e) and D.
  vec8 qf[QB][D / 16], df[QB][D / 16];
  float lse2[QB], drow[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + 32 * qb + l32;
    const uint32_t rowoff = (uint32_t)row * C::kRowBytes;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      qf[qb][c] = as_vec8<T>(buffer_load16(rq, rowoff + (16 * c + 8 * hi) * 2));
      df[qb][c] = as_vec8<T>(buffer_load16(rdo, rowoff + (16 * c + 8 * hi) * 2));
    }
    lse2[qb] = row < Nq ? LSE2[(size_t)bh * Nq + row] : 0.f;
    drow[qb] = row < Nq ? Dv[(size_t)bh * Nq + row] : 0.f;
  }

  f32x16 acc[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][t][r] = 0.f;

  int kt0 = 0;  // first key tile of the loop
  int n_kt = (Nk + C::kBC - 1) / C::kBC;
  if (CAUSAL) n_kt = min(n_kt, (q0 + C::kRows + C::kBC - 1) / C::kBC);

  // Interval masks (as in the forward): each row's keys lo .. hi (empty: lo = Nk,
  // hi = -1), the wave's union and intersection of its rows' intervals, and the
  // workgroup's tile range.
  int lo_r[QB], hi_r[QB];
  int w_lo = 0, w_hi = 0, w_maxlo = 0, w_minhi = 0;
  if constexpr (IMASK) {
    __shared__ int wg_bounds[2 * C::kNW];
    w_lo = w_maxlo = Nk;
    w_hi = w_minhi = -1;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = wrow0 + 32 * qb + l32;
      int lo = Nk, hi = -1;
      if (row < Nq) {
        lo = max(kv_lo[(size_t)b * Nq + row], 0);
        hi = min(kv_hi[(size_t)b * Nq + row], Nk - 1);
        if (lo > hi) {
          lo = Nk;
          hi = -1;
        }
      }
      lo_r[qb] = lo;
      hi_r[qb] = hi;
      w_lo = min(w_lo, lo);
      w_hi = max(w_hi, hi);
      w_maxlo = qb == 0 ? lo : max(w_maxlo, lo);
      w_minhi = qb == 0 ? hi : min(w_minhi, hi);
    }
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      w_lo = min(w_lo, __shfl_xor(w_lo, off));
      w_hi = max(w_hi, __shfl_xor(w_hi, off));
      w_maxlo = max(w_maxlo, __shfl_xor(w_maxlo, off));
      w_minhi = min(w_minhi, __shfl_xor(w_minhi, off));
    }
    // Both half-waves hold the same rows, so every lane now has the wave's values;
    // read them from lane 0 so that the per-tile tests are scalar branches.
    w_lo = __builtin_amdgcn_readfirstlane(w_lo);
    w_hi = __builtin_amdgcn_readfirstlane(w_hi);
    w_maxlo = __builtin_amdgcn_readfirstlane(w_maxlo);
    w_minhi = __builtin_amdgcn_readfirstlane(w_minhi);
    if (lane == 0) {
      wg_bounds[2 * wave] = w_lo;
      wg_bounds[2 * wave + 1] = w_hi;
    }
    __syncthreads();
    int g_lo = Nk, g_hi = -1;
#pragma unroll
    for (int w = 0; w < C::kNW; ++w) {
      g_lo = min(g_lo, wg_bounds[2 * w]);
      g_hi = max(g_hi, wg_bounds[2 * w + 1]);
    }
    kt0 = __builtin_amdgcn_readfirstlane(g_hi >= g_lo ? g_lo / C::kBC : 0);
    n_kt = __builtin_amdgcn_readfirstlane(g_hi >= g_lo ? g_hi / C::kBC + 1 - kt0 : 0);
  }

  uint32_t goff[C::kCPW];
#pragma unroll
  for (int i = 0; i < C::kCPW; ++i) {
    const int off = (wave * C::kCPW + i) * 1024 + lane * 16;
    const int r = off / C::kRowBytes;
    const int pg = (off % C::kRowBytes) / 16;
    goff[i] = r * C::kRowBytes + ((pg ^ bwd_swz<D>(r)) * 16);
  }
  auto issue = [&](int kt, uint16_t* lk, uint16_t* lv) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(kt0 + kt) * C::kBC * C::kRowBytes;
#pragma unroll
    for (int i = 0; i < C::kCPW; ++i) {
      const int ch = wave * C::kCPW + i;
      buffer_load16_lds(rk, lk + ch * 512, base + goff[i]);
      buffer_load16_lds(rv, lv + ch * 512, base + goff[i]);
    }
  };

  uint32_t roff[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) roff[c] = l32 * C::kRowBytes + (((2 * c + hi) ^ bwd_swz<D>(l32)) * 16);
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  //  The upper half (rows +8) has swizzle bwd_swz(row) ^ 2: granule bit 1, i.e. byte
  //  bit 5 of the in-row offset, flips.
  uint32_t toff[D / 32], toff8[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    const int col = 32 * t + tr_col;
    toff[t] = tr_row * C::kRowBytes + (((col >> 3) ^ bwd_swz<D>(tr_row)) * 16) + (col & 7) * 2;
    toff8[t] = (tr_row + 8) * C::kRowBytes + (((col >> 3) ^ bwd_swz<D>(tr_row + 8)) * 16) + (col & 7) * 2;
  }

  auto compute = [&](int kt, const char* kbase, const char* vbase) __attribute__((always_inline)) {
    const int k0 = (kt0 + kt) * C::kBC;
    if (CAUSAL && k0 > wrow0 + 32 * QB - 1) return;  // every key of the tile is after every row
    if (IMASK && (k0 > w_hi || k0 + C::kBC - 1 < w_lo)) return;  // no row of the wave sees it
    const bool need_mask = (k0 + C::kBC > Nk) || (CAUSAL && k0 + C::kBC - 1 > wrow0) ||
                           (IMASK && !(k0 >= w_maxlo && k0 + C::kBC - 1 <= w_minhi));
#pragma unroll
    for (int kb = 0; kb < C::kBC / 32; ++kb) {
      // S^T = K Q^T, dP^T = V dO^T (lane = query row, register = key); each K and V
      // operand read from LDS serves every row block.
      f32x16 s[QB], dp[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[qb][r] = 0.f;
          dp[qb][r] = 0.f;
        }
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const u32x4 ak = *(const u32x4*)(kbase + kb * 32 * C::kRowBytes + roff[c]);
        const u32x4 av = *(const u32x4*)(vbase + kb * 32 * C::kRowBytes + roff[c]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          s[qb] = M::mma32(as_vec8<T>(ak), qf[qb][c], s[qb]);
          dp[qb] = M::mma32(as_vec8<T>(av), df[qb][c], dp[qb]);
        }
      }
      // Masked scores become -inf (P = 0, so dS = 0) in a branch of their own: folded
      // into the loop below, the compiler would evaluate the key tests as selects on
      // every tile, needed or not.
      if (need_mask) {
        asm volatile("");  // keep this a branch
        // Key of element r: base + ko with ko a compile-time constant; the limits are
        // taken relative to base once per block.
        const int base = k0 + kb * 32 + 4 * hi;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int lim_hi = IMASK ? min(hi_r[qb] - base, Nk - 1 - base) : Nk - 1 - base;
          const int lim_lo = IMASK ? lo_r[qb] - base : 0;
          const int lim_c = wrow0 + 32 * qb + l32 - base;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = 8 * (r >> 2) + (r & 3);
            if (ko > lim_hi || (CAUSAL && ko > lim_c) || (IMASK && ko < lim_lo)) s[qb][r] = -INFINITY;
          }
        }
      }
      // dQ^T += K^T dS^T (reduction over the 32 keys of this block, 16 at a time); each
      // transposed K operand serves every row block.
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        vec8 ps[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float dsv[8];
#pragma unroll
          for (int r = 0; r < 8; ++r)
            dsv[r] = fast_exp2(fmaf(s[qb][8 * cc + r], scale_log2, -lse2[qb])) * (dp[qb][8 * cc + r] - drow[qb]);
          ps[qb] = pack8<T>(dsv);
        }
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const int rowb = (32 * kb + 16 * cc) * C::kRowBytes;
          const vec8 a = join8<T>(lds_read_tr4(kbase + rowb + toff[t]), lds_read_tr4(kbase + rowb + toff8[t]));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc[qb][t] = M::mma32(a, ps[qb], acc[qb][t]);
        }
      }
    }
  };

  auto stage_k = [&](auto sc) __attribute__((always_inline)) -> uint16_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return lk0;
    else if constexpr (S == 1) return lk1;
    else if constexpr (S == 2) return lk2;
    else return lk3;
  };
  auto stage_v = [&](auto sc) __attribute__((always_inline)) -> uint16_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return lv0;
    else if constexpr (S == 1) return lv1;
    else if constexpr (S == 2) return lv2;
    else return lv3;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if (0 < n_kt) issue(0, stage_k(I0{}), stage_v(I0{}));
  if (NBUF > 2 && 1 < n_kt) issue(1, stage_k(I1{}), stage_v(I1{}));
  if (NBUF > 3 && 2 < n_kt) issue(2, stage_k(I2{}), stage_v(I2{}));

  auto step = [&](auto sc, int kt) __attribute__((always_inline)) {
    constexpr int SN = (decltype(sc)::value + NBUF - 1) % NBUF;
    // Tile kt has landed once at most the loads of the (up to NBUF - 2) tiles
    // issued after it are outstanding.
    const int ahead = min(NBUF - 2, n_kt - 1 - kt);
    if (NBUF > 3 && ahead >= 2) wait_vmcnt<4 * C::kCPW>();
    else if (NBUF > 2 && ahead >= 1) wait_vmcnt<2 * C::kCPW>();
    else wait_vmcnt<0>();
    block_barrier();
    if (kt + NBUF - 1 < n_kt)
      issue(kt + NBUF - 1, stage_k(std::integral_constant<int, SN>{}),
            stage_v(std::integral_constant<int, SN>{}));
    compute(kt, (const char*)stage_k(sc), (const char*)stage_v(sc));
  };
  for (int kt = 0; kt < n_kt; kt += NBUF) {
    step(I0{}, kt);
    if (kt + 1 < n_kt) step(I1{}, kt + 1);
    if constexpr (NBUF > 2)
      if (kt + 2 < n_kt) step(I2{}, kt + 2);
    if constexpr (NBUF > 3)
      if (kt + 3 < n_kt) step(std::integral_constant<int, 3>{}, kt + 3);
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wrow0 + 32 * qb + l32;
    if (row < Nq) {
      uint16_t* qp = dQ + ((size_t)bh * Nq + row) * D;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = (uint32_t)to_bits<T>(acc[qb][t][4 * g + 0] * scale) |
                 ((uint32_t)to_bits<T>(acc[qb][t][4 * g + 1] * scale) << 16);
          w[1] = (uint32_t)to_bits<T>(acc[qb][t][4 * g + 2] * scale) |
                 ((uint32_t)to_bits<T>(acc[qb][t][4 * g + 3] * scale) << 16);
          *(u32x2*)(qp + 32 * t + 8 * g + 4 * hi) = w;
        }
    }
  }
}

// ---------------------------------------------------------------------------
template <typename E, int D>
static hipError_t preprocess_t(const BwdArgs& a) {
  constexpr int kTPR = D / (16 / sizeof(E));
  const long long rows = (long long)a.B * a.H * a.N;  // query rows
  const long long blocks = (rows + (256 / kTPR) - 1) / (256 / kTPR);
  hipLaunchKernelGGL((bwd_preprocess_kernel<E, D>), dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)a.stream, (const E*)a.o, (const E*)a.dO, a.lse, a.dvec, a.lse2,
                     rows);
  return hipGetLastError();
}

static hipError_t preprocess_dt(const BwdArgs& a) {
  if (a.dtype == 0) return a.d == 64 ? preprocess_t<float, 64>(a) : preprocess_t<float, 128>(a);
  if (a.dtype == 1) return a.d == 64 ? preprocess_t<_Float16, 64>(a) : preprocess_t<_Float16, 128>(a);
  return a.d == 64 ? preprocess_t<__bf16, 64>(a) : preprocess_t<__bf16, 128>(a);
}

hipError_t launch_bwd_preprocess(const BwdArgs& a) {
  hipError_t e = preprocess_dt(a);
  if (e != hipSuccess || !a.kv_lo) return e;
  const int n_qt = (a.N + 63) / 64;
  hipLaunchKernelGGL(mask_tiles_kernel, dim3((unsigned)n_qt, (unsigned)a.B), dim3(64), 0,
                     (hipStream_t)a.stream, a.kv_lo, a.kv_hi, (i32x4*)a.tile_sum, a.N,
                     a.Nk ? a.Nk : a.N, n_qt);
  return hipGetLastError();
}

#ifndef OSATTN_BWD_NBUF
#define OSATTN_BWD_NBUF 3
#endif
#ifndef OSATTN_DKDV_NBUF
#define OSATTN_DKDV_NBUF 4
#endif

#ifndef OSATTN_DQ64_QB
#define OSATTN_DQ64_QB 2
#endif

template <typename T, int D, int NB, int QB, bool CAUSAL, bool IMASK>
static hipError_t launch_dq_t(const BwdArgs& a, float sl2, int Nk) {
  using C = DqCfg<D, NB, QB>;
  const int n_qt = (a.N + C::kRows - 1) / C::kRows;
  const long long blocks = (long long)n_qt * a.B * a.H;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, NB, QB, CAUSAL, IMASK>), dim3((unsigned)blocks),
                     dim3(512), 0, (hipStream_t)a.stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dO, a.lse2,
                     a.dvec, (uint16_t*)a.dq, a.H, a.Hkv, a.N, n_qt, a.scale, sl2,
                     a.kv_lo, a.kv_hi, Nk);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL, bool IMASK>
static hipError_t bwd_t(const BwdArgs& a) {
  constexpr int NB = OSATTN_BWD_NBUF;
  constexpr int NBK = OSATTN_DKDV_NBUF;
  const float sl2 = a.scale * kLog2e;
  const int Nk = a.Nk ? a.Nk : a.N;
  if (a.stages & kStageDkdv) {
    using C = DkdvCfg<D, NBK>;
    const int n_kt = (Nk + C::kKeys - 1) / C::kKeys;
    const long long jobs = (long long)n_kt * a.B * a.Hkv;
    auto kernel = bwd_dkdv_kernel<T, D, NBK, CAUSAL, IMASK>;
    long long blocks = jobs;
    if (OSATTN_DKDV_PERSIST && CAUSAL && !IMASK) {
      static const int per_cu = resident_per_cu(kernel, 256);
      blocks = persistent_grid(per_cu, jobs);
    }
    const DkdvKernelArgs ka{(const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                            (const uint16_t*)a.dO, a.lse2, a.dvec, (uint16_t*)a.dk, (uint16_t*)a.dv,
                            a.H, a.Hkv, a.N, n_kt, a.scale, sl2, a.kv_lo, a.kv_hi,
                            (const i32x4*)a.tile_sum, Nk, (int)jobs, 0};
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)a.stream, ka);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.stages & kStageDq) {
    // d = 64 (not causal, no interval masks): two 32-row blocks per wave (512-row
    // workgroups), so that every K and V operand read from LDS feeds two MFMAs, unless
    // that grid would leave CUs without a workgroup.  (Under the causal mask the longer
    // staircase of 512-row tiles costs more than the reuse gains: 0.88 -> 0.99 ms on
    // fp16 B2 H32 N8192.)
    constexpr int QB2 = (D == 64 && !CAUSAL && !IMASK) ? OSATTN_DQ64_QB : 1;
    const long long wide = (long long)((a.N + DqCfg<D, NB, QB2>::kRows - 1) / DqCfg<D, NB, QB2>::kRows) *
                           a.B * a.H;
    if (QB2 > 1 && wide >= device_cus()) return launch_dq_t<T, D, NB, QB2, CAUSAL, IMASK>(a, sl2, Nk);
    return launch_dq_t<T, D, NB, 1, CAUSAL, IMASK>(a, sl2, Nk);
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t bwd_dt(const BwdArgs& a) {
  if (a.kv_lo) return a.d == 64 ? bwd_t<T, 64, false, true>(a) : bwd_t<T, 128, false, true>(a);
  if (a.d == 64) return a.causal ? bwd_t<T, 64, true, false>(a) : bwd_t<T, 64, false, false>(a);
  return a.causal ? bwd_t<T, 128, true, false>(a) : bwd_t<T, 128, false, false>(a);
}

hipError_t launch_bwd_mfma(const BwdArgs& a) {
  return a.dtype == 2 ? bwd_dt<__bf16>(a) : bwd_dt<_Float16>(a);
}

}  // namespace osattn
