// Split-KV forward for few queries against a long key/value sequence (decoding).
//
// With a handful of query rows per head the row-partitioned forward launches too
// few workgroups to fill 256 CUs, so the key axis is cut instead (ml-notes page,
// the split-K notes of the sparse-attention kernel: more independent blocks, each
// carrying the online-softmax state over its own key chunk, then an exact merge).
//
//  1. splitkv_partial_kernel: one to four waves per workgroup, 32 query rows per
//     wave, sharing the K/V tiles.  The rows are the n_rep query heads of one
//     key/value head times the Nq queries (grouped-query decoding reads each K/V
//     chunk once for the whole group); in memory these rows are contiguous,
//     [h_local][i].  Each wave walks the chunk of keys in 32-key tiles with the FlashAttention-2 online softmax
//     (FlashAttention-2 page, inner loop steps 1-5; the running max is a reference
//     that moves only when a tile's max exceeds it by more than 8 in log2 units)
//     and writes the chunk's normalised output O_s = Ot / l and LSE_s = m + ln l
//     in fp32 (LSE_s = -inf and O_s = 0 for rows that see no key of the chunk).
//  2. splitkv_merge_kernel: one wave per query row combines the chunks,
//     LSE = ln sum_s exp(LSE_s) taken about a running max, O = sum_s exp(LSE_s - LSE) O_s
//     (the exact rescale-to-a-common-max merge of the ml-notes page and of
//     "Phase 2" on the attnres-kernel-lab page), and writes O in the I/O dtype.
//
// Causal masks are aligned bottom-right: query i is position i + Nk - Nq.
// The step is HBM-bound (K and V are read once); K/V tiles go straight from
// memory into LDS with 16-byte DMA, three or four tiles staged, and the same
// MFMA layouts as the main forward: S^T = K Q^T with one query row per lane,
// O^T += V^T P^T with P from registers and V read transposed from LDS.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace osattn {

namespace {

constexpr int kSplitTile = 32;  // keys per tile
constexpr int kSplitNbuf = OSATTN_SPLIT_NBUF;  // tiles in flight (3 or 4)
// s_waitcnt lgkmcnt(0) with vmcnt and expcnt left at their maxima (gfx9 encoding).
constexpr int kWaitLgkm0 = 0xF | (0x7 << 4) | (0x3 << 14);

template <int D>
struct SplitSwizzle {
  // 16-byte granule XOR of tile row `row` (conflict-free 128-bit K reads and
  // transposed V reads; the V swizzle is equal for rows r and r + 8).
  static __device__ __forceinline__ int k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  static __device__ __forceinline__ int v(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
};

template <typename T, int D, int NW, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
void splitkv_partial_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                            const uint16_t* __restrict__ V, float* __restrict__ Opart,
                            float* __restrict__ Lpart, int H, int Hkv, int Nq, int Nk,
                            int n_rowblocks, int n_splits, int split_keys, long long rows_total,
                            float scale_log2) {
  using M = Mfma<T>;
  using vec8 = typename M::vec8;
  using Swz = SplitSwizzle<D>;
  constexpr int NBUF = kSplitNbuf;
  static_assert(NBUF == 3 || NBUF == 4, "three or four stages");
  constexpr int kRowBytes = D * 2;
  constexpr int kTileElems = kSplitTile * D;
  constexpr int kChunks = kSplitTile * kRowBytes / 1024;  // 1 KB DMA chunks per tile
  constexpr int kCPW = kChunks / NW;                       // of them per wave
  static_assert(kCPW >= 1 && kChunks % NW == 0, "tile must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) uint16_t lk0[kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lv0[kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lk1[kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lv1[kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lk2[kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lv2[kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lk3[NBUF > 3 ? kTileElems : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lv3[NBUF > 3 ? kTileElems : 8];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // blockIdx.x = (bg * n_splits + split) * n_rowblocks + rb: row blocks of one chunk
  // are adjacent (they read the same K/V tiles).
  const int rb = blockIdx.x % n_rowblocks;
  const int split = (blockIdx.x / n_rowblocks) % n_splits;
  const int bg = blockIdx.x / (n_rowblocks * n_splits);  // b * Hkv + g
  const int g = bg % Hkv;
  const int b = bg / Hkv;
  const int n_rep = H / Hkv;
  const int R = n_rep * Nq;                       // rows of this group
  const int wr0 = 32 * (NW * rb + wave);          // this wave's first row within the group
  const int r = wr0 + l32;                        // this lane's row
  const bool row_ok = r < R;
  const long long row0 = ((long long)b * H + (long long)g * n_rep) * Nq;  // group's first row

  // Query fragments (B operand of S^T = K Q^T); rows >= R read zero.
  const auto rq = make_rsrc(Q + row0 * D, (uint32_t)R * kRowBytes);
  vec8 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qf[c] = as_vec8<T>(buffer_load16(rq, (uint32_t)r * kRowBytes + (16 * c + 8 * hi) * 2));

  // Key range of this chunk, shortened (causal) to the last key any row of the
  // workgroup can see.
  const int ks = split * split_keys;
  const int ke = min(Nk, ks + split_keys);
  const int lim = (row_ok ? r % Nq : 0) + Nk - Nq;  // last visible key of this row (causal)
  int kend = ke;
  if (CAUSAL) {
    const int first = 32 * NW * rb, last = min(R, first + 32 * NW) - 1;
    int max_i;
    if (last - first + 1 >= Nq) max_i = Nq - 1;
    else max_i = (last % Nq >= first % Nq) ? last % Nq : Nq - 1;
    kend = min(ke, max_i + Nk - Nq + 1);
  }
  const int n_t = kend > ks ? (kend - ks + kSplitTile - 1) / kSplitTile : 0;

  const auto rk = make_rsrc(K + (size_t)bg * Nk * D, (uint32_t)Nk * kRowBytes);
  const auto rv = make_rsrc(V + (size_t)bg * Nk * D, (uint32_t)Nk * kRowBytes);
  uint32_t goff_k[kCPW], goff_v[kCPW];
#pragma unroll
  for (int i = 0; i < kCPW; ++i) {
    const int off = (wave * kCPW + i) * 1024 + lane * 16;
    const int row = off / kRowBytes;
    const int pg = (off % kRowBytes) / 16;
    goff_k[i] = row * kRowBytes + ((pg ^ Swz::k(row)) * 16);
    goff_v[i] = row * kRowBytes + ((pg ^ Swz::v(row)) * 16);
  }
  auto issue = [&](int t, uint16_t* lk, uint16_t* lv) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(ks + t * kSplitTile) * kRowBytes;
#pragma unroll
    for (int i = 0; i < kCPW; ++i) {
      const int ch = wave * kCPW + i;
      buffer_load16_lds(rk, lk + ch * 512, base + goff_k[i]);
      buffer_load16_lds(rv, lv + ch * 512, base + goff_v[i]);
    }
  };

  uint32_t koff[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) koff[c] = l32 * kRowBytes + (((2 * c + hi) ^ Swz::k(l32)) * 16);
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  uint32_t voff[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    const int col = 32 * t + tr_col;
    voff[t] = tr_row * kRowBytes + (((col >> 3) ^ Swz::v(tr_row)) * 16) + (col & 7) * 2;
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  // Running max (log2 units, finite sentinel) and this lane's half of the running sum.
  float m_run = -1e30f, l_run = 0.f;
  const bool wave_live = wr0 < R;  // waves whose rows are all padding only stage tiles

  auto compute = [&](int t, const char* kbase, const char* vbase) __attribute__((always_inline)) {
    if (!wave_live) return;
    const int k0 = ks + t * kSplitTile;
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const u32x4 a = *(const u32x4*)(kbase + koff[c]);
      s = M::mma32(as_vec8<T>(a), qf[c], s);
    }
    const bool need_mask = (k0 + kSplitTile > ke) || (CAUSAL && k0 + kSplitTile - 1 > Nk - Nq);
    if (need_mask) {
      asm volatile("");  // a branch: the key tests run only on tiles that need them
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + 8 * (e >> 2) + 4 * hi + (e & 3);
        if (key >= ke || (CAUSAL && key > lim)) s[e] = -INFINITY;
      }
    }
    // The tile's row max (log2 units).  The reference m moves to it (with the rescale
    // of Ot and l by exp2(m_old - m_new)) only when it exceeds m by more than 8: then
    // P <= 2^8, well inside the range of the rounded P and of l, and most tiles skip
    // the rescale of the accumulators.  Ot / l does not depend on the reference.
    float mx = s[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
    const float m_tile = wave_xor32_max(mx) * scale_log2;
    if (__any(m_tile > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int tt = 0; tt < D / 32; ++tt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[tt][e] *= alpha;
    }
    const float neg_m = -m_run;
    vec8 pf[2];
    float part = 0.f;
#pragma unroll
    for (int c4 = 0; c4 < 2; ++c4) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = fast_exp2(fmaf(s[8 * c4 + j], scale_log2, neg_m));
      pf[c4] = pack8<T>(p);
      part = sum8<T>(pf[c4], part);
    }
    l_run += part;
#pragma unroll
    for (int c4 = 0; c4 < 2; ++c4)
#pragma unroll
      for (int tt = 0; tt < D / 32; ++tt) {
        const char* vb = vbase + 16 * c4 * kRowBytes + voff[tt];
        const vec8 a = join8<T>(lds_read_tr4(vb), lds_read_tr4(vb + 8 * kRowBytes));
        acc[tt] = M::mma32(a, pf[c4], acc[tt]);
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
  using I3 = std::integral_constant<int, 3>;
  if (0 < n_t) issue(0, lk0, lv0);
  if (1 < n_t) issue(1, lk1, lv1);
  if (NBUF > 3 && 2 < n_t) issue(2, lk2, lv2);
  auto step = [&](auto sc, int t) __attribute__((always_inline)) {
    constexpr int SN = (decltype(sc)::value + NBUF - 1) % NBUF;
    // Tile t has landed once at most this wave's loads of the tiles issued after it
    // (up to NBUF - 2) are outstanding.
    const int ahead = min(NBUF - 2, n_t - 1 - t);
    if (NBUF > 3 && ahead >= 2) wait_vmcnt<4 * kCPW>();
    else if (ahead >= 1) wait_vmcnt<2 * kCPW>();
    else wait_vmcnt<0>();
    // The stage receiving tile t + NBUF - 1 was read for tile t - 1: those LDS reads
    // complete before any wave may overwrite it.
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if constexpr (NW > 1) block_barrier();  // every wave's share of tile t is in LDS
    if (t + NBUF - 1 < n_t)
      issue(t + NBUF - 1, stage_k(std::integral_constant<int, SN>{}),
            stage_v(std::integral_constant<int, SN>{}));
    compute(t, (const char*)stage_k(sc), (const char*)stage_v(sc));
  };
  for (int t = 0; t < n_t; t += NBUF) {
    step(I0{}, t);
    if (t + 1 < n_t) step(I1{}, t + 1);
    if (t + 2 < n_t) step(I2{}, t + 2);
    if constexpr (NBUF > 3)
      if (t + 3 < n_t) step(I3{}, t + 3);
  }

  // Chunk result: O_s = Ot / l and LSE_s = ln(2) * (m + log2 l), or 0 and -inf.
  const float l = wave_xor32_sum(l_run);
  if (row_ok) {
    const long long row = row0 + r;
    float* op = Opart + ((long long)split * rows_total + row) * D;
    const bool any = l > 0.f;
    const float inv = any ? 1.0f / l : 0.f;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = acc[t][4 * gq + e] * inv;
        *(f32x4*)(op + 32 * t + 8 * gq + 4 * hi) = w;
      }
    if (hi == 0)
      Lpart[(long long)split * rows_total + row] = any ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// One wave per query row: merge the n_splits chunk results of that row.  A chunk's
// output row is D fp32 values, read as 16-byte pieces by D/4 lanes, so a wave reads
// 64/(D/4) chunks side by side (lane group g takes chunks g, g + G, g + 2G, ...).
// Every lane keeps its own online-softmax state over the chunks it reads: the max
// m of their logsumexps, the weight sum z and the weighted sum o, each rescaled by
// exp(m_old - m_new) when m moves (the FlashAttention-2 page's running statistics,
// applied to chunk results).  Batches of eight chunks per lane are loaded before any
// of them is used, so a row with up to 8G chunks costs one memory round trip; the
// lane groups are then brought to the common max and summed across the wave.
template <typename T, int D>
__global__ __launch_bounds__(64) void splitkv_merge_kernel(const float* __restrict__ Opart,
                                                           const float* __restrict__ Lpart,
                                                           uint16_t* __restrict__ O,
                                                           float* __restrict__ LSE,
                                                           long long rows, int n_splits) {
  constexpr int kLanes = D / 4;        // lanes per chunk row (float4 each)
  constexpr int kGroups = 64 / kLanes;  // chunks read side by side
  constexpr int kBatch = 8;            // chunks per lane in flight
  const int lane = threadIdx.x;
  const int g = lane / kLanes;
  const int cl = lane % kLanes;
  const long long row = blockIdx.x;
  if (row >= rows) return;
  const long long stride = rows * D;  // floats between chunks of one row
  const float* obase = Opart + row * D + 4 * cl;
  float m = -INFINITY, z = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = g; s0 < n_splits; s0 += kGroups * kBatch) {
    float4 v[kBatch];
    float ls[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int s = s0 + u * kGroups;
      if (s < n_splits) {
        v[u] = *reinterpret_cast<const float4*>(obase + s * stride);
        ls[u] = Lpart[(long long)s * rows + row];
      } else {
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        ls[u] = -INFINITY;
      }
    }
    float bm = ls[0];
#pragma unroll
    for (int u = 1; u < kBatch; ++u) bm = fmaxf(bm, ls[u]);
    if (bm > m) {
      const float c = m > -INFINITY ? __expf(m - bm) : 0.f;
      o.x *= c; o.y *= c; o.z *= c; o.w *= c;
      z *= c;
      m = bm;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = ls[u] > -INFINITY ? __expf(ls[u] - m) : 0.f;
      o.x = fmaf(w, v[u].x, o.x); o.y = fmaf(w, v[u].y, o.y);
      o.z = fmaf(w, v[u].z, o.z); o.w = fmaf(w, v[u].w, o.w);
      z += w;
    }
  }
  // Bring the lane groups to the common max, then sum them.
  float mall = m;
#pragma unroll
  for (int off = kLanes; off < 64; off <<= 1) mall = fmaxf(mall, __shfl_xor(mall, off));
  const float c = m > -INFINITY ? __expf(m - mall) : 0.f;
  o.x *= c; o.y *= c; o.z *= c; o.w *= c;
  z *= c;
#pragma unroll
  for (int off = kLanes; off < 64; off <<= 1) {
    o.x += __shfl_xor(o.x, off); o.y += __shfl_xor(o.y, off);
    o.z += __shfl_xor(o.z, off); o.w += __shfl_xor(o.w, off);
    z += __shfl_xor(z, off);
  }
  if (g == 0) {
    const float inv = z > 0.f ? 1.0f / z : 0.f;
    const uint32_t lo = (uint32_t)to_bits<T>(o.x * inv) | ((uint32_t)to_bits<T>(o.y * inv) << 16);
    const uint32_t hi2 = (uint32_t)to_bits<T>(o.z * inv) | ((uint32_t)to_bits<T>(o.w * inv) << 16);
    *reinterpret_cast<uint2*>(O + row * D + 4 * cl) = make_uint2(lo, hi2);
  }
  if (lane == 0) LSE[row] = z > 0.f ? mall + __logf(z) : -INFINITY;
}

template <typename T, int D, int NW, bool CAUSAL>
hipError_t splitkv_t(const SplitArgs& a) {
  const int n_rep = a.H / a.Hkv;
  const int n_rb = (n_rep * a.Nq + 32 * NW - 1) / (32 * NW);
  const long long rows = (long long)a.B * a.H * a.Nq;
  const long long blocks = (long long)a.B * a.Hkv * a.n_splits * n_rb;
  hipLaunchKernelGGL((splitkv_partial_kernel<T, D, NW, CAUSAL>), dim3((unsigned)blocks),
                     dim3(NW * 64), 0, (hipStream_t)a.stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, a.o_part, a.lse_part, a.H, a.Hkv,
                     a.Nq, a.Nk, n_rb, a.n_splits, a.split_keys, rows, a.scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((splitkv_merge_kernel<T, D>), dim3((unsigned)rows), dim3(64), 0,
                     (hipStream_t)a.stream, a.o_part, a.lse_part, (uint16_t*)a.o, a.lse, rows,
                     a.n_splits);
  return hipGetLastError();
}

// Waves per workgroup: one per 32 rows of a query group, up to four.
template <typename T, int D, bool CAUSAL>
hipError_t splitkv_nw(const SplitArgs& a) {
  const int nw = splitkv_waves((a.H / a.Hkv) * a.Nq);
  if (nw == 4) return splitkv_t<T, D, 4, CAUSAL>(a);
  if (nw == 2) return splitkv_t<T, D, 2, CAUSAL>(a);
  return splitkv_t<T, D, 1, CAUSAL>(a);
}

template <typename T>
hipError_t splitkv_dt(const SplitArgs& a) {
  if (a.d == 64) return a.causal ? splitkv_nw<T, 64, true>(a) : splitkv_nw<T, 64, false>(a);
  return a.causal ? splitkv_nw<T, 128, true>(a) : splitkv_nw<T, 128, false>(a);
}

}  // namespace

hipError_t launch_splitkv(const SplitArgs& a) {
  return a.dtype == 2 ? splitkv_dt<__bf16>(a) : splitkv_dt<_Float16>(a);
}

}  // namespace osattn
