// Forward pass with fp8 (e4m3) Q, K, V on the gfx950 8-bit matrix cores.
//
// The same FlashAttention-2 forward as the bf16 kernel (FlashAttention-2 page,
// inner-loop steps 1-5 and the final normalisation), with the products done in
// 8-bit floats and everything else in fp32 (ml-notes page: low-precision multiply,
// high-precision accumulate, softmax statistics in fp32):
//  * S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales): 64 head
//    dimensions per instruction, exact products, fp32 sums.  S is then scaled by
//    scale * dq * dk (the tensors' dequantisation factors) in the exp2 argument.
//  * The probabilities are formed against a running reference m that follows the
//    row max (the page's m_new = max(m_old, rowmax), with its rescale of Ot and l)
//    but moves only when a tile's max exceeds it by more than 0.8 (log2 units):
//    then P <= 2^0.8 and P * 256 <= 446 stays below 448, the largest e4m3 value,
//    when rounded to e4m3 for O^T += V^T P^T.  Moving on every increase would
//    rescale Ot on most tiles (some of a wave's 32 rows nearly always gains); Ot / l
//    does not depend on the reference.  The factor 256 keeps small probabilities out
//    of the subnormal range.
//  * The row sum l is taken by the matrix core from the same 8-bit P (a row of
//    ones as an extra A operand), so O = Ot / l uses exactly the weights that
//    produced Ot; the 256 cancels.  LSE = ln 2 * (m + log2 l - 8).
//  * V^T is the A operand of the O update, with keys along each lane's bytes; a
//    small pass writes V transposed per (batch, kv head), keys of each 64-key
//    block in the order the probabilities sit in the registers (see vt_key), so
//    both operands of the O update are plain 16-byte LDS reads.
// d = 64 or 128.  Layouts: Q, K, V codes [B][H or Hkv][N][d] bytes, O bf16
// [B][H][N][d], LSE fp32 [B][H][N]; the workspace holds V^T, [B][Hkv][d][Np]
// bytes with Np = N rounded up to 128 (padding keys are zero).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace osattn {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kNW = 8;        // waves per workgroup (two per SIMD)
constexpr int kBR = kNW * 32; // query rows per workgroup
constexpr int kBC = 128;      // keys per tile
constexpr int kRowV = kBC;    // bytes per LDS row of V^T (the tile's 128 keys of one dim)

// Tile geometry for head dimension D (64 or 128): K rows are D bytes, V^T rows 128.
template <int D>
struct Fp8Cfg {
  static constexpr int kRowK = D;               // bytes per LDS row of K (a key's dims)
  static constexpr int kTile = kBC * D;         // bytes per K tile and per V^T tile
  static constexpr int kCPW = kTile / 1024 / kNW;  // 1 KB LDS-DMA chunks per wave per tensor
  static_assert(kCPW >= 1 && kTile % (1024 * kNW) == 0, "tile must split over the waves");
};

// Key (within a 64-key block) of byte b of the P^T operand held by lane half h:
// the S^T accumulator gives lane (row, h) keys 8g + 4h + e of each 32-key block in
// register 4g + e; bytes 0-15 are the first block's registers, 16-31 the second's.
__host__ __device__ constexpr int vt_key(int h, int b) {
  return 32 * (b / 16) + 8 * ((b % 16) / 4) + 4 * h + (b % 4);
}

// 16-byte granule swizzle of LDS rows of 128 bytes (two rows per 256-byte bank
// cycle) and of 64 bytes (four rows per cycle): consecutive rows reading the same
// logical granule land on distinct banks, so 128-bit reads by 32 lanes on 32
// consecutive rows are conflict-free.
template <int ROW>
__device__ __forceinline__ int swz(int row) {
  return ROW == 128 ? (row >> 1) & 7 : (row >> 2) & 3;
}

// ---- V -> V^T with the block key order --------------------------------------------
// One workgroup per (batch * kv head, 64-key block): the block's 64 x D bytes go
// through LDS; thread t < 2D writes dim t / 2, block positions 32 * (t % 2) .. +31.
template <int D>
__global__ __launch_bounds__(256) void vt_kernel(const uint8_t* __restrict__ V,
                                                 uint8_t* __restrict__ Vt, int N, int Np) {
  constexpr int kQ = D / 32;  // threads per row, 32 bytes each
  __shared__ uint8_t tile[64][D + 4];
  const int blk = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int k0 = blk * 64;
  const int t = threadIdx.x;
  // Load: thread t reads 32 bytes, row t / kQ, bytes 32 * (t % kQ) .. +31.
  if (t < 64 * kQ) {
    const int r = t / kQ, c = 32 * (t % kQ);
    u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (k0 + r < N) {
      const u32x4* src = (const u32x4*)(V + (bh * N + k0 + r) * D + c);
      a = src[0];
      b = src[1];
    }
    uint32_t* dst = (uint32_t*)&tile[r][c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dst[i] = a[i];
      dst[4 + i] = b[i];
    }
  }
  __syncthreads();
  if (t >= 2 * D) return;
  const int d = t / 2, h = t % 2;
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t v = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) v |= (uint32_t)tile[vt_key(h, 4 * j + e)][d] << (8 * e);
    w[j] = v;
  }
  u32x4* out = (u32x4*)(Vt + (bh * D + d) * Np + k0 + 32 * h);
  out[0] = u32x4{w[0], w[1], w[2], w[3]};
  out[1] = u32x4{w[4], w[5], w[6], w[7]};
}

__device__ __forceinline__ f32x16 mma8(i32x8 a, i32x8 b, f32x16 c) {
  // e4m3 x e4m3 (format selectors 0), unit block scales (E8M0 code 127 = 2^0).
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 lds_read32(const char* p0, const char* p1) {
  const u32x4 a = *(const u32x4*)p0, b = *(const u32x4*)p1;
  i32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (int)a[i];
    r[4 + i] = (int)b[i];
  }
  return r;
}

// Kernel arguments.
struct Fp8KernelArgs {
  const uint8_t* Q;
  const uint8_t* K;
  const uint8_t* Vt;
  uint16_t* O;
  float* LSE;
  int H, Hkv, N, Np, n_qtiles;
  float c_log2, dv;
  int n_jobs;  // logical tiles (query tiles x heads)
};

// Persistent grid (StaticSchedule in common.h) for the causal fp8 forward, whose query
// tiles differ in length.
#ifndef OSATTN_FP8_PERSIST
#define OSATTN_FP8_PERSIST 1
#endif

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kNW * 64, kNW * 64)))
__attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_fp8_kernel(const Fp8KernelArgs args) {
  constexpr bool PERSIST = OSATTN_FP8_PERSIST && CAUSAL;
  using C = Fp8Cfg<D>;
  constexpr int kD = D;
  constexpr int kRowK = C::kRowK;
  constexpr int kCPW = C::kCPW;
  constexpr int kNC = D / 64;  // 64-dim chunks of the score contraction
  __shared__ __attribute__((aligned(1024))) uint8_t lk0[C::kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t lv0[C::kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t lk1[C::kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t lv1[C::kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Logical tile L: query tile L % n_qtiles of head L / n_qtiles.  A persistent grid
  // (causal) walks its schedule, longest first within each head as below; otherwise
  // each workgroup runs one tile.
  StaticSchedule sched(args.n_jobs, blockIdx.x, gridDim.x);
  int L = PERSIST ? sched.next() : xcd_remap(blockIdx.x, gridDim.x);
  while (L >= 0) {
    // Arguments read afresh for each tile of a persistent grid (see fresh_kernel_args).
    const Fp8KernelArgs a = PERSIST ? fresh_kernel_args<Fp8KernelArgs>() : args;
    const uint8_t* __restrict__ Q = a.Q;
    const uint8_t* __restrict__ K = a.K;
    const uint8_t* __restrict__ Vt = a.Vt;
    uint16_t* __restrict__ O = a.O;
    float* __restrict__ LSE = a.LSE;
    const int H = a.H, Hkv = a.Hkv, N = a.N, Np = a.Np, n_qtiles = a.n_qtiles;
    const float c_log2 = a.c_log2, dv = a.dv;
    int qt = L % n_qtiles;
    const int bh = L / n_qtiles;
    if (CAUSAL) qt = n_qtiles - 1 - qt;  // longest rows first
    const int h = bh % H;
    const int b = bh / H;
    const int kvh = h / (H / Hkv);
    const int q0 = qt * kBR;
    const int wrow0 = q0 + wave * 32;
    const size_t g = (size_t)b * Hkv + kvh;

    const auto rq = make_rsrc(Q + (size_t)bh * N * kD, (uint32_t)N * kD);
    const auto rk = make_rsrc(K + g * N * kD, (uint32_t)N * kD);
    const auto rv = make_rsrc(Vt + g * kD * Np, (uint32_t)kD * Np);

    // Q fragments (B operand of S^T = K Q^T): row l32, dims 64c + 32hi .. +31.
    i32x8 qf[kNC];
#pragma unroll
    for (int c = 0; c < kNC; ++c) {
      const uint32_t off = (uint32_t)(wrow0 + l32) * kD + 64 * c + 32 * hi;
      const u32x4 a = buffer_load16(rq, off), bb = buffer_load16(rq, off + 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qf[c][i] = (int)a[i];
        qf[c][4 + i] = (int)bb[i];
      }
    }

    int n_kt = (N + kBC - 1) / kBC;
    if (CAUSAL) n_kt = min(n_kt, (q0 + kBR + kBC - 1) / kBC);

    // LDS-DMA: chunk ch of a tile is LDS bytes [ch * 1024, +1024); the lane's 16 bytes
    // are physical granule pg of its row, logical pg ^ swz(row).
    uint32_t goff_k[kCPW], goff_v[kCPW];
#pragma unroll
    for (int i = 0; i < kCPW; ++i) {
      const int off = (wave * kCPW + i) * 1024 + lane * 16;
      const int rk_ = off / kRowK;  // key row of the K tile
      goff_k[i] = rk_ * kRowK + (((off % kRowK) / 16) ^ swz<kRowK>(rk_)) * 16;  // + k0 * D (scalar)
      const int rv_ = off / kRowV;  // dim row of the V^T tile
      goff_v[i] = rv_ * Np + (((off % kRowV) / 16) ^ swz<kRowV>(rv_)) * 16;     // + k0 (scalar)
    }
    auto issue = [&](int kt, uint8_t* lk, uint8_t* lv) __attribute__((always_inline)) {
      const uint32_t k0 = (uint32_t)kt * kBC;
#pragma unroll
      for (int i = 0; i < kCPW; ++i) {
        const int ch = wave * kCPW + i;
        buffer_load16_lds(rk, lk + ch * 1024, goff_k[i], k0 * kRowK);
        buffer_load16_lds(rv, lv + ch * 1024, goff_v[i], k0);
      }
    };

    // LDS read offsets: row l32 of a 32-row block, logical granules 4c + 2hi, +1 (K:
    // dims 64c + 32hi .. +31; V^T: keys 64m + 32hi .. +31).
    uint32_t koff[kNC][2], voff[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int c = 0; c < kNC; ++c)
        koff[c][j] = l32 * kRowK + 16 * ((4 * c + 2 * hi + j) ^ swz<kRowK>(l32));
#pragma unroll
      for (int m = 0; m < 2; ++m) voff[m][j] = l32 * kRowV + 16 * ((4 * m + 2 * hi + j) ^ swz<kRowV>(l32));
    }

    f32x16 acc[kD / 32], lacc;
#pragma unroll
    for (int t = 0; t < kD / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) lacc[r] = 0.f;
    float m_run = -1e30f;  // finite: exp2(m_old - m_new) never sees inf - inf
    i32x8 ones;
#pragma unroll
    for (int i = 0; i < 8; ++i) ones[i] = 0x38383838;  // e4m3 1.0 in every byte

    // How far a tile's max may exceed the reference before it moves (log2 units):
    // 2^0.8 * 256 = 445.7 <= 448.
    constexpr float kSlack = 0.8f;
    auto compute = [&](int kt, const char* kbase, const char* vbase) __attribute__((always_inline)) {
      const int k0 = kt * kBC;
      if (CAUSAL && k0 > wrow0 + 31) return;  // every key after every row of the wave
      f32x16 s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int c = 0; c < kNC; ++c)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const char* base = kbase + kb * 32 * kRowK;
          s[kb] = mma8(lds_read32(base + koff[c][0], base + koff[c][1]), qf[c], s[kb]);
        }
      const bool need_mask = (k0 + kBC > N) || (CAUSAL && k0 + kBC - 1 > wrow0);
      if (need_mask) {
        asm volatile("");  // keep this a branch
        // Key of element r of block kb: base + ko with ko a compile-time constant.
        const int base = k0 + 4 * hi;
        const int lim_n = N - 1 - base, lim_c = wrow0 + l32 - base;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = kb * 32 + 8 * (r >> 2) + (r & 3);
            if (ko > lim_n || (CAUSAL && ko > lim_c)) s[kb][r] = -INFINITY;
          }
      }
      // The tile's row max (log2 units of the scaled scores) against the reference.
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      const float m_tile = wave_xor32_max(mx) * c_log2;
      if (__any(m_tile > m_run + kSlack)) {
        const float m_new = fmaxf(m_run, m_tile);
        const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
        for (int t = 0; t < kD / 32; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
        m_run = m_new;
      }
      // P * 256 in e4m3, bytes in vt_key order: pf[m] covers keys 64m .. 64m+63.
      const float bias = 8.0f - m_run;  // exp2(s*c - m + 8) = 256 * P
      i32x8 pf[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const f32x16& sb = s[2 * m + j / 4];
          const int r0 = 4 * (j % 4);
          const float p0 = fast_exp2(fmaf(sb[r0 + 0], c_log2, bias));
          const float p1 = fast_exp2(fmaf(sb[r0 + 1], c_log2, bias));
          const float p2 = fast_exp2(fmaf(sb[r0 + 2], c_log2, bias));
          const float p3 = fast_exp2(fmaf(sb[r0 + 3], c_log2, bias));
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
          pf[m][j] = w;
        }
      // O^T += V^T P^T (dims 32t .. 32t+31), and l += sum of the same 8-bit P.
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int t = 0; t < kD / 32; ++t) {
          const char* base = vbase + t * 32 * kRowV;
          acc[t] = mma8(lds_read32(base + voff[m][0], base + voff[m][1]), pf[m], acc[t]);
        }
        lacc = mma8(ones, pf[m], lacc);
      }
    };

    if (0 < n_kt) issue(0, lk0, lv0);
    auto step = [&](auto sc, int kt) __attribute__((always_inline)) {
      constexpr int S = decltype(sc)::value;
      uint8_t* lk = S == 0 ? lk0 : lk1;
      uint8_t* lv = S == 0 ? lv0 : lv1;
      uint8_t* nk = S == 0 ? lk1 : lk0;
      uint8_t* nv = S == 0 ? lv1 : lv0;
      wait_vmcnt<0>();
      block_barrier();  // tile kt is in LDS; the other stage is free
      if (kt + 1 < n_kt) issue(kt + 1, nk, nv);
      compute(kt, (const char*)lk, (const char*)lv);
    };
    for (int kt = 0; kt < n_kt; kt += 2) {
      step(std::integral_constant<int, 0>{}, kt);
      if (kt + 1 < n_kt) step(std::integral_constant<int, 1>{}, kt + 1);
    }

    // O = Ot * dv / l; LSE = ln 2 * (m + log2 l - 8).
    const int row = wrow0 + l32;
    const float l = lacc[0];
    const float inv = dv / l;
    if (row < N) {
      uint16_t* op = O + ((size_t)bh * N + row) * kD;
#pragma unroll
      for (int t = 0; t < kD / 32; ++t)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          u32x2 w;
          w[0] = (uint32_t)to_bits<__bf16>(acc[t][4 * gg + 0] * inv) |
                 ((uint32_t)to_bits<__bf16>(acc[t][4 * gg + 1] * inv) << 16);
          w[1] = (uint32_t)to_bits<__bf16>(acc[t][4 * gg + 2] * inv) |
                 ((uint32_t)to_bits<__bf16>(acc[t][4 * gg + 3] * inv) << 16);
          store_global(op + 32 * t + 8 * gg + 4 * hi, w);
        }
      if (hi == 0) store_global(LSE + (size_t)bh * N + row, (m_run + __log2f(l) - 8.0f) * kLn2);
    }
    if constexpr (!PERSIST) break;
    __syncthreads();  // every wave is done with the staged tiles
    L = sched.next();
  }
}

}  // namespace

size_t fp8_vt_bytes(int B, int Hkv, int N, int d) {
  const size_t np = ((size_t)N + kBC - 1) / kBC * kBC;
  return (size_t)B * Hkv * d * np;
}

namespace {

template <int D>
hipError_t launch_fp8_d(const Fp8Args& a) {
  const int np = (a.N + kBC - 1) / kBC * kBC;
  hipLaunchKernelGGL(vt_kernel<D>, dim3((unsigned)(np / 64), (unsigned)(a.B * a.Hkv)), dim3(256),
                     0, (hipStream_t)a.stream, (const uint8_t*)a.v, (uint8_t*)a.workspace, a.N, np);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_qtiles = (a.N + kBR - 1) / kBR;
  const long long jobs = (long long)n_qtiles * a.B * a.H;
  const float c_log2 = a.scale * a.descale_q * a.descale_k * kLog2e;
  const Fp8KernelArgs ka{(const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.workspace,
                         (uint16_t*)a.o, a.lse, a.H, a.Hkv, a.N, np, n_qtiles, c_log2,
                         a.descale_v, (int)jobs};
  if (a.causal) {
    auto kernel = fwd_fp8_kernel<D, true>;
    long long blocks = jobs;
    if (OSATTN_FP8_PERSIST) {
      static const int per_cu = resident_per_cu(kernel, kNW * 64);
      blocks = persistent_grid(per_cu, jobs);
    }
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kNW * 64), 0, (hipStream_t)a.stream, ka);
  } else {
    hipLaunchKernelGGL((fwd_fp8_kernel<D, false>), dim3((unsigned)jobs), dim3(kNW * 64), 0,
                       (hipStream_t)a.stream, ka);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Args& a) {
  return a.d == 64 ? launch_fp8_d<64>(a) : launch_fp8_d<128>(a);
}

}  // namespace osattn
