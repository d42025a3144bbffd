// Device-side building blocks shared by the osattn kernels (gfx950 / CDNA4 only).
//
// MFMA operand layouts used throughout (wave64, confirmed on gfx950):
//   v_mfma_f32_32x32x16_{bf16,f16}:  D[32x32] += A[32x16] * B[16x32]
//     lane l supplies A[m = l%32][k = 8*(l/32) + j] and B[k = 8*(l/32) + j][n = l%32]
//     for j = 0..7 (one 128-bit register quad each);
//     result register r of lane l is D[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32].
//   ds_read_b64_tr_b16 (LDS transpose read): inside each group of 16 lanes, lane i
//     receives element i%4 of the 4-element (64-bit) chunk addressed by lane
//     4*e + i/4, as its element e.  Pointing lane 4*a + b at row a, columns 4b..4b+3
//     of a row-major tile therefore hands lane i the column i of rows 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element traits: storage is 16-bit for bf16/fp16.
template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
  typedef bf16x8 vec8;
  static __device__ __forceinline__ f32x16 mma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<_Float16> {
  typedef f16x8 vec8;
  static __device__ __forceinline__ f32x16 mma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// fp32 -> 16-bit with round-to-nearest-even, returned as raw bits.
template <typename T> __device__ __forceinline__ uint16_t to_bits(float x);
template <> __device__ __forceinline__ uint16_t to_bits<__bf16>(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
template <> __device__ __forceinline__ uint16_t to_bits<_Float16>(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <typename T> __device__ __forceinline__ float from_bits(uint16_t b);
template <> __device__ __forceinline__ float from_bits<__bf16>(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
template <> __device__ __forceinline__ float from_bits<_Float16>(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// Pack 8 floats into an MFMA operand (round to nearest even).
template <typename T>
__device__ __forceinline__ typename Mfma<T>::vec8 pack8(const float* x) {
  typename Mfma<T>::vec8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (T)x[j];
  return r;
}

// LDS pointer helpers (address space 3).
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

// `p` must point into a __shared__ array; the cast is an address-space cast.
__device__ __forceinline__ i16x4 lds_read_tr4(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(void*)p);
}

// Combine two transposed 4-element reads into one 8-element MFMA operand.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::vec8 join8(i16x4 lo, i16x4 hi) {
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(typename Mfma<T>::vec8, v);
}

template <typename T>
__device__ __forceinline__ typename Mfma<T>::vec8 as_vec8(u32x4 x) {
  return __builtin_bit_cast(typename Mfma<T>::vec8, x);
}

__device__ __forceinline__ float wave_xor32_max(float x) {
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_xor32_sum(float x) {
  return x + __shfl_xor(x, 32);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum of the eight 16-bit values of an MFMA operand, accumulated in fp32 with
// v_dot2_f32_{bf16,f16} against (1, 1): two elements per instruction, and the
// sum is of exactly the rounded values the matrix core consumes.
template <typename T> __device__ __forceinline__ float sum8(typename Mfma<T>::vec8 v, float acc);
template <> __device__ __forceinline__ float sum8<__bf16>(bf16x8 v, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
  return acc;
}
template <> __device__ __forceinline__ float sum8<_Float16>(f16x8 v, float acc) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
  return acc;
}

// ---- buffer resources -------------------------------------------------------------
// A raw buffer over [base, base + bytes): loads at offsets >= bytes return zero,
// which is how rows past the end of a sequence are read without branches.
// Word 3 (0x00020000) is the raw-buffer configuration used for gfx9-family parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes lds_chunk + 16*i (lds_chunk is wave-uniform and 16-byte aligned).  The
// global offset is voff (per lane) + soff (wave-uniform, a scalar register): keeping
// the per-lane part loop-invariant and the tile base scalar leaves no short-lived
// address VGPR behind the DMA (the compiler treats the address register of an LDS
// DMA as busy until the load completes, so a reused temporary would make later
// LDS reads into it wait for the whole DMA).
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds_chunk,
                                                  uint32_t voff, uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_chunk, 16, voff, soff, 0, 0);
}

// 4 bytes per lane into LDS (lane i writes lds + 4*i); same offset split.
__device__ __forceinline__ void buffer_load4_lds(__amdgpu_buffer_rsrc_t r, void* lds,
                                                 uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                           voff, soff, 0, 0);
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence would
// wait for every outstanding global load, including prefetches still in flight.
// Callers order their own memory traffic (LDS reads are consumed before the
// barrier is reached; DMA writes are waited for with wait_vmcnt).
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Maps a linear workgroup index to a logical one so that the workgroups the
// hardware places on one XCD (dispatch is round-robin over the 8 XCDs) get a
// contiguous range of logical tiles, i.e. the same heads, sharing that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks >> 3;
  if (bid >= (per << 3)) return bid;
  return (bid & 7) * per + (bid >> 3);
}

// Workgroup order of the interval-masked attention kernels: 1 deals K/V-head groups to
// the XCDs round-robin (xcd_group_remap), 0 gives each XCD one contiguous block
// (xcd_remap, which the other kernels always use).
#ifndef OSATTN_XCD_GROUPS
#define OSATTN_XCD_GROUPS 1
#endif
// Interval-masked forward and dQ take their query tiles last-first (as causal does).
#ifndef OSATTN_MASK_LONGEST_FIRST
#define OSATTN_MASK_LONGEST_FIRST 1
#endif

// As xcd_remap, but over "groups" of consecutive logical tiles (a head, or the query
// heads sharing a K/V head, with all their tiles): when the group count is a multiple of
// 8, XCD x receives the groups g = x, x + 8, x + 16, ... (each one's tiles in order,
// for its L2), instead of one contiguous block of groups.  Work that differs between
// groups (packed documents of different lengths per batch entry, say) is then dealt
// over the XCDs instead of piling onto some.  Returns the logical tile index
// g * group_tiles + t.  Other group counts fall back to xcd_remap.
__device__ __forceinline__ int xcd_group_remap(int bid, int nblocks, int group_tiles) {
  const int L = xcd_remap(bid, nblocks);
  const int groups = nblocks / group_tiles;
  if (groups % 8 != 0 || groups * group_tiles != nblocks) return L;
  const int per_xcd = (groups / 8) * group_tiles;  // tiles of one residue class
  const int r = L / per_xcd;                       // = the XCD, for L from xcd_remap
  const int w = L % per_xcd;
  return ((w / group_tiles) * 8 + r) * group_tiles + w % group_tiles;
}

// ---------------------------------------------------------------------------
// Persistent grids.  The dispatcher hands workgroups to the 8 XCDs round-robin and in
// launch order, so a workgroup waits for a free CU on its own XCD even when other
// XCDs have one free.  With tiles of very different lengths (causal masks) the CUs
// then idle between workgroups: traced per workgroup, a causal forward left 6-7 us
// between one workgroup's end and the next one's start on a CU, against 0.2 us when
// all tiles are equal.  A persistent grid (one workgroup per resident slot) launches
// everything at once and walks a fixed schedule instead:
//   - the logical tiles are cut into one contiguous block per XCD (the heads that
//     xcd_remap gives that XCD, for its L2), and the workgroups that launch order
//     places on that XCD share its block;
//   - they take it in rounds, one tile each per round, in snake order (reversed
//     every other round).  Tiles come longest first within a head, so a workgroup
//     that gets a long tile in one round gets a short one in the next: under a causal
//     mask each pair of rounds gives every workgroup about the same work.
// The schedule is a fixed function of the launch index: no state in memory, nothing
// shared between launches (streams and graph replays may overlap freely).
struct StaticSchedule {
  int base;   // first logical tile of this workgroup's block
  int count;  // tiles in the block
  int nw;     // workgroups sharing the block
  int w;      // this workgroup's place among them
  int round;  // rounds taken so far

  __host__ __device__ StaticSchedule(int total, int bid, int grid) {
    const int k = grid < 8 ? grid : 8;  // blocks (one per XCD)
    const int per = (total + k - 1) / k;
    const int x = bid % k;
    base = x * per;
    count = total - base < per ? total - base : per;
    if (count < 0) count = 0;
    nw = (grid - x + k - 1) / k;
    w = bid / k;
    round = 0;
  }
  // Next logical tile of this workgroup, or -1 when it has none left.
  __host__ __device__ int next() {
    const int j = round * nw + ((round & 1) ? nw - 1 - w : w);
    ++round;
    return j < count ? base + j : -1;
  }
};

// Global-memory accesses through pointers the compiler cannot tell are global (ones
// loaded from memory, such as fresh_kernel_args gives): plain dereferences of those
// become flat instructions, which also count against the LDS wait counter.
template <typename V>
__device__ __forceinline__ void store_global(void* p, const V& v) {
  *(__attribute__((address_space(1))) V*)p = v;
}
template <typename V>
__device__ __forceinline__ V load_global(const void* p) {
  return *(const __attribute__((address_space(1))) V*)p;
}

// The kernel's arguments (a struct passed as its only argument), loaded anew from the
// kernel-argument segment: the empty asm hides that the pointer does not change, so
// the loads are not hoisted out of the caller's loop.  A persistent grid reads them
// once per tile: kept from one tile to the next, they would hold scalar registers
// through the tile loop, and the compiler gives up the LDS read-ahead there to make
// room.
template <typename A>
__device__ __forceinline__ A fresh_kernel_args() {
  static_assert(sizeof(A) % 4 == 0, "argument struct of whole words");
  auto p = (const __attribute__((address_space(4))) uint32_t*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  A a;
  uint32_t* w = reinterpret_cast<uint32_t*>(&a);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(A) / 4); ++i) w[i] = p[i];
  return a;
}

}  // namespace osattn
