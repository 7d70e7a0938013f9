// Device-side building blocks shared by the MoBA kernels (gfx950, wave64).
//
// Matrix-core convention used everywhere: one "k16 step" is a 32x32 output tile
// updated with a contraction of 16. For bf16 it is one v_mfma_f32_32x32x16_bf16;
// for fp32 it is eight v_mfma_f32_32x32x2_f32 over the same register data. In
// both cases lane l supplies, for operand A (32 x 16, row-major m x k),
// A[l % 32][8 * (l / 32) + e] for e = 0..7, and for operand B (16 x 32),
// B[8 * (l / 32) + e][l % 32]. The 16 accumulator floats of lane l hold
// C[8 * (i / 4) + 4 * (l / 32) + (i % 4)][l % 32], i = 0..15.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moba {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// Eight consecutive elements of the contraction dimension for one lane.
template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ f32x16 mma_k16(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mma_k16(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

// 16-byte vector loads/stores of "8 elements" (bf16: one 16 B access; fp32: two).
__device__ __forceinline__ bf16x8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 load8(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f32x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Streaming (non-temporal) variants for data read once, so that it does not
// push reusable K/V lines out of L2.
__device__ __forceinline__ bf16x8 load8_stream(const bf16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
}
__device__ __forceinline__ f32x8 load8_stream(const float* p) {
  f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  f32x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Eight consecutive partial-output values, read once (non-temporal), as fp32.
__device__ __forceinline__ void load8_part(const f16* p, float (&x)[8]) {
  typedef f16 f16x8 __attribute__((ext_vector_type(8)));
  const f16x8 v = __builtin_nontemporal_load(reinterpret_cast<const f16x8*>(p));
#pragma unroll
  for (int b = 0; b < 8; ++b) x[b] = (float)v[b];
}
__device__ __forceinline__ void load8_part(const float* p, float (&x)[8]) {
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
#pragma unroll
  for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
}

template <typename T> __device__ __forceinline__ T zero8();
template <> __device__ __forceinline__ bf16x8 zero8<bf16x8>() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
  return z;
}
template <> __device__ __forceinline__ f32x8 zero8<f32x8>() {
  f32x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = 0.0f;
  return z;
}

// Storage type of the per-part partial outputs: fp16 for bf16 inputs (normalised
// outputs are bounded by max |v|, so fp16's range is ample and its rounding is 4x
// finer than bf16's), fp32 for fp32 inputs.
template <typename T> struct PartType { typedef float type; };
template <> struct PartType<bf16> { typedef f16 type; };

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }     // RNE

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float swap_half(float x) { return __shfl_xor(x, 32, kWave); }
__device__ __forceinline__ int swap_half(int x) { return __shfl_xor(x, 32, kWave); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// IEEE 754-2019 maximum (NaN-propagating); gfx950 has a 3-input form, and unlike
// fmaxf it needs no canonicalising of its operands.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Workgroups are dispatched to the 8 XCDs round-robin (id % 8). Remap the
// dispatch id so that each XCD walks one contiguous range of logical tiles:
// neighbouring tiles (which share K/V or pooled keys) then share that XCD's L2.
// `padded` is the launched grid size, a multiple of 8.
__device__ __forceinline__ int64_t xcd_logical(int64_t id, int64_t padded) {
  return (id & 7) * (padded >> 3) + (id >> 3);
}

// Sequence index n with cu[n] <= tok < cu[n+1]; empty sequences are skipped.
__device__ __forceinline__ int seq_of_token(const int32_t* cu, int nseq, int64_t tok) {
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Largest index L in [0, n) with offs[L] <= x (offs ascending, offs[0] = 0).
__device__ __forceinline__ int upper_index(const int32_t* offs, int n, int64_t x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)offs[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// upper_index by the whole wave (x wave-uniform, every lane calls it): each round
// reads 64 evenly spaced entries of the range that holds the answer in one vector
// load, and the highest lane whose entry is <= x narrows the range to one stride,
// so n <= 4096 takes two dependent loads where the binary search takes twelve.
// Needs offs[0] <= x. Same result as upper_index.
__device__ __forceinline__ int upper_index_wave(const int32_t* offs, int n, int64_t x,
                                                int lane) {
  int lo = 0, len = n;                       // the answer lies in [lo, lo + len)
  while (len > 1) {
    const int step = (len + 63) / 64;
    const bool in = lane * step < len;
    const bool ok = in && (int64_t)offs[min(lo + lane * step, n - 1)] <= x;
    const uint64_t m = __ballot(ok);         // a prefix of the lanes; bit 0 is set
    const int hl = 63 - __clzll((unsigned long long)m);
    lo += hl * step;
    len = min(step, len - hl * step);
  }
  return lo;
}

// Eight fp32 values as one MFMA operand fragment of the input type.
template <typename T> __device__ __forceinline__ typename Frag<T>::type pack8(const float* x);
template <> __device__ __forceinline__ bf16x8 pack8<bf16>(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)x[e];
  return r;
}
template <> __device__ __forceinline__ f32x8 pack8<float>(const float* x) {
  f32x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = x[e];
  return r;
}

// Transposed copies of a matrix whose rows are the k index of an MFMA with a
// register operand from the 32x32 accumulator layout (P^T, dS^T, P, dS): lane
// l holds, per 16-row group, rows {4h..4h+3} and {8+4h..8+4h+3} (h = l / 32),
// and the operand wants k index 8h + e at element e. So inside each group of 16
// rows the transposed copy stores the four-row groups in the order 0, 2, 1, 3,
// i.e. bits 2 and 3 of the row index are swapped. Returns the position of the
// first row of four-row group kg (= row / 4).
__device__ __forceinline__ int vt_pos_of_group4(int kg) {
  return 16 * (kg >> 2) + 8 * (kg & 1) + 4 * ((kg >> 1) & 1);
}

// ---------------------------------------------------------------------------
// 16-bit inputs: K and V chunks go straight from global memory into LDS with
// gfx950's direct loads (global_load_lds_dwordx4: lane i's 16 bytes land at
// base + 16 i), so no registers hold chunks in flight and three chunks can be
// outstanding. Both are stored row-major, 256-byte rows (D = 128) of sixteen
// 16-byte pieces; piece p of row r sits at position p ^ swz(r). gfx950's LDS
// has 64 four-byte banks (one 256-byte row) and serves 16 lanes of a 16-byte
// read, or 32 lanes of an 8-byte read, per clock. The K reads put 16
// consecutive rows in one clock (swz must be a bijection on 0..15); the V^T
// reads put four pieces of each of 4 consecutive rows in one clock (the four
// rows must land in different piece quads). Transposing the row index's two
// 2-bit halves satisfies both. V^T fragments are
// read with ds_read_b64_tr_b16: within each 16-lane group, lane i receives
// element i % 4 of the 8-byte reads of lanes i/4, i/4+4, i/4+8, i/4+12, so
// pointing the group at a 4-row x 16-column block of V gives lane i column i of
// those four rows: four consecutive keys of one head dimension.
__device__ __forceinline__ int swz(int r) {
  return ((r & 3) << 2) | ((r >> 2) & 3);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One direct global->LDS load of 16 bytes per lane (lane i's bytes land at
// lds + 16 i). Issued from inline assembly so that the compiler, unaware of
// these LDS writes, does not pad every later LDS read with conservative waits;
// the caller orders them with an explicit vmcnt wait and a barrier. No register
// receives data, so nothing is left in flight in a register.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("global_load_lds_dwordx4 %1, off"
               :
               : "{m0}"(__builtin_amdgcn_readfirstlane(lds)), "v"(g)
               : "memory");
#endif
}

// The same direct load with the address split into a wave-uniform 64-bit base
// (read into SGPRs: it must be the same in every lane of the wave) and a 32-bit
// per-lane byte offset: a loop whose offsets are invariant then spends no vector
// instruction on addresses.
// When the base is held in VGPRs (it depends on the wave index) the compiler
// moves it to SGPRs with v_readfirstlane, a vector-ALU write of SGPRs, and a
// memory instruction may read such SGPRs only five wait states later. The
// compiler keeps that distance before its own memory instructions but cannot
// see into this asm (read sooner, the load took a stale base and faulted), so
// the first load from a newly formed base waits itself (kWait: s_nop 4); the
// following loads from the same base come after it. A host test compiles the
// kernels and checks that every such load has its five states.
template <bool kWait>
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint64_t b = (uint64_t)base;
  const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  if constexpr (kWait)
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "{m0}"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sb)
                 : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %1, %2"
                 :
                 : "{m0}"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sb)
                 : "memory");
#endif
}

// Lane i gets x of lane i ^ 32 (the other half of the wave), by the gfx950
// cross-half swap on the vector ALU rather than an LDS permute.
__device__ __forceinline__ float swap_half_valu(float x, int lane) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (lane < 32) ? r[1] : r[0]);
}

// Division of n in [0, 2^31) by a divisor d >= 1 fixed for a launch, as a
// multiply-high, an add and a shift (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994: the round-up multiplier with
// s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1; t + n cannot overflow
// because n < 2^31). Built on the host by make_fastdiv.
struct FastDiv {
  uint32_t m = 1, s = 0;
};
inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  if (d <= 1) return f;                            // m = 1, s = 0: n itself
  uint32_t sh = 0;
  while ((1ull << sh) < d) ++sh;
  f.s = sh;
  f.m = (uint32_t)((((1ull << sh) - d) << 32) / d + 1);
  return f;
}
__host__ __device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  const uint32_t hi = (uint32_t)(((uint64_t)n * f.m) >> 32);   // v_mul_hi_u32 on the GPU
  return (hi + n) >> f.s;
}

// A bare s_barrier (the host pass of the compiler sees only an empty body).
__device__ __forceinline__ void bare_barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_barrier" ::: "memory");
#endif
}

// s_waitcnt with vmcnt(n) (n < 64) and lgkmcnt(0), expcnt untouched (gfx9 encoding).
#define MOBA_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (((n) >> 4) << 14))

// One direct global->LDS load of 4 bytes per lane (lane i's dword lands at
// lds + 4 i); same conventions as dma16.
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("global_load_lds_dword %1, off"
               :
               : "{m0}"(__builtin_amdgcn_readfirstlane(lds)), "v"(g)
               : "memory");
#endif
}

}  // namespace moba
