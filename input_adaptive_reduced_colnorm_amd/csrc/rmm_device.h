// Device-side helpers shared by the RMM kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmm {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned long long)))) unsigned long long u64x2;

// Fourth descriptor word of a raw buffer resource on gfx9-family parts
// (32-bit data format, no swizzle): loads past num_records return zero.
constexpr int kBufferFlags = 0x00020000;
// Byte offset that is always past num_records (num_records < 2^31 is enforced
// by the host), so a load through it yields zeros.
constexpr uint32_t kOobOffset = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}

__device__ __forceinline__ i32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ i32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a buffer straight into LDS: lane l writes LDS bytes
// [dst + 16 l, dst + 16 l + 16) (dst uniform across the wave); an offset past
// the buffer end writes zeros.  Completion is counted by vmcnt.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, lds_void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}

// The same direct load issued from inline asm, for loops whose LDS reads
// must not wait for it: the compiler makes every LDS access wait for the
// direct loads it knows of (it cannot tell which LDS bytes they write), so
// a prefetch it sees would drain before each read.  The compiler neither
// sees nor counts this load; that only makes its own vmcnt waits stricter
// (the load lands in the in-order queue beside the ones it counts), and the
// caller orders the load's LDS bytes with wait_vmcnt and a barrier.  rsrc:
// buffer descriptor words (wave-uniform); lds: LDS byte address of lane 0
// (wave-uniform).  The nops cover the M0 and SGPR-to-VMEM read hazards.
__device__ __forceinline__ void load_lds16_async(i32x4 rsrc, uint32_t lds, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}

// Descriptor words of a raw buffer of `bytes` bytes at `base` (as make_rsrc).
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)((a >> 32) & 0xffffu), (int)bytes, kBufferFlags};
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// wait until at most N vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for data exchanged through LDS only: this wave's LDS
// accesses are complete (lgkmcnt(0); direct loads that must land are waited
// for by the caller), then s_barrier.  A release fence (as in
// __syncthreads) would also wait for every vector-memory access still in
// flight, prefetches included; the empty asm statements keep the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A row piece of 8 B-matrix elements while in flight: 8 bf16 (16 bytes) or
// 8 int8 weights (8 bytes).
template <bool I8> struct RowPiece { typedef i32x4 type; };
template <> struct RowPiece<true> { typedef i32x2 type; };

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round-to-nearest-even float -> bf16 (inputs are finite on every path that
// uses this; NaN is kept a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

// XOR swizzle of 16-byte chunks inside a 128-byte LDS row: makes both the
// row-wise fills and the 32-row MFMA operand reads free of bank conflicts.
__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row ^ (row >> 3)) & 7);
}

// 8 int8 values (two dwords, byte i = value i) -> 8 bf16 (four dwords, value
// 2w in the low half of dword w).  Exact: an int8 needs at most 8
// significant bits, which bf16 holds.  No integer-to-float conversion is
// used (the compiler folds a byte extract plus a signed conversion into an
// unsigned one that turns negative bytes into 2^32 - |q|): each byte b is
// offset to u = b ^ 0x80 in [0, 255] and placed under the exponent of
// 2^23, so the float is 2^23 + u exactly, and subtracting 2^23 + 128 gives
// the signed value q = u - 128 exactly.
__device__ __forceinline__ i32x4 i8x8_to_bf16x8(i32x2 v) {
  i32x4 o;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t u = (uint32_t)v[h] ^ 0x80808080u;
    float f[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      // bytes (low to high): u.byte b, 0x00, 0x00, 0x4B  ->  2^23 + u_b
      const uint32_t bits = __builtin_amdgcn_perm(0x4B000000u, u, 0x070c0c00u | (uint32_t)b);
      f[b] = __uint_as_float(bits) - 8388736.0f;
    }
    o[2 * h] = (int)__builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
    o[2 * h + 1] = (int)__builtin_amdgcn_perm(__float_as_uint(f[3]), __float_as_uint(f[2]), 0x07060302u);
  }
  return o;
}

// 8x8 transpose of bf16 held as 8 rows x 4 dwords: out[c] holds column c
// (the 8 values along the former rows) as 4 dwords, i.e. the 8-deep K run
// of one column that a matrix-core operand lane takes.
__device__ __forceinline__ void transpose8x8(const i32x4 (&in)[8], i32x4 (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = (uint32_t)in[2 * p][c >> 1];
      const uint32_t hi = (uint32_t)in[2 * p + 1][c >> 1];
      out[c][p] = (int)__builtin_amdgcn_perm(hi, lo, sel);
    }
  }
}

}  // namespace rmm
