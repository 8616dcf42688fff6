// Global loads, block numbering and the swizzled LDS tile layout shared by
// the per-tile backward kernels and the forward (gfx950).
#pragma once

#include "common.h"

namespace swa {

// Loads 8 contiguous 16-bit elements (16 bytes) from global memory.
template <typename T>
__device__ __forceinline__ typename Elem<T>::vec8 ld8(const T* p) {
  return *reinterpret_cast<const typename Elem<T>::vec8*>(p);
}
template <typename T>
__device__ __forceinline__ void st8(T* p, const typename Elem<T>::vec8& v) {
  *reinterpret_cast<typename Elem<T>::vec8*>(p) = v;
}

// 16 bytes from global memory straight into LDS: lane l of the wave writes
// bytes [16 l, 16 l + 16) after the wave-uniform LDS address `lds`.  (A
// plain function: called with dependent pointer types inside a kernel
// template, the builtin keeps the host pass from emitting the launch stub.)
__device__ __forceinline__ void ld16_to_lds(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

// Row `row` (>= 0) of a tensor whose row stride fits in 32 bits (checked
// when a plan is made): one 32 x 32 -> 64-bit multiply-add.
template <typename T>
__device__ __forceinline__ const T* row_at(const T* base, int row, int64_t stride) {
  return base + (uint64_t)(uint32_t)row * (uint32_t)stride;
}
template <typename T>
__device__ __forceinline__ T* row_at(T* base, int row, int64_t stride) {
  return base + (uint64_t)(uint32_t)row * (uint32_t)stride;
}

// Blocks are dealt to the 8 XCDs round-robin; renumber them so that each XCD
// runs one contiguous range of logical tiles (neighbouring tiles of one head
// then share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int base = n >> 3, extra = n & 7;
  return xcd * base + (xcd < extra ? xcd : extra) + slot;
}

// Tiles are row-major with the 16-byte chunks of row r permuted by XOR with
// (r mod 8) (64-wide rows) or 2 (r mod 8) (128-wide rows, moving whole
// 32-byte pairs): the 8 rows a half-wave's transposed read touches then
// fall on disjoint banks, and so do the 16 rows of a row read.
template <int D>
__device__ __forceinline__ int tsw(int r) { return D == 64 ? (r & 7) : ((r & 7) << 1); }
// element offset of (row r, 16-byte chunk ch) in a D-wide swizzled tile
template <int D>
__device__ __forceinline__ int toff(int r, int ch) { return r * D + ((ch ^ tsw<D>(r)) << 3); }
// lane offset of a transposed read: row 4 g + c / 4, column 16 cb + 4 (c % 4)
template <int D>
__device__ __forceinline__ int troff(int c, int g, int cb) {
  const int r = 4 * g + (c >> 2);
  return r * D + (((2 * cb + ((c & 3) >> 1)) ^ tsw<D>(r)) << 3) + 4 * (c & 1);
}

// ds_read_b64_tr_b16: the lane at row r0 + i / 4, column c0 + 4 (i % 4) of
// a 16-lane group receives rows r0..r0+3 of column c0 + i.
typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));
template <typename T>
__device__ __forceinline__ u32x2 ldtr(const T* p) {
  v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  return __builtin_bit_cast(u32x2, v);
}
// 8 contraction values for lane (c, g): e < 4 from the read at p0, e >= 4
// from p1 -- the layout that pairs with two stacked 16-row accumulator tiles
// used as the other operand (rows 4 g..4 g + 3 of each)
template <typename T>
__device__ __forceinline__ typename Elem<T>::vec8 trpair(const T* p0, const T* p1) {
  const u32x2 lo = ldtr(p0), hi = ldtr(p1);
  return __builtin_bit_cast(typename Elem<T>::vec8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Max / sum over the 4 lanes c, c + 16, c + 32, c + 48 of a wave, in every
// one of them: v_permlane16_swap exchanges 16-lane rows 2k + 1 of its first
// operand and 2k of its second, v_permlane32_swap the upper half of the
// first and the lower half of the second; given two copies of x, each pair
// of results holds both operands of a butterfly step (in the same order in
// every lane).  The second copy is made opaque: the compiler otherwise takes
// the two results of a swap of equal operands to be equal, and drops the
// step.
__device__ __forceinline__ void swap_pair(unsigned (&r)[2], float x, bool halves) {
  unsigned y = __builtin_bit_cast(unsigned, x);
  asm volatile("" : "+v"(y));
  const auto a = halves ? __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), y, false, false)
                        : __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), y, false, false);
  r[0] = a[0];
  r[1] = a[1];
}
__device__ __forceinline__ float col4_max(float x) {
  unsigned r[2];
  swap_pair(r, x, false);
  x = fmaxf(__builtin_bit_cast(float, r[0]), __builtin_bit_cast(float, r[1]));
  swap_pair(r, x, true);
  return fmaxf(__builtin_bit_cast(float, r[0]), __builtin_bit_cast(float, r[1]));
}
__device__ __forceinline__ float col4_sum(float x) {
  unsigned r[2];
  swap_pair(r, x, false);
  x = __builtin_bit_cast(float, r[0]) + __builtin_bit_cast(float, r[1]);
  swap_pair(r, x, true);
  return __builtin_bit_cast(float, r[0]) + __builtin_bit_cast(float, r[1]);
}

// Sums over 8 (16) consecutive lanes, in every one of them, by DPP (no LDS
// traffic): swaps within quads, then the mirror of each half-row, which pairs
// the two quads (and of the row, which pairs the two halves).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lanes8_sum(float x) { return dpp_add<0x141>(dpp_add<0x4E>(dpp_add<0xB1>(x))); }
__device__ __forceinline__ float lanes16_sum(float x) { return dpp_add<0x140>(lanes8_sum(x)); }

}  // namespace swa
