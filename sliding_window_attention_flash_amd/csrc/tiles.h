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

}  // namespace swa
