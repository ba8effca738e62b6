// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>
#include <utility>

namespace kvc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kNumXcd = 8;   // MI355X: 8 accelerator complex dies, 32 CUs each

// The dispatcher hands workgroups to the XCDs round-robin (linear id mod 8).
// Remap so that each XCD receives a contiguous range of logical work ids:
// consecutive ids (the query tiles of one head) then share one L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int nblk) {
  const int xcd = bid % kNumXcd;
  const int slot = bid / kNumXcd;
  const int per = nblk / kNumXcd;
  const int rem = nblk % kNumXcd;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(void* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace kvc
