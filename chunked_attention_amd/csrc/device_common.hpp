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

// Rotary encoding of one 16-byte chunk of bf16 features (pairs p .. p+3 of a
// token) by the angles of a float32 table row: cs = (cos, sin) of the four
// pairs.  x' = x cos - y sin, y' = x sin + y cos, each product and the
// sum/difference rounded to float32 on its own (no fused multiply-add), then
// rounded to bf16 (nearest, ties to even).
struct RopeRow {
  float cs[8];
};
__device__ __forceinline__ RopeRow rope_row(const float* __restrict__ t) {
  const float4 t0 = *reinterpret_cast<const float4*>(t);
  const float4 t1 = *reinterpret_cast<const float4*>(t + 4);
  return RopeRow{{t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w}};
}
__device__ __forceinline__ uint4 rope8(uint4 x, const RopeRow& row) {
#pragma clang fp contract(off)
  const float* cs = row.cs;
  uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float xe = bf16_bits_to_float(w[p] & 0xFFFFu);
    const float xo = bf16_bits_to_float(w[p] >> 16);
    const float c = cs[2 * p], s = cs[2 * p + 1];
    // plain operators under contract(off): HIP's __fmul_rn is a plain
    // multiply defined outside this pragma, which the compiler would fuse
    const float ec = xe * c, os = xo * s, es = xe * s, oc = xo * c;
    const float re = ec - os;
    const float ro = es + oc;
    const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(re));
    const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(ro));
    w[p] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}
// the same with the table row read from t
__device__ __forceinline__ uint4 rope8(uint4 x, const float* __restrict__ t) {
  return rope8(x, rope_row(t));
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
