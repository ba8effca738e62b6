// K1: fused cache write.  Moves a chunk's K/V from the caller's token-major
// layout [rows][H][d] into a ring slot: K head-major [H][pitch][d] and V
// transposed per head and tiled by the attention kernel's step, [H][pitch/T]
// [d][T] with T = 32 keys (bf16) or 64 (fp8), so that the V operand of one
// step is one contiguous 8 KB block, as the K operand is; padded rows are
// zero-filled.  Within every group of 16
// keys the bf16 V columns are stored in the order kappa (swap of key-index
// bits 2 and 3), which is the order in which the attention kernel's score
// accumulator hands keys to the PV product.  The fp8 variant quantises to
// E4M3 with one float32 scale per (head, slot) and stores the V columns of
// every 64-key tile in the order pi that the fp8 kernel's 64-deep PV product
// needs.
//
// The cached state is the clean K/V of each generated chunk, kept for the
// chunks that follow (discuss.pytorch.kr "JoyAI-Video-Edit 소개", real-time
// deployment section: after generation the clean KV is cached; the pages'
// per-chunk table lists this save step as its own stage).
//
// With a rotation table the keys are stored rotary-encoded (the fused M-RoPE
// of the same page's architecture section; the angles come from the caller,
// the rounding is that of rope8: float32 then bf16).  fp8 rings quantise the
// rotated keys, their scale taken over the rotated values.
//
// HBM-bound: each element is read once and written once.  One workgroup
// handles 64 rows of one head (bf16 keys with a rotation table: 64/G rows of
// G heads, so that each table row is read once for G heads); V goes through
// LDS for the transpose.
#include "device_common.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace {

constexpr int kRowsPerBlock = kTileKeys;   // 64
constexpr int kThreads = 256;

// key stored in V column p of a tile: swap bits 2 and 3 (an involution)
__device__ __forceinline__ int kappa(int p) {
  return (p & ~0xC) | ((p & 4) << 1) | ((p & 8) >> 1);
}
// fp8 rings: key stored in V column p (0..63) of a 64-key tile, the order in
// which the fp8 attention kernel's accumulators hand keys to its 64-deep PV
// product (bit permutation: key bits 5,4,3,2 = p bits 4,3,2,5)
__device__ __forceinline__ int pi64(int p) {
  return ((p & 0x1C) << 1) | ((p & 0x20) >> 3) | (p & 3);
}

// ---------------------------------------------------------------- bf16 ----

// Transposed store of a block's V (64 keys of one head, staged in LDS rows of
// D + 2 features): the block's keys are two 32-key tiles; row dd of tile b
// gets its 32 keys (4 chunks of 8), in kappa order.
template <int D>
__device__ __forceinline__ void store_vt_bf16(const uint16_t* vtile, uint16_t* __restrict__ vtd,
                                              int h, int pitch, int r0, int tid) {
  constexpr int kLdsPitch = D + 2;
  for (int c = tid; c < D * 8; c += kThreads) {
    const int dd = c / 8;
    const int ch = c % 8;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = vtile[kappa(ch * 8 + 2 * j) * kLdsPitch + dd];
      const uint32_t hi = vtile[kappa(ch * 8 + 2 * j + 1) * kLdsPitch + dd];
      w[j] = lo | (hi << 16);
    }
    const int tile = (r0 >> 5) + (ch >> 2);
    st16(vtd + static_cast<size_t>(h) * D * pitch + (static_cast<size_t>(tile) * D + dd) * 32 +
             (ch & 3) * 8,
         make_uint4(w[0], w[1], w[2], w[3]));
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void cache_write_bf16(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int rows, int pitch,
    int heads, uint16_t* __restrict__ kd, uint16_t* __restrict__ vtd) {
  constexpr int kChunks = D / 8;         // 16-byte chunks per row
  constexpr int kLdsPitch = D + 2;       // u16 per LDS row; odd word count avoids conflicts
  __shared__ uint32_t vtile32[kRowsPerBlock * kLdsPitch / 2];
  uint16_t* vtile = reinterpret_cast<uint16_t*>(vtile32);

  const int h = blockIdx.y;
  const int r0 = blockIdx.x * kRowsPerBlock;
  const int tid = threadIdx.x;

  for (int c = tid; c < kRowsPerBlock * kChunks; c += kThreads) {
    const int row = c / kChunks;
    const int ch = c % kChunks;
    const int r = r0 + row;
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (r < rows) {
      const size_t src = (static_cast<size_t>(r) * heads + h) * D + ch * 8;
      kv = ld16(k + src);
      vv = ld16(v + src);
    }
    st16(kd + (static_cast<size_t>(h) * pitch + r) * D + ch * 8, kv);
    uint32_t* dst = reinterpret_cast<uint32_t*>(vtile + row * kLdsPitch + ch * 8);
    dst[0] = vv.x;
    dst[1] = vv.y;
    dst[2] = vv.z;
    dst[3] = vv.w;
  }
  __syncthreads();
  store_vt_bf16<D>(vtile, vtd, h, pitch, r0, tid);
}

// The same write for keys with a rotation table.  The table row of a token
// is the same for every head, so within each group of G heads (G divides
// H) the G workgroups over one block of 64 rows split the keys by rows, not
// by heads: workgroup (block, h) rotates rows g*64/G .. (g+1)*64/G - 1 of
// the block (g = h mod G) for all G heads of its group, reading each table
// row once for G heads.  V is handled per head as above.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void cache_write_bf16_rope(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int rows, int pitch,
    int heads, uint16_t* __restrict__ kd, uint16_t* __restrict__ vtd,
    const float* __restrict__ rope) {
  constexpr int kChunks = D / 8;
  constexpr int kLdsPitch = D + 2;
  constexpr int kRowsK = kRowsPerBlock / G;
  static_assert(kRowsPerBlock % G == 0, "row share per head group");
  __shared__ uint32_t vtile32[kRowsPerBlock * kLdsPitch / 2];
  uint16_t* vtile = reinterpret_cast<uint16_t*>(vtile32);

  const int h = blockIdx.y;
  const int r0 = blockIdx.x * kRowsPerBlock;
  const int tid = threadIdx.x;
  const int h0 = h - h % G;
  const int rk0 = r0 + (h % G) * kRowsK;

  for (int c = tid; c < kRowsK * kChunks; c += kThreads) {
    const int r = rk0 + c / kChunks;
    const int ch = c % kChunks;
    uint4 kv[G];
#pragma unroll
    for (int j = 0; j < G; ++j) kv[j] = make_uint4(0, 0, 0, 0);
    if (r < rows) {
#pragma unroll
      for (int j = 0; j < G; ++j) kv[j] = ld16(k + (static_cast<size_t>(r) * heads + h0 + j) * D + ch * 8);
      const RopeRow cs = rope_row(rope + (static_cast<size_t>(r) * (D / 2) + ch * 4) * 2);
#pragma unroll
      for (int j = 0; j < G; ++j) kv[j] = rope8(kv[j], cs);
    }
#pragma unroll
    for (int j = 0; j < G; ++j)
      st16(kd + (static_cast<size_t>(h0 + j) * pitch + r) * D + ch * 8, kv[j]);
  }
  for (int c = tid; c < kRowsPerBlock * kChunks; c += kThreads) {
    const int row = c / kChunks;
    const int ch = c % kChunks;
    const int r = r0 + row;
    uint4 vv = make_uint4(0, 0, 0, 0);
    if (r < rows) vv = ld16(v + (static_cast<size_t>(r) * heads + h) * D + ch * 8);
    uint32_t* dst = reinterpret_cast<uint32_t*>(vtile + row * kLdsPitch + ch * 8);
    dst[0] = vv.x;
    dst[1] = vv.y;
    dst[2] = vv.z;
    dst[3] = vv.w;
  }
  __syncthreads();
  store_vt_bf16<D>(vtile, vtd, h, pitch, r0, tid);
}

// ----------------------------------------------------------------- fp8 ----

// E4M3 codes of two float32 values (byte 0: a, byte 1: b): nearest, ties to
// even, saturating at +-448, NaN -> 0x7F with the sign kept, taken by the
// hardware conversion (nearest-even on finite values up to 448) after an
// explicit saturation.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  const float ca = fminf(fmaxf(a, -448.0f), 448.0f);
  const float cb = fminf(fmaxf(b, -448.0f), 448.0f);
  uint32_t r = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false)) & 0xFFFFu;
  if (a != a) r = (r & 0xFF00u) | ((__float_as_uint(a) >> 24) & 0x80u) | 0x7Fu;
  if (b != b) r = (r & 0x00FFu) | (((__float_as_uint(b) >> 24) & 0x80u) | 0x7Fu) << 8;
  return r;
}
// x / s for the quantiser, from r = 1/s (correctly rounded): y = x r, the
// residual x - s y in one fused multiply-add, and one correction step y +
// r (x - s y), with the sign of x (so that -0 stays -0).  This is not always
// the correctly rounded quotient (the residual can underflow for tiny x), but
// its E4M3 code is: an exhaustive check on MI355X over every bf16 x with
// |x| <= amax and every bf16 amax found different codes only for amax below
// 2^-104.  The caller uses it for scales s >= 2^-108 (amax >= 2^-100) and
// finite; anything else takes the exact division.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
#pragma clang fp contract(off)
  const float y = x * r;
  const float e = fmaf(-s, y, x);
  return copysignf(fmaf(e, r, y), x);
}
__device__ __forceinline__ bool fast_scale(float s) {
  return s >= 0x1p-108f && s <= 0x1p+120f;
}

// Pass 1: per (head, 64-row block) largest magnitude of K and of V.

template <int D>
__global__ __launch_bounds__(kThreads) void cache_amax_fp8(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int rows, int heads,
    float* __restrict__ partial /* [2][H][nblk] */, const float* __restrict__ rope) {
  constexpr int kChunks = D / 8;
  __shared__ float red[2][kThreads / 64];
  const int h = blockIdx.y;
  const int r0 = blockIdx.x * kRowsPerBlock;
  const int nblk = gridDim.x;
  const int tid = threadIdx.x;
  float ak = 0.f, av = 0.f;
  for (int c = tid; c < kRowsPerBlock * kChunks; c += kThreads) {
    const int r = r0 + c / kChunks;
    if (r >= rows) break;
    const size_t src = (static_cast<size_t>(r) * heads + h) * D + (c % kChunks) * 8;
    uint4 kv = ld16(k + src);
    const uint4 vv = ld16(v + src);
    if (rope) kv = rope8(kv, rope + (static_cast<size_t>(r) * (D / 2) + (c % kChunks) * 4) * 2);
    const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
    const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ak = fmaxf(ak, fabsf(bf16_bits_to_float(kw[j] & 0xFFFFu)));
      ak = fmaxf(ak, fabsf(bf16_bits_to_float(kw[j] >> 16)));
      av = fmaxf(av, fabsf(bf16_bits_to_float(vw[j] & 0xFFFFu)));
      av = fmaxf(av, fabsf(bf16_bits_to_float(vw[j] >> 16)));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    ak = fmaxf(ak, __shfl_xor(ak, off));
    av = fmaxf(av, __shfl_xor(av, off));
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = ak;
    red[1][tid >> 6] = av;
  }
  __syncthreads();
  if (tid == 0) {
    float mk = 0.f, mv = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) {
      mk = fmaxf(mk, red[0][w]);
      mv = fmaxf(mv, red[1][w]);
    }
    partial[(0 * heads + h) * nblk + blockIdx.x] = mk;
    partial[(1 * heads + h) * nblk + blockIdx.x] = mv;
  }
}

// Pass 2: reduce the partials of the head, derive s = amax / 448 (float32,
// correctly rounded; 1 when amax = 0), write E4M3 codes of x / s.

template <int D>
__global__ __launch_bounds__(kThreads) void cache_quant_fp8(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int rows, int pitch,
    int heads, int nblk_rows, const float* __restrict__ partial, uint8_t* __restrict__ kd,
    uint8_t* __restrict__ vtd, float* __restrict__ k_scale, float* __restrict__ v_scale,
    const float* __restrict__ rope) {
  constexpr int kChunks = D / 8;         // 8-element chunks per row
  constexpr int kLdsPitch = D + 4;       // bytes per LDS row of codes
  __shared__ __attribute__((aligned(16))) uint8_t vtile[kRowsPerBlock * kLdsPitch];
  __shared__ float sc[2];
  const int h = blockIdx.y;
  const int r0 = blockIdx.x * kRowsPerBlock;
  const int tid = threadIdx.x;

  if (tid < 64) {
    float mk = 0.f, mv = 0.f;
    for (int b = tid; b < nblk_rows; b += 64) {
      mk = fmaxf(mk, partial[(0 * heads + h) * nblk_rows + b]);
      mv = fmaxf(mv, partial[(1 * heads + h) * nblk_rows + b]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      mk = fmaxf(mk, __shfl_xor(mk, off));
      mv = fmaxf(mv, __shfl_xor(mv, off));
    }
    if (tid == 0) {
      const float sk = mk > 0.f ? __fdiv_rn(mk, 448.0f) : 1.0f;
      const float sv = mv > 0.f ? __fdiv_rn(mv, 448.0f) : 1.0f;
      sc[0] = sk;
      sc[1] = sv;
      if (blockIdx.x == 0) {
        k_scale[h] = sk;
        v_scale[h] = sv;
      }
    }
  }
  __syncthreads();
  const float sk = sc[0], sv = sc[1];
  // x / s: reciprocal and one correction step when the scale allows it
  // (uniform per head), else the correctly rounded division
  const bool fast = fast_scale(sk) && fast_scale(sv);
  const float rk = __fdiv_rn(1.0f, sk), rv = __fdiv_rn(1.0f, sv);
  // the rows, encoded with one of the two divisions (chosen once, so that
  // the loop body is one straight block)
  auto encode = [&](auto fast_tag) {
    constexpr bool kFast = decltype(fast_tag)::value;
    auto qk = [&](float x) { return kFast ? div_by_scale(x, sk, rk) : __fdiv_rn(x, sk); };
    auto qv = [&](float x) { return kFast ? div_by_scale(x, sv, rv) : __fdiv_rn(x, sv); };
    for (int c = tid; c < kRowsPerBlock * kChunks; c += kThreads) {
      const int row = c / kChunks;
      const int ch = c % kChunks;
      const int r = r0 + row;
      uint32_t kc[2] = {0u, 0u}, vc[2] = {0u, 0u};
      if (r < rows) {
        const size_t src = (static_cast<size_t>(r) * heads + h) * D + ch * 8;
        uint4 kv = ld16(k + src);
        const uint4 vv = ld16(v + src);
        if (rope) kv = rope8(kv, rope + (static_cast<size_t>(r) * (D / 2) + ch * 4) * 2);
        const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
        const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t k01 = e4m3x2(qk(bf16_bits_to_float(kw[j] & 0xFFFFu)),
                                      qk(bf16_bits_to_float(kw[j] >> 16)));
          const uint32_t v01 = e4m3x2(qv(bf16_bits_to_float(vw[j] & 0xFFFFu)),
                                      qv(bf16_bits_to_float(vw[j] >> 16)));
          kc[j >> 1] |= k01 << (16 * (j & 1));
          vc[j >> 1] |= v01 << (16 * (j & 1));
        }
      }
      *reinterpret_cast<uint2*>(kd + (static_cast<size_t>(h) * pitch + r) * D + ch * 8) =
          make_uint2(kc[0], kc[1]);
      // LDS rows are 4-byte aligned only: two 32-bit stores
      uint32_t* vdst = reinterpret_cast<uint32_t*>(vtile + row * kLdsPitch + ch * 8);
      vdst[0] = vc[0];
      vdst[1] = vc[1];
    }
  };
  if (fast)
    encode(std::true_type{});
  else
    encode(std::false_type{});
  __syncthreads();
  // transposed store: the block is one 64-key tile; row dd gets its 64
  // keys (4 chunks of 16)
  for (int c = tid; c < D * 4; c += kThreads) {
    const int dd = c / 4;
    const int ch = c % 4;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t x = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        x |= static_cast<uint32_t>(vtile[pi64(ch * 16 + 4 * j + b) * kLdsPitch + dd]) << (8 * b);
      w[j] = x;
    }
    st16(vtd + static_cast<size_t>(h) * D * pitch + (static_cast<size_t>(r0 >> 6) * D + dd) * 64 +
             ch * 16,
         make_uint4(w[0], w[1], w[2], w[3]));
  }
}

template <int D>
kvc_status launch_write(const CacheWriteDesc& d, hipStream_t s) {
  const dim3 block(kThreads);
  const dim3 grid(d.pitch / kRowsPerBlock, d.heads);
  if (d.kv_dtype == KVC_KV_BF16) {
    const uint16_t* k = static_cast<const uint16_t*>(d.k);
    const uint16_t* v = static_cast<const uint16_t*>(d.v);
    uint16_t* kd = static_cast<uint16_t*>(d.k_dst);
    uint16_t* vtd = static_cast<uint16_t*>(d.vt_dst);
    if (!d.rope)
      hipLaunchKernelGGL(cache_write_bf16<D>, grid, block, 0, s, k, v, d.rows, d.pitch, d.heads,
                         kd, vtd);
    else if (d.heads % 4 == 0)
      hipLaunchKernelGGL((cache_write_bf16_rope<D, 4>), grid, block, 0, s, k, v, d.rows, d.pitch,
                         d.heads, kd, vtd, d.rope);
    else if (d.heads % 2 == 0)
      hipLaunchKernelGGL((cache_write_bf16_rope<D, 2>), grid, block, 0, s, k, v, d.rows, d.pitch,
                         d.heads, kd, vtd, d.rope);
    else
      hipLaunchKernelGGL((cache_write_bf16_rope<D, 1>), grid, block, 0, s, k, v, d.rows, d.pitch,
                         d.heads, kd, vtd, d.rope);
  } else {
    const int nblk = (d.rows + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(cache_amax_fp8<D>, dim3(nblk, d.heads), block, 0, s,
                       static_cast<const uint16_t*>(d.k), static_cast<const uint16_t*>(d.v),
                       d.rows, d.heads, d.scratch, d.rope);
    hipLaunchKernelGGL(cache_quant_fp8<D>, grid, block, 0, s,
                       static_cast<const uint16_t*>(d.k), static_cast<const uint16_t*>(d.v),
                       d.rows, d.pitch, d.heads, nblk, d.scratch,
                       static_cast<uint8_t*>(d.k_dst), static_cast<uint8_t*>(d.vt_dst),
                       d.k_scale, d.v_scale, d.rope);
  }
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_E_DEVICE;
}

}  // namespace

kvc_status launch_cache_write(const CacheWriteDesc& d, void* stream) {
  if (d.rows <= 0 || d.pitch % kRowsPerBlock || d.pitch < d.rows) return KVC_E_INVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d.head_dim) {
    case 64: return launch_write<64>(d, s);
    case 128: return launch_write<128>(d, s);
    default: return KVC_E_UNSUPPORTED;
  }
}

}  // namespace kvc
