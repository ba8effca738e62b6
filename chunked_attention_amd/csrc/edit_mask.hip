// LiveEdit's active-row mask (aitrends.kr, "LiveEdit 실시간 Diffusion 기반
// 스트리밍 비디오 편집", the AR-oriented Mask Cache paragraphs of the
// methodology and technical-detail sections): for the next chunk, a token is
// recomputed only where the previous chunk's edited latent differs from its
// source latent by more than a threshold in L2 distance; the threshold is
// set dynamically so that about 70% of the tokens are pruned.  The pruned
// rows keep their cached outputs.
//
// Output: the active token indices in increasing order (the row map of an
// active-row attention call) and their count, both in device memory, so the
// next kernel on the stream can size its work without a host round trip.
//
// One workgroup of 1024 threads does it all (a chunk has at most 16384
// tokens; the work is microseconds next to the attention it feeds):
//   1. squared distance of every token into LDS (float64, channels summed in
//      order, every operation rounded on its own, so a plain CPU loop gets
//      the same bits);
//   2. threshold mode: flag distances above tau^2.  Top-k mode: radix-select
//      the keep-th largest distance over its 64-bit order-preserving key
//      (eight 8-bit digit passes with an LDS histogram), flag every larger
//      key and, among keys equal to it, the lowest indices up to keep;
//   3. compact: thread t owns tokens 16t .. 16t+15; a prefix sum of the flag
//      counts gives each thread its output position.
#include "device_common.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace {

constexpr int kThreads = 1024;
constexpr int kPerThread = KVC_MAX_MASK_TOKENS / kThreads;   // 16
static_assert(kPerThread <= 32, "flags of a thread fit one word");

// acc + (e - s)^2 in float64 for one channel (bf16 bit patterns), each
// operation rounded on its own
__device__ __forceinline__ double add_sq(double acc, uint32_t e, uint32_t s) {
#pragma clang fp contract(off)
  const double d = static_cast<double>(bf16_bits_to_float(e)) -
                   static_cast<double>(bf16_bits_to_float(s));
  const double sq = d * d;
  return acc + sq;
}

// sum_c (e_c - s_c)^2 for one token, float64, channels in order; NaN -> -1
// (a NaN distance is never above the threshold and ranks last).  `vec`:
// rows are whole 16-byte chunks (8 channels), read 16 bytes at a time.
__device__ double distance_sq(const uint16_t* __restrict__ zs, const uint16_t* __restrict__ ze,
                              int channels, int token, bool vec) {
  const uint16_t* s = zs + static_cast<size_t>(token) * channels;
  const uint16_t* e = ze + static_cast<size_t>(token) * channels;
  double acc = 0.0;
  if (vec) {
    for (int c = 0; c < channels; c += 8) {
      const uint4 ev = ld16(e + c), sv = ld16(s + c);
      const uint32_t ew[4] = {ev.x, ev.y, ev.z, ev.w};
      const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc = add_sq(acc, ew[q] & 0xFFFFu, sw[q] & 0xFFFFu);
        acc = add_sq(acc, ew[q] >> 16, sw[q] >> 16);
      }
    }
  } else {
    for (int c = 0; c < channels; ++c) acc = add_sq(acc, e[c], s[c]);
  }
  return acc != acc ? -1.0 : acc;
}

// unsigned key with the order of the float64 value
__device__ __forceinline__ unsigned long long order_key(double d) {
  const unsigned long long u = __double_as_longlong(d);
  return (u >> 63) ? ~u : (u | (1ULL << 63));
}

// exclusive prefix sum of v over the workgroup (Hillis-Steele in LDS); also
// returns the total
__device__ int exclusive_scan(int v, int (&buf)[kThreads], int& total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  total = buf[kThreads - 1];
  const int incl = buf[tid];
  __syncthreads();
  return incl - v;
}

template <bool kTopK>
__global__ __launch_bounds__(kThreads) void edit_mask_kernel(
    const uint16_t* __restrict__ zs, const uint16_t* __restrict__ ze, int tokens, int channels,
    double tau2, int keep, bool vec, int* __restrict__ rows, int* __restrict__ count) {
  __shared__ double dist[KVC_MAX_MASK_TOKENS];
  __shared__ int scan[kThreads];
  __shared__ unsigned hist[256];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_need;
  const int tid = threadIdx.x;
  for (int i = tid; i < tokens; i += kThreads) dist[i] = distance_sq(zs, ze, channels, i, vec);
  __syncthreads();

  const int lo = tid * kPerThread;
  unsigned flags = 0;
  if constexpr (!kTopK) {
    for (int j = 0; j < kPerThread; ++j)
      if (lo + j < tokens && dist[lo + j] > tau2) flags |= 1u << j;
  } else {
    const int k = min(keep, tokens);
    if (k > 0) {
      // the k-th largest key: fix 8 bits per pass from the top, keeping
      // `need` = how many of the keys matching the prefix are still wanted
      unsigned long long prefix = 0, pmask = 0;
      int need = k;
      for (int p = 56; p >= 0; p -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int j = 0; j < kPerThread; ++j) {
          if (lo + j >= tokens) break;
          const unsigned long long u = order_key(dist[lo + j]);
          if ((u & pmask) == prefix) atomicAdd(&hist[(u >> p) & 255], 1u);
        }
        __syncthreads();
        if (tid < 64) {
          // the bin holding the need-th largest key, searched by one wave:
          // lane l holds bins 4l .. 4l+3; `above` = keys in higher lanes' bins
          const int l = tid;
          int hb[4], mine = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            hb[q] = static_cast<int>(hist[4 * l + q]);
            mine += hb[q];
          }
          int suffix = mine;
#pragma unroll
          for (int dl = 1; dl < 64; dl <<= 1) {
            const int y = __shfl_down(suffix, dl);
            if (l + dl < 64) suffix += y;
          }
          int above = suffix - mine;
#pragma unroll
          for (int q = 3; q >= 0; --q) {
            if (above < need && above + hb[q] >= need) {
              s_prefix = prefix | (static_cast<unsigned long long>(4 * l + q) << p);
              s_need = need - above;
            }
            above += hb[q];
          }
        }
        __syncthreads();
        prefix = s_prefix;
        need = s_need;
        pmask |= 255ULL << p;
      }
      // larger keys are in; of the keys equal to the k-th, the first `need`
      // by index
      unsigned eq = 0;
      for (int j = 0; j < kPerThread; ++j) {
        if (lo + j >= tokens) break;
        const unsigned long long u = order_key(dist[lo + j]);
        if (u > prefix) flags |= 1u << j;
        else if (u == prefix) eq |= 1u << j;
      }
      int unused;
      int before = exclusive_scan(__popc(eq), scan, unused);
      for (int j = 0; j < kPerThread; ++j)
        if ((eq >> j) & 1u) {
          if (before < need) flags |= 1u << j;
          ++before;
        }
    }
  }

  int total;
  int pos = exclusive_scan(__popc(flags), scan, total);
  for (int j = 0; j < kPerThread; ++j)
    if ((flags >> j) & 1u) rows[pos++] = lo + j;
  for (int j = total + tid; j < tokens; j += kThreads) rows[j] = -1;
  if (tid == 0) *count = total;
}

}  // namespace

kvc_status launch_edit_mask(const EditMaskDesc& d, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* zs = static_cast<const uint16_t*>(d.z_src);
  const auto* ze = static_cast<const uint16_t*>(d.z_edit);
  const double t = static_cast<double>(d.tau);
  // 16-byte reads when every row is a whole number of aligned 16-byte chunks
  const bool vec = d.channels % 8 == 0 && (reinterpret_cast<uintptr_t>(zs) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(ze) & 15u) == 0;
  if (d.keep < 0)
    hipLaunchKernelGGL(edit_mask_kernel<false>, dim3(1), dim3(kThreads), 0, s, zs, ze, d.tokens,
                       d.channels, t * t, 0, vec, d.rows, d.count);
  else
    hipLaunchKernelGGL(edit_mask_kernel<true>, dim3(1), dim3(kThreads), 0, s, zs, ze, d.tokens,
                       d.channels, 0.0, d.keep, vec, d.rows, d.count);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_E_DEVICE;
}

}  // namespace kvc
