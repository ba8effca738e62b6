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
//      the same bits; four tokens per thread loaded at once);
//   2. threshold mode: flag distances above tau^2.  Top-k mode: radix-select
//      the keep-th largest distance over its 64-bit order-preserving key
//      (8-bit digits from the top; one LDS histogram per wave, so colliding
//      atomics stay within a wave, summed before one wave finds the bin;
//      done early once that bin holds exactly the keys still wanted), flag
//      every larger key and, among keys equal to it, the lowest indices up
//      to keep;
//   3. compact: thread t owns tokens 16t .. 16t+15; a prefix sum of the flag
//      counts (lane shuffles, then the waves' totals) gives each thread its
//      output position.
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

__device__ __forceinline__ double nan_last(double acc) { return acc != acc ? -1.0 : acc; }

// sum_c (e_c - s_c)^2 of the tokens i0 + u * kThreads (u < kTok) into dist[],
// float64, channels in order for each token; NaN -> -1 (a NaN distance is
// never above the threshold and ranks last).  `vec`: rows are whole
// 16-byte chunks (8 channels), read 16 bytes at a time, the chunks of all
// kTok tokens loaded before any is used so their latencies overlap.
template <int kTok>
__device__ void distances(const uint16_t* __restrict__ zs, const uint16_t* __restrict__ ze,
                          int tokens, int channels, int i0, bool vec, double* __restrict__ dist) {
  double acc[kTok];
#pragma unroll
  for (int u = 0; u < kTok; ++u) acc[u] = 0.0;
  if (vec) {
    for (int c = 0; c < channels; c += 8) {
      uint4 ev[kTok], sv[kTok];
#pragma unroll
      for (int u = 0; u < kTok; ++u) {
        const int i = min(i0 + u * kThreads, tokens - 1);   // in bounds; unused if past the end
        ev[u] = ld16(ze + static_cast<size_t>(i) * channels + c);
        sv[u] = ld16(zs + static_cast<size_t>(i) * channels + c);
      }
#pragma unroll
      for (int u = 0; u < kTok; ++u) {
        const uint32_t ew[4] = {ev[u].x, ev[u].y, ev[u].z, ev[u].w};
        const uint32_t sw[4] = {sv[u].x, sv[u].y, sv[u].z, sv[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[u] = add_sq(acc[u], ew[q] & 0xFFFFu, sw[q] & 0xFFFFu);
          acc[u] = add_sq(acc[u], ew[q] >> 16, sw[q] >> 16);
        }
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      const int i = min(i0 + u * kThreads, tokens - 1);
      const uint16_t* s = zs + static_cast<size_t>(i) * channels;
      const uint16_t* e = ze + static_cast<size_t>(i) * channels;
      for (int c = 0; c < channels; ++c) acc[u] = add_sq(acc[u], e[c], s[c]);
    }
  }
#pragma unroll
  for (int u = 0; u < kTok; ++u) {
    const int i = i0 + u * kThreads;
    if (i < tokens) dist[i] = nan_last(acc[u]);
  }
}

// unsigned key with the order of the float64 value
__device__ __forceinline__ unsigned long long order_key(double d) {
  const unsigned long long u = __double_as_longlong(d);
  return (u >> 63) ? ~u : (u | (1ULL << 63));
}

constexpr int kWaves = kThreads / 64;

// exclusive prefix sum of v over the workgroup, and its total: an inclusive
// scan inside each wave (lane shuffles), then the waves' totals through LDS
__device__ int exclusive_scan(int v, int (&wave_sum)[kWaves], int& total) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_sum[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int ws = wave_sum[w];
    before += w < wave ? ws : 0;
    total += ws;
  }
  __syncthreads();   // wave_sum may be reused by the next scan
  return before + x - v;
}

template <bool kTopK>
__global__ __launch_bounds__(kThreads) void edit_mask_kernel(
    const uint16_t* __restrict__ zs, const uint16_t* __restrict__ ze, int tokens, int channels,
    double tau2, int keep, bool vec, int* __restrict__ rows, int* __restrict__ count) {
  __shared__ double dist[KVC_MAX_MASK_TOKENS];
  __shared__ int scan[kWaves];
  __shared__ unsigned whist[kWaves][256];   // per-wave histograms (less atomic contention)
  __shared__ unsigned hist[256];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_need, s_cnt;
  const int tid = threadIdx.x;
  for (int i0 = tid; i0 < tokens; i0 += 4 * kThreads)
    distances<4>(zs, ze, tokens, channels, i0, vec, dist);
  __syncthreads();

  const int lo = tid * kPerThread;
  unsigned flags = 0;
  if constexpr (!kTopK) {
    for (int j = 0; j < kPerThread; ++j)
      if (lo + j < tokens && dist[lo + j] > tau2) flags |= 1u << j;
  } else {
    const int k = min(keep, tokens);
    if (k > 0) {
      // this thread's keys, in registers for all passes (tokens past the end
      // get key 0, below every real key, and are never counted)
      unsigned long long key[kPerThread];
#pragma unroll
      for (int j = 0; j < kPerThread; ++j)
        key[j] = lo + j < tokens ? order_key(dist[lo + j]) : 0ULL;
      // the k-th largest key: fix 8 bits per pass from the top, keeping
      // `need` = how many of the keys matching the prefix are still wanted
      unsigned long long prefix = 0, pmask = 0;
      int need = k;
      bool whole_bin = false;   // every key matching the prefix is wanted
      const int wv = tid >> 6;
      for (int p = 56; p >= 0; p -= 8) {
        for (int b = tid; b < kWaves * 256; b += kThreads) (&whist[0][0])[b] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
          const unsigned long long u = key[j];
          if (lo + j < tokens && (u & pmask) == prefix) atomicAdd(&whist[wv][(u >> p) & 255], 1u);
        }
        __syncthreads();
        if (tid < 256) {
          unsigned sum = 0;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) sum += whist[w][tid];
          hist[tid] = sum;
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
              s_cnt = hb[q];
            }
            above += hb[q];
          }
        }
        __syncthreads();
        prefix = s_prefix;
        need = s_need;
        pmask |= 255ULL << p;
        // the bin holds exactly the keys still wanted: all of them are in,
        // so the lower digits cannot change the selection (for continuous
        // distances this ends the select after two or three digits)
        if (s_cnt == need) {
          whole_bin = true;
          break;
        }
      }
      // larger keys are in; of the keys equal to the k-th, the first `need`
      // by index (all of them when the select ended on a whole bin)
      unsigned eq = 0;
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const unsigned long long u = key[j];
        if (lo + j < tokens) {
          const unsigned long long um = u & pmask;
          if (um > prefix || (whole_bin && um == prefix)) flags |= 1u << j;
          else if (um == prefix) eq |= 1u << j;
        }
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
