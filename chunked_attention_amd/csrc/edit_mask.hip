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
// tokens; the work is microseconds next to the attention it feeds, so the
// kernel is built for latency: few barriers, wave-level scans on DPP lane
// moves, loads of a thread's tokens in flight together).  Thread t owns
// tokens t, t + 1024, t + 2048, ... ("rounds"), so every phase keeps all
// sixteen waves busy and a wave's accesses are to consecutive tokens:
//   1. squared distance of each owned token (float64, channels summed in
//      order, every operation rounded on its own, so a plain CPU loop gets
//      the same bits).  Threshold mode: a flag bit per round.  Top-k mode:
//      the 64-bit order-preserving key into LDS, and the AND and OR of all
//      keys (the bits where they all agree);
//   2. top-k mode: radix-select the keep-th largest key with 8-bit digits,
//      starting at the highest digit where the keys are not all equal; one
//      LDS histogram per pass (all cleared up front), lanes of a wave with
//      the same digit as the first lane adding their count once; one
//      barrier per pass, after which every wave finds the bin on its own;
//      the select ends early once the chosen bin holds exactly the keys
//      still wanted.  Every larger key is in and, among keys equal to the
//      last one, the lowest indices up to keep;
//   3. compact: the rank of a chosen token among the chosen ones in index
//      order is a ballot count within its wave plus a prefix over the
//      (round, wave) counts, which every wave scans for itself.
#include <algorithm>
#include <mutex>
#include <vector>

#include "device_common.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kRounds = KVC_MAX_MASK_TOKENS / kThreads;   // 16 tokens per thread at most
constexpr int kGroup = 4;                                  // tokens whose loads overlap
static_assert(kRounds <= 32, "flags of a thread fit one word");
static_assert(kRounds * kWaves == 4 * 64, "a wave scans the (round, wave) table, 4 per lane");

// acc + (e - s)^2 in float64 for one channel (bf16 bit patterns), each
// operation rounded on its own
__device__ __forceinline__ double add_sq(double acc, uint32_t e, uint32_t s) {
#pragma clang fp contract(off)
  const double d = static_cast<double>(bf16_bits_to_float(e)) -
                   static_cast<double>(bf16_bits_to_float(s));
  const double sq = d * d;
  return acc + sq;
}

// unsigned key with the order of the float64 value
__device__ __forceinline__ unsigned long long order_key(double d) {
  const unsigned long long u = __double_as_longlong(d);
  return (u >> 63) ? ~u : (u | (1ULL << 63));
}

// number of set bits of b in the lanes below this one
__device__ __forceinline__ int lanes_below(unsigned long long b) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(
      static_cast<unsigned>(b >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(b), 0u)));
}

// DPP lane moves (GCN data-parallel primitives): row_shr:n takes the value of
// the lane n below within its row of 16 lanes; row_bcast:15 / row_bcast:31
// take lane 15 / 31 of the wave (for the rows selected by the row mask).
// A lane whose source is outside the row, or whose row is masked off, gets
// `id`.
constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ unsigned dpp(unsigned id, unsigned x) {
  return static_cast<unsigned>(__builtin_amdgcn_update_dpp(static_cast<int>(id), static_cast<int>(x),
                                                           kCtrl, kRowMask, 0xf, false));
}

// inclusive scan over the 64 lanes of an associative operation with identity id
template <typename Op>
__device__ __forceinline__ unsigned wave_scan(unsigned x, unsigned id, Op op) {
  x = op(x, dpp<kRowShr + 1>(id, x));
  x = op(x, dpp<kRowShr + 2>(id, x));
  x = op(x, dpp<kRowShr + 4>(id, x));
  x = op(x, dpp<kRowShr + 8>(id, x));     // inclusive within each row of 16
  x = op(x, dpp<kRowBcast15, 0xa>(id, x));   // rows 1, 3 take the end of rows 0, 2
  x = op(x, dpp<kRowBcast31, 0xc>(id, x));   // rows 2, 3 take the end of rows 0-1
  return x;
}

__device__ __forceinline__ int wave_incl_sum(int x) {
  return static_cast<int>(wave_scan(static_cast<unsigned>(x), 0u,
                                    [](unsigned a, unsigned b) { return a + b; }));
}

__device__ __forceinline__ unsigned lane63(unsigned x) {
  return static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}

// sum_c (e_c - s_c)^2 of this thread's tokens of rounds g .. g+kTok-1:
// acc[u] for token (g + u) * kThreads + tid (a lane with fewer tokens
// computes clamped in-bounds tokens it never uses).  `vec`: rows are whole
// aligned 16-byte chunks (8 channels), read 16 bytes at a time, two chunks
// of every token loaded before any is used so that their latencies overlap.
template <int kTok>
__device__ __forceinline__ void group_distances(const uint16_t* __restrict__ zs,
                                                const uint16_t* __restrict__ ze, int tokens,
                                                int channels, int g, bool vec,
                                                double (&acc)[kGroup]) {
  const int tid = threadIdx.x;
  size_t row[kTok];
#pragma unroll
  for (int u = 0; u < kTok; ++u) {
    acc[u] = 0.0;
    row[u] = static_cast<size_t>(min((g + u) * kThreads + tid, tokens - 1)) * channels;
  }
  if (vec) {
    int c = 0;
    for (; c + 16 <= channels; c += 16) {
      uint4 ev[kTok][2], sv[kTok][2];
#pragma unroll
      for (int u = 0; u < kTok; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          ev[u][h] = ld16(ze + row[u] + c + 8 * h);
          sv[u][h] = ld16(zs + row[u] + c + 8 * h);
        }
#pragma unroll
      for (int u = 0; u < kTok; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t ew[4] = {ev[u][h].x, ev[u][h].y, ev[u][h].z, ev[u][h].w};
          const uint32_t sw[4] = {sv[u][h].x, sv[u][h].y, sv[u][h].z, sv[u][h].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[u] = add_sq(acc[u], ew[q] & 0xFFFFu, sw[q] & 0xFFFFu);
            acc[u] = add_sq(acc[u], ew[q] >> 16, sw[q] >> 16);
          }
        }
    }
    if (c < channels) {   // one chunk left
      uint4 ev[kTok], sv[kTok];
#pragma unroll
      for (int u = 0; u < kTok; ++u) {
        ev[u] = ld16(ze + row[u] + c);
        sv[u] = ld16(zs + row[u] + c);
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
    for (int c = 0; c < channels; ++c) {
      uint32_t e[kTok], s[kTok];
#pragma unroll
      for (int u = 0; u < kTok; ++u) {
        e[u] = ze[row[u] + c];
        s[u] = zs[row[u] + c];
      }
#pragma unroll
      for (int u = 0; u < kTok; ++u) acc[u] = add_sq(acc[u], e[u], s[u]);
    }
  }
}

// Counts of the chosen tokens per (round, wave), for ranks in index order:
// bit r of `pick` chooses this thread's token r * kThreads + tid (rounds
// < nr).  Lane 0 of each wave stores its wave's count of every round in
// table[r * kWaves + wave]; after the barrier every wave scans the table
// itself.
__device__ __forceinline__ void count_table(unsigned pick, int nr, int* table) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int r = 0; r < nr; ++r) {
    const unsigned long long b = __ballot((pick >> r) & 1u);
    if (lane == 0) table[r * kWaves + wave] = __popcll(b);
  }
  __syncthreads();
}

// The table's exclusive prefix (round-major order, so index order) for this
// wave: lane l holds entries 4l .. 4l+3, and returns the prefix of entry
// 4l + (wave mod 4), so that round r's base of this wave is in lane
// 4r + wave / 4.  *total = the sum of the table.
__device__ __forceinline__ int table_prefix(const int* table, int nr, int* total) {
  const int lane = threadIdx.x & 63;
  const int q = (threadIdx.x >> 6) & 3;
  int v[4], mine = 0, part = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    v[i] = e < nr * kWaves ? table[e] : 0;
    mine += v[i];
    part += i < q ? v[i] : 0;
  }
  const int incl = wave_incl_sum(mine);
  *total = static_cast<int>(lane63(static_cast<unsigned>(incl)));
  return incl - mine + part;
}

__device__ __forceinline__ int round_base(int prefix, int r) {
  return __builtin_amdgcn_readlane(prefix, 4 * r + (threadIdx.x >> 6) / 4);
}

template <bool kTopK>
__global__ __launch_bounds__(kThreads) void edit_mask_kernel(
    const uint16_t* __restrict__ zs, const uint16_t* __restrict__ ze, int tokens, int channels,
    double tau2, int keep, bool vec, int* __restrict__ rows, int* __restrict__ count) {
  constexpr int kPasses = 8;   // 8-bit digits of a 64-bit key
  // top-k mode: the keys, [round][thread] for the tokens that exist (dynamic
  // LDS of tokens * 8 bytes, so that a small call leaves room on its CU for
  // other kernels' workgroups)
  extern __shared__ unsigned long long keys[];
  __shared__ unsigned hist[kTopK ? kPasses : 1][256];                  // one per pass
  __shared__ int table[2][kRounds * kWaves];
  __shared__ unsigned long long wand[kWaves], wor[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nr = (tokens + kThreads - 1) / kThreads;   // rounds with any token
  const int mine = tokens > tid ? (tokens - tid + kThreads - 1) / kThreads : 0;   // this thread's
  const int mine_w = __builtin_amdgcn_readfirstlane(mine);                       // lane 0's: most
  if constexpr (kTopK) {
    for (int b = tid; b < kPasses * 256; b += kThreads) (&hist[0][0])[b] = 0;
  }

  unsigned pick = 0;   // bit r: token r * kThreads + tid is chosen
  unsigned long long kand = ~0ULL, kor = 0;
  for (int g = 0; g < mine_w; g += kGroup) {
    // as many tokens as lane 0 of the wave has in the group (the most)
    double acc[kGroup];
    const int n = min(mine_w - g, kGroup);
    switch (n) {
      case 1: group_distances<1>(zs, ze, tokens, channels, g, vec, acc); break;
      case 2: group_distances<2>(zs, ze, tokens, channels, g, vec, acc); break;
      case 3: group_distances<3>(zs, ze, tokens, channels, g, vec, acc); break;
      default: group_distances<4>(zs, ze, tokens, channels, g, vec, acc); break;
    }
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int r = g + u;
      if (u < n && r < mine) {
        if constexpr (kTopK) {
          // a NaN distance ranks below every real one (as -1)
          const unsigned long long key = order_key(acc[u] != acc[u] ? -1.0 : acc[u]);
          keys[r * kThreads + tid] = key;
          kand &= key;
          kor |= key;
        } else {
          // NaN is never above the threshold
          if (acc[u] > tau2) pick |= 1u << r;
        }
      }
    }
  }

  if constexpr (kTopK) {
    const int k = min(keep, tokens);
    const auto band = [](unsigned a, unsigned b) { return a & b; };
    const auto bor = [](unsigned a, unsigned b) { return a | b; };
    {
      const unsigned al = lane63(wave_scan(static_cast<unsigned>(kand), ~0u, band));
      const unsigned ah = lane63(wave_scan(static_cast<unsigned>(kand >> 32), ~0u, band));
      const unsigned ol = lane63(wave_scan(static_cast<unsigned>(kor), 0u, bor));
      const unsigned oh = lane63(wave_scan(static_cast<unsigned>(kor >> 32), 0u, bor));
      if (lane == 0) {
        wand[wave] = (static_cast<unsigned long long>(ah) << 32) | al;
        wor[wave] = (static_cast<unsigned long long>(oh) << 32) | ol;
      }
    }
    __syncthreads();
    if (k > 0) {
      // the AND and OR of every key: lanes 0-15 hold the waves' values
      kand = lane < kWaves ? wand[lane] : ~0ULL;
      kor = lane < kWaves ? wor[lane] : 0ULL;
      kand = (static_cast<unsigned long long>(lane63(wave_scan(static_cast<unsigned>(kand >> 32), ~0u, band))) << 32) |
             lane63(wave_scan(static_cast<unsigned>(kand), ~0u, band));
      kor = (static_cast<unsigned long long>(lane63(wave_scan(static_cast<unsigned>(kor >> 32), 0u, bor))) << 32) |
            lane63(wave_scan(static_cast<unsigned>(kor), 0u, bor));
      // digits above the highest one where some keys differ are common to
      // all keys; with no difference at all every key is a tie
      const unsigned long long x = kand ^ kor;
      int p = x ? ((63 - __clzll(x)) & ~7) : -8;
      unsigned long long pmask = p >= 56 ? 0ULL : ~0ULL << (p + 8);
      unsigned long long prefix = kand & pmask;
      int need = k;
      bool whole = tokens == k;   // every key matching the prefix is wanted
      for (int pass = 0; p >= 0 && !whole; p -= 8, ++pass) {
        unsigned* h = hist[pass];
        for (int r = 0; r < mine; ++r) {
          const unsigned long long u = keys[r * kThreads + tid];
          if ((u & pmask) == prefix) {
            // lanes sharing the first active lane's digit add once
            const unsigned dg = static_cast<unsigned>(u >> p) & 255u;
            const unsigned lead = __builtin_amdgcn_readfirstlane(dg);
            const unsigned long long same = __ballot(dg == lead);
            if (dg != lead)
              atomicAdd(&h[dg], 1u);
            else if (lanes_below(same) == 0)
              atomicAdd(&h[lead], static_cast<unsigned>(__popcll(same)));
          }
        }
        __syncthreads();
        // every wave finds the bin holding the need-th largest key: lane l
        // holds bins 4l .. 4l+3; `above` = keys in higher lanes' bins
        int hb[4], sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hb[q] = static_cast<int>(h[4 * lane + q]);
          sum += hb[q];
        }
        const int incl = wave_incl_sum(sum);
        int above = static_cast<int>(lane63(static_cast<unsigned>(incl))) - incl;
        int fbin = -1, fneed = 0, fcnt = 0;
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          if (above < need && above + hb[q] >= need) {
            fbin = 4 * lane + q;
            fneed = need - above;
            fcnt = hb[q];
          }
          above += hb[q];
        }
        const int src = __ffsll(static_cast<long long>(__ballot(fbin >= 0))) - 1;   // one lane
        prefix |= static_cast<unsigned long long>(__builtin_amdgcn_readlane(fbin, src)) << p;
        need = __builtin_amdgcn_readlane(fneed, src);
        whole = __builtin_amdgcn_readlane(fcnt, src) == need;
        pmask |= 255ULL << p;
      }
      // larger keys are in; of the keys equal to the k-th, the first `need`
      // by index (all of them when the select ended on a whole bin)
      unsigned eq = 0;
      for (int r = 0; r < mine; ++r) {
        const unsigned long long um = keys[r * kThreads + tid] & pmask;
        if (um > prefix || (whole && um == prefix)) pick |= 1u << r;
        else if (um == prefix) eq |= 1u << r;
      }
      if (!whole) {
        count_table(eq, nr, table[1]);
        int unused;
        const int pre = table_prefix(table[1], nr, &unused);
        for (int r = 0; r < nr; ++r) {
          const unsigned long long b = __ballot((eq >> r) & 1u);
          if (((eq >> r) & 1u) && round_base(pre, r) + lanes_below(b) < need) pick |= 1u << r;
        }
      }
    }
  }

  count_table(pick, nr, table[0]);
  int total;
  const int pre = table_prefix(table[0], nr, &total);
  for (int r = 0; r < nr; ++r) {
    const unsigned long long b = __ballot((pick >> r) & 1u);
    const int base = round_base(pre, r);
    if ((pick >> r) & 1u) rows[base + lanes_below(b)] = r * kThreads + tid;
  }
  for (int j = total + tid; j < tokens; j += kThreads) rows[j] = -1;
  if (tid == 0) *count = total;
}

}  // namespace

// The top-k kernel's keys may take up to 128 KB of dynamic LDS: allow it
// once per device (the first call on each device).
static kvc_status allow_mask_lds() {
  static std::mutex mu;
  static std::vector<int> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVC_E_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (std::find(done.begin(), done.end(), dev) != done.end()) return KVC_OK;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(edit_mask_kernel<true>),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(sizeof(unsigned long long) * KVC_MAX_MASK_TOKENS)) !=
      hipSuccess)
    return KVC_E_DEVICE;
  done.push_back(dev);
  return KVC_OK;
}

kvc_status launch_edit_mask(const EditMaskDesc& d, void* stream) {
  if (d.keep >= 0) {
    if (kvc_status st = allow_mask_lds()) return st;
  }
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
    hipLaunchKernelGGL(edit_mask_kernel<true>, dim3(1), dim3(kThreads),
                       sizeof(unsigned long long) * static_cast<size_t>(d.tokens), s, zs, ze,
                       d.tokens, d.channels, 0.0, d.keep, vec, d.rows, d.count);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_E_DEVICE;
}

}  // namespace kvc
