// K2: chunk-causal sink+window attention forward, bf16 MFMA, gfx950.
//
// For every query of the current chunk and every head, softmax attention over
// the visible keys: condition tokens, the sink chunk, the window chunks and
// the current chunk (discuss.pytorch.kr "JoyAI-Video-Edit 소개", chunk-wise
// autoregressive adaptation section: bidirectional within the chunk, causal
// across chunks through a sliding window plus the first chunk as global
// sink).  The visible set is never concatenated: the kernel walks the ring's
// segment table (slots in logical order) tile by tile.
//
// Work decomposition: one workgroup = 4 waves = 128 queries of one head; each
// wave owns 32 queries for the whole key range.  Keys stream through LDS in
// tiles of 64, double-buffered (the next tile's global loads are in flight
// while the current one is computed).
//
// Per tile and wave, with 32x32x16 bf16 MFMAs (fp32 accumulate):
//   S^T[64 keys x 32 q] = K_tile[64 x d] . Q^T[d x 32]     (A = K from LDS, B = Q in VGPRs)
//   online softmax on S^T: each lane holds one query column, 32 key values
//   O^T[d x 32 q]      += Vt_tile[d x 64] . P^T[64 x 32]    (A = Vt from LDS, B = P in VGPRs)
// Computing the transposed scores puts P^T straight into the B-operand
// layout of the PV product (no shuffle through LDS).  The 32x32 accumulator
// holds rows (i/4)*8 + (lane/32)*4 + i%4 in register i; reading K rows through
// the permutation pi (swap of row bits 2 and 3) makes the 8 keys each lane
// contributes to one PV step consecutive, so the Vt operand is one 16-byte
// LDS read.  Both LDS tiles are XOR-swizzled per row so the 16-byte reads of
// 16 consecutive lanes hit distinct bank groups.
//
// Online softmax in base 2: t = s * scale * log2(e); the running max is only
// raised (and O, l rescaled) when a tile's max exceeds it by more than 8,
// which keeps p = 2^(t - m) <= 2^8 and skips nearly every rescale after the
// first tiles.  The row sum l is kept per lane and combined across the two
// lane halves at the end.
#include "device_common.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace {

constexpr int kThreads = 256;
constexpr int kBq = 128;          // queries per workgroup
constexpr int kBk = kTileKeys;    // keys per tile (64)
constexpr float kRescaleThreshold = 8.0f;

struct SegArg {
  const unsigned char* k;   // [H][pitch][d]
  const unsigned char* vt;  // [H][d][pitch]
  int rows;
  int pitch;
};

struct AttnArgs {
  const uint16_t* q;
  uint16_t* o;
  float* lse;
  int n;
  int heads;
  float c;          // softmax scale * log2(e)
  int nseg;
  int ntiles;       // total key tiles over all segments
  int nqt;          // query tiles per head
  SegArg seg[kMaxSegments];
};

// swap bits 2 and 3 of a row index
__device__ __forceinline__ int pi_row(int r) {
  return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1);
}
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return pi_row(row & 15) & (D / 8 - 1);
}
__device__ __forceinline__ int swz_v(int row) { return (row ^ (row >> 3)) & 7; }

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16(const AttnArgs a) {
  constexpr int kKRow = D * 2;                  // bytes per K row in LDS
  constexpr int kKChunks = D / 8;               // 16-byte chunks per K row
  constexpr int kKTile = kBk * kKRow;           // bytes of a K tile
  constexpr int kVTile = D * kBk * 2;           // bytes of a Vt tile (D rows x 128 B)
  constexpr int kKLoads = kBk * kKChunks / kThreads;   // 16-byte loads per thread
  constexpr int kVLoads = D * 8 / kThreads;
  constexpr int kDS = D / 16;                   // MFMA k-steps over d
  constexpr int kDB = D / 32;                   // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) unsigned char smem[2][kKTile + kVTile];

  const int L = xcd_contiguous(blockIdx.x, gridDim.x);
  const int h = L / a.nqt;
  const int qt = L - h * a.nqt;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int qi = qt * kBq + wave * 32 + col;
  const bool qvalid = qi < a.n;

  // Q^T as B operand: lane holds query qi, features ks*16 + half*8 .. +7
  bf16x8_t qreg[kDS];
  {
    const uint16_t* qrow = a.q + (static_cast<size_t>(qi) * a.heads + h) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < kDS; ++ks) {
      if (qvalid) {
        qreg[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) qreg[ks][j] = static_cast<__bf16>(0.0f);
      }
    }
  }

  f32x16_t oacc[kDB];
#pragma unroll
  for (int b = 0; b < kDB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[b][i] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  uint4 kst[kKLoads], vst[kVLoads];
  int ls = 0, lk = 0;   // load cursor: segment, first key of the tile
  int cs = 0, ck = 0;   // compute cursor

  auto load_tile = [&](int s, int k0) {
    const SegArg g = a.seg[s];
    const unsigned char* kb = g.k + (static_cast<size_t>(h) * g.pitch + k0) * kKRow;
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int c = tid + kThreads * i;
      kst[i] = ld16(kb + (c / kKChunks) * kKRow + (c % kKChunks) * 16);
    }
    const unsigned char* vb = g.vt + (static_cast<size_t>(h) * D * g.pitch + k0) * 2;
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
      const int c = tid + kThreads * i;
      vst[i] = ld16(vb + static_cast<size_t>(c / 8) * g.pitch * 2 + (c % 8) * 16);
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* kl = smem[buf];
    unsigned char* vl = smem[buf] + kKTile;
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / kKChunks;
      st16(kl + row * kKRow + (((c % kKChunks) ^ swz_k<D>(row)) * 16), kst[i]);
    }
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / 8;
      st16(vl + row * 128 + (((c % 8) ^ swz_v(row)) * 16), vst[i]);
    }
  };
  auto advance = [&](int& s, int& k0) {
    k0 += kBk;
    if (k0 >= a.seg[s].rows) {
      ++s;
      k0 = 0;
    }
  };

  load_tile(ls, lk);
  store_tile(0);
  advance(ls, lk);
  __syncthreads();

  for (int j = 0; j < a.ntiles; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < a.ntiles;
    if (more) load_tile(ls, lk);

    const unsigned char* kl = smem[buf];
    const unsigned char* vl = smem[buf] + kKTile;

    // ---- S^T = K . Q^T
    f32x16_t sacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[b][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kDS; ++ks) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int row = b * 32 + pi_row(col);
        const int chunk = ks * 2 + half;
        const bf16x8_t kop = *reinterpret_cast<const bf16x8_t*>(
            kl + row * kKRow + ((chunk ^ swz_k<D>(row)) * 16));
        sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[ks], sacc[b], 0, 0, 0);
      }
    }

    // ---- mask the padded keys of a segment's last tile
    const int valid = a.seg[cs].rows - ck;
    if (valid < kBk) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = b * 32 + pi_row((i >> 2) * 8 + half * 4 + (i & 3));
          if (key >= valid) sacc[b][i] = -INFINITY;
        }
    }

    // ---- online softmax (base 2, lazy rescale)
    float mx = sacc[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[b][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * a.c;
    if (__any(mt > m_run + kRescaleThreshold)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int b = 0; b < kDB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[b][i] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float neg_m = -m_run;
    bf16x8_t pb[4];
    float lsum = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[b][i], a.c, neg_m));
        lsum += p;
        pb[b * 2 + (i >> 3)][i & 7] = static_cast<__bf16>(p);
      }
    l_run += lsum;

    // ---- O^T += Vt . P^T
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int row = db * 32 + col;
        const int chunk = ps * 2 + half;
        const bf16x8_t vop = *reinterpret_cast<const bf16x8_t*>(
            vl + row * 128 + ((chunk ^ swz_v(row)) * 16));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[ps], oacc[db], 0, 0, 0);
      }
    }

    if (more) {
      store_tile(buf ^ 1);
      advance(ls, lk);
    }
    advance(cs, ck);
    __syncthreads();
  }

  // ---- epilogue: O /= l, store bf16; lse = (m + log2 l) * ln 2
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (qvalid) {
    uint16_t* orow = a.o + (static_cast<size_t>(qi) * a.heads + h) * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t w[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const __bf16 lo = static_cast<__bf16>(oacc[db][g * 4 + 2 * e] * inv);
          const __bf16 hi = static_cast<__bf16>(oacc[db][g * 4 + 2 * e + 1] * inv);
          w[e] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                 (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
        }
        *reinterpret_cast<uint2*>(orow + db * 32 + g * 8 + half * 4) = make_uint2(w[0], w[1]);
      }
    if (a.lse && half == 0) {
      a.lse[static_cast<size_t>(h) * a.n + qi] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
    }
  }
}

template <int D>
kvc_status launch_bf16(const AttnDesc& d, hipStream_t stream) {
  AttnArgs a;
  a.q = static_cast<const uint16_t*>(d.q);
  a.o = static_cast<uint16_t*>(d.o);
  a.lse = d.lse;
  a.n = d.n;
  a.heads = d.heads;
  a.c = d.scale * 1.4426950408889634f;
  a.nseg = d.nseg;
  a.ntiles = 0;
  for (int s = 0; s < d.nseg; ++s) {
    a.seg[s].k = static_cast<const unsigned char*>(d.seg[s].k);
    a.seg[s].vt = static_cast<const unsigned char*>(d.seg[s].vt);
    a.seg[s].rows = d.seg[s].rows;
    a.seg[s].pitch = d.seg[s].pitch;
    if (d.seg[s].rows <= 0 || d.seg[s].pitch < d.seg[s].rows || d.seg[s].pitch % kBk)
      return KVC_E_INVAL;
    a.ntiles += (d.seg[s].rows + kBk - 1) / kBk;
  }
  a.nqt = (d.n + kBq - 1) / kBq;
  const int nblk = a.nqt * d.heads;
  hipLaunchKernelGGL(attn_fwd_bf16<D>, dim3(nblk), dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_E_DEVICE;
}

}  // namespace

kvc_status launch_attention(const AttnDesc& d, void* stream) {
  if (d.nseg < 1 || d.nseg > kMaxSegments || d.n < 1) return KVC_E_INVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d.kv_dtype != KVC_KV_BF16) return KVC_E_UNSUPPORTED;
  switch (d.head_dim) {
    case 64: return launch_bf16<64>(d, s);
    case 128: return launch_bf16<128>(d, s);
    default: return KVC_E_UNSUPPORTED;
  }
}

}  // namespace kvc
