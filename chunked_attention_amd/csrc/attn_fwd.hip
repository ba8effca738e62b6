// K2: chunk-causal sink+window attention forward, bf16 MFMA, gfx950.
//
// For every query of the current chunk and every head, softmax attention over
// the visible keys: condition tokens, the sink chunk, the window chunks and
// the current chunk (discuss.pytorch.kr "JoyAI-Video-Edit 소개", chunk-wise
// autoregressive adaptation section: bidirectional within the chunk, causal
// across chunks through a sliding window plus the first chunk as global
// sink).  The visible set is never concatenated: the kernel walks the ring's
// segment table (cache slots in logical order) tile by tile.
//
// Work: a "row" is 128 queries of one head; its keys are T tiles of 64 keys
// over all segments (a segment's last tile is masked).  A workgroup runs one
// row at a time with 128 / (32 NCQ) waves of 32 NCQ queries each.  With
// NCQ = 1 a workgroup has 4 waves and two workgroups share a CU, so every
// SIMD holds two waves and interleaves one wave's softmax (VALU) with the
// other's matrix products (MFMA).  The grid is persistent: nwg workgroups
// (two per CU) split the R*T (row, tile) steps into equal contiguous ranges
// (stream-K), so the whole GPU stays busy whatever R is.  A row cut between
// workgroups is finished by the last piece to arrive, which merges all
// partial (O, reference, sums) in piece order.
//
// Per tile and wave (32 NCQ queries = NCQ column blocks of 32), with
// 32x32x16 bf16 MFMAs (fp32 accumulate):
//   S^T[64 keys x 32 q] = K_tile . Q^T      A = K from LDS, B = Q in VGPRs
//   O^T[d x 32 q]      += Vt_tile . P^T     A = Vt from LDS, B = P in VGPRs
// Computing transposed scores puts P^T straight into the B-operand layout of
// the PV product.  The accumulator holds key rows (i/4)*8 + (lane/32)*4 + i%4
// in register i; the ring stores V's key columns in exactly that order within
// each group of 16 (kappa, a swap of index bits 2 and 3), so the 8 keys a
// lane feeds to one PV step are consecutive and each Vt operand is one
// 16-byte LDS read.  Tiles are XOR-swizzled per row (16-byte chunk c of row r
// lives at c ^ (r & 7)) so 8 consecutive lanes' 16-byte reads hit distinct
// bank groups; the swizzle depends only on the lane, so the unrolled reads of
// one lane differ by immediate offsets.  K and Vt tiles are copied from
// global memory straight into LDS (buffer_load ... lds, scalar base and
// offset, per-lane 32-bit offset), two buffers each.
//
// Software pipeline: while the softmax of half tile u runs on the VALU, the
// QK^T MFMAs of half tile u+1 are issued; then the PV MFMAs of half tile u.
// So K runs one tile ahead of V: tile j reads K_{j+1} and V_j while K_{j+2}
// and V_{j+1} stream in.
//
// Softmax in base 2 with a fixed reference per row piece: t = s*scale*log2(e)
// and p = 2^(t - m_ref), where m_ref is the max of the piece's first 32 keys,
// so the largest p is at least 1.  No running max is kept: O is never
// rescaled in the loop.  A key far above m_ref shows up in the row sum
// instead: if any row sum exceeds 2^64 (or overflows) the workgroup computes
// the piece again, with m_ref raised by log2 of that sum (then no p exceeds
// 1), or, if a sum overflowed, once more tracking the true max first.  Below
// 2^64 every p, every sum and every accumulator is finite in fp32 and bf16.
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace {

constexpr int kBq = kAttnRowQueries;    // queries per row (128)
constexpr int kBk = kTileKeys;          // keys per tile (64)
constexpr int kMaxWg = kAttnMaxWg;      // persistent workgroups at most (2 per CU)
constexpr int kMinPieceTiles = 16;      // smallest share of a row worth splitting off
constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kMaxPasses = 4;

// Geometry of one variant: head dim D, NCQ column blocks of 32 queries per
// wave.
template <int D, int NCQ>
struct Geo {
  static constexpr int kWaves = 4 / NCQ;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kQW = 32 * NCQ;              // queries per wave
  static constexpr int kKRow = 2 * D;               // bytes per K row
  static constexpr int kKBytes = kBk * kKRow;       // K tile bytes
  static constexpr int kVBytes = D * kBk * 2;       // Vt tile bytes (D rows of 128 B)
  static constexpr int kKInstr = kKBytes / 1024 / kWaves;   // 1 KB copy per wave-instruction
  static constexpr int kVInstr = kVBytes / 1024 / kWaves;
  static constexpr int kDS = D / 16;                // k-steps over d for QK^T
  static constexpr int kDB = D / 32;                // 32-row blocks of O^T
  static constexpr int kMl = NCQ * 3 * 32;          // per wave: (ref, sum, exact sum) per query
  static constexpr int kBufFloats = kKBytes / 4;    // floats per LDS tile buffer
  static_assert(kKBytes == kVBytes, "K and Vt tiles have the same size");
  static_assert(kWaves * kQW == kBq, "row = waves x queries per wave");
  static_assert(kKInstr >= 1 && kVInstr >= 1, "whole 1 KB copies per wave");
  static_assert(kQW * D == NCQ * kBufFloats, "a wave's partial O fills NCQ tile buffers");
};

struct SegArg {
  const unsigned char* k;   // [H][pitch][d]
  const unsigned char* vt;  // [H][d][pitch]
  int rows;
  int pitch;
  int tile0;                // first tile of this segment in the row's tile list
  int pad_;
};

struct AttnArgs {
  const uint16_t* q;
  uint16_t* o;
  float* lse;
  float* part_o;            // [2*nwg][kBq*D] partial O, accumulator layout
  float* part_ml;           // [2*nwg][waves][NCQ][3][32] partial ref, sum, exact sum
  unsigned* counters;       // [nrows][2]: arrived, partials written
  int n;
  int heads;
  float c;                  // softmax scale * log2(e)
  int nseg;
  int ntiles;               // tiles per row (T)
  int nqt;                  // rows per head
  int nrows;                // heads * nqt
  int nwg;                  // persistent workgroups
  long long total;          // nrows * ntiles
  SegArg seg[kMaxSegments];
};

// max / sum of a value with the one held by lane ^ 32 (v_permlane32_swap
// exchanges the two 32-lane halves)
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// first step of workgroup w's range, and the owner of step x
__device__ __forceinline__ long long range_begin(long long w, const AttnArgs& a) {
  return w * a.total / a.nwg;
}
__device__ __forceinline__ int owner_of(long long x, const AttnArgs& a) {
  return static_cast<int>(((x + 1) * a.nwg - 1) / a.total);
}

typedef __attribute__((address_space(3))) void lds_void;

// buffer resource over `bytes` bytes at `base` (raw buffer: stride 0, offsets
// in bytes; 0x00020000 = 32-bit data format, the gfx9 setting for raw access)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// 16 bytes per lane from the buffer at voff + soff into LDS at lds + 16*lane
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, static_cast<int>(voff),
                                           static_cast<int>(soff), 0, 0);
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt low bits [3:0], high
// bits [15:14]; expcnt [6:4], left at its maximum; lgkmcnt [11:8])
template <int N>
__device__ __forceinline__ void wait_vm_keep_lds_done() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// Workgroup barrier without a memory fence (a fence would make the compiler
// wait for every copy in flight).  Written as an asm statement with a memory
// clobber so that no memory access is moved across it at any compiler level;
// it emits no wait of its own.  The caller has already waited for its own LDS
// accesses and for the copies the next step reads.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("s_barrier" ::: "memory");
}

// Cursor over one row's key tiles: segment, first key of the tile, and that
// segment's fields, all wave-uniform (scalar registers).  Moving to the next
// tile touches no memory except when a segment ends.
struct TileCursor {
  int t;                    // tile index within the row
  int s;                    // segment
  int k0;                   // first key of the tile within the segment
  int rows;
  int pitch;
  __amdgpu_buffer_rsrc_t rk;   // this head's K plane of the segment
  __amdgpu_buffer_rsrc_t rv;   // this head's Vt plane
};

template <int D>
__device__ __forceinline__ void cursor_fields(const AttnArgs& a, TileCursor& c, int h) {
  const SegArg& s = a.seg[c.s];
  c.rows = s.rows;
  c.pitch = s.pitch;
  const uint32_t plane = static_cast<uint32_t>(s.pitch) * D * 2;
  c.rk = make_rsrc(s.k + static_cast<size_t>(h) * plane, plane);
  c.rv = make_rsrc(s.vt + static_cast<size_t>(h) * plane, plane);
}
template <int D>
__device__ __forceinline__ void cursor_seek(const AttnArgs& a, TileCursor& c, int t, int h) {
  int s = 0;
  while (s + 1 < a.nseg && a.seg[s + 1].tile0 <= t) ++s;
  c.t = t;
  c.s = s;
  c.k0 = (t - a.seg[s].tile0) * kBk;
  cursor_fields<D>(a, c, h);
}
// one tile on, but never past tile `last`
template <int D>
__device__ __forceinline__ void cursor_next(const AttnArgs& a, TileCursor& c, int last, int h) {
  if (c.t >= last) return;
  ++c.t;
  c.k0 += kBk;
  if (c.k0 >= c.rows) {
    ++c.s;
    c.k0 = 0;
    cursor_fields<D>(a, c, h);
  }
}

template <int D, int NCQ, bool kLse>
__global__ __launch_bounds__(64 * 4 / NCQ)
__attribute__((amdgpu_waves_per_eu(NCQ == 1 ? 2 : 1, NCQ == 1 ? 2 : 1)))
void attn_fwd_bf16(const AttnArgs a) {
  using G = Geo<D, NCQ>;
  constexpr int kWaves = G::kWaves;
  constexpr int kQW = G::kQW;
  constexpr int kDS = G::kDS;
  constexpr int kDB = G::kDB;
  // LDS: two K tiles and two Vt tiles, as four separate arrays so that the
  // compiler can tell reads of one buffer from copies landing in another
  // (a single array would make it wait for every copy in flight before any
  // LDS read).  kK0.. name the buffers.
  constexpr int kK0 = 0, kK1 = 1, kV0 = 2, kV1 = 3;
  __shared__ __attribute__((aligned(1024))) unsigned char kb0[G::kKBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char kb1[G::kKBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vb0[G::kVBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vb1[G::kVBytes];
  auto buf = [&](int b) -> unsigned char* {
    return b == kK0 ? kb0 : b == kK1 ? kb1 : b == kV0 ? vb0 : vb1;
  };
  __shared__ unsigned s_ticket;
  __shared__ int s_vote[kWaves][2];

  const int w = xcd_contiguous(blockIdx.x, gridDim.x);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  // Per-lane byte offsets of the copies.  K: a 1 KB block holds 1024 / (2D)
  // consecutive key rows; lane l fills 16-byte chunk l % (D/8) of row
  // l / (D/8), which takes logical chunk pc ^ (row & 7).  The row's low 3
  // bits depend on the block only through its parity (D = 128) or not at all
  // (D = 64).  Vt: a 1 KB block holds 8 rows d of 128 bytes; lane l fills
  // chunk l % 8 of row l / 8 with logical chunk (l % 8) ^ (l / 8).
  constexpr int kKLanesPerRow = D / 8;
  constexpr int kKRowsPerBlk = 1024 / G::kKRow;
  uint32_t koff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int row = par * kKRowsPerBlk + lane / kKLanesPerRow;
    const int pc = lane % kKLanesPerRow;
    koff[par] = (lane / kKLanesPerRow) * G::kKRow + ((pc ^ (row & 7)) * 16);
  }
  const uint32_t vrow = lane >> 3;
  const uint32_t vchunk16 = (((lane & 7) ^ vrow) & 7) * 16;

  // copies of one tile into LDS buffer DST; this wave's share of the 1 KB
  // blocks
  auto dma_k = [&](auto dst_tag, const TileCursor& c) {
    constexpr int DST = decltype(dst_tag)::value;
    const uint32_t sbase = static_cast<uint32_t>(c.k0) * G::kKRow;
#pragma unroll
    for (int u = 0; u < G::kKInstr; ++u) {
      const int blk = wave * G::kKInstr + u;
      // the block's row parity: kKInstr is even for D = 128, and D = 64 has
      // 8 rows per block
      const int par = kKRowsPerBlk == 4 ? (u & 1) : 0;
      static_assert(kKRowsPerBlk == 8 || (G::kKInstr % 2) == 0, "row parity per block");
      dma16(c.rk, buf(DST) + blk * 1024, koff[par], sbase + blk * 1024);
    }
  };
  auto dma_v = [&](auto dst_tag, const TileCursor& c) {
    constexpr int DST = decltype(dst_tag)::value;
    const uint32_t pitch2 = static_cast<uint32_t>(c.pitch) * 2;
    const uint32_t voff = vrow * pitch2 + vchunk16;
#pragma unroll
    for (int u = 0; u < G::kVInstr; ++u) {
      const int blk = wave * G::kVInstr + u;
      dma16(c.rv, buf(DST) + blk * 1024, voff,
            static_cast<uint32_t>(blk) * 8 * pitch2 + static_cast<uint32_t>(c.k0) * 2);
    }
  };

  // K operands of one 32-key half tile: rows col of the half at kl
  auto read_kops = [&](const unsigned char* kl, bf16x8_t (&kops)[kDS]) {
    const unsigned char* rowp = kl + col * G::kKRow;
#pragma unroll
    for (int ks = 0; ks < kDS; ++ks)
      kops[ks] = *reinterpret_cast<const bf16x8_t*>(rowp + (((ks * 2 + half) ^ (col & 7)) * 16));
  };
  auto qk = [&](const bf16x8_t (&kops)[kDS], const bf16x8_t (&qreg)[NCQ][kDS],
                f32x16_t (&s)[NCQ]) {
#pragma unroll
    for (int cq = 0; cq < NCQ; ++cq)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[cq][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kDS; ++ks)
#pragma unroll
      for (int cq = 0; cq < NCQ; ++cq)
        s[cq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kops[ks], qreg[cq][ks], s[cq], 0, 0, 0);
  };
  // the scores of one half tile with the padded keys of a segment's last
  // tile set to -inf; `valid` = keys of this half that exist.  Register i
  // holds key (i/4)*8 + half*4 + i%4.
  auto mask = [&](f32x16_t (&sc)[NCQ], int valid) {
    if (valid < 32) {
      const int lim = valid - half * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool keep = (i >> 2) * 8 + (i & 3) < lim;
#pragma unroll
        for (int cq = 0; cq < NCQ; ++cq) sc[cq][i] = keep ? sc[cq][i] : -INFINITY;
      }
    }
  };
  // scaled max over the 32 keys of a half tile, per query block
  auto half_max = [&](const f32x16_t (&sc)[NCQ], float (&mt)[NCQ]) {
#pragma unroll
    for (int cq = 0; cq < NCQ; ++cq) {
      float mx = fmaxf(sc[cq][0], sc[cq][1]);
#pragma unroll
      for (int i = 2; i < 16; ++i) mx = fmaxf(mx, sc[cq][i]);
      mt[cq] = xor32_max(mx) * a.c;
    }
  };
  // workgroup-wide OR of two per-lane flags (every wave must take the same
  // path: the passes contain barriers)
  auto vote2 = [&](bool p0, bool p1, bool& any0, bool& any1) {
    const bool w0 = __any(p0), w1 = __any(p1);
    if (lane == 0) {
      s_vote[wave][0] = w0;
      s_vote[wave][1] = w1;
    }
    __syncthreads();
    any0 = any1 = false;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      any0 = any0 || s_vote[v][0];
      any1 = any1 || s_vote[v][1];
    }
  };

  for (long long x = range_begin(w, a), xe = range_begin(w + 1, a); x < xe;) {
    const int r = static_cast<int>(x / a.ntiles);
    const int t0 = static_cast<int>(x % a.ntiles);
    const long long rest = xe - x;
    const int t1 = rest < a.ntiles - t0 ? t0 + static_cast<int>(rest) : a.ntiles;
    const bool first_piece = x == range_begin(w, a);
    x += t1 - t0;
    const int h = r / a.nqt;
    const int qbase = (r - h * a.nqt) * kBq + wave * kQW;

    // Q^T as B operand: lane holds query qbase + cq*32 + col, features
    // ks*16 + half*8 .. +7
    bf16x8_t qreg[NCQ][kDS];
#pragma unroll
    for (int cq = 0; cq < NCQ; ++cq) {
      const int qi = qbase + cq * 32 + col;
      const uint16_t* qrow = a.q + (static_cast<size_t>(qi) * a.heads + h) * D + half * 8;
#pragma unroll
      for (int ks = 0; ks < kDS; ++ks) {
        if (qi < a.n) {
          qreg[cq][ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) qreg[cq][ks][j] = static_cast<__bf16>(0.0f);
        }
      }
    }

    f32x16_t oacc[kDB][NCQ];
    float m_ref[NCQ];
    float m_seen[NCQ];
    float l_tot[NCQ], le_tot[NCQ];
    bool track_max = false;
    const int tlast = t1 - 1;
    for (int pass = 0;; ++pass) {
      float l_run[NCQ], l_exact[NCQ];
#pragma unroll
      for (int cq = 0; cq < NCQ; ++cq) {
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][cq][i] = 0.f;
        l_run[cq] = 0.f;
        l_exact[cq] = 0.f;
        m_seen[cq] = -INFINITY;
      }
      f32x16_t sacc[2][NCQ];   // [buffer][cq] scores of a 32-key half tile

      // cursors: tile j (scores, mask), tile j+1 (V copy), tile j+2 (K
      // copy); the copy cursors stop at the piece's last tile, so every step
      // issues the same number of copies (the extra ones land in a buffer
      // that is not read again) and the vmcnt waits stay exact
      TileCursor cj, cv, ck;
      cursor_seek<D>(a, cj, t0, h);
      cv = cj;
      cursor_next<D>(a, cv, tlast, h);
      ck = cv;
      cursor_next<D>(a, ck, tlast, h);

      // ---- prologue: K_t0, V_t0, K_t0+1 in LDS; scores of the first half
      // tile, whose max is the reference of the piece
      __syncthreads();
      dma_k(std::integral_constant<int, kK0>{}, cj);
      dma_v(std::integral_constant<int, kV0>{}, cj);
      dma_k(std::integral_constant<int, kK1>{}, cv);
      wait_dma();
      __syncthreads();
      {
        bf16x8_t kops[kDS];
        read_kops(buf(kK0), kops);
        qk(kops, qreg, sacc[0]);
      }
      if (pass == 0) {
        f32x16_t first[NCQ];
#pragma unroll
        for (int cq = 0; cq < NCQ; ++cq) first[cq] = sacc[0][cq];
        mask(first, cj.rows - cj.k0);
        half_max(first, m_ref);
      }

      // ---- one pipelined half step.  Half step u = 2i + hh covers keys
      // [32 hh, 32 hh + 32) of tile j = t0 + i.  It issues the next copies,
      // reads the operands it needs, computes the scores of half step u+1
      // while running the softmax of half step u, then adds P V of half step u.
      auto half_step = [&](auto u_tag) {
        constexpr int U = decltype(u_tag)::value;     // u mod 4
        constexpr int HH = U & 1;                      // which half of the tile
        constexpr int TP = (U >> 1) & 1;               // parity of the tile
        constexpr int CUR = U & 1;                     // score buffer of this half
        constexpr int KJ = TP == 0 ? kK0 : kK1;        // K of tile j
        constexpr int KN = TP == 0 ? kK1 : kK0;        // K of tile j+1
        constexpr int VJ = TP == 0 ? kV0 : kV1;        // V of tile j
        constexpr int VN = TP == 0 ? kV1 : kV0;        // V of tile j+1
        if (HH == 0) {
          dma_v(std::integral_constant<int, VN>{}, cv);   // V_{j+1}; V_{j-1} is done
        } else {
          dma_k(std::integral_constant<int, KJ>{}, ck);   // K_{j+2}; K_j is done
        }
        // operands: K rows of the next half step, Vt columns of this one
        bf16x8_t kops[kDS];
        if (HH == 0) {
          read_kops(buf(KJ) + 32 * G::kKRow, kops);
        } else {
          read_kops(buf(KN), kops);
        }
        bf16x8_t vops[2][kDB];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int db = 0; db < kDB; ++db) {
            const int ps = HH * 2 + pp;
            vops[pp][db] = *reinterpret_cast<const bf16x8_t*>(
                buf(VJ) + (db * 32 + col) * 128 + (((ps * 2 + half) ^ (col & 7)) * 16));
          }

        f32x16_t (&sc)[NCQ] = sacc[CUR];
        mask(sc, cj.rows - cj.k0 - HH * 32);
        if (track_max) {
          float mt[NCQ];
          half_max(sc, mt);
#pragma unroll
          for (int cq = 0; cq < NCQ; ++cq) m_seen[cq] = fmaxf(m_seen[cq], mt[cq]);
        }

        // scores of the next half step (discarded after the last one)
        qk(kops, qreg, sacc[1 - CUR]);

        // probabilities as bf16 P^T, and their row sums taken over the
        // rounded values the PV product uses (so O is an exact convex
        // combination of the weights applied): bf16 pairs dotted with (1, 1)
        bf16x8_t pb[NCQ][2];
        const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
        for (int cq = 0; cq < NCQ; ++cq) {
          const float neg_m = -m_ref[cq];
#pragma unroll
          for (int i = 0; i < 16; ++i)
            pb[cq][i >> 3][i & 7] =
                static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sc[cq][i], a.c, neg_m)));
          float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const bf16x8_t v = pb[cq][g];
            acc0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), ones, acc0, false);
            acc1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), ones, acc1, false);
            acc0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), ones, acc0, false);
            acc1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), ones, acc1, false);
          }
          l_run[cq] += acc0 + acc1;
          if constexpr (kLse) {
            // the log-sum-exp output wants the exact sum of the unrounded p
            float p[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(sc[cq][i], a.c, neg_m));
#pragma unroll
            for (int st = 8; st >= 1; st >>= 1)
#pragma unroll
              for (int i = 0; i < st; ++i) p[i] += p[i + st];
            l_exact[cq] += p[0];
          }
        }

        // O^T += Vt . P^T over these 32 keys
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int cq = 0; cq < NCQ; ++cq)
              oacc[db][cq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vops[pp][db], pb[cq][pp],
                                                                    oacc[db][cq], 0, 0, 0);
        // the copies issued one half step earlier must have landed (the ones
        // just issued, of the other kind, may stay in flight) and this wave's
        // LDS reads must be done before any wave starts overwriting buffers
        if (HH == 0) {
          wait_vm_keep_lds_done<G::kVInstr>();
        } else {
          wait_vm_keep_lds_done<G::kKInstr>();
        }
        barrier_no_fence();
        if (HH == 1) {
          cursor_next<D>(a, cj, tlast, h);
          cursor_next<D>(a, cv, tlast, h);
          cursor_next<D>(a, ck, tlast, h);
        }
      };

      int j = t0;
      for (; j + 1 < t1; j += 2) {
        half_step(std::integral_constant<int, 0>{});
        half_step(std::integral_constant<int, 1>{});
        half_step(std::integral_constant<int, 2>{});
        half_step(std::integral_constant<int, 3>{});
      }
      if (j < t1) {
        half_step(std::integral_constant<int, 0>{});
        half_step(std::integral_constant<int, 1>{});
      }
      // no copy may still land in a buffer the next pass or piece refills
      wait_dma();

#pragma unroll
      for (int cq = 0; cq < NCQ; ++cq) {
        l_tot[cq] = xor32_sum(l_run[cq]);
        le_tot[cq] = kLse ? xor32_sum(l_exact[cq]) : 0.f;
      }
      if (pass + 1 >= kMaxPasses) break;
      if (track_max) {
        // the true max is known now: no p of the next pass exceeds 1
#pragma unroll
        for (int cq = 0; cq < NCQ; ++cq) m_ref[cq] = m_seen[cq];
        track_max = false;
        continue;
      }
      // a key far above the reference: shift the reference by log2 of the
      // sum (the largest p is at most the sum), or find the true max first
      // if the sum overflowed.  NaN sums pass.
      bool over = false, inf = false;
#pragma unroll
      for (int cq = 0; cq < NCQ; ++cq) {
        over = over || l_tot[cq] > kSumLimit;
        inf = inf || l_tot[cq] == INFINITY;
      }
      bool any_over, any_inf;
      vote2(over, inf, any_over, any_inf);
      if (!any_over) break;
      if (any_inf) {
        track_max = true;
      } else {
#pragma unroll
        for (int cq = 0; cq < NCQ; ++cq)
          if (l_tot[cq] > kSumLimit) m_ref[cq] += __log2f(l_tot[cq]);
      }
    }
    float m_run[NCQ];
#pragma unroll
    for (int cq = 0; cq < NCQ; ++cq) m_run[cq] = m_ref[cq];

    // ---- finish the piece
    const long long rs = static_cast<long long>(r) * a.ntiles;
    const int w_lo = owner_of(rs, a);
    const int w_hi = owner_of(rs + a.ntiles - 1, a);
    bool write_final = true;
    if (w_hi > w_lo) {
      // this row is split: the last piece to arrive merges the others
      unsigned* arrived = a.counters + 2 * r;
      unsigned* written = arrived + 1;
      const unsigned npieces = static_cast<unsigned>(w_hi - w_lo + 1);
      __syncthreads();
      if (tid == 0)
        s_ticket = __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const bool last = s_ticket == npieces - 1;
      const int slot = first_piece ? 0 : 1;
      const size_t o_wave = static_cast<size_t>(wave) * kQW * D;
      const size_t ml_wave = static_cast<size_t>(wave) * G::kMl;
      if (!last) {
        write_final = false;
        // Partials are written and read with device-scope relaxed atomics
        // (write-through, coherent across the XCDs' L2s), ordered by waiting
        // for completion before the counter update: no cache writeback needed.
        float* po = a.part_o + static_cast<size_t>(2 * w + slot) * kBq * D + o_wave;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int cq = 0; cq < NCQ; ++cq)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              __hip_atomic_store(po + ((db * NCQ + cq) * 16 + i) * 64 + lane, oacc[db][cq][i],
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        float* pml = a.part_ml + static_cast<size_t>(2 * w + slot) * kWaves * G::kMl + ml_wave;
        if (half == 0) {
#pragma unroll
          for (int cq = 0; cq < NCQ; ++cq) {
            __hip_atomic_store(pml + (cq * 3 + 0) * 32 + col, m_run[cq], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(pml + (cq * 3 + 1) * 32 + col, l_tot[cq], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(pml + (cq * 3 + 2) * 32 + col, le_tot[cq], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): stores complete
        __syncthreads();
        if (tid == 0)
          __hip_atomic_fetch_add(written, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        // wait until every other piece has stored its partial (they have all
        // arrived already, so this is a short wait), then merge
        if (tid == 0) {
          for (int spin = 0; spin < (1 << 26); ++spin) {
            if (__hip_atomic_load(written, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                npieces - 1)
              break;
            __builtin_amdgcn_s_sleep(1);
          }
        }
        __syncthreads();
        // Merge in piece order whoever merges, so the result is bitwise the
        // same from run to run: sum_i O_i 2^(m_i - m_max), starting from the
        // first piece.  This wave's own partial waits in LDS (the tile
        // buffers are idle now: no copy is in flight after the loop); wave w
        // uses buffers w*NCQ .. w*NCQ + NCQ - 1.
        auto own_at = [&](int db, int cq, int i) -> float* {
          const int e = (db * NCQ + cq) * 1024;   // first float of the 16 x 64 block
          return reinterpret_cast<float*>(buf(wave * NCQ + e / G::kBufFloats)) +
                 e % G::kBufFloats + i * 64 + lane;
        };
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int cq = 0; cq < NCQ; ++cq)
#pragma unroll
            for (int i = 0; i < 16; ++i) *own_at(db, cq, i) = oacc[db][cq][i];
        float mmax[NCQ];
#pragma unroll
        for (int cq = 0; cq < NCQ; ++cq) mmax[cq] = m_run[cq];
        for (int ow = w_lo; ow <= w_hi; ++ow) {
          if (ow == w) continue;
          const int oslot = range_begin(ow, a) >= rs ? 0 : 1;
          const float* pml =
              a.part_ml + static_cast<size_t>(2 * ow + oslot) * kWaves * G::kMl + ml_wave;
#pragma unroll
          for (int cq = 0; cq < NCQ; ++cq)
            mmax[cq] = fmaxf(mmax[cq], __hip_atomic_load(pml + (cq * 3 + 0) * 32 + col,
                                                         __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT));
        }
        float own_m[NCQ], own_l[NCQ], own_le[NCQ];
#pragma unroll
        for (int cq = 0; cq < NCQ; ++cq) {
          own_m[cq] = m_run[cq];
          own_l[cq] = l_tot[cq];
          own_le[cq] = le_tot[cq];
        }
        for (int ow = w_lo; ow <= w_hi; ++ow) {
          const bool mine = ow == w;
          const bool first = ow == w_lo;
          const int oslot = range_begin(ow, a) >= rs ? 0 : 1;
          const float* po = a.part_o + static_cast<size_t>(2 * ow + oslot) * kBq * D + o_wave;
          const float* pml =
              a.part_ml + static_cast<size_t>(2 * ow + oslot) * kWaves * G::kMl + ml_wave;
#pragma unroll
          for (int cq = 0; cq < NCQ; ++cq) {
            float mo, lo, leo;
            if (mine) {
              mo = own_m[cq];
              lo = own_l[cq];
              leo = own_le[cq];
            } else {
              mo = __hip_atomic_load(pml + (cq * 3 + 0) * 32 + col, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
              lo = __hip_atomic_load(pml + (cq * 3 + 1) * 32 + col, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
              leo = __hip_atomic_load(pml + (cq * 3 + 2) * 32 + col, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
            }
            const float f = __builtin_amdgcn_exp2f(mo - mmax[cq]);
#pragma unroll
            for (int db = 0; db < kDB; ++db)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const float v = mine ? *own_at(db, cq, i)
                                     : __hip_atomic_load(po + ((db * NCQ + cq) * 16 + i) * 64 + lane,
                                                         __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
                oacc[db][cq][i] = first ? v * f : fmaf(v, f, oacc[db][cq][i]);
              }
            l_tot[cq] = first ? lo * f : fmaf(lo, f, l_tot[cq]);
            le_tot[cq] = first ? leo * f : fmaf(leo, f, le_tot[cq]);
          }
        }
#pragma unroll
        for (int cq = 0; cq < NCQ; ++cq) m_run[cq] = mmax[cq];
        if (tid == 0) {
          __hip_atomic_store(arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(written, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }

    if (write_final) {
#pragma unroll
      for (int cq = 0; cq < NCQ; ++cq) {
        const int qi = qbase + cq * 32 + col;
        if (qi >= a.n) continue;
        const float inv = 1.0f / l_tot[cq];
        uint16_t* orow = a.o + (static_cast<size_t>(qi) * a.heads + h) * D;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint32_t wv[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const __bf16 lo = static_cast<__bf16>(oacc[db][cq][g * 4 + 2 * e] * inv);
              const __bf16 hi = static_cast<__bf16>(oacc[db][cq][g * 4 + 2 * e + 1] * inv);
              wv[e] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                      (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
            }
            *reinterpret_cast<uint2*>(orow + db * 32 + g * 8 + half * 4) = make_uint2(wv[0], wv[1]);
          }
        if (kLse && half == 0)
          a.lse[static_cast<size_t>(h) * a.n + qi] = (m_run[cq] + __log2f(le_tot[cq])) * kLn2;
      }
    }
  }
}

__global__ void fill_u32(unsigned* p, int n, unsigned v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

// query blocks of 32 per wave for each head dim
template <int D>
constexpr int kNcq = 1;

template <int D>
kvc_status launch_bf16(const AttnDesc& d, hipStream_t stream) {
  constexpr int NCQ = kNcq<D>;
  using G = Geo<D, NCQ>;
  AttnArgs a;
  a.q = static_cast<const uint16_t*>(d.q);
  a.o = static_cast<uint16_t*>(d.o);
  a.lse = d.lse;
  a.n = d.n;
  a.heads = d.heads;
  a.c = d.scale * 1.4426950408889634f;
  a.nseg = d.nseg;
  int tiles = 0;
  for (int s = 0; s < d.nseg; ++s) {
    if (d.seg[s].rows <= 0 || d.seg[s].pitch < d.seg[s].rows || d.seg[s].pitch % kBk)
      return KVC_E_INVAL;
    a.seg[s].k = static_cast<const unsigned char*>(d.seg[s].k);
    a.seg[s].vt = static_cast<const unsigned char*>(d.seg[s].vt);
    a.seg[s].rows = d.seg[s].rows;
    a.seg[s].pitch = d.seg[s].pitch;
    a.seg[s].tile0 = tiles;
    a.seg[s].pad_ = 0;
    tiles += (d.seg[s].rows + kBk - 1) / kBk;
  }
  a.ntiles = tiles;
  a.nqt = (d.n + kBq - 1) / kBq;
  a.nrows = a.nqt * d.heads;
  a.total = static_cast<long long>(a.nrows) * a.ntiles;
  const long long slots = std::min(2 * device_cus(), kMaxWg);
  const long long by_size = std::max<long long>(1, a.total / kMinPieceTiles);
  a.nwg = static_cast<int>(std::min(slots, by_size));
  // workspace: counters, then partial ref/sums, then partial O
  unsigned char* ws = static_cast<unsigned char*>(d.workspace);
  const size_t cnt_bytes = align_up(sizeof(unsigned) * 2 * a.nrows, 256);
  const size_t ml_bytes = align_up(sizeof(float) * 2 * kMaxWg * G::kWaves * G::kMl, 256);
  const size_t po_bytes = sizeof(float) * 2 * kMaxWg * kBq * D;
  if (d.workspace_bytes < cnt_bytes + ml_bytes + po_bytes) return KVC_E_INVAL;
  a.counters = reinterpret_cast<unsigned*>(ws);
  a.part_ml = reinterpret_cast<float*>(ws + cnt_bytes);
  a.part_o = reinterpret_cast<float*>(ws + cnt_bytes + ml_bytes);
  if (!d.workspace_ready) {
    const int nc = 2 * a.nrows;
    hipLaunchKernelGGL(fill_u32, dim3((nc + 255) / 256), dim3(256), 0, stream, a.counters, nc,
                       0u);
  }
  if (a.lse)
    hipLaunchKernelGGL((attn_fwd_bf16<D, NCQ, true>), dim3(a.nwg), dim3(G::kThreads), 0, stream,
                       a);
  else
    hipLaunchKernelGGL((attn_fwd_bf16<D, NCQ, false>), dim3(a.nwg), dim3(G::kThreads), 0, stream,
                       a);
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
