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
// row at a time with 4 waves of 32 queries; two workgroups share a CU, so
// every SIMD holds two waves and interleaves one wave's softmax (VALU) with
// the other's matrix products (MFMA).  The grid is persistent: nwg
// workgroups (two per CU) split the R*T (row, tile) steps into equal
// contiguous ranges (stream-K), so the whole GPU stays busy whatever R is;
// the split and the merge of split rows live in attn_common.hpp.
//
// Per tile and wave (32 queries), with 32x32x16 bf16 MFMAs (fp32
// accumulate):
//   S^T[64 keys x 32 q] = K_tile . Q^T      A = K from LDS, B = Q in VGPRs
//   O^T[d x 32 q]      += Vt_tile . P^T     A = Vt from LDS, B = P in VGPRs
// Computing transposed scores puts P^T straight into the B-operand layout of
// the PV product.  The accumulator holds key rows (i/4)*8 + (lane/32)*4 + i%4
// in register i; the ring stores V's key columns in exactly that order within
// each group of 16 (kappa, a swap of index bits 2 and 3), so the 8 keys a
// lane feeds to one PV step are consecutive and each Vt operand is one
// 16-byte LDS read.  Tiles are XOR-swizzled per row (swz_chunk in
// attn_common.hpp) so the 16 lanes an LDS clock serves hit distinct bank
// groups; the swizzle depends only on the lane, so the unrolled reads of one
// lane differ by immediate offsets.  K and Vt tiles are copied from
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
#include "attn_common.hpp"

namespace kvc {
namespace attn {
namespace {

constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64
constexpr int kMaxPasses = 4;

// Geometry of the bf16 tiles for head dim D.
template <int D>
struct Geo {
  static constexpr int kKRow = 2 * D;               // bytes per K row
  static constexpr int kKBytes = kBk * kKRow;       // K tile bytes
  static constexpr int kVBytes = D * kBk * 2;       // Vt tile bytes (D rows of 128 B)
  static constexpr int kKInstr = kKBytes / 1024 / kWaves;   // 1 KB copy per wave-instruction
  static constexpr int kVInstr = kVBytes / 1024 / kWaves;
  static constexpr int kDS = D / 16;                // k-steps over d for QK^T
  static constexpr int kDB = D / 32;                // 32-row blocks of O^T
  static_assert(kKInstr >= 1 && kVInstr >= 1, "whole 1 KB copies per wave");
};

template <int D, bool kLse>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16(const AttnArgs a) {
  using G = Geo<D>;
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

  // Per-lane byte offsets of the copies (16 bytes per lane, 1 KB per wave
  // instruction).  K: a block holds 1024 / (2D) rows of 2D bytes; lane l
  // fills physical chunk l % (D/8) of row l / (D/8) and fetches the logical
  // chunk the swizzle puts there.  Vt: a block holds 8 rows of 128 bytes.
  // Each wave's blocks start on a multiple of 16 rows, so copy u of a wave
  // sees the same swizzle phase in every wave.
  constexpr int kKLanesPerRow = D / 8;
  constexpr int kKRowsPerBlk = 1024 / G::kKRow;
  static_assert(G::kKInstr * kKRowsPerBlk % kSwizzleRows == 0, "K swizzle phase per copy");
  static_assert(G::kVInstr * 8 % kSwizzleRows == 0, "Vt swizzle phase per copy");
  // Copy u (in 0..3) of a wave covers rows whose swizzle phase differs from
  // copy 0's by u << 2 in the chunk index for both K row sizes (rows 4u.. of
  // 256 bytes: r & 15 gains 4u; rows 8u.. of 128 bytes: (r >> 1) & 7 gains
  // 4u), i.e. by u << 6 in the byte offset; likewise the Vt copies by
  // (u & 1) << 6.
  const uint32_t koff0 = (lane / kKLanesPerRow) * G::kKRow +
                         swz_chunk<G::kKRow>(lane / kKLanesPerRow, lane % kKLanesPerRow) * 16;
  const uint32_t vrow = lane >> 3;
  const uint32_t vchunk0 = swz_chunk<128>(lane >> 3, lane & 7) * 16;

  // copies of one tile into LDS buffer DST; this wave's share of the 1 KB
  // blocks
  auto dma_k = [&](auto dst_tag, const TileCursor& c) {
    constexpr int DST = decltype(dst_tag)::value;
    const uint32_t sbase = static_cast<uint32_t>(c.k0) * G::kKRow;
#pragma unroll
    for (int u = 0; u < G::kKInstr; ++u) {
      const int blk = wave * G::kKInstr + u;
      dma16(c.rk, buf(DST) + blk * 1024, koff0 ^ (u << 6), sbase + blk * 1024);
    }
  };
  auto dma_v = [&](auto dst_tag, const TileCursor& c) {
    constexpr int DST = decltype(dst_tag)::value;
    const uint32_t pitch2 = static_cast<uint32_t>(c.pitch) * 2;
    const uint32_t voff = vrow * pitch2 + vchunk0;
#pragma unroll
    for (int u = 0; u < G::kVInstr; ++u) {
      const int blk = wave * G::kVInstr + u;
      dma16(c.rv, buf(DST) + blk * 1024, voff ^ ((u & 1) << 6),
            static_cast<uint32_t>(blk) * 8 * pitch2 + static_cast<uint32_t>(c.k0) * 2);
    }
  };

  // LDS reads.  Logical chunk ks*2 + half of row r sits at chunk
  // (half ^ s(r)) ^ (ks*2), so each read is one per-lane offset XORed with
  // ks << 5 (bits 5..7; row offsets and buffer bases leave them clear).
  const uint32_t krd = col * G::kKRow + swz_chunk<G::kKRow>(col, half) * 16;
  const uint32_t vrd = col * 128 + swz_chunk<128>(col, half) * 16;
  // K operands of one 32-key half tile: rows col of the half at kl
  auto read_kops = [&](const unsigned char* kl, bf16x8_t (&kops)[kDS]) {
    kvc::static_for<kDS>([&](auto ks_tag) {
      constexpr int ks = decltype(ks_tag)::value;
      kops[ks] = *reinterpret_cast<const bf16x8_t*>(kl + xor_here<ks * 32>(krd));
    });
  };
  auto qk = [&](const bf16x8_t (&kops)[kDS], const bf16x8_t (&qreg)[kDS], f32x16_t& s) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kDS; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kops[ks], qreg[ks], s, 0, 0, 0);
  };
  // the scores of one half tile with the padded keys of a segment's last
  // tile set to -inf; `valid` = keys of this half that exist.  Register i
  // holds key (i/4)*8 + half*4 + i%4.
  auto mask = [&](f32x16_t& sc, int valid) {
    if (valid < 32) {
      const int lim = valid - half * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool keep = (i >> 2) * 8 + (i & 3) < lim;
        sc[i] = keep ? sc[i] : -INFINITY;
      }
    }
  };
  // scaled max over the 32 keys of a half tile
  auto half_max = [&](const f32x16_t& sc) -> float {
    float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = fmaxf(mx, sc[i]);
    return xor32_max(mx) * a.c;
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

    // Q^T as B operand: lane holds query qbase + col, features
    // ks*16 + half*8 .. +7
    bf16x8_t qreg[kDS];
    {
      const int qi = qbase + col;
      const uint16_t* qrow = a.q + (static_cast<size_t>(qi) * a.heads + h) * D + half * 8;
#pragma unroll
      for (int ks = 0; ks < kDS; ++ks) {
        if (qi < a.n) {
          qreg[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) qreg[ks][j] = static_cast<__bf16>(0.0f);
        }
      }
    }

    f32x16_t oacc[kDB];
    float m_ref = 0.f, m_seen = -INFINITY;
    float l_tot = 0.f, le_tot = 0.f;
    bool track_max = false;
    const int tlast = t1 - 1;
    for (int pass = 0;; ++pass) {
      float l_run = 0.f, l_exact = 0.f;
      m_seen = -INFINITY;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
      f32x16_t sacc[2];   // scores of a 32-key half tile, double-buffered

      // cursors: tile j (scores, mask), tile j+1 (V copy), tile j+2 (K
      // copy); the copy cursors stop at the piece's last tile, so every step
      // issues the same number of copies (the extra ones land in a buffer
      // that is not read again) and the vmcnt waits stay exact
      TileCursor cj, cv, ck;
      cursor_seek<D, 2>(a, cj, t0, h);
      cv = cj;
      cursor_next<D, 2>(a, cv, tlast, h);
      ck = cv;
      cursor_next<D, 2>(a, ck, tlast, h);

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
        f32x16_t first = sacc[0];
        mask(first, cj.rows - cj.k0);
        m_ref = half_max(first);
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
        kvc::static_for<2>([&](auto pp_tag) {
          constexpr int pp = decltype(pp_tag)::value;
          // key chunk (HH*2 + pp)*2 + half of rows db*32 + col
          const uint32_t vo = xor_here<(HH * 2 + pp) * 32>(vrd);
#pragma unroll
          for (int db = 0; db < kDB; ++db)
            vops[pp][db] = *reinterpret_cast<const bf16x8_t*>(buf(VJ) + db * 4096 + vo);
        });

        f32x16_t& sc = sacc[CUR];
        mask(sc, cj.rows - cj.k0 - HH * 32);
        if (track_max) m_seen = fmaxf(m_seen, half_max(sc));

        // scores of the next half step (discarded after the last one)
        qk(kops, qreg, sacc[1 - CUR]);

        // probabilities as bf16 P^T, and their row sums taken over the
        // rounded values the PV product uses (so O is an exact convex
        // combination of the weights applied): bf16 pairs dotted with (1, 1)
        bf16x8_t pb[2];
        const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
        const float neg_m = -m_ref;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          pb[i >> 3][i & 7] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sc[i], a.c, neg_m)));
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const bf16x8_t v = pb[g];
          acc0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), ones, acc0, false);
          acc1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), ones, acc1, false);
          acc0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), ones, acc0, false);
          acc1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), ones, acc1, false);
        }
        l_run += acc0 + acc1;
        if constexpr (kLse) {
          // the log-sum-exp output wants the exact sum of the unrounded p
          float p[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], a.c, neg_m));
#pragma unroll
          for (int st = 8; st >= 1; st >>= 1)
#pragma unroll
            for (int i = 0; i < st; ++i) p[i] += p[i + st];
          l_exact += p[0];
        }

        // O^T += Vt . P^T over these 32 keys
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int db = 0; db < kDB; ++db)
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vops[pp][db], pb[pp], oacc[db],
                                                              0, 0, 0);
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
          cursor_next<D, 2>(a, cj, tlast, h);
          cursor_next<D, 2>(a, cv, tlast, h);
          cursor_next<D, 2>(a, ck, tlast, h);
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

      l_tot = xor32_sum(l_run);
      le_tot = kLse ? xor32_sum(l_exact) : 0.f;
      if (pass + 1 >= kMaxPasses) break;
      if (track_max) {
        // the true max is known now: no p of the next pass exceeds 1
        m_ref = m_seen;
        track_max = false;
        continue;
      }
      // a key far above the reference: shift the reference by log2 of the
      // sum (the largest p is at most the sum), or find the true max first
      // if the sum overflowed.  NaN sums pass.
      bool any_over, any_inf;
      vote2(s_vote, wave, lane, l_tot > kSumLimit, l_tot == INFINITY, any_over, any_inf);
      if (!any_over) break;
      if (any_inf)
        track_max = true;
      else if (l_tot > kSumLimit)
        m_ref += __log2f(l_tot);
    }

    finish_piece<D, kLse>(a, oacc, m_ref, l_tot, le_tot, r, h, qbase, first_piece, w, wave,
                          lane, s_ticket);
  }
}

template <int D>
kvc_status launch_bf16(const AttnDesc& d, hipStream_t stream) {
  AttnArgs a;
  const kvc_status st = fill_args(d, a);
  if (st != KVC_OK) return st;
  if (!d.workspace_ready) launch_fill_u32(a.counters, 2 * a.nrows, 0u, stream);
  if (a.lse)
    hipLaunchKernelGGL((attn_fwd_bf16<D, true>), dim3(a.nwg), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_fwd_bf16<D, false>), dim3(a.nwg), dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_E_DEVICE;
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

}  // namespace

void launch_fill_u32(unsigned* p, int n, unsigned v, hipStream_t stream) {
  hipLaunchKernelGGL(fill_u32, dim3((n + 255) / 256), dim3(256), 0, stream, p, n, v);
}

kvc_status fill_args(const AttnDesc& d, AttnArgs& a) {
  a.q = static_cast<const uint16_t*>(d.q);
  a.o = static_cast<uint16_t*>(d.o);
  a.lse = d.lse;
  a.n = d.n;
  a.heads = d.heads;
  a.c = d.scale * kLog2e;
  a.nseg = d.nseg;
  int tiles = 0;
  for (int s = 0; s < d.nseg; ++s) {
    if (d.seg[s].rows <= 0 || d.seg[s].pitch < d.seg[s].rows || d.seg[s].pitch % kBk)
      return KVC_E_INVAL;
    a.seg[s].k = static_cast<const unsigned char*>(d.seg[s].k);
    a.seg[s].vt = static_cast<const unsigned char*>(d.seg[s].vt);
    a.seg[s].ks = d.seg[s].k_scale;
    a.seg[s].vs = d.seg[s].v_scale;
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
  // workspace: counters, then partial reference/sums, then partial O
  unsigned char* ws = static_cast<unsigned char*>(d.workspace);
  const size_t cnt_bytes = align_up(sizeof(unsigned) * 2 * a.nrows, 256);
  const size_t ml_bytes = align_up(sizeof(float) * 2 * kMaxWg * kWaves * kMl, 256);
  const size_t po_bytes = sizeof(float) * 2 * kMaxWg * kBq * d.head_dim;
  if (d.workspace_bytes < cnt_bytes + ml_bytes + po_bytes) return KVC_E_INVAL;
  a.counters = reinterpret_cast<unsigned*>(ws);
  a.part_ml = reinterpret_cast<float*>(ws + cnt_bytes);
  a.part_o = reinterpret_cast<float*>(ws + cnt_bytes + ml_bytes);
  return KVC_OK;
}

}  // namespace attn

kvc_status launch_attention(const AttnDesc& d, void* stream) {
  if (d.nseg < 1 || d.nseg > kMaxSegments || d.n < 1) return KVC_E_INVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d.kv_dtype == KVC_KV_FP8_E4M3) return attn::launch_fp8(d, s);
  if (d.kv_dtype != KVC_KV_BF16) return KVC_E_UNSUPPORTED;
  switch (d.head_dim) {
    case 64: return attn::launch_bf16<64>(d, s);
    case 128: return attn::launch_bf16<128>(d, s);
    default: return KVC_E_UNSUPPORTED;
  }
}

}  // namespace kvc
