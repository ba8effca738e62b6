// K3: chunk-causal sink+window attention forward over an fp8 (E4M3) KV
// cache, fp8 MFMA, gfx950.
//
// Same visible set, work split and pipeline as the bf16 kernel (see
// attn_fwd.hip and attn_common.hpp); the KV cache holds E4M3 codes with one
// float32 scale per (head, stored segment), so a segment's keys are
// k = s_k * code and its values v = s_v * code.  Q stays bf16 in memory
// (discuss.pytorch.kr "JoyAI-Video-Edit 소개", real-time deployment section:
// the deployed pipeline runs with FP8 quantisation and a bounded KV cache).
//
// Per tile and wave (32 queries), with 32x32x64 fp8 MFMAs
// (v_mfma_f32_32x32x64_f8f6f4, E4M3 x E4M3, fp32 accumulate):
//   S^T[32 keys x 32 q] = K_half . Q8^T      (2 D/64 MFMAs per half tile)
//   O^T[d x 32 q]      += Vt_tile . P8^T     (D/32 MFMAs per 64-key tile)
//   l[32 q]            += 1 . P8^T           (one MFMA: an all-ones A operand
//                                            gives every row the column sums)
// The MFMA pairs byte j of A lane (row r, half h) with byte j of B lane
// (column c, half h) over k = 64.
// - Q is quantised per query when a row piece starts, in two parts:
//   y = q * 448 / amax|q|, Q8hi = E4M3(y), Q8lo = E4M3(16 (y - Q8hi)); the
//   scores take K . Q8hi + (K . Q8lo) / 16, the second product on the MFMA's
//   block-scaled form (B scale 2^-4), so Q keeps about 8 significant bits.
//   The logit is s = acc * s_q * s_k and the softmax multiplier is
//   scale * log2(e) * s_q * s_k per segment.
// - P is quantised to E4M3 and the row sum is taken over those same codes
//   (by the ones MFMA), so O is an exact convex combination of the weights
//   applied.  E4M3 saturates at 448: the piece's reference m_ref (max of its
//   first 32 keys) must stay within 8 (log2 units) of every logit; the max
//   is tracked and a piece that exceeds it is computed again with its true
//   max as reference (then p <= 1).
// - O accumulates in units of the current segment's V scale; when the tiles
//   move to a segment with another scale, O is multiplied by s_old / s_new
//   (at most once per segment, W+3 times per row), and by the last scale at
//   the end.
// Layout of the fp8 tiles in LDS: K rows of D bytes and Vt rows of 64 bytes,
// 16-byte chunks XOR-swizzled (swz_chunk in attn_common.hpp) so that the 16
// lanes an LDS clock serves hit distinct bank groups.  The ring stores the
// Vt columns of every 64-key tile in the order pi: column p holds key
// ((p & 0x1C) << 1) | ((p & 0x20) >> 3) | (p & 3), which is the key a
// lane's accumulator register delivers to B-operand byte p % 32 of lane half
// p / 32.
#include "attn_common.hpp"

namespace kvc {
namespace attn {
namespace {

constexpr float kP8Margin = 8.0f;   // largest p allowed before recomputing: 2^8
constexpr int kMaxPasses = 3;

typedef int i32x8_t __attribute__((ext_vector_type(8)));

template <int D>
struct Geo8 {
  static constexpr int kKRow = D;                   // bytes per K row
  static constexpr int kKBytes = kBk * kKRow;       // K tile bytes
  static constexpr int kVBytes = D * kBk;           // Vt tile bytes (D rows of 64 B)
  static constexpr int kKInstr = kKBytes / 1024 / kWaves;
  static constexpr int kVInstr = kVBytes / 1024 / kWaves;
  static constexpr int kKS = D / 64;                // MFMA k-steps over d for QK^T
  static constexpr int kDB = D / 32;                // 32-row blocks of O^T
  static_assert(kKInstr >= 1 && kVInstr >= 1, "whole 1 KB copies per wave");
};


__device__ __forceinline__ i32x8_t ld32(const unsigned char* p0, const unsigned char* p1) {
  const uint4 a = *reinterpret_cast<const uint4*>(p0);
  const uint4 b = *reinterpret_cast<const uint4*>(p1);
  i32x8_t v;
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  return v;
}

__device__ __forceinline__ f32x16_t mfma8(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// the same product with B scaled by 2^-4 (block scale E8M0 123; A scale 127 = 1)
__device__ __forceinline__ f32x16_t mfma8_b16th(const i32x8_t& a, const i32x8_t& b,
                                               const f32x16_t& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 123);
}

// two floats to E4M3 codes (nearest, ties to even) in the low or high half
template <bool kHigh>
__device__ __forceinline__ int pack8(float x, float y, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(x, y, old, kHigh);
}

// This wave's lane index, computed afresh where it is called (volatile, so
// the compiler can neither merge it with another call nor hoist it): at the
// register limit, per-lane values kept from the prologue across the piece
// loop would otherwise be spilled.
__device__ __forceinline__ int lane_now() {
  int r;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
  return r;
}

template <int D, bool kLse, bool kRope, bool kRowsFirst>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_fp8(const AttnArgs a) {
  using G = Geo8<D>;
  constexpr int kKS = G::kKS;
  constexpr int kDB = G::kDB;
  // LDS: rings of four K slots and four Vt slots (one 64-key tile each), as
  // eight separate arrays so that the compiler can tell reads of one slot
  // from copies landing in another.
  __shared__ __attribute__((aligned(1024))) unsigned char kb0[G::kKBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char kb1[G::kKBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char kb2[G::kKBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char kb3[G::kKBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vb0[G::kVBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vb1[G::kVBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vb2[G::kVBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vb3[G::kVBytes];
  auto kslot = [&](int b) -> unsigned char* {
    return b == 0 ? kb0 : b == 1 ? kb1 : b == 2 ? kb2 : kb3;
  };
  auto vslot = [&](int b) -> unsigned char* {
    return b == 0 ? vb0 : b == 1 ? vb1 : b == 2 ? vb2 : vb3;
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
  // instruction).  K: a 1 KB block holds 1024 / D rows; lane l fills chunk
  // l % (D/16) of row l / (D/16) and fetches the logical chunk that the
  // swizzle puts there; the swizzle of a row depends on the lane only.  Vt:
  // a 1 KB block holds 16 rows of 64 bytes.
  constexpr int kKLanesPerRow = D / 16;
  constexpr int kKRowsPerBlk = 1024 / D;
  static_assert(G::kKInstr * kKRowsPerBlk % kSwizzleRows == 0, "K swizzle phase per copy");
  static_assert(G::kVInstr * 16 % kSwizzleRows == 0, "Vt swizzle phase per copy");
  uint32_t koff[G::kKInstr];
#pragma unroll
  for (int u = 0; u < G::kKInstr; ++u) {
    const int row = u * kKRowsPerBlk + lane / kKLanesPerRow;
    koff[u] = static_cast<uint32_t>((lane / kKLanesPerRow) * D +
                                    swz_chunk<D>(row, lane % kKLanesPerRow) * 16);
  }
  const int vrow = lane >> 2;
  const int vlog = swz_chunk<64>(vrow, lane & 3);

  auto dma_k = [&](auto dst_tag, const TileCursor& c) {
    constexpr int DST = decltype(dst_tag)::value;
    const uint32_t sbase = static_cast<uint32_t>(c.k0) * G::kKRow;
#pragma unroll
    for (int u = 0; u < G::kKInstr; ++u) {
      const int blk = wave * G::kKInstr + u;
      dma16(c.rk, kslot(DST) + blk * 1024, koff[u], sbase + blk * 1024);
    }
  };
  // Vt is stored in 64-key tiles of D rows x 64 bytes: the tile is one
  // contiguous block and block blk of it holds rows 16*blk .. +15
  const uint32_t voff = static_cast<uint32_t>(vrow) * 64 + vlog * 16;
  auto dma_v = [&](auto dst_tag, const TileCursor& c) {
    constexpr int DST = decltype(dst_tag)::value;
    const uint32_t sbase = static_cast<uint32_t>(c.k0) * D;   // (k0 / 64) * D * 64 bytes
#pragma unroll
    for (int u = 0; u < G::kVInstr; ++u) {
      const int blk = wave * G::kVInstr + u;
      dma16(c.rv, vslot(DST) + blk * 1024, voff, sbase + blk * 1024);
    }
  };

  // K operands of one 32-key half tile (rows hh*32 + col): 32 bytes of
  // features ks*64 + half*32 .. +31 per k-step
  auto read_kops = [&](const unsigned char* kt, int hh, i32x8_t (&kops)[kKS]) {
    const int r = hh * 32 + col;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      kops[ks] = ld32(kt + swz_off<D>(r, ks * 4 + half * 2), kt + swz_off<D>(r, ks * 4 + half * 2 + 1));
  };
  // scores: K . (Q8hi + Q8lo / 16)^T
  auto qk = [&](const i32x8_t (&kops)[kKS], const i32x8_t (&qhi)[kKS], const i32x8_t (&qlo)[kKS],
                f32x16_t& s) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      s = mfma8(kops[ks], qhi[ks], s);
      s = mfma8_b16th(kops[ks], qlo[ks], s);
    }
  };
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
  auto raw_max = [&](const f32x16_t& sc) -> float {
    float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = fmaxf(mx, sc[i]);
    return xor32_max(mx);
  };

  i32x8_t ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = 0x38383838;   // E4M3 1.0 in every byte

  const Split sp = make_split(a);
  if (w >= sp.nwg) return;
  // one piece: tiles [t0, t1) of row r; first_piece if it holds the first
  // tile of this workgroup's range (the partial slot it uses if split)
  auto piece = [&](const int r, const int t0, const int t1, const bool first_piece) {
    // the row count and the epoch are read as scalars in every piece: the
    // division's reciprocal and a vector copy of the epoch, hoisted out of
    // the piece loop, would each take a register across it
    int nqt = sp.nqt;
    asm volatile("" : "+s"(nqt));
    const int h = r / nqt;
    const int qbase = (r - h * nqt) * kBq + wave * kQW;

    // Q^T as B operands: lane holds query qbase + col, byte j of k-step ks
    // = feature ks*64 + half*32 + j.  q / s_q = Q8hi + Q8lo / 16 (E4M3 of
    // the value, then E4M3 of 16 x the remainder): about 8 significant bits,
    // like bf16, for two fp8 MFMAs per k-step
    i32x8_t q8[kKS], q8lo[kKS];
    float cq;   // scale * log2(e) * s_q
    {
      const int ln = lane_now();
      const int qcol = ln & 31;
      const int qhalf = ln >> 5;
      const int g = query_row(a, sp, qbase + qcol);
      float qv[kKS][32];
      const uint16_t* qrow = a.q + (static_cast<size_t>(g < 0 ? 0 : g) * a.heads + h) * D +
                             qhalf * 32;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          uint4 u = make_uint4(0, 0, 0, 0);
          if (g >= 0) {
            u = ld16(qrow + ks * 64 + c4 * 8);
            if constexpr (kRope)
              u = rope8(u, a.qrope + (static_cast<size_t>(g) * (D / 2) + ks * 32 + qhalf * 16 +
                                      c4 * 4) * 2);
          }
          const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            qv[ks][c4 * 8 + 2 * e] = bf16_bits_to_float(wv[e] & 0xFFFFu);
            qv[ks][c4 * 8 + 2 * e + 1] = bf16_bits_to_float(wv[e] >> 16);
          }
        }
      float amax = 0.f;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(qv[ks][j]));
      amax = xor32_max(amax);
      const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
      cq = a.c * (amax > 0.f ? amax / 448.0f : 1.0f);
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = qv[ks][4 * v + e] * inv;
          const int hi = pack8<true>(y[2], y[3], pack8<false>(y[0], y[1], 0));
          const auto d01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
          const auto d23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
          q8[ks][v] = hi;
          q8lo[ks][v] = pack8<true>((y[2] - d23[0]) * 16.0f, (y[3] - d23[1]) * 16.0f,
                                    pack8<false>((y[0] - d01[0]) * 16.0f,
                                                 (y[1] - d01[1]) * 16.0f, 0));
        }
    }

    f32x16_t oacc[kDB];
    f32x16_t lacc;
    float m_ref = 0.f, m_seen = -INFINITY;
    float vs_cur = 1.f;
    const int tlast = t1 - 1;
    for (int pass = 0;; ++pass) {
      m_seen = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) lacc[i] = 0.f;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
      int pv_seg = -1;
      f32x16_t sacc[2];
      int pf[2][4] = {};   // E4M3 P of the two half tiles: byte (i%4) of word i/4

      // softmax multiplier of the tile whose scores are being consumed
      auto ceff = [&](const TileCursor& c) { return cq * a.seg[c.s].ks[h]; };

      // ---- prologue.  Ring slots are indexed by (tile - t0) mod 4.  Copy
      // K of tiles t0..t0+2 and Vt of tiles t0, t0+1 in the order K0 V0 K1
      // V1 K2, so that from the first tile on the two most recent copy
      // groups are always those of the current tile (cursors stop at the
      // piece's last tile, so every copy happens and the vmcnt counts stay
      // exact); wait for K0, V0, K1 and take the scores of the first half
      // tile, whose max is the reference.
      TileCursor cj, cv, ck;
      cursor_seek<D, 1, kBk>(a, cj, t0, h);
      __syncthreads();
      ck = cj;
      cv = cj;
      dma_k(std::integral_constant<int, 0>{}, ck);
      dma_v(std::integral_constant<int, 0>{}, cv);
      cursor_next<D, 1, kBk>(a, ck, tlast, h);
      cursor_next<D, 1, kBk>(a, cv, tlast, h);
      dma_k(std::integral_constant<int, 1>{}, ck);
      dma_v(std::integral_constant<int, 1>{}, cv);
      cursor_next<D, 1, kBk>(a, ck, tlast, h);
      cursor_next<D, 1, kBk>(a, cv, tlast, h);      // tile t0+2: next Vt copy
      dma_k(std::integral_constant<int, 2>{}, ck);
      cursor_next<D, 1, kBk>(a, ck, tlast, h);      // tile t0+3: next K copy
      wait_vm_keep_lds_done<G::kVInstr + G::kKInstr>();
      __syncthreads();
      {
        i32x8_t kops[kKS];
        read_kops(kslot(0), 0, kops);
        qk(kops, q8, q8lo, sacc[0]);
      }
      if (pass == 0) {
        f32x16_t first = sacc[0];
        mask(first, cj.rows - cj.k0);
        m_ref = raw_max(first) * ceff(cj);
      }

      // ---- one tile j (U = (j - t0) mod 4): copy K of tile j+3 (into the
      // slot tile j-1 used) and Vt of tile j+2 (slot of tile j-2).  Half 0:
      // softmax of keys 0..31 while computing the scores of keys 32..63 (K
      // of tile j); half 1: softmax of keys 32..63 while computing the scores
      // of the next tile's keys 0..31 (K of tile j+1); then P V of the tile.
      // One wait and one barrier per tile.
      auto half_tile = [&](auto u_tag, auto hh_tag) {
        constexpr int U = decltype(u_tag)::value;
        constexpr int HH = decltype(hh_tag)::value;
        constexpr int CUR = HH;
        i32x8_t kops[kKS];
        if (HH == 0) {
          read_kops(kslot(U), 1, kops);
        } else {
          read_kops(kslot((U + 1) & 3), 0, kops);
        }

        f32x16_t& sc = sacc[CUR];
        mask(sc, cj.rows - cj.k0 - HH * 32);
        const float c_eff = ceff(cj);
        m_seen = fmaxf(m_seen, raw_max(sc) * c_eff);

        qk(kops, q8, q8lo, sacc[1 - CUR]);

        const float neg_m = -m_ref;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[4 * v + 0], c_eff, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[4 * v + 1], c_eff, neg_m));
          const float p2 = __builtin_amdgcn_exp2f(fmaf(sc[4 * v + 2], c_eff, neg_m));
          const float p3 = __builtin_amdgcn_exp2f(fmaf(sc[4 * v + 3], c_eff, neg_m));
          // the second conversion overwrites bytes 2-3 of the first's result, so
          // the first may write into last tile's (dead) word: no zeroing copy
          pf[HH][v] = pack8<true>(p2, p3, pack8<false>(p0, p1, pf[HH][v]));
        }
      };
      auto tile = [&](auto u_tag) {
        constexpr int U = decltype(u_tag)::value;
        // take turns with the other workgroup's wave on this SIMD (the
        // arbiter favours the older wave; see the bf16 kernel)
        __builtin_amdgcn_s_setprio(U & 1);
        dma_k(std::integral_constant<int, (U + 3) & 3>{}, ck);
        dma_v(std::integral_constant<int, (U + 2) & 3>{}, cv);
        half_tile(u_tag, std::integral_constant<int, 0>{});
        half_tile(u_tag, std::integral_constant<int, 1>{});
        // this tile's values: rescale O if the tile starts a segment with
        // another V scale, then O^T += Vt . P^T and l += 1 . P^T
        if (cj.s != pv_seg) {
          const float vs_new = a.seg[cj.s].vs[h];
          if (pv_seg >= 0) {
            const float f = vs_cur / vs_new;
#pragma unroll
            for (int db = 0; db < kDB; ++db)
#pragma unroll
              for (int i = 0; i < 16; ++i) oacc[db][i] *= f;
          }
          vs_cur = vs_new;
          pv_seg = cj.s;
        }
        i32x8_t pb;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          pb[v] = pf[0][v];
          pb[4 + v] = pf[1][v];
        }
        const unsigned char* vt = vslot(U);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const int rr = db * 32 + col;
          const i32x8_t vops = ld32(vt + swz_off<64>(rr, half * 2), vt + swz_off<64>(rr, half * 2 + 1));
          oacc[db] = mfma8(vops, pb, oacc[db]);
        }
        lacc = mfma8(ones, pb, lacc);
        // the next tile reads K of tile j+2 and Vt of tile j+1 (copied one
        // tile ago: only this tile's copies may stay in flight), and this
        // wave's LDS reads must be done before any wave refills a slot
        wait_vm_keep_lds_done<G::kKInstr + G::kVInstr>();
        barrier_no_fence();
        cursor_next<D, 1, kBk>(a, cj, tlast, h);
        cursor_next<D, 1, kBk>(a, cv, tlast, h);
        cursor_next<D, 1, kBk>(a, ck, tlast, h);
        wait_scalar_loads();
      };

      int j = t0;
      for (; j + 3 < t1; j += 4) {
        tile(std::integral_constant<int, 0>{});
        tile(std::integral_constant<int, 1>{});
        tile(std::integral_constant<int, 2>{});
        tile(std::integral_constant<int, 3>{});
      }
      if (j < t1) tile(std::integral_constant<int, 0>{});
      if (j + 1 < t1) tile(std::integral_constant<int, 1>{});
      if (j + 2 < t1) tile(std::integral_constant<int, 2>{});
      wait_dma();
      if (pass + 1 >= kMaxPasses) break;
      // a logit more than 2^8 above the reference would saturate E4M3 P:
      // recompute with the true max (NaN passes)
      const bool over = m_seen > m_ref + kP8Margin;
      bool any_over, unused;
      vote2(s_vote, wave, lane, over, false, any_over, unused);
      if (!any_over) break;
      if (over) m_ref = m_seen;
    }
    // O in true units; the row sum is the same in every accumulator row
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= vs_cur;
    const float l_tot = lacc[0];
    unsigned epoch = a.epoch;
    asm volatile("" : "+s"(epoch));
    finish_piece<D, kLse>(a, oacc, m_ref, l_tot, r, h, qbase, first_piece, w, wave, lane_now(),
                          s_ticket, sp, epoch);
  };

  // The pieces of this workgroup's range (one per row it touches).
  const long long xb = range_begin(w, sp);
  if constexpr (kRowsFirst) {
    // whole rows first, then the last piece, then the first
    RowsFirst pieces(xb, range_begin(w + 1, sp), a.ntiles);
    for (int i = 0; i < pieces.np; ++i) {
      int r, t0, t1;
      bool first_piece;
      pieces.get(i, r, t0, t1, first_piece);
      piece(r, t0, t1, first_piece);
    }
  } else {
    // last first: every workgroup then starts at the first tile of a row,
    // and the workgroups sharing a head walk its keys nearly in step, so one
    // copy of each tile in L2 serves them all
    for (long long e = range_begin(w + 1, sp); e > xb;) {
      const int r = static_cast<int>((e - 1) / a.ntiles);
      const long long row_start = static_cast<long long>(r) * a.ntiles;
      const long long s0 = xb > row_start ? xb : row_start;
      const int t0 = static_cast<int>(s0 - row_start);
      const int t1 = static_cast<int>(e - row_start);
      const bool first_piece = s0 == xb;
      e = s0;
      piece(r, t0, t1, first_piece);
    }
  }
}

template <int D>
kvc_status launch_fp8_d(const AttnDesc& d, hipStream_t stream) {
  AttnArgs a;
  for (int s = 0; s < d.nseg; ++s)
    if (!d.seg[s].k_scale || !d.seg[s].v_scale) return KVC_E_INVAL;
  const kvc_status st = fill_args(d, kBk, a, stream);
  if (st != KVC_OK) return st;
  const dim3 grid(a.nwg), block(kThreads);
  // whole rows first on the plain and RoPE calls whose ranges span more
  // than two rows (active-row calls share the last-first instances)
  if (a.qrope) {
    if (!a.qcount && rows_first(a.total, a.nwg, a.ntiles)) {
      if (a.lse) hipLaunchKernelGGL((attn_fwd_fp8<D, true, true, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((attn_fwd_fp8<D, false, true, true>), grid, block, 0, stream, a);
    } else {
      if (a.lse) hipLaunchKernelGGL((attn_fwd_fp8<D, true, true, false>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((attn_fwd_fp8<D, false, true, false>), grid, block, 0, stream, a);
    }
  } else if (!a.qcount && rows_first(a.total, a.nwg, a.ntiles)) {
    if (a.lse) hipLaunchKernelGGL((attn_fwd_fp8<D, true, false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_fwd_fp8<D, false, false, true>), grid, block, 0, stream, a);
  } else {
    if (a.lse) hipLaunchKernelGGL((attn_fwd_fp8<D, true, false, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_fwd_fp8<D, false, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_E_DEVICE;
}

}  // namespace

kvc_status launch_fp8(const AttnDesc& d, hipStream_t stream) {
  switch (d.head_dim) {
    case 64: return launch_fp8_d<64>(d, stream);
    case 128: return launch_fp8_d<128>(d, stream);
    default: return KVC_E_UNSUPPORTED;
  }
}

}  // namespace attn
}  // namespace kvc
