// K2: chunk-causal sink+window attention forward, bf16 MFMA, gfx950.
//
// For every query of the current chunk (and of its source tokens) and every
// head, softmax attention over the visible keys: condition and reference
// tokens, the sink chunk, the window chunks, the current chunk and its source
// tokens (discuss.pytorch.kr "JoyAI-Video-Edit 소개", chunk-wise
// autoregressive adaptation section: bidirectional within the chunk, causal
// across chunks through a sliding window plus the first chunk as global sink;
// architecture section: the token groups and the mask between them).  The
// visible set is never concatenated: the kernel walks the ring's segment
// table (cache slots in logical order) tile by tile.
//
// Work: a "row" is 128 queries of one head; its keys are T steps of 32 keys
// over all segments (a segment's last step is masked).  A workgroup runs one
// row at a time with 4 waves of 32 queries; two workgroups share a CU, so
// every SIMD holds two waves and interleaves one wave's softmax (VALU) with
// the other's matrix products (MFMA).  The grid is persistent: nwg
// workgroups (two per CU) split the R*T (row, step) pairs into equal
// contiguous ranges (stream-K), so the whole GPU stays busy whatever R is;
// the split and the merge of split rows live in attn_common.hpp.
//
// Instances (template flags): kLse (log-sum-exp output), kRope (q rotated at
// its load), kRowsFirst (plain and RoPE calls over ranges of more than two
// rows walk a workgroup's pieces whole rows first; otherwise last first) and
// kActive (active-row calls: the split is taken in the kernel from the
// device-side row count, with ranges kept inside one row where that costs
// few steps).  Each is its own instance so that the others' code stays as
// it is: the kernel sits at the register limit, and code added for one case
// moved the schedule of the rest.
//
// Per step and wave (32 keys x 32 queries), with 32x32x16 bf16 MFMAs (fp32
// accumulate):
//   S^T[32 keys x 32 q] = K_step . Q^T      A = K from LDS, B = Q in VGPRs
//   O^T[d x 32 q]      += Vt_step . P^T     A = Vt from LDS, B = P in VGPRs
// Computing transposed scores puts P^T straight into the B-operand layout of
// the PV product.  The accumulator holds key rows (i/4)*8 + (lane/32)*4 + i%4
// in register i; the ring stores V's key columns in exactly that order within
// each group of 16 (kappa, a swap of index bits 2 and 3), so the 8 keys a
// lane feeds to one PV step are consecutive and each Vt operand is one
// 16-byte LDS read.  Tiles are XOR-swizzled per row (swz_chunk in
// attn_common.hpp) so the 16 lanes an LDS clock serves hit distinct bank
// groups; the reads of one operand differ by an XOR of one per-lane offset.
// K and Vt are copied from global memory straight into LDS (buffer_load ...
// lds, scalar base and offset, per-lane 32-bit offset); the ring stores Vt in
// 32-key tiles, so both operands of a step are contiguous 8 KB blocks.
//
// Software pipeline over steps of 32 keys, with K and Vt in rings of four
// LDS slots each: while the softmax of step s runs on the VALU, the QK^T
// MFMAs of step s+1 are issued, then the PV MFMAs of step s (scheduling
// groups ask the compiler to put six softmax VALU instructions after each
// QK^T MFMA).  K copies run four steps ahead and Vt copies three, so every
// copy has two steps to land; one barrier per step.  The two waves sharing a
// SIMD (one from each of the CU's workgroups) take turns at the higher issue
// priority, step by step, so that neither workgroup runs ahead and leaves
// the other to finish its range alone.
//
// Softmax in base 2 with a fixed reference per row piece: t = s*scale*log2(e)
// and p = 2^(t - m_ref), where m_ref is the max of the piece's first 32 keys,
// so the largest p is at least 1.  No running max is kept: O is never
// rescaled in the loop.  A key far above m_ref shows up in the row sum
// instead: if any row sum exceeds 2^64 (or overflows) the workgroup computes
// the piece again, with m_ref raised by log2 of that sum (then no p exceeds
// 1), or, if a sum overflowed, once more tracking the true max first.  Below
// 2^64 every p, every sum and every accumulator is finite in fp32 and bf16.
// The row sum adds the bf16-rounded p the PV product uses, and the optional
// log-sum-exp output is reference + log of that same sum.
#include "attn_common.hpp"

namespace kvc {
namespace attn {
namespace {

constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64
constexpr int kMaxPasses = 4;

// Geometry of the bf16 pipeline for head dim D: steps of 32 keys; K and Vt
// of a step each fill one LDS slot, four slots per ring.
template <int D>
struct Geo {
  static constexpr int kStep = 32;                  // keys per step
  static constexpr int kKRow = 2 * D;               // bytes per K row
  static constexpr int kKBytes = kStep * kKRow;     // K slot bytes
  static constexpr int kVRow = 2 * kStep;           // bytes per Vt row (64)
  static constexpr int kVBytes = D * kVRow;         // Vt slot bytes
  static constexpr int kKInstr = kKBytes / 1024 / kWaves;   // 1 KB copy per wave-instruction
  static constexpr int kVInstr = kVBytes / 1024 / kWaves;
  static constexpr int kDS = D / 16;                // k-steps over d for QK^T
  static constexpr int kDB = D / 32;                // 32-row blocks of O^T
  static constexpr int kSlots = 4;                  // ring slots for K and for Vt
  static_assert(kKInstr >= 1 && kVInstr >= 1 && kKInstr == kVInstr, "copy counts");
};

template <int D, bool kLse, bool kRope, bool kRowsFirst, bool kActive>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16(const AttnArgs a) {
  using G = Geo<D>;
  constexpr int kDS = G::kDS;
  constexpr int kDB = G::kDB;
  constexpr int kStep = G::kStep;
  // LDS: two rings of four slots (K, Vt), as eight separate arrays so that
  // the compiler can tell reads of one slot from copies landing in another
  // (one array would make it wait for every copy in flight before any LDS
  // read).  Slot b of K is buffer b, slot b of Vt is buffer 4 + b.
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
  // instruction).  K: a block holds 1024 / (2D) rows of 2D bytes; lane l
  // fills physical chunk l % (D/8) of its row and fetches the logical chunk
  // the swizzle puts there.  Copy u of wave w covers block w*kKInstr + u; its
  // swizzle phase differs from copy 0's by u << 2 in the chunk index (4 rows
  // of 256 bytes), i.e. by u << 6 in the byte offset.  Vt: a block holds 16
  // rows of 64 bytes; the swizzle phase of a row is lane-only there.
  constexpr int kKLanesPerRow = D / 8;
  constexpr int kKRowsPerBlk = 1024 / G::kKRow;
  static_assert(G::kKInstr == 1 || kKRowsPerBlk == 4, "K copy phase by XOR");
  const int krow0 = wave * G::kKInstr * kKRowsPerBlk + lane / kKLanesPerRow;
  const uint32_t koff0 = (lane / kKLanesPerRow) * G::kKRow +
                         swz_chunk<G::kKRow>(krow0, lane % kKLanesPerRow) * 16;
  const uint32_t vrow = lane >> 2;
  const uint32_t vchunk = swz_chunk<G::kVRow>(vrow, lane & 3) * 16;

  auto dma_k = [&](auto dst_tag, const TileCursor& c) {
    constexpr int DST = decltype(dst_tag)::value;
    const uint32_t sbase = static_cast<uint32_t>(c.k0) * G::kKRow;
#pragma unroll
    for (int u = 0; u < G::kKInstr; ++u) {
      const int blk = wave * G::kKInstr + u;
      dma16(c.rk, kslot(DST) + blk * 1024, koff0 ^ (u << 6), sbase + blk * 1024);
    }
  };
  // Vt is stored in 32-key tiles of D rows x 64 bytes: the step's tile is
  // one contiguous 8 KB block and block blk of it holds rows 16*blk .. +15
  const uint32_t voff = vrow * G::kVRow + vchunk;
  auto dma_v = [&](auto dst_tag, const TileCursor& c) {
    constexpr int DST = decltype(dst_tag)::value;
    const uint32_t sbase = static_cast<uint32_t>(c.k0) * (2 * D);   // (k0 / 32) * 8 KB
#pragma unroll
    for (int u = 0; u < G::kVInstr; ++u) {
      const int blk = wave * G::kVInstr + u;
      dma16(c.rv, vslot(DST) + blk * 1024, voff, sbase + blk * 1024);
    }
  };

  // LDS reads.  Logical chunk 2j + half of row r sits at chunk
  // (half ^ s(r)) ^ 2j, so each read is one per-lane offset XORed with j << 5
  // (row offsets and slot bases leave those bits clear).
  const uint32_t krd = col * G::kKRow + swz_chunk<G::kKRow>(col, half) * 16;
  const uint32_t vrd = col * G::kVRow + swz_chunk<G::kVRow>(col, half) * 16;
  // K operands of one step (rows col of the slot)
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
  // the scores of one step with the padded keys of a segment's last step
  // set to -inf; `valid` = keys of this step that exist.  Register i holds
  // key (i/4)*8 + half*4 + i%4.
  auto mask = [&](f32x16_t& sc, int valid) {
    if (valid < kStep) {
      const int lim = valid - half * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool keep = (i >> 2) * 8 + (i & 3) < lim;
        sc[i] = keep ? sc[i] : -INFINITY;
      }
    }
  };
  // scaled max over the 32 keys of a step
  auto step_max = [&](const f32x16_t& sc) -> float {
    float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = fmaxf(mx, sc[i]);
    return xor32_max(mx) * a.c;
  };

  const Split sp = kActive ? make_split_active(a) : make_split(a);
  if (w >= sp.nwg) return;
  // one piece: steps [t0, t1) of row r; first_piece if it holds the first
  // step of this workgroup's range (the partial slot it uses if split)
  auto piece = [&](const int r, const int t0, const int t1, const bool first_piece) {
    const int h = r / sp.nqt;
    const int qbase = (r - h * sp.nqt) * kBq + wave * kQW;

    // Q^T as B operand: lane holds query qbase + col, features
    // ks*16 + half*8 .. +7
    bf16x8_t qreg[kDS];
    {
      const int g = query_row(a, sp, qbase + col);
      const uint16_t* qrow = a.q + (static_cast<size_t>(g < 0 ? 0 : g) * a.heads + h) * D +
                             half * 8;
#pragma unroll
      for (int ks = 0; ks < kDS; ++ks) {
        if (g >= 0) {
          uint4 u = ld16(qrow + ks * 16);
          if constexpr (kRope)
            u = rope8(u, a.qrope + (static_cast<size_t>(g) * (D / 2) + ks * 8 + half * 4) * 2);
          qreg[ks] = __builtin_bit_cast(bf16x8_t, u);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) qreg[ks][j] = static_cast<__bf16>(0.0f);
        }
      }
    }

    f32x16_t oacc[kDB];
    float m_ref = 0.f, m_seen = -INFINITY;
    float l_tot = 0.f;
    bool track_max = false;
    const int tlast = t1 - 1;
    for (int pass = 0;; ++pass) {
      float l_run = 0.f;
      m_seen = -INFINITY;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
      f32x16_t sacc[2];   // scores of a step, double-buffered

      // ---- prologue.  Ring slots are indexed by (step - t0) mod 4.  Copy
      // K of steps t0..t0+3 and Vt of steps t0..t0+2 (in the order K0 V0 K1
      // V1 K2 V2 K3; cursors stop at the piece's last step, so every slot
      // copy happens and the vmcnt counts stay exact), wait for K0, V0, K1,
      // and take the scores of step t0, whose max is the reference.
      TileCursor cj, cv, ck;
      cursor_seek<D, 2, kStep>(a, cj, t0, h);
      __syncthreads();
      ck = cj;
      dma_k(std::integral_constant<int, 0>{}, ck);
      dma_v(std::integral_constant<int, 0>{}, ck);
      cursor_next<D, 2, kStep>(a, ck, tlast, h);
      dma_k(std::integral_constant<int, 1>{}, ck);
      dma_v(std::integral_constant<int, 1>{}, ck);
      cursor_next<D, 2, kStep>(a, ck, tlast, h);
      dma_k(std::integral_constant<int, 2>{}, ck);
      dma_v(std::integral_constant<int, 2>{}, ck);
      cv = ck;
      cursor_next<D, 2, kStep>(a, cv, tlast, h);      // step t0+3: next V copy
      cursor_next<D, 2, kStep>(a, ck, tlast, h);
      dma_k(std::integral_constant<int, 3>{}, ck);
      cursor_next<D, 2, kStep>(a, ck, tlast, h);      // step t0+4: next K copy
      wait_vm_keep_lds_done<4 * G::kKInstr>();
      __syncthreads();
      {
        bf16x8_t kops[kDS];
        read_kops(kslot(0), kops);
        qk(kops, qreg, sacc[0]);
      }
      if (pass == 0) {
        f32x16_t first = sacc[0];
        mask(first, cj.rows - cj.k0);
        m_ref = step_max(first);
      }
      // slot 0 of K is refilled by the first step: every wave's reads of it
      // must be done
      wait_vm_keep_lds_done<4 * G::kKInstr>();
      barrier_no_fence();

      // ---- one pipelined step s (U = (s - t0) mod 4): copy K of step s+4
      // (into the slot step s used) and Vt of step s+3 (into the slot step
      // s-1 used); read K of step s+1 and Vt of step s; compute the scores
      // of step s+1 while running the softmax of step s, then add P V.
      auto step = [&](auto u_tag) {
        constexpr int U = decltype(u_tag)::value;
        constexpr int CUR = U & 1;
        // Two workgroups share each CU, one wave of each per SIMD.  The
        // issue arbiter favours the older wave, so with equal priorities one
        // workgroup runs well ahead and the other finishes its (equal) range
        // alone at one wave per SIMD.  Raising the priority on every other
        // step lets the two waves take turns being favoured, and the pair
        // ends together.
        __builtin_amdgcn_s_setprio(U & 1);
        dma_k(std::integral_constant<int, U>{}, ck);
        dma_v(std::integral_constant<int, (U + 3) & 3>{}, cv);
        bf16x8_t kops[kDS];
        read_kops(kslot((U + 1) & 3), kops);
        bf16x8_t vops[2][kDB];
        kvc::static_for<2>([&](auto pp_tag) {
          constexpr int pp = decltype(pp_tag)::value;
          // key chunk 2pp + half of Vt rows db*32 + col
          const uint32_t vo = xor_here<pp * 32>(vrd);
#pragma unroll
          for (int db = 0; db < kDB; ++db)
            vops[pp][db] = *reinterpret_cast<const bf16x8_t*>(vslot(U) + db * 32 * G::kVRow + vo);
        });

        f32x16_t& sc = sacc[CUR];
        mask(sc, cj.rows - cj.k0);
        if (track_max) m_seen = fmaxf(m_seen, step_max(sc));

        // scores of the next step (discarded after the last one)
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

        // O^T += Vt . P^T over these 32 keys
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int db = 0; db < kDB; ++db)
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vops[pp][db], pb[pp], oacc[db],
                                                              0, 0, 0);
        // Order for the scheduler: each QK^T MFMA of the next step followed
        // by six VALU instructions of this step's softmax, then the rest of
        // the VALU work, then the PV MFMAs (2% faster on MI355X than the
        // order the compiler picks by itself).  Masks: 0x008 MFMA, 0x002 VALU.
#pragma unroll
        for (int i = 0; i < kDS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * kDB, 0);
        // the next step reads K of step s+2 and Vt of step s+1 (copied two
        // steps ago: only the last two steps' copies may stay in flight),
        // and this wave's LDS reads must be done before any wave refills a
        // slot
        wait_vm_keep_lds_done<2 * (G::kKInstr + G::kVInstr)>();
        barrier_no_fence();
        cursor_next<D, 2, kStep>(a, cj, tlast, h);
        cursor_next<D, 2, kStep>(a, cv, tlast, h);
        cursor_next<D, 2, kStep>(a, ck, tlast, h);
        wait_scalar_loads();
      };

      int j = t0;
      for (; j + 3 < t1; j += 4) {
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
      }
      if (j < t1) step(std::integral_constant<int, 0>{});
      if (j + 1 < t1) step(std::integral_constant<int, 1>{});
      if (j + 2 < t1) step(std::integral_constant<int, 2>{});
      // no copy may still land in a slot the next pass or piece refills
      wait_dma();

      l_tot = xor32_sum(l_run);
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

    // the log-sum-exp output is that of the weights applied: reference +
    // log of the same sum O is divided by (within ln(1 + 2^-8) of the sum
    // of the unrounded p, each weight being rounded to bf16 once)
    finish_piece<D, kLse>(a, oacc, m_ref, l_tot, r, h, qbase, first_piece, w, wave, lane,
                          s_ticket, sp, a.epoch);
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
    // last first: every workgroup then starts at the first step of a row,
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
kvc_status launch_bf16(const AttnDesc& d, hipStream_t stream) {
  AttnArgs a;
  const kvc_status st = fill_args(d, Geo<D>::kStep, a, stream);
  if (st != KVC_OK) return st;
  const dim3 grid(a.nwg), block(kThreads);
  // active-row calls have instances of their own (their split is taken in
  // the kernel); whole rows first on the plain and RoPE calls whose ranges
  // span more than two rows
  if (a.qcount) {
    if (a.qrope) {
      if (a.lse) hipLaunchKernelGGL((attn_fwd_bf16<D, true, true, false, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((attn_fwd_bf16<D, false, true, false, true>), grid, block, 0, stream, a);
    } else {
      if (a.lse) hipLaunchKernelGGL((attn_fwd_bf16<D, true, false, false, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((attn_fwd_bf16<D, false, false, false, true>), grid, block, 0, stream, a);
    }
  } else if (a.qrope) {
    if (rows_first(a.total, a.nwg, a.ntiles)) {
      if (a.lse) hipLaunchKernelGGL((attn_fwd_bf16<D, true, true, true, false>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((attn_fwd_bf16<D, false, true, true, false>), grid, block, 0, stream, a);
    } else {
      if (a.lse) hipLaunchKernelGGL((attn_fwd_bf16<D, true, true, false, false>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((attn_fwd_bf16<D, false, true, false, false>), grid, block, 0, stream, a);
    }
  } else if (rows_first(a.total, a.nwg, a.ntiles)) {
    if (a.lse) hipLaunchKernelGGL((attn_fwd_bf16<D, true, false, true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_fwd_bf16<D, false, false, true, false>), grid, block, 0, stream, a);
  } else {
    if (a.lse) hipLaunchKernelGGL((attn_fwd_bf16<D, true, false, false, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_fwd_bf16<D, false, false, false, false>), grid, block, 0, stream, a);
  }
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

kvc_status fill_args(const AttnDesc& d, int step_keys, AttnArgs& a, hipStream_t stream) {
  a.q = static_cast<const uint16_t*>(d.q);
  a.o = static_cast<uint16_t*>(d.o);
  a.lse = d.lse;
  a.qrows = d.qrows;
  a.qcount = d.qcount;
  a.qrope = d.qrope;
  a.n = d.n;
  a.ld = d.n;
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
    tiles += (d.seg[s].rows + step_keys - 1) / step_keys;
  }
  a.ntiles = tiles;
  a.step_keys = step_keys;
  a.nqt = (d.n + kBq - 1) / kBq;
  a.nrows = a.nqt * d.heads;
  a.total = static_cast<long long>(a.nrows) * a.ntiles;
  const long long slots = std::min(2 * device_cus(), kMaxWg);
  const long long by_size = std::max<long long>(1, a.total * step_keys / kMinPieceKeys);
  a.nwg = static_cast<int>(std::min(slots, by_size));
  // workspace: arrival words, partial tags, partial reference/sums, partial O
  const WorkLayout L = attention_workspace_layout(d.heads, d.head_dim, d.n);
  static_assert(sizeof(float) * kWaves * kMl == sizeof(float) * 2 * kAttnRowQueries,
                "partial reference/sum slot size");
  if (L.rows < a.nrows || d.workspace_bytes < L.total || d.epoch == 0) return KVC_E_INVAL;
  unsigned char* ws = static_cast<unsigned char*>(d.workspace);
  a.arrive = reinterpret_cast<unsigned long long*>(ws + L.arrive_off);
  a.tags = reinterpret_cast<unsigned*>(ws + L.tags_off);
  a.part_ml = reinterpret_cast<float*>(ws + L.ml_off);
  a.part_o = reinterpret_cast<float*>(ws + L.po_off);
  a.epoch = d.epoch;
  if (!d.workspace_ready)
    hipLaunchKernelGGL(fill_u32, dim3((L.zero_words + 255) / 256), dim3(256), 0, stream,
                       reinterpret_cast<unsigned*>(ws), L.zero_words, 0u);
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
