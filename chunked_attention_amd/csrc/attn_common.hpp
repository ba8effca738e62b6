// Pieces shared by the bf16 (attn_fwd.hip) and fp8 (attn_fwd_fp8.hip)
// attention kernels: kernel arguments, the persistent stream-K work split,
// tile cursors over the ring's segments, LDS copies, waits and barriers, and
// the end of a row piece (normalise and store, or hand a partial result to
// the piece that merges the row).
//
// Work: a "row" is 128 queries of one head; its keys are T steps (a kernel-
// defined number of keys: 32 for bf16, 64 for fp8) over all visible
// segments.  A workgroup of 4 waves (32 queries each) runs one row piece at a
// time; nwg persistent workgroups split the R*T (row, step) pairs into equal
// contiguous ranges.  A row cut between workgroups is finished by the last
// piece to arrive, which merges every piece's partial (O, reference, sums) in
// piece order, so results do not depend on timing.  Active-row calls take
// the split at run time from a device-side query count (make_split).
#pragma once

#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace attn {

constexpr int kBq = kAttnRowQueries;    // queries per row (128)
constexpr int kBk = kTileKeys;          // keys per stored tile (64): segment padding
constexpr int kWaves = 4;               // waves per workgroup, 32 queries each
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 32;                 // queries per wave
constexpr int kMaxWg = kAttnMaxWg;      // persistent workgroups at most (2 per CU)
constexpr int kMinPieceKeys = 1024;    // smallest share of a row worth splitting off
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMl = 2 * 32;             // per wave: (reference, sum) per query
static_assert(kWaves * kQW == kBq, "row = waves x queries per wave");

struct SegArg {
  const unsigned char* k;   // [H][pitch][d]
  const unsigned char* vt;  // [H][pitch/T][d][T], T = 32 (bf16) or 64 (fp8) keys
  const float* ks;          // [H] K scales (fp8 rings)
  const float* vs;          // [H] V scales (fp8 rings)
  int rows;
  int pitch;
  int tile0;                // first step of this segment in the row's step list
  int pad_;
};

struct AttnArgs {
  const uint16_t* q;
  uint16_t* o;
  float* lse;
  const int* qrows;         // active-row calls: query i is row qrows[i] of q / o / lse
  const int* qcount;        // active-row calls: number of active rows (device memory)
  const float* qrope;       // optional rotation of q rows: [ld][D/2][(cos, sin)]
  float* part_o;            // [2*kMaxWg][kBq*D] partial O, accumulator layout
  float* part_ml;           // [2*kMaxWg][waves][2][32] partial reference and sum
  unsigned long long* arrive;   // [nrows]: (epoch << 32) | pieces of the row arrived
  unsigned* tags;           // [2*kMaxWg]: epoch of the call that stored each partial
  unsigned epoch;           // this call's epoch (nonzero)
  int n;                    // queries of the call (active-row calls: at most)
  int ld;                   // rows of q / o; row stride of lse
  int heads;
  float c;                  // softmax scale * log2(e)
  int nseg;
  int ntiles;               // steps per row (T; a step is a kernel-defined key count)
  int step_keys;            // keys per step
  int nqt;                  // rows per head
  int nrows;                // heads * nqt (active-row calls: at most)
  int nwg;                  // persistent workgroups
  long long total;          // nrows * ntiles (active-row calls: at most)
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

// The call's work: queries, 128-query rows per head and (row, step) pairs.
// An active-row call reads its query count from device memory (written by an
// earlier kernel on the stream), so the split is taken at run time: the grid
// is sized for every row, and workgroups whose range is empty exit.
struct Split {
  long long total;          // heads * nqt * ntiles
  int nqt;
  int nq;
  int nwg;                  // workgroups with work (the rest exit)
};
__device__ __forceinline__ Split make_split(const AttnArgs& a) {
  if (!a.qcount) return Split{a.total, a.nqt, a.n, a.nwg};
  const int nq = min(max(*a.qcount, 0), a.n);
  const int nqt = (nq + kBq - 1) / kBq;
  const long long total = static_cast<long long>(a.heads) * nqt * a.ntiles;
  // as on the host: pieces of at least kMinPieceKeys keys
  const long long by_size = max(1LL, total * a.step_keys / kMinPieceKeys);
  return Split{total, nqt, nq, static_cast<int>(min(static_cast<long long>(a.nwg), by_size))};
}
// Workgroups for a split of `rows` rows of `steps` steps over at most `cap`.
// When the rows fit, the largest multiple m of the row count within cap:
// range w starts at step w * rows * steps / m, a row start whenever w is a
// multiple of m / rows, so every range lies inside one row and no workgroup
// pays the fixed cost of a second piece (its opening copies, a partial or a
// merge; about kPieceCostSteps steps) while the others have one.  Taken when
// the longer ranges cost fewer steps than that: rows * steps * (1/m - 1/cap)
// <= kPieceCostSteps.
constexpr long long kPieceCostSteps = 6;
__device__ __forceinline__ int split_workgroups(int rows, int steps, int cap) {
  if (rows > 0 && rows <= cap) {
    const int m = cap / rows * rows;
    if (static_cast<long long>(rows) * steps * (cap - m) <=
        kPieceCostSteps * static_cast<long long>(m) * cap)
      return m;
  }
  return cap;
}
// The split of an active-row call (its own kernel instance; a.qcount is
// set): from the device-side count, with ranges inside one row where that
// costs few steps.
__device__ __forceinline__ Split make_split_active(const AttnArgs& a) {
  const int nq = min(max(*a.qcount, 0), a.n);
  const int nqt = (nq + kBq - 1) / kBq;
  const long long total = static_cast<long long>(a.heads) * nqt * a.ntiles;
  const long long by_size = max(1LL, total * a.step_keys / kMinPieceKeys);
  const int cap = static_cast<int>(min(static_cast<long long>(a.nwg), by_size));
  return Split{total, nqt, nq, split_workgroups(a.heads * nqt, a.ntiles, cap)};
}
// row of q / o / lse that query qi of the call stands for, or -1 if none
// (past the active count, or an index outside the tensors)
__device__ __forceinline__ int query_row(const AttnArgs& a, const Split& sp, int qi) {
  if (qi >= sp.nq) return -1;
  if (!a.qrows) return qi;
  const int g = a.qrows[qi];
  return g >= 0 && g < a.ld ? g : -1;
}

// first step of workgroup w's range, and the owner of step x
__device__ __forceinline__ long long range_begin(long long w, const Split& sp) {
  return w * sp.total / sp.nwg;
}
__device__ __forceinline__ int owner_of(long long x, const Split& sp) {
  return static_cast<int>(((x + 1) * sp.nwg - 1) / sp.total);
}

// The pieces of workgroup w's range [xb, xe) of the flattened (row, step)
// space, one per row it touches, taken whole rows first, then the last
// piece, then the first (with two or fewer, last first).  For ranges over
// several long rows: the partial first piece, taken first, would set the
// workgroups out of step for the rest of the call; whole rows first keep the
// workgroups that share a head on the same keys at once.  get(i) gives the
// i-th piece's row, its steps [t0, t1) and whether it holds the range's first
// step (the partial slot it uses when its row is split); the merge does not
// depend on the order.
struct RowsFirst {
  int rb, np, tf, tl, ntiles;
  __device__ __forceinline__ RowsFirst(long long xb, long long xe, int nt) : ntiles(nt) {
    rb = static_cast<int>(xb / nt);
    const int rl = xe > xb ? static_cast<int>((xe - 1) / nt) : rb - 1;
    np = rl - rb + 1;
    tf = static_cast<int>(xb - static_cast<long long>(rb) * nt);
    tl = static_cast<int>(xe - static_cast<long long>(rl) * nt);
  }
  __device__ __forceinline__ void get(int i, int& r, int& t0, int& t1, bool& first) const {
    const int pi = np <= 2 ? np - 1 - i : (i < np - 2 ? i + 1 : (i == np - 2 ? np - 1 : 0));
    r = rb + pi;
    t0 = pi == 0 ? tf : 0;
    t1 = pi == np - 1 ? tl : ntiles;
    first = pi == 0;
  }
};
// whether whole rows first pays: ranges that span more than two rows
inline bool rows_first(long long total, int nwg, int ntiles) {
  return total > 2LL * ntiles * nwg;
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
// s_waitcnt lgkmcnt(0) at the end of a step, right after the cursors moved:
// a cursor that entered a new segment loaded its fields with scalar loads,
// and scalar loads share the counter with LDS reads.  Waiting here, where no
// LDS read is in flight, keeps the compiler from waiting for all of the next
// step's LDS reads at the first use of those fields.
__device__ __forceinline__ void wait_scalar_loads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// LDS tiles are stored as rows of RB bytes in 16-byte chunks; logical chunk c
// of row r sits at physical chunk swz_chunk<RB>(r, c) (an XOR, so the same
// function maps back).  gfx950's LDS serves a 128-bit read for 16 lanes (256
// bytes over 64 banks of 4 bytes) per clock; when 16 lanes read the same
// logical chunk of 16 consecutive rows, these swizzles put the 16 physical
// chunks in 16 distinct 16-byte bank groups of a 256-byte period.  All three
// repeat every 16 rows.
template <int RB>
__device__ __forceinline__ int swz_chunk(int r, int c) {
  static_assert(RB == 256 || RB == 128 || RB == 64, "row size");
  if constexpr (RB == 256) return c ^ (r & 15);
  else if constexpr (RB == 128) return c ^ ((r >> 1) & 7);
  else return c ^ ((r >> 2) & 3);
}
template <int RB>
__device__ __forceinline__ uint32_t swz_off(int r, int c) {
  return static_cast<uint32_t>(r * RB + swz_chunk<RB>(r, c) * 16);
}
constexpr int kSwizzleRows = 16;

// a ^ imm, computed where it is used: the asm keeps the compiler from
// hoisting one register per immediate out of the loop (the reads of one
// operand differ only by such an XOR, see swz_chunk)
template <uint32_t kImm>
__device__ __forceinline__ uint32_t xor_here(uint32_t a) {
  if constexpr (kImm == 0) {
    return a;
  } else {
    uint32_t r;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "i"(kImm), "v"(a));
    return r;
  }
}

// Workgroup barrier without a memory fence (a fence would make the compiler
// wait for every copy in flight).  Written as an asm statement with a memory
// clobber so that no memory access is moved across it at any compiler level;
// it emits no wait of its own.  The caller has already waited for its own LDS
// accesses and for the copies the next step reads.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("s_barrier" ::: "memory");
}

// Cursor over one row's key steps (SK keys each): segment, first key of the
// step, and that segment's fields, all wave-uniform (scalar registers).
// Moving to the next step touches no memory except when a segment ends.
// E = bytes per stored element.
struct TileCursor {
  int t;                    // step index within the row
  int s;                    // segment
  int k0;                   // first key of the step within the segment
  int rows;
  int pitch;
  __amdgpu_buffer_rsrc_t rk;   // this head's K plane of the segment
  __amdgpu_buffer_rsrc_t rv;   // this head's Vt plane
};

template <int D, int E>
__device__ __forceinline__ void cursor_fields(const AttnArgs& a, TileCursor& c, int h) {
  const SegArg& s = a.seg[c.s];
  c.rows = s.rows;
  c.pitch = s.pitch;
  const uint32_t plane = static_cast<uint32_t>(s.pitch) * D * E;
  c.rk = make_rsrc(s.k + static_cast<size_t>(h) * plane, plane);
  c.rv = make_rsrc(s.vt + static_cast<size_t>(h) * plane, plane);
}
template <int D, int E, int SK>
__device__ __forceinline__ void cursor_seek(const AttnArgs& a, TileCursor& c, int t, int h) {
  int s = 0;
  while (s + 1 < a.nseg && a.seg[s + 1].tile0 <= t) ++s;
  c.t = t;
  c.s = s;
  c.k0 = (t - a.seg[s].tile0) * SK;
  cursor_fields<D, E>(a, c, h);
}
// one step on, but never past step `last`
template <int D, int E, int SK>
__device__ __forceinline__ void cursor_next(const AttnArgs& a, TileCursor& c, int last, int h) {
  if (c.t >= last) return;
  ++c.t;
  c.k0 += SK;
  if (c.k0 >= c.rows) {
    ++c.s;
    c.k0 = 0;
    cursor_fields<D, E>(a, c, h);
  }
}

// x, as a value the compiler cannot see through.  Addresses derived from it
// are computed where they are used: left to itself, the compiler hoists the
// per-lane addresses of the code after the step loop (partial stores, vote
// slots) out of every loop and keeps them in VGPRs across the whole loop,
// which at this register budget spilled other long-lived values to scratch.
template <typename T>
__device__ __forceinline__ T opaque(T x) {
  asm volatile("" : "+v"(x));
  return x;
}

// workgroup-wide OR of two per-wave flags (every wave must take the same path
// when the paths contain barriers)
__device__ __forceinline__ void vote2(int (&slot)[kWaves][2], int wave, int lane, bool p0,
                                      bool p1, bool& any0, bool& any1) {
  const bool w0 = __any(p0), w1 = __any(p1);
  if (lane == 0) {
    slot[wave][0] = w0;
    slot[wave][1] = w1;
  }
  __syncthreads();
  any0 = any1 = false;
  const int z = opaque(0);
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    any0 = any0 || slot[v + z][0];
    any1 = any1 || slot[v + z][1];
  }
}

// End of a row piece.  oacc holds this wave's unnormalised O^T (accumulator
// layout: register i of block db is feature db*32 + (i/4)*8 + (lane/32)*4 +
// i%4 of query qbase + lane%32), m_run the reference (log2 units) and l_tot
// the row sum that normalises O (the lse output is m_run + log2 l_tot, in
// natural-log units).  A piece that covers its whole row writes O / l (bf16)
// and lse; otherwise the last piece of the row to arrive merges every
// piece's partial in piece order, and the others store theirs.  epoch is the
// call's epoch (a.epoch; a caller at the register limit may pass a copy it
// keeps in a scalar register).
//
// Protocol (every word tagged with the call's epoch, so nothing is reset and
// stale words from earlier calls are told apart):
//   - arrival: one 64-bit compare-and-swap on the row's word, which holds
//     (epoch << 32) | pieces arrived; a word of another epoch counts as zero.
//     The piece that makes the count npieces merges.
//   - a storing piece writes its partial with agent-scope atomic stores,
//     every wave waits for their completion, and then the tag of its slot is
//     set to the epoch with release ordering at agent scope.
//   - the merging piece waits until every other piece's tag holds the epoch
//     (relaxed loads, bounded), takes an agent-scope acquire fence, and reads
//     the partials with agent-scope atomic loads.  Should the bound ever be
//     reached, the row is written as NaN rather than silently missing a
//     partial; a late store can only set a tag to this epoch, which no later
//     call takes for its own.
// `s_ticket` is a workgroup-shared word.
template <int D, bool kLse>
__device__ __forceinline__ void finish_piece(const AttnArgs& a, f32x16_t (&oacc)[D / 32],
                                             float m_run, float l_tot, int r, int h, int qbase,
                                             bool first_piece, int w, int wave, int lane,
                                             unsigned& s_ticket, const Split& sp,
                                             const unsigned epoch) {
  constexpr int kDB = D / 32;
  const int tid = threadIdx.x;
  lane = opaque(lane);
  const int col = lane & 31;
  const int half = lane >> 5;
  const long long rs = static_cast<long long>(r) * a.ntiles;
  const int w_lo = owner_of(rs, sp);
  const int w_hi = owner_of(rs + a.ntiles - 1, sp);
  if (w_hi > w_lo) {
    // this row is split: the last piece to arrive merges the others
    const unsigned npieces = static_cast<unsigned>(w_hi - w_lo + 1);
    __syncthreads();
    if (tid == 0) {
      unsigned long long* word = a.arrive + r;
      const unsigned long long mine = static_cast<unsigned long long>(epoch) << 32;
      unsigned long long old = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      unsigned long long next;
      do {
        next = (old >> 32) == epoch ? old + 1 : mine | 1u;
      } while (!__hip_atomic_compare_exchange_strong(word, &old, next, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      s_ticket = static_cast<unsigned>(next);
    }
    __syncthreads();
    const bool last = s_ticket == npieces;
    const size_t o_wave = static_cast<size_t>(wave) * kQW * D;
    const size_t ml_wave = static_cast<size_t>(wave) * kMl;
    if (!last) {
      const int slot = 2 * w + (first_piece ? 0 : 1);
      float* po = a.part_o + static_cast<size_t>(slot) * kBq * D + o_wave;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          __hip_atomic_store(po + (db * 16 + i) * 64 + lane, oacc[db][i], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      float* pml = a.part_ml + static_cast<size_t>(slot) * kWaves * kMl + ml_wave;
      if (half == 0) {
        __hip_atomic_store(pml + 0 * 32 + col, m_run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(pml + 1 * 32 + col, l_tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): stores complete
      __syncthreads();
      if (tid == 0)
        __hip_atomic_store(a.tags + slot, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    // wait until every other piece has stored its partial (they have all
    // arrived already, so this is a short wait), then merge in piece order
    // whoever merges, so the result is bitwise the same from run to run:
    // sum_i O_i 2^(m_i - m_max), starting from the first piece.  (The flag
    // has a word of its own: other waves may still be reading s_ticket.)
    __shared__ unsigned s_missing;
    if (tid == 0) {
      unsigned missing = 0;
      int budget = 1 << 26;
      for (int ow = w_lo; ow <= w_hi; ++ow) {
        if (ow == w) continue;
        const int oslot = 2 * ow + (range_begin(ow, sp) >= rs ? 0 : 1);
        while (__hip_atomic_load(a.tags + oslot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
               epoch) {
          if (--budget <= 0) {
            missing = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (missing) break;
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      s_missing = missing;
    }
    __syncthreads();
    const bool poisoned = s_missing != 0;
    float mmax = m_run;
    for (int ow = w_lo; ow <= w_hi; ++ow) {
      if (ow == w) continue;
      const int oslot = 2 * ow + (range_begin(ow, sp) >= rs ? 0 : 1);
      const float* pml = a.part_ml + static_cast<size_t>(oslot) * kWaves * kMl + ml_wave;
      mmax = fmaxf(mmax, __hip_atomic_load(pml + col, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
    f32x16_t acc[kDB];
    float l_acc = 0.f;
    for (int ow = w_lo; ow <= w_hi; ++ow) {
      const bool first = ow == w_lo;
      float mo = m_run, lo = l_tot;
      f32x16_t v[kDB];
      if (ow == w) {
#pragma unroll
        for (int db = 0; db < kDB; ++db) v[db] = oacc[db];
      } else {
        const int oslot = 2 * ow + (range_begin(ow, sp) >= rs ? 0 : 1);
        const float* po = a.part_o + static_cast<size_t>(oslot) * kBq * D + o_wave;
        const float* pml = a.part_ml + static_cast<size_t>(oslot) * kWaves * kMl + ml_wave;
        mo = __hip_atomic_load(pml + 0 * 32 + col, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lo = __hip_atomic_load(pml + 1 * 32 + col, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            v[db][i] = __hip_atomic_load(po + (db * 16 + i) * 64 + lane, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      }
      const float f = __builtin_amdgcn_exp2f(mo - mmax);
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = first ? v[db][i] * f : fmaf(v[db][i], f, acc[db][i]);
      l_acc = first ? lo * f : fmaf(lo, f, l_acc);
    }
#pragma unroll
    for (int db = 0; db < kDB; ++db) oacc[db] = acc[db];
    m_run = mmax;
    l_tot = poisoned ? __builtin_nanf("") : l_acc;
  }

  const int g = query_row(a, sp, qbase + col);
  if (g < 0) return;
  const float inv = 1.0f / l_tot;
  uint16_t* orow = a.o + (static_cast<size_t>(g) * a.heads + h) * D;
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t wv[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const __bf16 lo = static_cast<__bf16>(oacc[db][g * 4 + 2 * e] * inv);
        const __bf16 hi = static_cast<__bf16>(oacc[db][g * 4 + 2 * e + 1] * inv);
        wv[e] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
      }
      *reinterpret_cast<uint2*>(orow + db * 32 + g * 8 + half * 4) = make_uint2(wv[0], wv[1]);
    }
  if (kLse && half == 0)
    a.lse[static_cast<size_t>(h) * a.ld + g] = (m_run + __log2f(l_tot)) * kLn2;
}

// Host side: kernel arguments from a launch description (segment table in
// steps of step_keys keys, rows, grid, workspace); before a ring's first call
// (workspace not ready) it also zeroes the workspace's arrival words and tags
// on the stream.  Returns KVC_OK or KVC_E_INVAL.
kvc_status fill_args(const AttnDesc& d, int step_keys, AttnArgs& a, hipStream_t stream);

// the fp8 launcher (attn_fwd_fp8.hip)
kvc_status launch_fp8(const AttnDesc& d, hipStream_t stream);

}  // namespace attn
}  // namespace kvc
