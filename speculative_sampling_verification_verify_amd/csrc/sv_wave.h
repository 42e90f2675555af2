// Streaming top-k select, one wavefront per (logit row, row part).
//
// Every wavefront works alone: no workgroup barrier is ever taken, so the
// memory pipe never drains while lanes wait for each other.  A wavefront
// streams its part of a logit row once from HBM in steps of 64 lanes x 8
// non-temporal 16-byte loads, double-buffered in registers (one step in
// flight while the previous one is examined).
//
// Threshold logic (exact).  A "certified" bound t is a key with at least k
// elements of the row >= t; it never exceeds the row's k-th largest key, so
// every element of the kept set (all keys >= the k-th largest, ties kept) is
// >= t.  The first step certifies the k-th largest of its lane (or vector)
// maxima; each step then marks the keys >= t and appends them to the
// wavefront's LDS candidate buffer.  Whenever the buffer passes a refresh
// level, t is raised to the exact k-th largest of the buffer (a radix select
// on a wave-private histogram) and the buffer is compacted; when a step's
// marked keys would overflow the buffer, t is first raised to the exact k-th
// largest of buffer + marked keys.  So the buffer never overflows unless
// more than its capacity of keys tie at the k-th largest value; then the
// sequence is handed to the multi-pass path.
//
// At the end the part writes the keys >= its exact k-th largest (finite ones
// only) to its survivor list in the workspace; the finisher kernel merges
// the parts of a row after the kernel boundary.
#pragma once

#include "sv_common.h"

#include <type_traits>

namespace sv {

constexpr int K1_WAVES = 4;              // wavefronts per workgroup
constexpr int K1_NT = 64 * K1_WAVES;
constexpr int WVPL = 8;                  // 16-byte vectors per lane per step (packed bf16 path)
constexpr int WVPL_GENERIC = 4;          // the same for fp32 and unaligned rows
constexpr int WCB = 768;                 // candidate slots per wavefront (LDS)
constexpr int SCAP = 128;                // staged vectors per wavefront (LDS)
static_assert(WCB <= SEG, "a part's kept set must fit one list segment");

struct WaveSmem {
  uint2 cand[WCB];                       // (key, vocabulary id)
  uint4 stage[SCAP];                     // flagged 16-byte vectors awaiting the drain
  uint32_t sidx[SCAP];                   // their vector index in the row
  struct {
    uint32_t hist[256];                  // radix-select histogram
  } h;
};

// Wavefront priority from the work left (left of total steps, both
// wavefront-uniform): the issue arbiter favours older wavefronts, so without
// this the first-launched ones finish their parts long before the
// last-launched ones and the memory system idles in the tail.  A wavefront
// with more of its part left ranks higher (the four priority levels, at
// half, a quarter and an eighth of the part left, so the levels are finest
// where the parts end).
__device__ __forceinline__ void progress_prio(int left, int total) {
  const int q = (left * 8) / total;
  if (q >= 4) __builtin_amdgcn_s_setprio(3);
  else if (q >= 2) __builtin_amdgcn_s_setprio(2);
  else if (q == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// ---------------------------------------------------------------------------
// One step of a part, held in registers: lane l holds vectors
// first + 64 j (j < WVPL) of the row, where first = step start + l, so every
// load instruction of the wavefront reads 1 KiB of consecutive bytes.
// ---------------------------------------------------------------------------
template <typename ET, bool VECTOR>
struct GChunk {
  static constexpr int VEC = Key<ET>::VEC;
  static constexpr int NV = WVPL_GENERIC;   // vectors per lane per step
  uint4 raw[NV];
  int first;   // vector index of raw[0]
  int lim;     // one past the part's last vector
  int eend;    // one past the part's last element

  __device__ __forceinline__ void load(const ET* rp, int v0, int lim_, int eend_) {
    first = v0 + (int)(threadIdx.x & 63);
    lim = lim_;
    eend = eend_;
    if constexpr (VECTOR) {
      const uint4* vp = reinterpret_cast<const uint4*>(rp);
#pragma unroll
      for (int j = 0; j < NV; ++j) raw[j] = load_nt(vp + min(first + 64 * j, lim - 1));
    } else {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        uint32_t w4[4] = {0u, 0u, 0u, 0u};
        const int i0 = (first + 64 * j) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int i = i0 + e;
          if (i < eend) {
            if constexpr (sizeof(ET) == 2)
              w4[e >> 1] |= (uint32_t)reinterpret_cast<const uint16_t*>(rp)[i] << (16 * (e & 1));
            else
              w4[e] = __float_as_uint(reinterpret_cast<const float*>(rp)[i]);
          }
        }
        raw[j] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
    }
  }

  __device__ __forceinline__ bool valid(int j, int e) const { return (first + 64 * j) * VEC + e < eend; }
  __device__ __forceinline__ int index_of(int j, int e) const { return (first + 64 * j) * VEC + e; }

  __device__ __forceinline__ uint32_t key(int j, int e) const {
    const uint4 r = raw[j];
    if constexpr (sizeof(ET) == 2) {
      const int q = e >> 1;
      const uint32_t w = q == 0 ? r.x : q == 1 ? r.y : q == 2 ? r.z : r.w;
      return Key<ET>::of_bits((e & 1) ? (w >> 16) : (w & 0xFFFFu));
    } else {
      const uint32_t w = e == 0 ? r.x : e == 1 ? r.y : e == 2 ? r.z : r.w;
      return Key<ET>::of_bits(w);
    }
  }

  // Bit (j * VEC + e) set when element e of vector j is valid with key >= t;
  // lo tracks the smallest valid key.
  __device__ __forceinline__ uint64_t mask_ge(uint32_t t, uint32_t& lo) const {
    uint64_t m = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const uint32_t kk = key(j, e);
        const bool ok = valid(j, e);
        lo = ok ? min(lo, kk) : lo;
        m |= (ok && kk >= t) ? (1ull << (j * VEC + e)) : 0ull;
      }
    }
    return m;
  }

  // Largest key of vector j (0 when it holds no valid element).
  __device__ __forceinline__ uint32_t vec_max_key(int j) const {
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) m = valid(j, e) ? max(m, key(j, e)) : m;
    return m;
  }

  // fn(key, index) for every marked element.
  template <class F>
  __device__ __forceinline__ void for_marked(uint64_t mask, bool, F fn) const {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      uint32_t mb = (uint32_t)(mask >> (j * VEC)) & ((1u << VEC) - 1u);
      while (mb) {
        const int e = __builtin_ctz(mb);
        mb &= mb - 1u;
        fn(key(j, e), index_of(j, e));
      }
    }
  }
};

// bf16 with 16-byte vectors: the hot path compares raw 16-bit patterns of
// packed pairs with one test, chosen by the sign of the bound.  With key(x)
// the order-preserving key of x and t a bound key:
//  * t > 0x8000 (the bound stands for a value > 0): key(x) >= t exactly when
//    the pattern read as int16 is >= t - 0x8000 (positive values order like
//    their patterns; every negative pattern reads as a negative int16);
//  * t <= 0x8000 (a value <= 0): key(x) >= t exactly when the pattern read
//    as uint16 is <= 0x10000 - t (all positive patterns lie below 0x8000,
//    and a negative value of magnitude m has pattern 0x8000 + m).
// So per 16-byte vector a packed max (int16) or min (uint16) tree decides
// whether any element reaches t; a packed uint16 max tree over all patterns
// finds negative NaNs (patterns >= 0xFF81).  Positive NaN and +inf always
// reach t and are caught as candidates.
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lo16(uint32_t w) { return (int)(short)(w & 0xFFFFu); }
__device__ __forceinline__ int hi16(uint32_t w) { return (int)(short)(w >> 16); }
constexpr uint32_t RAW_NEG_NAN = 0xFF81u; // smallest negative NaN pattern (as unsigned 16 bits)

// The compare of one 16-bit pattern h with the bound in the form above:
// pos: (int16)h >= T; else: (uint16)h <= T.
__device__ __forceinline__ bool reaches(uint32_t h, bool pos, int T) {
  return pos ? (int)(short)h >= T : (int)h <= T;
}
__device__ __forceinline__ int bound_of(uint32_t t, bool pos) { return pos ? (int)t - 0x8000 : 0x10000 - (int)t; }

struct PChunk {
  static constexpr int VEC = 8;
  static constexpr int NV = WVPL;   // vectors per lane per step
  uint4 raw[NV];   // bf16 patterns
  int first, lim;

  // Buffer loads through the row's resource descriptor: one 32-bit offset
  // per lane plus immediates, and vectors past the part (num_records) read
  // as zero without touching memory (valid() excludes them).
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, int v0, int lim_) {
    first = v0 + (int)(threadIdx.x & 63);
    lim = lim_;
    const uint32_t off = (uint32_t)first * 16u;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(off + 1024u * (uint32_t)j), 0, BUF_NT);
      raw[j] = make_uint4(v.x, v.y, v.z, v.w);
    }
  }
  __device__ __forceinline__ bool valid(int j) const { return first + 64 * j < lim; }

  __device__ __forceinline__ s16x2 smax(int j) const {
    const s16x2 a = __builtin_elementwise_max(__builtin_bit_cast(s16x2, raw[j].x), __builtin_bit_cast(s16x2, raw[j].y));
    const s16x2 b = __builtin_elementwise_max(__builtin_bit_cast(s16x2, raw[j].z), __builtin_bit_cast(s16x2, raw[j].w));
    return __builtin_elementwise_max(a, b);
  }
  __device__ __forceinline__ u16x2 umin(int j) const {
    const u16x2 a = __builtin_elementwise_min(__builtin_bit_cast(u16x2, raw[j].x), __builtin_bit_cast(u16x2, raw[j].y));
    const u16x2 b = __builtin_elementwise_min(__builtin_bit_cast(u16x2, raw[j].z), __builtin_bit_cast(u16x2, raw[j].w));
    return __builtin_elementwise_min(a, b);
  }
  __device__ __forceinline__ u16x2 umax(int j) const {
    const u16x2 a = __builtin_elementwise_max(__builtin_bit_cast(u16x2, raw[j].x), __builtin_bit_cast(u16x2, raw[j].y));
    const u16x2 b = __builtin_elementwise_max(__builtin_bit_cast(u16x2, raw[j].z), __builtin_bit_cast(u16x2, raw[j].w));
    return __builtin_elementwise_max(a, b);
  }

  // Key of the largest element of vector j (0 when past the part): the
  // largest non-negative pattern if there is one, else the negative pattern
  // of smallest magnitude.
  __device__ __forceinline__ uint32_t vec_max_key(int j) const {
    const s16x2 s = smax(j);
    const int m = max((int)s.x, (int)s.y);
    const u16x2 u = umin(j);
    const uint32_t h = m >= 0 ? (uint32_t)m : (uint32_t)min((int)u.x, (int)u.y);
    return valid(j) ? Key<uint16_t>::of_bits(h) : 0u;
  }

  // Bit j set when vector j holds an element reaching the bound; folds the
  // unsigned maxima into um (negative NaN check).
  __device__ __forceinline__ uint32_t scan(bool pos, int T, u16x2& um) const {
    uint32_t vf = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (!valid(j)) continue;
      um = __builtin_elementwise_max(um, umax(j));
      bool hit;
      if (pos) {
        const s16x2 s = smax(j);
        hit = max((int)s.x, (int)s.y) >= T;
      } else {
        const u16x2 u = umin(j);
        hit = min((int)u.x, (int)u.y) <= T;
      }
      vf |= hit ? (1u << j) : 0u;
    }
    return vf;
  }

  // Copy the flagged vectors of the step to staging slots base, base + 1,
  // ... in ascending vector index (vector slot j major, lane minor), with
  // their vector index in the row, so the candidates drained from them come
  // out in ascending vocabulary id.  Returns the number staged.
  __device__ __forceinline__ uint32_t stage(uint32_t vf, uint32_t base, uint4* dst, uint32_t* didx) const {
    const uint64_t below = lanemask_lt();
    uint32_t n = base;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const bool f = (vf >> j) & 1u;
      const uint64_t bal = __ballot(f);
      if (f) {
        const uint32_t slot = n + (uint32_t)__popcll(bal & below);
        dst[slot] = raw[j];
        didx[slot] = (uint32_t)(first + 64 * j);
      }
      n += (uint32_t)__popcll(bal);
    }
    return n - base;
  }
};

// Keep the buffer entries with key >= t, in order, in place.  Returns the
// new fill.  Entries move only downwards and each round reads its 64 slots
// before writing, so no slot is overwritten before it is read.
__device__ __forceinline__ uint32_t wave_compact(uint2* cand, uint32_t fill, uint32_t t) {
  const int lane = threadIdx.x & 63;
  uint32_t outn = 0;
  for (uint32_t base = 0; base < fill; base += 64) {
    const uint32_t i = base + lane;
    const uint2 e = i < fill ? cand[i] : make_uint2(0u, 0u);
    const bool keep = i < fill && e.x >= t;
    const uint64_t bal = __ballot(keep);
    if (keep) cand[outn + (uint32_t)__popcll(bal & lanemask_lt())] = e;
    outn += (uint32_t)__popcll(bal);
  }
  wave_sync_lds();
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)outn);
}

// Raise t to the exact k-th largest key of the buffer and keep the entries
// >= it.  Wavefront-uniform.
template <int LEVELS>
__device__ __forceinline__ void buffer_select(WaveSmem& w, uint32_t k, uint32_t& t, uint32_t& fill) {
  const int lane = threadIdx.x & 63;
  const uint32_t fl = fill;
  const uint32_t kth = wave_kth<LEVELS>(
      [&](auto fn) {
        for (uint32_t i = lane; i < fl; i += 64) fn(w.cand[i].x);
      },
      k, w.h.hist);
  t = max(t, (uint32_t)__builtin_amdgcn_readfirstlane((int)kth));
  fill = wave_compact(w.cand, fill, t);
}

// The end of a part: flags, then the keys >= the part's exact k-th largest
// (finite only) written to its survivor list.
template <typename ET>
__device__ __forceinline__ void unit_finish(WaveSmem& w, uint32_t k, uint32_t t, uint32_t fill, bool demoted,
                                            bool isbad, uint2* out, int32_t* out_count, uint32_t* flags) {
  constexpr int LEVELS = Key<ET>::LEVELS;
  const int lane = threadIdx.x & 63;
  if (demoted || isbad) {
    if (lane == 0) {
      atomicOr(flags, isbad ? F_BAD : F_DEMOTE);
      *out_count = 0;
    }
    return;
  }
  uint32_t tf = t;
  if (fill > k) {
    const uint32_t fl = fill;
    tf = max(tf, wave_kth<LEVELS>(
                     [&](auto fn) {
                       for (uint32_t i = lane; i < fl; i += 64) fn(w.cand[i].x);
                     },
                     k, w.h.hist));
  }
  uint32_t outn = 0;
  for (uint32_t base = 0; base < fill; base += 64) {
    const uint32_t i = base + lane;
    const uint2 e = i < fill ? w.cand[i] : make_uint2(0u, 0u);
    const bool keep = i < fill && e.x >= tf && e.x != Key<ET>::NEG_INF;
    const uint64_t bal = __ballot(keep);
    const uint32_t pos = outn + (uint32_t)__popcll(bal & lanemask_lt());
    if (keep && pos < (uint32_t)SEG) out[pos] = e;
    outn += (uint32_t)__popcll(bal);
  }
  if (lane == 0) {
    *out_count = (int32_t)min(outn, (uint32_t)SEG);
    if (outn > (uint32_t)SEG) atomicOr(flags, F_DEMOTE);
  }
}

// ---------------------------------------------------------------------------
// One part [e0, e1) of one logit row, general element-by-element form (fp32
// rows and rows that are not 16-byte vectors).  Writes the part's survivors
// to out[0, *out_count); flags F_BAD / F_DEMOTE on the sequence when the
// logits hold NaN / +inf or the ties do not fit.  Wavefront-uniform control
// flow throughout.
// ---------------------------------------------------------------------------
template <typename ET, bool VECTOR>
__device__ __forceinline__ void unit_select(WaveSmem& w, const ET* rp, int e0, int e1, uint32_t k, uint2* out,
                                            int32_t* out_count, uint32_t* flags) {
  constexpr int LEVELS = Key<ET>::LEVELS;
  constexpr int VEC = Key<ET>::VEC;
  constexpr int NVC = GChunk<ET, VECTOR>::NV;
  constexpr int SPAN = 64 * NVC;         // vectors per step
  const int lane = threadIdx.x & 63;
  const int v0 = e0 / VEC;
  const int lim = (e1 + VEC - 1) / VEC;
  const int nsteps = (lim - v0 + SPAN - 1) / SPAN;
  uint32_t t = 1;                        // certified bound (wavefront-uniform; 1 = none yet)
  uint32_t fill = 0;                     // buffer fill (wavefront-uniform)
  uint32_t bad = 0;                      // lane: NaN / +inf among the marked keys
  uint32_t lo = 0xFFFFFFFFu;             // lane minimum key
  bool demoted = false;
  const uint32_t refresh_at = min(k + max(32u, k / 4), (uint32_t)WCB - 64u);

  auto examine = [&](GChunk<ET, VECTOR>& ch, bool first) {
    if (demoted) return;
    if (first) {
      // The k-th largest of the vector maxima is a certified bound: each
      // maximum is a distinct element of the part.
      uint32_t t0 = 0;
      if (k <= 64u * NVC)
        t0 = wave_kth<LEVELS>(
            [&](auto fn) {
#pragma unroll
              for (int j = 0; j < NVC; ++j) fn(ch.vec_max_key(j));
            },
            k, w.h.hist);
      t = max(t, (uint32_t)__builtin_amdgcn_readfirstlane((int)t0));
    }
    uint64_t mask = ch.mask_ge(t, lo);
    if (__ballot(mask != 0ull) == 0ull) return;
    uint32_t c = (uint32_t)__popcll(mask);
    uint32_t incl = wave_incl_scan_dpp(c);
    uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (fill + tot > (uint32_t)WCB) {
      // Raise t to the exact k-th largest of buffer + marked keys first.
      const uint32_t fl = fill;
      const uint32_t kth = wave_kth<LEVELS>(
          [&](auto fn) {
            for (uint32_t i = lane; i < fl; i += 64) fn(w.cand[i].x);
            ch.for_marked(mask, false, [&](uint32_t kk, int) { fn(kk); });
          },
          k, w.h.hist);
      t = max(t, (uint32_t)__builtin_amdgcn_readfirstlane((int)kth));
      fill = wave_compact(w.cand, fill, t);
      uint32_t dummy = 0;
      mask = ch.mask_ge(t, dummy);
      c = (uint32_t)__popcll(mask);
      incl = wave_incl_scan_dpp(c);
      tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      if (fill + tot > (uint32_t)WCB) {   // more ties at the k-th largest than the buffer holds
        demoted = true;
        return;
      }
    }
    if (tot) {
      uint32_t slot = fill + incl - c;
      ch.for_marked(mask, false, [&](uint32_t kk, int idx) {
        bad |= kk >= Key<ET>::POS_INF ? 1u : 0u;
        w.cand[slot++] = make_uint2(kk, (uint32_t)idx);
      });
      fill += tot;
      wave_sync_lds();
      if (fill >= refresh_at) buffer_select<LEVELS>(w, k, t, fill);
    }
  };

  // The loop body is straight-line: both buffers are examined every
  // iteration (a step past the part holds no valid element and marks
  // nothing), every load is issued unconditionally (a step past the part
  // re-reads its last vector) and demotion only turns examine() into a
  // no-op.  An early exit or a load under a branch would make the compiler
  // wait for both buffers before examining either.
  GChunk<ET, VECTOR> A, B;
  A.load(rp, v0, lim, e1);
  __builtin_amdgcn_sched_barrier(0);   // keep A's loads ahead of B's
  B.load(rp, v0 + SPAN, lim, e1);
  for (int s = 0; s < nsteps; s += 2) {
    progress_prio(nsteps - s, nsteps);
    examine(A, s == 0);
    A.load(rp, v0 + (s + 2) * SPAN, lim, e1);
    examine(B, false);
    B.load(rp, v0 + (s + 3) * SPAN, lim, e1);
  }
  const bool isbad = __ballot(bad != 0 || lo < Key<ET>::NEG_INF) != 0ull;
  unit_finish<ET>(w, k, t, fill, demoted, isbad, out, out_count, flags);
}

// ---------------------------------------------------------------------------
// The same for bf16 rows of 16-byte vectors, the hot path.  A step only
// flags the vectors whose maximum reaches t (packed max trees on the raw
// patterns once t is positive) and copies the flagged vectors to the
// wavefront's LDS staging area; a drain pass later gives each lane one
// staged vector, so element work runs once per flagged vector, and the
// step's registers are free again at once.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void unit_select_packed(WaveSmem& w, const uint16_t* rp, int e0, int e1, uint32_t k,
                                                   uint2* out, int32_t* out_count, uint32_t* flags) {
  constexpr int LEVELS = Key<uint16_t>::LEVELS;
  constexpr int NVC = WVPL;
  constexpr int SPAN = 64 * NVC;          // vectors per step
  // Staged vectors per drain round (<= 8 per vector appended): a full
  // wavefront when the buffer has the room, half of one for large k.
  const uint32_t db = k <= 160u ? 64u : 32u;
  const int lane = threadIdx.x & 63;
  const int v0 = e0 / 8;
  const int lim = e1 / 8;
  const int nsteps = (lim - v0 + SPAN - 1) / SPAN;
  uint32_t t = 1;                         // certified bound (wavefront-uniform; 1 = none yet)
  uint32_t fill = 0;                      // candidate buffer fill (wavefront-uniform)
  uint32_t staged = 0;                    // staged vectors (wavefront-uniform)
  bool demoted = false;
  uint32_t bad = 0;                       // lane: NaN / +inf among the candidates
  u16x2 um = {(unsigned short)0, (unsigned short)0};   // unsigned maxima of the patterns seen
  const uint32_t refresh_at = min(k + max(32u, k / 4), (uint32_t)WCB - 8u * db);

  // Turn the staged vectors into candidates (keys >= the current t).
  auto drain = [&]() {
    for (uint32_t r0 = 0; r0 < staged; r0 += db) {
      if (fill + 8u * db > (uint32_t)WCB) {
        buffer_select<LEVELS>(w, k, t, fill);
        if (fill + 8u * db > (uint32_t)WCB) {   // more ties at the k-th largest than the buffer holds
          demoted = true;
          staged = 0;
          return;
        }
      }
      const bool pos = t > 0x8000u;
      const int T = bound_of(t, pos);
      const uint32_t si = r0 + lane;
      const bool have = (uint32_t)lane < db && si < staged;
      uint4 d = make_uint4(0u, 0u, 0u, 0u);
      uint32_t vi = 0;
      if (have) {
        d = w.stage[si];
        vi = w.sidx[si];
      }
      const uint32_t wd[4] = {d.x, d.y, d.z, d.w};
      uint32_t mb = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        mb |= reaches(wd[q] & 0xFFFFu, pos, T) ? (1u << (2 * q)) : 0u;
        mb |= reaches(wd[q] >> 16, pos, T) ? (1u << (2 * q + 1)) : 0u;
      }
      if (!have) mb = 0;
      const uint32_t c = (uint32_t)__popc(mb);
      const uint32_t incl = wave_incl_scan_dpp(c);
      const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      uint32_t slot = fill + incl - c;
      while (mb) {
        const int e = __builtin_ctz(mb);
        mb &= mb - 1u;
        const int q = e >> 1;
        const uint32_t wq = q == 0 ? wd[0] : q == 1 ? wd[1] : q == 2 ? wd[2] : wd[3];
        const uint32_t kk = Key<uint16_t>::of_bits((e & 1) ? (wq >> 16) : (wq & 0xFFFFu));
        bad |= kk >= Key<uint16_t>::POS_INF ? 1u : 0u;
        w.cand[slot++] = make_uint2(kk, vi * 8u + (uint32_t)e);
      }
      fill += tot;
      wave_sync_lds();
    }
    staged = 0;
    if (fill >= refresh_at) buffer_select<LEVELS>(w, k, t, fill);
  };

  // Flag, then stage, the vectors of one step that reach t.
  auto examine = [&](PChunk& ch) {
    if (demoted) return;
    const bool pos = t > 0x8000u;
    uint32_t vf = ch.scan(pos, bound_of(t, pos), um);
    if (__ballot(vf != 0u) == 0ull) return;
    uint32_t nv = (uint32_t)__popc(vf);
    uint32_t vincl = wave_incl_scan_dpp(nv);
    uint32_t tv = (uint32_t)__builtin_amdgcn_readlane((int)vincl, 63);
    if (staged + tv > (uint32_t)SCAP) {
      if (staged) drain();
      if (demoted) return;
      if (tv > (uint32_t)SCAP) {
        // Too many flagged vectors: the k-th largest of their maxima is a
        // certified bound (each maximum is a distinct element); re-flag.
        if (tv > k) {
          const uint32_t kth = wave_kth<LEVELS>(
              [&](auto fn) {
#pragma unroll
                for (int j = 0; j < NVC; ++j)
                  if (vf & (1u << j)) fn(ch.vec_max_key(j));
              },
              k, w.h.hist);
          t = max(t, (uint32_t)__builtin_amdgcn_readfirstlane((int)kth));
          const bool p2 = t > 0x8000u;
          u16x2 dummy = um;
          vf &= ch.scan(p2, bound_of(t, p2), dummy);
          nv = (uint32_t)__popc(vf);
          vincl = wave_incl_scan_dpp(nv);
          tv = (uint32_t)__builtin_amdgcn_readlane((int)vincl, 63);
        }
        if (tv > (uint32_t)SCAP) {   // more tied maxima than the staging area holds
          demoted = true;
          return;
        }
      }
    }
    staged += ch.stage(vf, staged, w.stage, w.sidx);
    wave_sync_lds();
    if (staged >= (uint32_t)SCAP - 32u) drain();   // drain in large batches
  };

  // The descriptor covers the row up to the part's end.
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(rp), (short)0, e1 * 2, BUF_WORD3);
  PChunk A, B;
  A.load(rsrc, v0, lim);
  __builtin_amdgcn_sched_barrier(0);   // keep A's loads ahead of B's
  B.load(rsrc, v0 + SPAN, lim);
  {
    // First step: the k-th largest of the vector maxima is a certified
    // bound (each maximum is a distinct element of the part).
    uint32_t t0 = 0;
    if (k <= 64u * NVC)
      t0 = wave_kth<LEVELS>(
          [&](auto fn) {
#pragma unroll
            for (int j = 0; j < NVC; ++j) fn(A.vec_max_key(j));
          },
          k, w.h.hist);
    t = max(t, (uint32_t)__builtin_amdgcn_readfirstlane((int)t0));
    examine(A);
  }
  A.load(rsrc, v0 + 2 * SPAN, lim);
  // The loop body is straight-line: both buffers are examined every
  // iteration (a step past the part holds no valid element and flags
  // nothing), every load is issued unconditionally (a step past the part
  // reads zeros through the descriptor) and demotion only turns the
  // examination into a no-op.  An early exit or a load under a branch would
  // make the compiler wait for both buffers before examining either.
  for (int s = 1; s < nsteps; s += 2) {
    progress_prio(nsteps - s, nsteps);
    examine(B);
    B.load(rsrc, v0 + (s + 2) * SPAN, lim);
    examine(A);
    A.load(rsrc, v0 + (s + 3) * SPAN, lim);
  }
  if (!demoted && staged) drain();
  const bool negnan = max((uint32_t)um.x, (uint32_t)um.y) >= RAW_NEG_NAN;
  const bool isbad = __ballot(bad != 0 || negnan) != 0ull;
  unit_finish<uint16_t>(w, k, t, fill, demoted, isbad, out, out_count, flags);
}

// ---------------------------------------------------------------------------
// The streaming kernel: K1_WAVES independent wavefronts per workgroup, one
// (logit row, row part) unit each; units of sequences that are neither
// top-k nor argmax exit at once (the finisher takes them whole).
// ---------------------------------------------------------------------------
// Workgroups past the streaming ones list the dense sequences' (sequence,
// position) pairs for the pair kernel, one sequence per thread.  Draft
// positions (a target and a draft row) fill the list from the front, bonus
// positions (a target row only, about half the work) from the back, so the
// pair kernel takes the cheap ones last.  Each wavefront reserves its slots
// with one atomic per end; the order within an end is arbitrary (every pair
// writes its own result record).
__device__ __forceinline__ void list_dense_pairs(const Args& a, long long blk) {
  const int lane = threadIdx.x & 63;
  const long long bl = blk * K1_NT + threadIdx.x;
  uint32_t cf = 0, cb = 0;
  int g = 0;
  if (bl < a.B) {
    const Mode m = seq_mode(a, (int)bl);
    if (m.mode == MODE_DENSE) {
      g = m.g;
      cf = (uint32_t)m.g;
      cb = 1u;
    }
  }
  const uint32_t inf = wave_incl_scan_dpp(cf);
  const uint32_t inb = wave_incl_scan_dpp(cb);
  const uint32_t totf = (uint32_t)__builtin_amdgcn_readlane((int)inf, 63);
  const uint32_t totb = (uint32_t)__builtin_amdgcn_readlane((int)inb, 63);
  if (totb == 0) return;   // no dense sequence in this wavefront
  uint32_t basef = 0, baseb = 0;
  if (lane == 63) {
    basef = atomicAdd(&a.dense_count[0], totf);
    baseb = atomicAdd(&a.dense_count[1], totb);
  }
  basef = (uint32_t)__builtin_amdgcn_readlane((int)basef, 63);
  baseb = (uint32_t)__builtin_amdgcn_readlane((int)baseb, 63);
  const int b = (int)bl;
  const int G1 = a.G + 1;
  const uint32_t npairs = (uint32_t)a.B * (uint32_t)G1;
  for (uint32_t j = 0; j < cf; ++j) a.dense_list[basef + inf - cf + j] = b * G1 + (int)j;
  if (cb) a.dense_list[npairs - 1u - (baseb + inb - 1u)] = b * G1 + g;
}

// One streaming unit (logit row, row part) by the calling wavefront, with
// its LDS w; units of sequences that are neither top-k nor argmax, and
// padding rows, return at once.
template <typename ET, bool VECTOR>
__device__ __forceinline__ void select_unit(const Args& a, long long unit, WaveSmem& w) {
  const int lane = threadIdx.x & 63;
  const int RS = a.RS;
  const long long rowid_ll = unit / a.NP;
  if (rowid_ll >= (long long)a.B * RS) return;
  const int rowid = (int)rowid_ll;
  const int part = (int)(unit - rowid_ll * a.NP);
  const int b = rowid / RS;
  const int slot = rowid - b * RS;
  const Mode m = seq_mode(a, b);
  if (m.mode != MODE_GREEDY && m.mode != MODE_SPARSE) return;
  const bool isP = slot <= a.G;
  const int pos = isP ? slot : slot - a.G - 1;
  if (isP ? pos > m.g : pos >= m.g) return;   // padding rows are never read
  int e0 = part * a.PL;
  int e1 = min(a.V, e0 + a.PL);
  // Under the small-call split, a top-k sequence whose part lists might not
  // fit the finisher's pool together streams each row as one part.
  if (a.split && m.mode == MODE_SPARSE && (long long)m.k * a.RS * a.NP > POOL) {
    e0 = part == 0 ? 0 : a.V;
    e1 = a.V;
  }
  int32_t* cnt = a.counts + (size_t)rowid * a.NP + part;
  if (e0 < e1) {
    if constexpr (VECTOR && sizeof(ET) == 2)
      unit_select_packed(w, row_ptr<ET>(a, b, isP, pos), e0, e1, m.k, a.lists + list_index(a, rowid, part), cnt,
                         a.seq_flags + b);
    else
      unit_select<ET, VECTOR>(w, row_ptr<ET>(a, b, isP, pos), e0, e1, m.k, a.lists + list_index(a, rowid, part),
                              cnt, a.seq_flags + b);
  } else if (lane == 0) {
    *cnt = 0;
  }
}

template <typename ET, bool VECTOR>
__global__ __launch_bounds__(K1_NT) __attribute__((amdgpu_waves_per_eu(4, 8))) void select_kernel(Args a) {
  __shared__ WaveSmem smem[K1_WAVES];
  if ((long long)blockIdx.x >= a.sel_blocks) {
    list_dense_pairs(a, (long long)blockIdx.x - a.sel_blocks);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  select_unit<ET, VECTOR>(a, (long long)blockIdx.x * K1_WAVES + wave, smem[wave]);
}

}  // namespace sv
