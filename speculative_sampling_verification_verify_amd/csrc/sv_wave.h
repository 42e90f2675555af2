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

namespace sv {

constexpr int K1_WAVES = 4;              // wavefronts per workgroup
constexpr int K1_NT = 64 * K1_WAVES;
constexpr int WVPL = 8;                  // 16-byte vectors per lane per step (packed bf16 path)
constexpr int WVPL_GENERIC = 4;          // the same for fp32 and unaligned rows
constexpr int WCB = 1024;                // candidate slots per wavefront (LDS)
static_assert(WCB <= SEG, "a part's kept set must fit one list segment");

struct WaveSmem {
  uint2 cand[WCB];                       // (key, vocabulary id)
  struct {
    uint32_t hist[256];                  // radix-select histogram
  } h;
};

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
struct WChunk {
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
  __device__ __forceinline__ void for_marked(uint64_t mask, F fn) const {
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

// bf16 with 16-byte vectors: the hot path works on packed pairs.  Each dword
// holds two bf16 values; x ^ ((x >> 15) & 0x7FFF) per 16-bit half turns
// sign-magnitude into a two's-complement int16 s' that orders like the
// values, except that every negative value lands one below its key:
// s' = K for K >= 0 and s' = K - 1 for K < 0, where K = key - 0x8000.  A test
// key >= t is then s' >= T' with T = t - 0x8000 and T' = T if T >= 1, else
// T - 1.  Lane minima and maxima use packed min / max; per-element compares
// run only in lanes whose packed maximum reaches T'.
typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t ordered_pair(uint32_t w) {
  const s16x2 v = __builtin_bit_cast(s16x2, w);
  const s16x2 m = (v >> (short)15) & (short)0x7FFF;
  return __builtin_bit_cast(uint32_t, v ^ m);
}
__device__ __forceinline__ int lo16(uint32_t w) { return (int)(short)(w & 0xFFFFu); }
__device__ __forceinline__ int hi16(uint32_t w) { return (int)(short)(w >> 16); }
__device__ __forceinline__ uint32_t key_of_ordered(int sp) { return (uint32_t)(0x8000 + (sp >= 0 ? sp : sp + 1)); }
__device__ __forceinline__ int ordered_threshold(uint32_t t) {
  const int T = (int)t - 0x8000;
  return T >= 1 ? T : T - 1;
}
constexpr int ORDERED_NEG_INF = -32641;   // s' of -inf; a negative NaN orders below it

template <>
struct WChunk<uint16_t, true> {
  static constexpr int VEC = 8;
  static constexpr int NV = WVPL;   // vectors per lane per step
  uint4 raw[NV];   // ordered int16 pairs after prepare()
  int first, lim;

  __device__ __forceinline__ void load(const uint16_t* rp, int v0, int lim_, int) {
    first = v0 + (int)(threadIdx.x & 63);
    lim = lim_;
    const uint4* vp = reinterpret_cast<const uint4*>(rp);
#pragma unroll
    for (int j = 0; j < NV; ++j) raw[j] = load_nt(vp + min(first + 64 * j, lim - 1));
  }
  __device__ __forceinline__ bool valid(int j) const { return first + 64 * j < lim; }
  __device__ __forceinline__ int index_of(int j, int e) const { return (first + 64 * j) * VEC + e; }

  // Convert in place; fold the valid pairs into the packed minimum / maximum.
  __device__ __forceinline__ void prepare(s16x2& mn, s16x2& mx) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[q] = ordered_pair(w[q]);
        if (valid(j)) {
          const s16x2 v = __builtin_bit_cast(s16x2, w[q]);
          mn = __builtin_elementwise_min(mn, v);
          mx = __builtin_elementwise_max(mx, v);
        }
      }
      raw[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }

  __device__ __forceinline__ s16x2 vec_max(int j) const {
    const s16x2 a = __builtin_elementwise_max(__builtin_bit_cast(s16x2, raw[j].x), __builtin_bit_cast(s16x2, raw[j].y));
    const s16x2 b = __builtin_elementwise_max(__builtin_bit_cast(s16x2, raw[j].z), __builtin_bit_cast(s16x2, raw[j].w));
    return __builtin_elementwise_max(a, b);
  }

  // Largest key of vector j (0 when the vector is past the part).
  __device__ __forceinline__ uint32_t vec_max_key(int j) const {
    const s16x2 v = vec_max(j);
    return valid(j) ? key_of_ordered(max((int)v.x, (int)v.y)) : 0u;
  }

  // Per-element compares run only in lanes whose maximum reaches the bound,
  // and there only for the vectors whose own maximum does.
  __device__ __forceinline__ uint64_t mask_ge(uint32_t t, s16x2 mx) const {
    const int Tp = ordered_threshold(t);
    if (max((int)mx.x, (int)mx.y) < Tp) return 0ull;
    uint64_t m = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (!valid(j)) continue;
      const s16x2 v = vec_max(j);
      if (max((int)v.x, (int)v.y) < Tp) continue;
      const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
      uint32_t mb = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        mb |= lo16(w[q]) >= Tp ? (1u << (2 * q)) : 0u;
        mb |= hi16(w[q]) >= Tp ? (1u << (2 * q + 1)) : 0u;
      }
      m |= (uint64_t)mb << (8 * j);
    }
    return m;
  }

  template <class F>
  __device__ __forceinline__ void for_marked(uint64_t mask, F fn) const {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      uint32_t mb = (uint32_t)(mask >> (8 * j)) & 0xFFu;
      const uint4 r = raw[j];
      while (mb) {
        const int e = __builtin_ctz(mb);
        mb &= mb - 1u;
        const int q = e >> 1;
        const uint32_t w = q == 0 ? r.x : q == 1 ? r.y : q == 2 ? r.z : r.w;
        fn(key_of_ordered((e & 1) ? hi16(w) : lo16(w)), index_of(j, e));
      }
    }
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

// ---------------------------------------------------------------------------
// One part [e0, e1) of one logit row.  Writes the part's survivors (keys >=
// its exact k-th largest, finite only) to out[0, *out_count); flags F_BAD /
// F_DEMOTE on the sequence when the logits hold NaN / +inf or the ties do
// not fit.  Wavefront-uniform control flow throughout.
// ---------------------------------------------------------------------------
template <typename ET, bool VECTOR>
__device__ __forceinline__ void unit_select(WaveSmem& w, const ET* rp, int e0, int e1, uint32_t k, uint2* out,
                                            int32_t* out_count, uint32_t* flags) {
  constexpr int LEVELS = Key<ET>::LEVELS;
  constexpr int VEC = Key<ET>::VEC;
  constexpr int SPAN = 64 * WChunk<ET, VECTOR>::NV;   // vectors per step
  constexpr bool PACKED = VECTOR && sizeof(ET) == 2;
  const int lane = threadIdx.x & 63;
  const int v0 = e0 / VEC;
  const int lim = (e1 + VEC - 1) / VEC;
  const int nsteps = (lim - v0 + SPAN - 1) / SPAN;
  uint32_t t = 1;                        // certified bound (wavefront-uniform; 1 = none yet)
  uint32_t fill = 0;                     // buffer fill (wavefront-uniform)
  uint32_t bad = 0;                      // lane: NaN / +inf among the marked keys
  uint32_t lo = 0xFFFFFFFFu;             // lane minimum key (generic path)
  bool demoted = false;
  s16x2 pmin = {(short)32767, (short)32767};

  constexpr int NVC = WChunk<ET, VECTOR>::NV;
  // Buffer fill at which t is raised again (keeps candidates rare).
  const uint32_t refresh_at = min(k + max(64u, k / 2), (uint32_t)WCB - 64u);
  auto examine = [&](WChunk<ET, VECTOR>& ch, bool first) {
    if (demoted) return;
    uint64_t mask;
    s16x2 mx = {(short)-32768, (short)-32768};
    if constexpr (PACKED) ch.prepare(pmin, mx);
    if (first) {
      // The k-th largest of the lane maxima (or of the vector maxima) is a
      // certified bound: each maximum is a distinct element of the part.
      uint32_t t0 = 0;
      if (k <= 64) {
        uint32_t lm = 0;
#pragma unroll
        for (int j = 0; j < NVC; ++j) lm = max(lm, ch.vec_max_key(j));
        t0 = wave_kth<LEVELS>([&](auto fn) { fn(lm); }, k, w.h.hist);
      } else if (k <= 64u * NVC) {
        t0 = wave_kth<LEVELS>(
            [&](auto fn) {
#pragma unroll
              for (int j = 0; j < NVC; ++j) fn(ch.vec_max_key(j));
            },
            k, w.h.hist);
      }
      t = max(t, (uint32_t)__builtin_amdgcn_readfirstlane((int)t0));
    }
    if constexpr (PACKED) {
      mask = ch.mask_ge(t, mx);
    } else {
      mask = ch.mask_ge(t, lo);
    }
    if (__ballot(mask != 0ull) == 0ull) return;
    uint32_t c = (uint32_t)__popcll(mask);
    uint32_t incl = wave_incl_scan(c);
    uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (fill + tot > (uint32_t)WCB) {
      // Raise t to the exact k-th largest of buffer + marked keys first.
      const uint32_t fl = fill;
      const uint32_t kth = wave_kth<LEVELS>(
          [&](auto fn) {
            for (uint32_t i = lane; i < fl; i += 64) fn(w.cand[i].x);
            ch.for_marked(mask, [&](uint32_t kk, int) { fn(kk); });
          },
          k, w.h.hist);
      t = max(t, (uint32_t)__builtin_amdgcn_readfirstlane((int)kth));
      fill = wave_compact(w.cand, fill, t);
      if constexpr (PACKED) {
        mask = ch.mask_ge(t, mx);
      } else {
        uint32_t dummy = 0;
        mask = ch.mask_ge(t, dummy);
      }
      c = (uint32_t)__popcll(mask);
      incl = wave_incl_scan(c);
      tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      if (fill + tot > (uint32_t)WCB) {   // more ties at the k-th largest than the buffer holds
        demoted = true;
        return;
      }
    }
    if (tot) {
      uint32_t slot = fill + incl - c;
      ch.for_marked(mask, [&](uint32_t kk, int idx) {
        bad |= kk >= Key<ET>::POS_INF ? 1u : 0u;
        w.cand[slot++] = make_uint2(kk, (uint32_t)idx);
      });
      fill += tot;
      wave_sync_lds();
      if (fill >= refresh_at) {
        // Raise t to the exact k-th largest of the buffer and drop the rest.
        const uint32_t fl = fill;
        const uint32_t kth = wave_kth<LEVELS>(
            [&](auto fn) {
              for (uint32_t i = lane; i < fl; i += 64) fn(w.cand[i].x);
            },
            k, w.h.hist);
        t = max(t, (uint32_t)__builtin_amdgcn_readfirstlane((int)kth));
        fill = wave_compact(w.cand, fill, t);
      }
    }
  };

  // The loop body is straight-line: both buffers are examined every
  // iteration (a step past the part holds no valid element and marks
  // nothing), every load is issued unconditionally (a step past the part
  // re-reads its last vector) and demotion only turns examine() into a
  // no-op.  An early exit or a load under a branch would make the compiler
  // wait for both buffers before examining either.
  WChunk<ET, VECTOR> A, B;
  A.load(rp, v0, lim, e1);
  __builtin_amdgcn_sched_barrier(0);   // keep A's loads ahead of B's
  B.load(rp, v0 + SPAN, lim, e1);
  for (int s = 0; s < nsteps; s += 2) {
    examine(A, s == 0);
    A.load(rp, v0 + (s + 2) * SPAN, lim, e1);
    examine(B, false);
    B.load(rp, v0 + (s + 3) * SPAN, lim, e1);
  }
  if constexpr (PACKED) lo = min((int)pmin.x, (int)pmin.y) < ORDERED_NEG_INF ? 0u : 0xFFFFFFFFu;

  const bool isbad = __ballot(bad != 0 || lo < Key<ET>::NEG_INF) != 0ull;
  if (demoted || isbad) {
    if (lane == 0) {
      atomicOr(flags, isbad ? F_BAD : F_DEMOTE);
      *out_count = 0;
    }
    return;
  }
  // The part's exact kept set among its candidates.
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
// The streaming kernel: K1_WAVES independent wavefronts per workgroup, one
// (logit row, row part) unit each; units of sequences that are neither
// top-k nor argmax exit at once (the finisher takes them whole).
// ---------------------------------------------------------------------------
template <typename ET, bool VECTOR>
__global__ __launch_bounds__(K1_NT) __attribute__((amdgpu_waves_per_eu(4, 8))) void select_kernel(Args a) {
  __shared__ WaveSmem smem[K1_WAVES];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  WaveSmem& w = smem[wave];
  const int RS = 2 * a.G + 1;
  const long long unit = (long long)blockIdx.x * K1_WAVES + wave;
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
  const int e0 = part * a.PL;
  const int e1 = min(a.V, e0 + a.PL);
  int32_t* cnt = a.counts + (size_t)rowid * a.NP + part;
  if (e0 < e1) {
    unit_select<ET, VECTOR>(w, row_ptr<ET>(a, b, isP, pos), e0, e1, m.k, a.lists + list_index(a, rowid, part), cnt,
                            a.seq_flags + b);
  } else if (lane == 0) {
    *cnt = 0;
  }
}

}  // namespace sv
