// Streaming top-k select: one pass over each logit row.
//
// One workgroup handles one part (CPP consecutive chunks) of one logit row.
// A chunk is NT lanes x VPL 16-byte vectors: each lane holds its VPL vectors
// in registers while the next chunk's non-temporal loads are in flight, so
// the row is read from HBM once and the memory pipe stays busy while keys
// are compared.
//
// Threshold logic (exact, no sampling heuristics).  A "certified" bound t is
// a key with at least k elements of the row >= t; it never exceeds the row's
// k-th largest key, so every element of the kept set (all keys >= the k-th
// largest, ties included) is >= t.
//  * The first chunk certifies the k-th largest of the lanes' maxima (each
//    lane maximum is a distinct element).
//  * Lanes mark the keys >= t of their chunk in a bit mask; each wavefront
//    reserves room for its marked keys with one LDS atomic and writes them to
//    the workgroup's candidate buffer.  No block barrier is needed for this.
//  * At check points (every `sync` chunks and after the last one) the
//    workgroup reads the buffer's fill; when it holds >= k keys their k-th
//    largest is certified and the buffer is compacted to the keys >= it.
//    Appends that found the buffer full were dropped: the check point then
//    rebuilds the buffer from a re-read of the part so far.
// At the end the part keeps its candidates >= their exact k-th largest and
// writes them to its own segment of the row's list; parts of a row never talk
// to each other (the finisher merges them after the kernel boundary).  Keys
// equal to -inf carry no probability mass and are dropped.
#pragma once

#include "sv_common.h"

namespace sv {

template <typename ET, bool VECTOR>
struct Chunk {
  static constexpr int VEC = Key<ET>::VEC;
  static constexpr int EPL = VPL * VEC;   // elements per lane (<= 32: one mask bit each)
  uint4 raw[VPL];
  int first;   // this lane's first vector index; vector j is first + j * NT
  int lim;     // one past the chunk's last vector
  int V;

  // Vectors [start / VEC, ceil(end / VEC)) of the row; start is a multiple of
  // VEC.  The vector path requires V % VEC == 0 and 16-byte aligned rows;
  // the scalar path packs the elements the same way with 2- or 4-byte loads.
  __device__ __forceinline__ void load(const ET* rp, int start, int end, int Vrow) {
    first = start / VEC + (int)threadIdx.x;
    lim = (end + VEC - 1) / VEC;
    V = Vrow;
    if constexpr (VECTOR) {
      // Branch-free: lanes past the chunk's end re-load its last vector
      // (never marked), so the loads form one group.
      const uint4* vp = reinterpret_cast<const uint4*>(rp);
#pragma unroll
      for (int j = 0; j < VPL; ++j) raw[j] = load_nt(vp + min(first + j * NT, lim - 1));
    } else {
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        uint32_t w4[4] = {0u, 0u, 0u, 0u};
        const int e0 = (first + j * NT) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int i = e0 + e;
          if (first + j * NT < lim && i < V) {
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

  __device__ __forceinline__ void keys_of(int j, uint32_t* kk) const {
    const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
    if constexpr (sizeof(ET) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kk[2 * e] = Key<ET>::of_bits(w[e] & 0xFFFFu);
        kk[2 * e + 1] = Key<ET>::of_bits(w[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) kk[e] = Key<ET>::of_bits(w[e]);
    }
  }

  __device__ __forceinline__ bool valid(int j, int e) const {
    const int v = first + j * NT;
    if constexpr (VECTOR) return v < lim;
    else return v < lim && v * VEC + e < V;
  }

  __device__ __forceinline__ int index_of(int j, int e) const { return (first + j * NT) * VEC + e; }

  // fn(key) for every valid element of the lane.
  template <class F>
  __device__ __forceinline__ void visit(F fn) const {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      uint32_t kk[VEC];
      keys_of(j, kk);
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        if (valid(j, e)) fn(kk[e]);
    }
  }

  // Bit (j * VEC + e) is set when element e of vector j is valid and >= t.
  // lo tracks the smallest valid key.
  __device__ __forceinline__ uint32_t mask_ge(uint32_t t, uint32_t& lo) const {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      uint32_t kk[VEC];
      keys_of(j, kk);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const bool ok = valid(j, e);
        lo = ok ? min(lo, kk[e]) : lo;
        m |= (ok && kk[e] >= t) ? (1u << (j * VEC + e)) : 0u;
      }
    }
    return m;
  }

  // Key of element bit b (= j * VEC + e).
  __device__ __forceinline__ uint32_t key_at(int b) const {
    const int j = b / VEC, e = b % VEC;
    const uint4 r = j == 0 ? raw[0] : j == 1 ? raw[1] : j == 2 ? raw[2] : raw[VPL - 1];
    if constexpr (sizeof(ET) == 2) {
      const int q = e >> 1;
      const uint32_t w = q == 0 ? r.x : q == 1 ? r.y : q == 2 ? r.z : r.w;
      return Key<ET>::of_bits((e & 1) ? (w >> 16) : (w & 0xFFFFu));
    } else {
      const uint32_t w = e == 0 ? r.x : e == 1 ? r.y : e == 2 ? r.z : r.w;
      return Key<ET>::of_bits(w);
    }
  }
};
static_assert(VPL == 4, "key_at selects among four vectors");

// bf16 with 16-byte vectors: the hot path works on packed pairs.  Each dword
// holds two bf16 values; x ^ ((x >> 15) & 0x7FFF) per 16-bit half (three
// packed instructions) turns sign-magnitude into a two's-complement int16 s'
// that orders like the values, except that every negative value lands one
// below its key: s' = K for K >= 0 and s' = K - 1 for K < 0, where
// K = key - 0x8000 (so -0 and +0 differ only here).  A test key >= t is then
// s' >= T' with T = t - 0x8000 and T' = T if T >= 1, else T - 1.  Lane
// minima and maxima use packed min / max; per-element compares run only in
// lanes whose packed maximum reaches T'.
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

template <>
struct Chunk<uint16_t, true> {
  static constexpr int VEC = 8;
  uint4 raw[VPL];   // ordered int16 pairs after load()
  int first, lim, V;

  __device__ __forceinline__ void load(const uint16_t* rp, int start, int end, int Vrow) {
    first = start / VEC + (int)threadIdx.x;
    lim = (end + VEC - 1) / VEC;
    V = Vrow;
    const uint4* vp = reinterpret_cast<const uint4*>(rp);
#pragma unroll
    for (int j = 0; j < VPL; ++j) raw[j] = load_nt(vp + min(first + j * NT, lim - 1));
  }
  __device__ __forceinline__ bool valid(int j, int) const { return first + j * NT < lim; }
  __device__ __forceinline__ int index_of(int j, int e) const { return (first + j * NT) * VEC + e; }

  // Packed min / max of the lane's valid pairs, after converting in place.
  __device__ __forceinline__ void prepare(s16x2& mn, s16x2& mx) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[q] = ordered_pair(w[q]);
        if (valid(j, 0)) {
          const s16x2 v = __builtin_bit_cast(s16x2, w[q]);
          mn = __builtin_elementwise_min(mn, v);
          mx = __builtin_elementwise_max(mx, v);
        }
      }
      raw[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }

  // Largest key of the lane (0 when it holds no element).
  __device__ __forceinline__ uint32_t lane_max_key(s16x2 mx) const {
    return valid(0, 0) ? key_of_ordered(max((int)mx.x, (int)mx.y)) : 0u;
  }

  // Bit (j * 8 + e) set when element e of vector j is valid with key >= t.
  __device__ __forceinline__ uint32_t mask_ge(uint32_t t, s16x2 mx) const {
    const int Tp = ordered_threshold(t);
    if (max((int)mx.x, (int)mx.y) < Tp) return 0u;
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      if (!valid(j, 0)) continue;
      const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        m |= lo16(w[q]) >= Tp ? (1u << (j * 8 + 2 * q)) : 0u;
        m |= hi16(w[q]) >= Tp ? (1u << (j * 8 + 2 * q + 1)) : 0u;
      }
    }
    return m;
  }

  __device__ __forceinline__ uint32_t key_at(int b) const {
    const int j = b >> 3, e = b & 7;
    const uint4 r = j == 0 ? raw[0] : j == 1 ? raw[1] : j == 2 ? raw[2] : raw[3];
    const int q = e >> 1;
    const uint32_t w = q == 0 ? r.x : q == 1 ? r.y : q == 2 ? r.z : r.w;
    return key_of_ordered((e & 1) ? hi16(w) : lo16(w));
  }

  // fn(key) for every valid element (cold paths only).
  template <class F>
  __device__ __forceinline__ void visit(F fn) const {
#pragma unroll
    for (int b = 0; b < VPL * VEC; ++b)
      if (valid(b >> 3, 0)) fn(key_at(b));
  }
};


struct SelSmem {
  uint2 cand[CCAP];        // (key, vocabulary id)
  uint32_t hist[256];
  uint32_t red[NWAVE];
  uint32_t bc[4];
  uint32_t cnt, cnt2;
};

// Write the lane's marked keys to the buffer: one LDS atomic per wavefront
// reserves the wave's slots.  Slots at or past the capacity are dropped (the
// next check point sees the count).  bad collects NaN / +inf candidates.
template <typename ET, bool VECTOR>
__device__ __forceinline__ void append_marked(const Chunk<ET, VECTOR>& ch, uint32_t mask, SelSmem& s,
                                              uint32_t& bad) {
  const uint32_t mine = (uint32_t)__popc(mask);
  if (__ballot(mine != 0) == 0ull) return;
  const uint32_t incl = wave_incl_scan(mine);
  const uint32_t total = (uint32_t)__shfl((int)incl, 63, 64);
  uint32_t base = 0;
  if ((threadIdx.x & 63) == 0) base = atomicAdd(&s.cnt, total);
  uint32_t slot = (uint32_t)__shfl((int)base, 0, 64) + incl - mine;
  while (mask) {
    const int b = __builtin_ctz(mask);
    mask &= mask - 1u;
    const uint32_t key = ch.key_at(b);
    bad |= key >= Key<ET>::POS_INF ? 1u : 0u;
    if (slot < (uint32_t)CCAP)
      s.cand[slot] = make_uint2(key, (uint32_t)ch.index_of(b / Key<ET>::VEC, b % Key<ET>::VEC));
    ++slot;
  }
}

// Raise t to the k-th largest key of cand[0, n) when n >= k (certified), then
// keep only entries >= t.  Returns the new count.  Block-uniform.
template <typename ET>
__device__ __forceinline__ uint32_t compact_buffer(SelSmem& s, uint32_t n, uint32_t k, uint32_t& t) {
  constexpr int LEVELS = Key<ET>::LEVELS;
  if (n >= k) {
    const uint32_t kth = block_kth_largest<LEVELS>(
        [&](auto fn) {
          for (uint32_t i = threadIdx.x; i < n; i += NT) fn(s.cand[i].x);
        },
        k, s.hist, s.bc);
    t = max(t, kth);
  }
  constexpr int OWN = CCAP / NT;
  uint2 mine[OWN];
#pragma unroll
  for (int l = 0; l < OWN; ++l) {
    const uint32_t i = threadIdx.x + l * NT;
    mine[l] = i < n ? s.cand[i] : make_uint2(0u, 0u);
  }
  if (threadIdx.x == 0) s.cnt2 = 0;
  __syncthreads();
#pragma unroll
  for (int l = 0; l < OWN; ++l) {
    const uint32_t i = threadIdx.x + l * NT;
    if (i < n && mine[l].x >= t) s.cand[atomicAdd(&s.cnt2, 1u)] = mine[l];
  }
  __syncthreads();
  const uint32_t m = s.cnt2;
  __syncthreads();
  return m;
}

// fn(key, index) for the elements [start, end) of a row, this thread's share,
// read with plain loads (recovery path only).
template <typename ET, class F>
__device__ __forceinline__ void reread_range(const ET* rp, int start, int end, F fn) {
#pragma unroll 1
  for (int i = start + (int)threadIdx.x; i < end; i += NT) fn(Key<ET>::load_key(rp, i), i);
}

template <typename ET, bool VECTOR>
__device__ __forceinline__ void select_part(const Args& a, SelSmem& s, RowInfo& ri, int rowid, int part,
                                            const ET* rp, int c0, int c1, uint32_t k) {
  constexpr int LEVELS = Key<ET>::LEVELS;
  uint32_t t = 1;             // block-uniform certified bound (1 = none yet)
  uint32_t lo = 0xFFFFFFFFu;  // lane minimum key (negative NaN sorts below -inf)
  uint32_t bad = 0;           // NaN / +inf among the candidates
  bool demoted = false;
  uint32_t n = 0;             // block-uniform candidate count (valid at check points)
  uint32_t refresh_at = min((uint32_t)CCAP / 2, 2 * k + 256);
  auto cstart = [&](int c) { return c * a.L; };
  auto cend = [&](int c) { return min(a.V, (c + 1) * a.L); };

  auto check = [&](int c) {
    __syncthreads();
    n = s.cnt;
    __syncthreads();
    if (n > (uint32_t)CCAP) {
      // Rebuild from a re-read of chunks [c0, c]: their exact k-th largest is
      // certified; keep what reaches it.
      const int e0 = cstart(c0), e1 = cend(c);
      const uint32_t kth = block_kth_largest<LEVELS>(
          [&](auto fn) { reread_range<ET>(rp, e0, e1, [&](uint32_t uk, int) { fn(uk); }); }, k, s.hist, s.bc);
      t = max(t, kth);
      if (threadIdx.x == 0) s.cnt = 0;
      __syncthreads();
      reread_range<ET>(rp, e0, e1, [&](uint32_t uk, int idx) {
        if (uk >= t) {
          bad |= uk >= Key<ET>::POS_INF ? 1u : 0u;
          const uint32_t slot = atomicAdd(&s.cnt, 1u);
          if (slot < (uint32_t)CCAP) s.cand[slot] = make_uint2(uk, (uint32_t)idx);
        }
      });
      __syncthreads();
      n = s.cnt;
      __syncthreads();
      if (n > (uint32_t)CCAP) {   // ties beyond the buffer: the multi-pass path takes the sequence
        demoted = true;
        return;
      }
    }
    if (n >= refresh_at) {
      n = compact_buffer<ET>(s, n, k, t);
      if (threadIdx.x == 0) s.cnt = n;
      __syncthreads();
      refresh_at = min((uint32_t)CCAP / 2 + n, n + 2 * k + 256);
    }
  };
  auto due = [&](int c) { return c == c1 - 1 || ((c - c0) % a.sync) == a.sync - 1; };

  constexpr bool PACKED = VECTOR && sizeof(ET) == 2;
  s16x2 pmin = {(short)32767, (short)32767};   // packed lane minimum (ordered pairs)
  // Examine one chunk: mark the keys >= t and append them; returns the lane's
  // largest key (used for the first chunk's bound).
  auto examine = [&](Chunk<ET, VECTOR>& ch, bool first_chunk) {
    uint32_t mask;
    if constexpr (PACKED) {
      s16x2 mx = {(short)-32768, (short)-32768};
      ch.prepare(pmin, mx);
      if (first_chunk) {
        const uint32_t t0 = block_kth_largest<LEVELS>([&](auto fn) { fn(ch.lane_max_key(mx)); }, k, s.hist, s.bc);
        t = max(t, t0);
      }
      mask = ch.mask_ge(t, mx);
    } else {
      if (first_chunk) {
        uint32_t lmax = 0;
        ch.visit([&](uint32_t uk) { lmax = max(lmax, uk); });
        const uint32_t t0 = block_kth_largest<LEVELS>([&](auto fn) { fn(lmax); }, k, s.hist, s.bc);
        t = max(t, t0);
      }
      mask = ch.mask_ge(t, lo);
    }
    append_marked(ch, mask, s, bad);
  };

  if (threadIdx.x == 0) s.cnt = 0;
  Chunk<ET, VECTOR> A, B;
  A.load(rp, cstart(c0), cend(c0), a.V);
  if (c0 + 1 < c1) B.load(rp, cstart(c0 + 1), cend(c0 + 1), a.V);
  // First chunk: the k-th largest lane maximum is a certified bound.
  examine(A, true);
  check(c0);
  // Steady state: B holds chunk c while A is refilled with chunk c+1.
  int c = c0 + 1;
  while (c < c1 && !demoted) {
    if (c + 1 < c1) A.load(rp, cstart(c + 1), cend(c + 1), a.V);
    examine(B, false);
    if (due(c)) check(c);
    if (++c >= c1 || demoted) break;
    if (c + 1 < c1) B.load(rp, cstart(c + 1), cend(c + 1), a.V);
    examine(A, false);
    if (due(c)) check(c);
    ++c;
  }
  if constexpr (PACKED) {
    // A negative NaN orders below -inf (ordered value -32641).
    lo = min((int)pmin.x, (int)pmin.y) < -32641 ? 0u : 0xFFFFFFFFu;
  }

  // Validity: NaN / +inf reached the test, or a key below -inf (negative NaN).
  const uint32_t flag = block_or_u32(bad | (lo < Key<ET>::NEG_INF ? 1u : 0u), s.red);
  if (flag || demoted) {
    if (threadIdx.x == 0) atomicOr(&ri.flags, flag ? F_BAD : F_DEMOTE);
    return;
  }
  // The part's exact kept set among its candidates.
  uint32_t tf = t;
  if (n > k) {
    const uint32_t kth = block_kth_largest<LEVELS>(
        [&](auto fn) {
          for (uint32_t i = threadIdx.x; i < n; i += NT) fn(s.cand[i].x);
        },
        k, s.hist, s.bc);
    tf = max(tf, kth);
  }
  if (threadIdx.x == 0) s.cnt2 = 0;
  __syncthreads();
  uint2* out = a.cand + (size_t)rowid * RCAP + (size_t)part * a.seg;
  const uint32_t cap = (uint32_t)a.seg;
  for (uint32_t i = threadIdx.x; i < n; i += NT) {
    const uint2 e = s.cand[i];
    if (e.x >= tf && e.x != Key<ET>::NEG_INF) {
      const uint32_t slot = atomicAdd(&s.cnt2, 1u);
      if (slot < cap) out[slot] = e;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t ns = s.cnt2;
    if (ns > cap) atomicOr(&ri.flags, F_DEMOTE);
    ri.nsurv[part] = (int32_t)min(ns, cap);
  }
}

template <typename ET, bool VECTOR>
__global__ __launch_bounds__(NT) void select_kernel(Args a) {
  __shared__ SelSmem s;
  const int RS = 2 * a.G + 1;
  const int rowid = blockIdx.x / a.NP;
  const int part = blockIdx.x - rowid * a.NP;
  const int b = rowid / RS;
  const int slot = rowid - b * RS;
  const Mode m = seq_mode(a, b);
  if (m.mode != MODE_GREEDY && m.mode != MODE_SPARSE) return;
  const bool isP = slot <= a.G;
  const int pos = isP ? slot : slot - a.G - 1;
  if (isP ? pos > m.g : pos >= m.g) return;   // padding rows are never read
  const int c0 = part * a.CPP;
  const int c1 = min(a.NC, c0 + a.CPP);
  if (c0 >= c1) {
    if (threadIdx.x == 0) a.rows[rowid].nsurv[part] = 0;
    return;
  }
  select_part<ET, VECTOR>(a, s, a.rows[rowid], rowid, part, row_ptr<ET>(a, b, isP, pos), c0, c1, m.k);
}

}  // namespace sv
