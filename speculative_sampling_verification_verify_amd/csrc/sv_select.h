// Streaming top-k select (one pass over each logit row).
//
// One workgroup handles one part of one logit row: CPP consecutive chunks of
// at most NT * VPL * VEC elements.  The chunk being examined is held in
// registers while the next chunk's 16-byte non-temporal loads are already in
// flight, so the row is read from HBM once and the memory pipe stays busy
// while keys are compared.
//
// Threshold logic (exact, no sampling heuristics):
//  * a "certified" bound t is a key such that at least k elements of the row
//    are >= t; it never exceeds the row's k-th largest key, so every element
//    of the kept set (all keys >= the k-th largest) is >= t;
//  * the first chunk certifies the k-th largest of the lanes' maxima (each
//    lane maximum is a distinct element);
//  * whenever the candidate buffer holds >= k keys, its k-th largest is
//    certified too, and the buffer is compacted to the keys >= it;
//  * parts of the same row share their bounds through an atomic maximum.
// At the end the part's survivors (>= the exact k-th largest of its
// candidates) go to the row's list; with several parts the last one to
// finish (completion ticket) reduces the merged list to the row's exact
// kept set.  Keys equal to -inf carry no probability mass and are dropped.
#pragma once

#include "sv_common.h"

namespace sv {

template <typename ET, bool VECTOR>
struct Chunk {
  static constexpr int VEC = Key<ET>::VEC;
  static constexpr int EPL = VPL * VEC;   // elements per lane
  uint4 raw[VECTOR ? VPL : 1];
  uint32_t sraw[VECTOR ? 1 : EPL];
  int first;                              // this lane's first vector (or element) index
  int lim;                                // one past the chunk's last vector (or element)

  __device__ __forceinline__ void load(const ET* rp, int start, int end) {
    if constexpr (VECTOR) {
      const uint4* vp = reinterpret_cast<const uint4*>(rp);
      first = start / VEC + (int)threadIdx.x;
      lim = end / VEC;
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int vi = first + j * NT;
        raw[j] = vi < lim ? load_nt(vp + vi) : make_uint4(0u, 0u, 0u, 0u);
      }
    } else {
      first = start + (int)threadIdx.x;
      lim = end;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = first + j * NT;
        uint32_t bits = 0;
        if (e < lim) {
          if constexpr (sizeof(ET) == 2) bits = reinterpret_cast<const uint16_t*>(rp)[e];
          else bits = __float_as_uint(reinterpret_cast<const float*>(rp)[e]);
        }
        sraw[j] = bits;
      }
    }
  }

  // fn(key, vocabulary index) for every element this lane holds.
  template <class F>
  __device__ __forceinline__ void visit(F fn) const {
    if constexpr (VECTOR) {
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int vi = first + j * NT;
        if (vi < lim) {
          const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
          if constexpr (sizeof(ET) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              fn(Key<ET>::of_bits(w[e] & 0xFFFFu), vi * VEC + 2 * e);
              fn(Key<ET>::of_bits(w[e] >> 16), vi * VEC + 2 * e + 1);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) fn(Key<ET>::of_bits(w[e]), vi * VEC + e);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = first + j * NT;
        if (e < lim) fn(Key<ET>::of_bits(sraw[j]), e);
      }
    }
  }

  // Like visit, but one test per 16-byte vector first: fn runs only for the
  // elements of vectors whose largest key reaches t.  lo tracks the lane's
  // smallest key (to catch negative NaN, which sorts below -inf).
  template <class F>
  __device__ __forceinline__ void visit_at_least(uint32_t t, uint32_t& lo, F fn) const {
    if constexpr (VECTOR) {
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int vi = first + j * NT;
        if (vi < lim) {
          uint32_t kk[VEC];
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
          uint32_t mx = kk[0], mn = kk[0];
#pragma unroll
          for (int e = 1; e < VEC; ++e) {
            mx = max(mx, kk[e]);
            mn = min(mn, kk[e]);
          }
          lo = min(lo, mn);
          if (mx >= t) {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
              if (kk[e] >= t) fn(kk[e], vi * VEC + e);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = first + j * NT;
        if (e < lim) {
          const uint32_t uk = Key<ET>::of_bits(sraw[j]);
          lo = min(lo, uk);
          if (uk >= t) fn(uk, e);
        }
      }
    }
  }
};

struct SelSmem {
  uint2 cand[CCAP];        // (key, vocabulary id)
  uint32_t hist[256];
  uint32_t red[NWAVE];
  uint32_t bc[4];
  uint32_t cnt, cnt2, flag, t;
};

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
  // Two-phase in-place compaction: read everything first, then write.
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
// read from global memory with plain loads (used by rare recovery paths, so
// that they do not need the chunk's registers).
template <typename ET, class F>
__device__ __forceinline__ void reread_range(const ET* rp, int start, int end, F fn) {
#pragma unroll 1
  for (int i = start + (int)threadIdx.x; i < end; i += NT) fn(Key<ET>::load_key(rp, i), i);
}

template <typename ET, bool VECTOR>
__device__ __forceinline__ void select_part(const Args& a, SelSmem& s, RowInfo& ri, int rowid, const ET* rp,
                                            int c0, int c1, uint32_t k) {
  constexpr int LEVELS = Key<ET>::LEVELS;
  uint32_t t = 1;             // block-uniform certified bound (1 = none yet)
  uint32_t lo = 0xFFFFFFFFu;  // lane minimum key
  uint32_t hi_bad = 0;        // a NaN / +inf reached the candidate test
  bool demoted = false;
  uint32_t n = 0;             // block-uniform candidate count
  uint32_t refresh_at = min((uint32_t)CCAP / 2, 2 * k + 256);
  if (threadIdx.x == 0) s.cnt = 0;

  auto cstart = [&](int c) { return c * a.L; };
  auto cend = [&](int c) { return min(a.V, (c + 1) * a.L); };
  auto push = [&](uint32_t uk, int idx) {
    hi_bad |= uk >= Key<ET>::POS_INF ? 1u : 0u;
    const uint32_t slot = atomicAdd(&s.cnt, 1u);
    if (slot < (uint32_t)CCAP) s.cand[slot] = make_uint2(uk, (uint32_t)idx);
  };

  // After a chunk's candidates are appended: overflow recovery, buffer
  // refresh, and bounds from the row's other parts.  Block-uniform.
  auto settle = [&](int c, uint32_t before) {
    __syncthreads();
    n = s.cnt;
    __syncthreads();
    if (n > (uint32_t)CCAP) {
      // This chunk alone overflowed the buffer: drop its partial entries,
      // certify the chunk's own k-th largest (re-reading it), compact the
      // older entries and append the chunk again at the higher bound.
      const uint32_t kc = block_kth_largest<LEVELS>(
          [&](auto fn) { reread_range<ET>(rp, cstart(c), cend(c), [&](uint32_t uk, int) { fn(uk); }); }, k,
          s.hist, s.bc);
      t = max(t, kc);
      n = compact_buffer<ET>(s, before, k, t);
      if (threadIdx.x == 0) s.cnt = n;
      __syncthreads();
      reread_range<ET>(rp, cstart(c), cend(c), [&](uint32_t uk, int idx) {
        if (uk >= t) push(uk, idx);
      });
      __syncthreads();
      n = s.cnt;
      __syncthreads();
      if (n > (uint32_t)CCAP) {   // ties beyond the buffer: leave it to the multi-pass path
        demoted = true;
        return;
      }
    }
    if (n >= refresh_at) {
      n = compact_buffer<ET>(s, n, k, t);
      if (threadIdx.x == 0) {
        s.cnt = n;
        if (n >= k) __hip_atomic_fetch_max(&ri.thr, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      refresh_at = min((uint32_t)CCAP / 2 + n, n + 2 * k + 256);
    }
    // Bounds published by the row's other parts.
    if (threadIdx.x == 0) s.t = atomic_load_u32(&ri.thr);
    __syncthreads();
    t = max(t, s.t);
    __syncthreads();
  };

  Chunk<ET, VECTOR> A, B;
  A.load(rp, cstart(c0), cend(c0));
  if (c0 + 1 < c1) B.load(rp, cstart(c0 + 1), cend(c0 + 1));
  // First chunk: the k-th largest lane maximum is a certified bound.
  {
    uint32_t lmax = 0;
    A.visit([&](uint32_t uk, int) { lmax = max(lmax, uk); });
    const uint32_t t0 = block_kth_largest<LEVELS>([&](auto fn) { fn(lmax); }, k, s.hist, s.bc);
    t = max(t, t0);
    A.visit_at_least(t, lo, push);
    settle(c0, 0);
  }
  // Steady state: B holds chunk c; A is refilled with chunk c+1 meanwhile.
  int c = c0 + 1;
  while (c < c1 && !demoted) {
    if (c + 1 < c1) A.load(rp, cstart(c + 1), cend(c + 1));
    {
      const uint32_t before = n;
      B.visit_at_least(t, lo, push);
      settle(c, before);
    }
    if (++c >= c1 || demoted) break;
    if (c + 1 < c1) B.load(rp, cstart(c + 1), cend(c + 1));
    {
      const uint32_t before = n;
      A.visit_at_least(t, lo, push);
      settle(c, before);
    }
    ++c;
  }

  // Validity: NaN / +inf reached the test, or a key below -inf (negative NaN).
  const uint32_t bad = block_or_u32(hi_bad | (lo < Key<ET>::NEG_INF ? 1u : 0u), s.red);
  if (bad || demoted) {
    if (threadIdx.x == 0) atomicOr(&ri.flags, bad ? F_BAD : F_DEMOTE);
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
  if (threadIdx.x == 0) {
    s.cnt2 = 0;
    if (a.NP > 1 && n >= k) __hip_atomic_fetch_max(&ri.thr, tf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s.t = a.NP > 1 ? atomic_load_u32(&ri.thr) : 0u;
  }
  __syncthreads();
  tf = max(tf, s.t);   // any certified bound of the row is safe to apply
  uint2* list = a.cand + (size_t)rowid * RCAP;
  // Survivors with mass, compacted at the front of the LDS buffer.
  constexpr int OWN = CCAP / NT;
  uint2 mine[OWN];
#pragma unroll
  for (int l = 0; l < OWN; ++l) {
    const uint32_t i = threadIdx.x + l * NT;
    mine[l] = i < n ? s.cand[i] : make_uint2(0u, 0u);
  }
  __syncthreads();
#pragma unroll
  for (int l = 0; l < OWN; ++l) {
    const uint32_t i = threadIdx.x + l * NT;
    if (i < n && mine[l].x >= tf && mine[l].x != Key<ET>::NEG_INF) s.cand[atomicAdd(&s.cnt2, 1u)] = mine[l];
  }
  __syncthreads();
  const uint32_t ns = s.cnt2;
  if (a.NP == 1) {
    for (uint32_t i = threadIdx.x; i < ns; i += NT) list[i] = s.cand[i];
    if (threadIdx.x == 0) ri.nsurv = (int32_t)ns;
    return;
  }
  if (threadIdx.x == 0)
    s.bc[2] = ns ? __hip_atomic_fetch_add(&ri.cnt, ns, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
  __syncthreads();
  const uint32_t base = s.bc[2];
  if (base + ns > (uint32_t)RCAP) {
    if (threadIdx.x == 0) atomicOr(&ri.flags, F_DEMOTE);
    return;
  }
  for (uint32_t i = threadIdx.x; i < ns; i += NT) list[base + i] = s.cand[i];
}

// Last part of a row: exact k-th largest of the merged list; survivors are
// written back to the front of the list.
template <typename ET>
__device__ __forceinline__ void merge_row(const Args& a, SelSmem& s, RowInfo& ri, int rowid, uint32_t k) {
  constexpr int LEVELS = Key<ET>::LEVELS;
  const uint32_t flags = atomic_load_u32(&ri.flags);
  const uint32_t n = min(atomic_load_u32(&ri.cnt), (uint32_t)RCAP);
  if (flags) return;
  uint2* list = a.cand + (size_t)rowid * RCAP;
  for (uint32_t i = threadIdx.x; i < n; i += NT) s.cand[i] = list[i];
  __syncthreads();
  uint32_t kth = 1;
  if (n > k) {
    kth = block_kth_largest<LEVELS>(
        [&](auto fn) {
          for (uint32_t i = threadIdx.x; i < n; i += NT) fn(s.cand[i].x);
        },
        k, s.hist, s.bc);
  }
  if (threadIdx.x == 0) s.cnt2 = 0;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < n; i += NT) {
    const uint2 e = s.cand[i];
    if (e.x >= kth) list[atomicAdd(&s.cnt2, 1u)] = e;
  }
  __syncthreads();
  if (threadIdx.x == 0) ri.nsurv = (int32_t)s.cnt2;
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
  RowInfo& ri = a.rows[rowid];
  const int c0 = part * a.CPP;
  const int c1 = min(a.NC, c0 + a.CPP);
  select_part<ET, VECTOR>(a, s, ri, rowid, row_ptr<ET>(a, b, isP, pos), c0, c1, m.k);
  if (a.NP > 1) {
    if (!block_ticket(&ri.done, (uint32_t)a.NP, &s.flag)) return;
    merge_row<ET>(a, s, ri, rowid, m.k);
  }
}

}  // namespace sv
