// Per-sequence finisher: acceptance, first rejection, overlap, residual or
// bonus draw.  One workgroup (NT threads) per sequence.
//
// Top-k and argmax sequences work from the survivor lists left by the
// streaming select.  Without top-p, and when every part list fits, the
// register path takes them: one wavefront per position holds its two rows'
// lists in registers and computes everything for that position with no
// block barrier; one barrier then gives wavefront 0 every position for the
// acceptance test (fast_position).  Otherwise the LDS list path: every
// (row, part) list of the sequence is brought into LDS in one round trip;
// each wavefront takes whole rows (the row's exact kept set from the union
// of its part lists, normaliser, top-p cut) and whole positions (p(x),
// q(x), overlap), and one wavefront takes the acceptance test and the draw.
// Entries are broadcast to the wavefront through registers (readlane), so
// the all-pairs loops over a row's survivors do not wait on LDS once per
// entry.
//
// Sequences without top-k (or whose lists overflowed) run a multi-pass
// procedure over the logits in one workgroup: maximum, count-based radix
// select for top-k, mass-weighted radix select for top-p (fixed-point 64-bit
// masses, so the result does not depend on summation order), normalisers,
// overlap, and a tiled inverse-CDF scan in ascending id order.
#pragma once

#include "sv_common.h"

namespace sv {

constexpr int MAXROWS = 2 * SV_MAX_GAMMA + 1;
constexpr int MAXSEG = 512;                     // (row, part) lists of one sequence on the list path

struct FinSmem {
  uint2 pool[POOL];                             // (key, id) of every survivor of the sequence
  float pv[POOL];                               // exp((z - zmax) / T) per kept survivor
  double wts[POOL];                             // residual / bonus weights of a row (draws)
  uint32_t soff[MAXSEG + 1];                    // pool offset of each (row, part) list
  uint32_t cslot[MAXSEG];                       // survivor count of every (slot, part) of the sequence
  uint32_t off[MAXROWS + 1];                    // pool offset of each used row
  uint32_t whist[NWAVE][256];                   // per-wavefront radix histograms
  uint32_t st_thr[MAXROWS];                     // kept keys are >= st_thr (multi-pass path)
  uint32_t st_cnt[MAXROWS];                     // kept survivors of each row (list path)
  uint32_t st_sorted[MAXROWS];                  // 1 when the row's kept survivors are in ascending id
  uint32_t st_arg[MAXROWS];                     // argmax (T == 0)
  float st_zmax[MAXROWS];
  double st_S[MAXROWS];                         // normaliser over the kept keys
  double st_invS[MAXROWS];
  double pos_p[SV_MAX_GAMMA];
  double pos_q[SV_MAX_GAMMA];
  double pos_alpha[SV_MAX_GAMMA];
  int32_t cand_tok[SV_MAX_GAMMA + 1];           // drawn token if the first rejection is at i (i = g: bonus)
  int32_t xs[SV_MAX_GAMMA];                     // the drafts, staged once
  union {
    uint32_t h32[256];
    unsigned long long h64[256];
  } hist;
  double red_d[NWAVE];
  unsigned long long red_u64[NWAVE];
  uint32_t red_u[NWAVE];
  uint32_t red_or[NWAVE];
  uint32_t fflag[NWAVE];                        // register path: per-wavefront input / list checks
  uint32_t fempty[NWAVE];                       // register path: position i has a row without survivors
  uint32_t bc[8];
  uint32_t flag;
};

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ===========================================================================
// List path.
// ===========================================================================

// fn(key, id, val) for every entry of ents[o, o+n) in order, seen by every
// lane of the wavefront through readlane (no LDS access per entry).  Must be
// called with the whole wavefront active and wavefront-uniform o, n.
template <typename VT, class F>
__device__ __forceinline__ void wave_broadcast(const uint2* ents, const VT* vals, int o, int n, F fn) {
  const int lane = threadIdx.x & 63;
  for (int b = 0; b < n; b += 64) {
    const int i = b + lane;
    const uint2 e = i < n ? ents[o + i] : make_uint2(0u, 0u);
    const VT v = i < n ? vals[o + i] : (VT)0;
    const int m = min(64, n - b);
    for (int l = 0; l < m; ++l) {
      const uint32_t key = (uint32_t)__builtin_amdgcn_readlane((int)e.x, l);
      const uint32_t id = (uint32_t)__builtin_amdgcn_readlane((int)e.y, l);
      VT val;
      if constexpr (sizeof(VT) == 4) {
        val = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
      } else {
        const long long bv = __double_as_longlong(v);
        val = __longlong_as_double(((long long)__builtin_amdgcn_readlane((int)(bv >> 32), l) << 32) |
                                   (unsigned int)__builtin_amdgcn_readlane((int)(bv & 0xFFFFFFFFll), l));
      }
      fn(key, id, val);
    }
  }
}

// The k-th largest key (1-based) of ents[0, n) by one wavefront, with a
// wave-private 256-bin histogram; 0 when n < k.
template <int LEVELS>
__device__ __forceinline__ uint32_t wave_kth_largest(const uint2* ents, int n, uint32_t k, uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  return wave_kth<LEVELS>(
      [&](auto fn) {
        for (int i = lane; i < n; i += 64) fn(ents[i].x);
      },
      k, hist);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Keep the entries of [o, o+n) (pool and pv together) whose key is >= t, in
// order, at the start of the range; returns their number.
__device__ __forceinline__ int wave_keep(FinSmem& s, int o, int n, uint32_t t) {
  const int lane = threadIdx.x & 63;
  int outn = 0;
  for (int b = 0; b < n; b += 64) {
    const int i = b + lane;
    const uint2 e = i < n ? s.pool[o + i] : make_uint2(0u, 0u);
    const float v = i < n ? s.pv[o + i] : 0.0f;
    const bool keep = i < n && e.x >= t;
    const unsigned long long bal = __ballot(keep);
    const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
    if (keep) {
      const int d = o + outn + __popcll(bal & below);
      s.pool[d] = e;
      s.pv[d] = v;
    }
    outn += __popcll(bal);
  }
  wave_lds_sync();
  return outn;
}

// Statistics of row r, by one wavefront.  The row's kept set is every key >=
// the k-th largest of the union of its part lists (ties kept), then cut by
// top-p when asked for; it is left compacted at the start of the row's pool
// range (cnt[r] entries, exp((z - zmax) / T) of each in pv) with its
// normaliser.
template <typename ET>
__device__ __forceinline__ void pool_row_stats(FinSmem& s, int r, const Mode& m, int np) {
  const int lane = threadIdx.x & 63;
  const int o = (int)s.off[r];
  int n = (int)(s.off[r + 1] - s.off[r]);
  uint32_t* hist = s.whist[threadIdx.x >> 6];
  // A row streamed as one part already holds exactly its kept set (the k-th
  // largest and everything above, ties included); the union of several
  // parts is cut to the k-th largest here.
  const uint32_t kth =
      (np > 1 && n > (int)m.k) ? wave_kth_largest<Key<ET>::LEVELS>(s.pool + o, n, m.k, hist) : 1u;
  uint32_t kmax = 0;
  for (int i = lane; i < n; i += 64) kmax = max(kmax, s.pool[o + i].x);
  kmax = wave_max_dpp(kmax);
  if (m.mode == MODE_GREEDY) {
    uint32_t best = 0xFFFFFFFFu;
    for (int i = lane; i < n; i += 64)
      if (s.pool[o + i].x == kmax) best = min(best, s.pool[o + i].y);
    best = wave_min_dpp(best);
    if (lane == 0) s.st_arg[r] = best;
    return;
  }
  const float invT = 1.0f / m.T;
  const float zmax = Key<ET>::value(kmax);
  if (kth > 1u) n = wave_keep(s, o, n, kth);   // kth == 1: every listed (finite) key is kept
  double S = 0.0;
  for (int i = lane; i < n; i += 64) {
    const float e = expf((Key<ET>::value(s.pool[o + i].x) - zmax) * invT);
    s.pv[o + i] = e;
    S += (double)e;
  }
  S = wave_sum_dpp(S);
  wave_lds_sync();
  if (m.tp < 1.0f) {
    // The nucleus: order the survivors by (value desc, id asc); the cut is
    // the first entry whose running mass reaches top_p; every value >= the
    // cut's value is kept.
    const double target = (double)m.tp * S;
    uint32_t cut_rank = 0xFFFFFFFFu, cut_key = 0;
    for (int b = 0; b < n; b += 64) {
      const int i = b + lane;
      const uint2 e = i < n ? s.pool[o + i] : make_uint2(0u, 0u);
      uint32_t rank = 0;
      double run = 0.0;
      wave_broadcast(s.pool, s.pv, o, n, [&](uint32_t key, uint32_t id, float val) {
        const bool before = key > e.x || (key == e.x && id <= e.y);
        rank += (before && id != e.y) ? 1u : 0u;
        run += before ? (double)val : 0.0;
      });
      const bool reach = m.tp <= 0.0f ? rank == 0 : run >= target;
      if (i < n && reach && rank < cut_rank) {
        cut_rank = rank;
        cut_key = e.x;
      }
    }
    const uint32_t best = wave_min_dpp(cut_rank);
    const unsigned long long who = __ballot(cut_rank == best && best != 0xFFFFFFFFu);
    if (best != 0xFFFFFFFFu) {
      const int src = __ffsll((long long)who) - 1;
      const uint32_t thr = (uint32_t)__builtin_amdgcn_readlane((int)cut_key, src);
      n = wave_keep(s, o, n, thr);
      double S2 = 0.0;
      for (int i = lane; i < n; i += 64) S2 += (double)s.pv[o + i];
      S = wave_sum_dpp(S2);
    }
  }
  // Are the kept survivors in ascending id (the streaming select leaves them
  // so)?
  bool unsorted = false;
  for (int b = 0; b < n; b += 64) {
    const int i = b + lane;
    unsorted |= i > 0 && i < n && s.pool[o + i].y <= s.pool[o + i - 1].y;
  }
  unsorted = __ballot(unsorted) != 0ull;
  if (lane == 0) {
    s.st_cnt[r] = (uint32_t)n;
    s.st_sorted[r] = unsorted ? 0u : 1u;
    s.st_zmax[r] = zmax;
    s.st_S[r] = S;
    s.st_invS[r] = 1.0 / S;
  }
}

// Position of vocabulary id v among the ascending ids pool[o, o+n), or -1.
__device__ __forceinline__ int find_sorted(const FinSmem& s, int o, int n, uint32_t v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s.pool[o + mid].y < v) lo = mid + 1;
    else hi = mid;
  }
  return (lo < n && s.pool[o + lo].y == v) ? lo : -1;
}

// Rows with survivors in ascending id, by one wavefront: for i < g, p_i(x_i),
// q_i(x_i), alpha_i and the residual draw at i (weights max(0, p_i - q_i));
// for i == g the bonus draw (weights p_g).  q(v) is found by binary search
// in q's ascending ids, and the inverse CDF in ascending id is a prefix scan
// of the weights in list order.  Returns the drawn token.
__device__ __forceinline__ int wave_position_draw_sorted(FinSmem& s, int i, int x, const Mode& m, float ures) {
  const int lane = threadIdx.x & 63;
  const bool resid = i < m.g;
  const int rp = i, rq = m.g + 1 + i;
  const int op = (int)s.off[rp], np = (int)s.st_cnt[rp];
  const int oq = resid ? (int)s.off[rq] : 0, nq = resid ? (int)s.st_cnt[rq] : 0;
  const double ip = s.st_invS[rp], iq = resid ? s.st_invS[rq] : 0.0;
  double al = 0.0, px = 0.0, qx = 0.0, zl = 0.0, zp = 0.0;
  for (int b = 0; b < np; b += 64) {
    const int j = b + lane;
    if (j < np) {
      const uint32_t id = s.pool[op + j].y;
      const double p = (double)s.pv[op + j] * ip;
      double q = 0.0;
      if (resid) {
        const int qi = find_sorted(s, oq, nq, id);
        q = qi >= 0 ? (double)s.pv[oq + qi] * iq : 0.0;
      }
      al += fmin(p, q);
      if (id == (uint32_t)x) px = p;
      const double w = resid ? fmax(p - q, 0.0) : p;
      s.wts[op + j] = w;
      zl += w;
      zp += p;
    }
  }
  if (resid) {
    for (int j = lane; j < nq; j += 64)
      if (s.pool[oq + j].y == (uint32_t)x) qx = (double)s.pv[oq + j] * iq;
    al = wave_sum_dpp(al);
    px = wave_sum_dpp(px);
    qx = wave_sum_dpp(qx);
    if (lane == 0) {
      s.pos_p[i] = px;
      s.pos_q[i] = qx;
      s.pos_alpha[i] = al;
    }
  }
  double Z = wave_sum_dpp(zl);
  const bool fallback = !(Z > 0.0);   // zero residual mass: draw from the target itself
  if (fallback) Z = wave_sum_dpp(zp);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const double target = (double)ures * Z;
  double base = 0.0;
  int lastpos = -1;
  for (int b = 0; b < np; b += 64) {
    const int j = b + lane;
    double w = 0.0;
    if (j < np) w = fallback ? (double)s.pv[op + j] * ip : s.wts[op + j];
    const double c = base + wave_incl_scan_f64(w);
    const unsigned long long hit = __ballot(j < np && c > target);
    if (hit) return (int)s.pool[op + b + __ffsll((long long)hit) - 1].y;
    const unsigned long long posw = __ballot(w > 0.0);
    if (posw) lastpos = b + 63 - __clzll((long long)posw);
    const long long cb = __double_as_longlong(c);
    base = __longlong_as_double(((long long)__builtin_amdgcn_readlane((int)(cb >> 32), 63) << 32) |
                                (unsigned int)__builtin_amdgcn_readlane((int)(cb & 0xFFFFFFFFll), 63));
  }
  return lastpos >= 0 ? (int)s.pool[op + lastpos].y : (int)s.pool[op + np - 1].y;   // rounding left no crossing
}

// p_i(x_i), q_i(x_i) and alpha_i for one position, by one wavefront.
__device__ __forceinline__ void wave_position(FinSmem& s, int i, int x, const Mode& m) {
  const int lane = threadIdx.x & 63;
  const int rp = i, rq = m.g + 1 + i;
  if (m.mode == MODE_GREEDY) {
    if (lane == 0) {
      s.pos_p[i] = (uint32_t)x == s.st_arg[rp] ? 1.0 : 0.0;
      s.pos_q[i] = (uint32_t)x == s.st_arg[rq] ? 1.0 : 0.0;
      s.pos_alpha[i] = s.st_arg[rp] == s.st_arg[rq] ? 1.0 : 0.0;
    }
    return;
  }
  const int op = (int)s.off[rp], np = (int)s.st_cnt[rp];
  const int oq = (int)s.off[rq], nq = (int)s.st_cnt[rq];
  const double ip = s.st_invS[rp], iq = s.st_invS[rq];
  double al = 0.0, px = 0.0, qx = 0.0;
  for (int b = 0; b < np; b += 64) {
    const int j = b + lane;
    const uint32_t id = j < np ? s.pool[op + j].y : 0xFFFFFFFFu;
    const double pv = j < np ? (double)s.pv[op + j] * ip : 0.0;
    float qe = 0.0f;
    wave_broadcast(s.pool, s.pv, oq, nq, [&](uint32_t, uint32_t qid, float val) { qe = qid == id ? val : qe; });
    if (id == (uint32_t)x) px = pv;
    al += fmin(pv, (double)qe * iq);
  }
  for (int j = lane; j < nq; j += 64)
    if (s.pool[oq + j].y == (uint32_t)x) qx = (double)s.pv[oq + j] * iq;
  al = wave_sum_dpp(al);
  px = wave_sum_dpp(px);
  qx = wave_sum_dpp(qx);
  if (lane == 0) {
    s.pos_p[i] = px;
    s.pos_q[i] = qx;
    s.pos_alpha[i] = al;
  }
}

// Residual (n < g) or bonus (n == g) draw from the lists, by one wavefront.
// weight(v) = max(0, p_n(v) - q_n(v)) (or p_g(v)); token = the smallest id
// whose running weight in ascending id order exceeds u * Z.
__device__ __forceinline__ int pool_draw(FinSmem& s, const Mode& m, int n, float ures) {
  const int lane = threadIdx.x & 63;
  if (m.mode == MODE_GREEDY) return (int)s.st_arg[n];
  const bool resid = n < m.g;
  const int rp = n, rq = m.g + 1 + n;
  const int op = (int)s.off[rp], np = (int)s.st_cnt[rp];
  const int oq = resid ? (int)s.off[rq] : 0, nq = resid ? (int)s.st_cnt[rq] : 0;
  const double ip = s.st_invS[rp], iq = resid ? s.st_invS[rq] : 0.0;
  double zl = 0.0, zp = 0.0;
  for (int b = 0; b < np; b += 64) {
    const int j = b + lane;
    const uint32_t id = j < np ? s.pool[op + j].y : 0xFFFFFFFFu;
    const double p = j < np ? (double)s.pv[op + j] * ip : 0.0;
    float qe = 0.0f;
    wave_broadcast(s.pool, s.pv, oq, nq, [&](uint32_t, uint32_t qid, float val) { qe = qid == id ? val : qe; });
    const double w = resid ? fmax(p - (double)qe * iq, 0.0) : p;
    if (j < np) s.wts[op + j] = w;
    zl += w;
    zp += p;
  }
  double Z = wave_sum_dpp(zl);
  if (!(Z > 0.0)) {   // zero residual mass: draw from the target itself
    for (int j = lane; j < np; j += 64) s.wts[op + j] = (double)s.pv[op + j] * ip;
    Z = wave_sum_dpp(zp);
  }
  wave_lds_sync();
  const double target = (double)ures * Z;
  uint32_t best = 0xFFFFFFFFu, lastpos = 0;
  for (int b = 0; b < np; b += 64) {
    const int j = b + lane;
    const uint32_t v = j < np ? s.pool[op + j].y : 0xFFFFFFFFu;
    double run = 0.0;
    wave_broadcast(s.pool, s.wts, op, np, [&](uint32_t, uint32_t id, double w) { run += id <= v ? w : 0.0; });
    if (j < np) {
      if (s.wts[op + j] > 0.0) lastpos = max(lastpos, v + 1u);
      if (run > target) best = min(best, v);
    }
  }
  best = wave_min_dpp(best);
  if (best != 0xFFFFFFFFu) return (int)best;
  return (int)wave_max_dpp(lastpos) - 1;   // rounding left no crossing
}

// ===========================================================================
// Register path: one wavefront per position, survivor lists in registers.
// ===========================================================================

// Chunks of 64 list entries a position wavefront holds per row: a row of NP
// parts keeps FAST_CH / NP chunks of each part, so a part list of at most
// 64 * FAST_CH / NP entries fits.
constexpr int FAST_CH = 4;
static_assert(64 * FAST_CH <= SEG, "a row part's register chunks stay inside its list segment");

// The k-th largest keys of two key sets by one wavefront, one radix level
// of both per round so that the two selects' LDS round trips overlap (as
// wave_kth, each on its own 256-word histogram).  feed(h, fn) calls fn(key)
// for every key of set h this lane holds; set h is skipped (result 0) when
// !on[h]; a set with fewer than k keys gives 0.
template <int LEVELS, class Feed>
__device__ __forceinline__ void wave_kth_pair(Feed feed, uint32_t k, uint32_t* hist0, uint32_t* hist1, const bool (&on)[2],
                                              uint32_t (&out)[2]) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix[2] = {0u, 0u}, pmask = 0u, krem[2] = {k, k};
  bool live[2] = {on[0], on[1]};
  for (int lvl = 0; lvl < LEVELS; ++lvl) {
    const int shift = 8 * (LEVELS - 1 - lvl);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hist0[lane + 64 * i] = 0u;
      hist1[lane + 64 * i] = 0u;
    }
    wave_sync_lds();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (live[h]) {
        uint32_t* hist = h ? hist1 : hist0;
        const uint32_t pf = prefix[h];
        feed(h, [&](uint32_t key) {
          if (key != 0 && (key & pmask) == pf) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        });
      }
    }
    wave_sync_lds();
    const int top = 255 - 4 * lane;
    uint32_t c[2][4], incl[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t* hist = h ? hist1 : hist0;
#pragma unroll
      for (int j = 0; j < 4; ++j) c[h][j] = hist[top - j];
      incl[h] = wave_incl_scan_dpp(c[h][0] + c[h][1] + c[h][2] + c[h][3]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t sum = c[h][0] + c[h][1] + c[h][2] + c[h][3];
      const uint32_t excl = incl[h] - sum;
      const bool hit = excl < krem[h] && incl[h] >= krem[h];
      const unsigned long long any = __ballot(hit);
      uint32_t d = 0, r = 0;
      if (hit) {
        r = krem[h] - excl;
        if (c[h][0] >= r) {
          d = top;
        } else if (c[h][0] + c[h][1] >= r) {
          d = top - 1; r -= c[h][0];
        } else if (c[h][0] + c[h][1] + c[h][2] >= r) {
          d = top - 2; r -= c[h][0] + c[h][1];
        } else {
          d = top - 3; r -= c[h][0] + c[h][1] + c[h][2];
        }
      }
      if (any == 0ull) {
        live[h] = false;
        prefix[h] = 0u;
      } else {
        const int src = __ffsll((long long)any) - 1;
        d = (uint32_t)__builtin_amdgcn_readlane((int)d, src);
        r = (uint32_t)__builtin_amdgcn_readlane((int)r, src);
        prefix[h] |= live[h] ? d << shift : 0u;
        krem[h] = r;
      }
    }
    pmask |= 255u << shift;
    wave_sync_lds();
  }
  out[0] = on[0] && live[0] ? prefix[0] : 0u;
  out[1] = on[1] && live[1] ? prefix[1] : 0u;
}

// Position i of a top-k (top-p off) or argmax sequence by one wavefront,
// from the survivor lists of its target row (h = 0) and draft row (h = 1,
// used when i < g) in registers, for rows of NP parts.  Chunk c of a row is
// part c / FC, entries (c % FC) * 64 + lane, FC = FAST_CH / NP; f0[h][p]
// holds part p's first chunk (loaded by the caller), the others are loaded
// here when the part's size (cnt, lane h * NP + p) reaches them; lp[h] is
// row h's part-0 list (parts SEG apart).  The same quantities as the LDS
// list path: the row's kept set (the k-th largest key of the union of its
// parts and everything above), p = exp((z - zmax)/T)/S, p_i(x_i),
// q_i(x_i), the overlap, and the draw at i (residual weights
// max(0, p_i - q_i), or p_g at the bonus) by an inverse CDF in ascending id.
// Results go to pos_p / pos_q / pos_alpha / cand_tok[i]; fempty[i] = 1 when
// a row has no survivor, 2 when a list does not fit the registers or is not
// in ascending id (the sequence then takes the LDS list path).  i is
// wavefront-uniform.
template <typename ET, int NP>
__device__ __forceinline__ void fast_position(FinSmem& s, const Mode& m, int i, const uint2 (&f0)[2][FAST_CH],
                                              uint32_t cnt, const uint2* lp0, const uint2* lp1, int x, float ures) {
  constexpr int FC = FAST_CH / NP;
  const int lane = threadIdx.x & 63;
  const bool resid = i < m.g;
  // Entries per chunk (wave-uniform) and the rows' list totals.
  int ccnt[2][FAST_CH];
  uint32_t total[2] = {0u, 0u};
  bool fits = true;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t pc = (h == 0 || resid) ? (uint32_t)__builtin_amdgcn_readlane((int)cnt, h * NP + p) : 0u;
      total[h] += pc;
      fits = fits && pc <= (uint32_t)(64 * FC);
#pragma unroll
      for (int sub = 0; sub < FC; ++sub) ccnt[h][p * FC + sub] = (int)min(pc - min(pc, (uint32_t)(sub * 64)), 64u);
    }
#pragma unroll
    for (int c = NP * FC; c < FAST_CH; ++c) ccnt[h][c] = 0;
  }
  if (!fits) {
    if (lane == 0) s.fempty[i] = 2u;
    return;
  }
  // The parts' later chunks, then the order check over every chunk.
  uint2 e[2][FAST_CH];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint2* lp = h ? lp1 : lp0;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      e[h][p * FC] = f0[h][p];
#pragma unroll
      for (int sub = 1; sub < FC; ++sub)
        e[h][p * FC + sub] = ccnt[h][p * FC + sub] > 0 ? lp[(size_t)p * SEG + sub * 64 + lane] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int c = NP * FC; c < FAST_CH; ++c) e[h][c] = make_uint2(0u, 0u);
  }
  bool unsorted = false;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int c = 0; c < NP * FC; ++c) {
      const uint32_t id = e[h][c].y;
      uint32_t prev = (uint32_t)__shfl_up((int)id, 1, 64);
      if (c % FC > 0) {
        const uint32_t last = (uint32_t)__builtin_amdgcn_readlane((int)e[h][c > 0 ? c - 1 : 0].y, 63);
        prev = lane == 0 ? last : prev;
      }
      unsorted |= lane < ccnt[h][c] && (lane > 0 || c % FC > 0) && id <= prev;
    }
  }
  if (__ballot(unsorted) != 0ull) {
    if (lane == 0) s.fempty[i] = 2u;
    return;
  }
  if (total[0] == 0u || (resid && total[1] == 0u)) {
    if (lane == 0) s.fempty[i] = 1u;
    return;
  }
  // Kept set: for several parts, every key >= the k-th largest of their union.
  uint32_t kth[2] = {0u, 0u};
  if (NP > 1 && m.mode != MODE_GREEDY) {
    const bool on[2] = {total[0] > m.k, resid && total[1] > m.k};
    if (on[0] || on[1]) {
      // The draft row's histogram in the wavefront's pool range (free until
      // the q lookup below).
      wave_kth_pair<Key<ET>::LEVELS>(
          [&](int h, auto fn) {
#pragma unroll
            for (int c = 0; c < NP * FC; ++c)
              if (lane < ccnt[h][c]) fn(e[h][c].x);
          },
          m.k, s.whist[i], reinterpret_cast<uint32_t*>(s.pool + i * (64 * FAST_CH)), on, kth);
    }
  }
  bool kp[2][FAST_CH];
  uint32_t km[2] = {0u, 0u};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int c = 0; c < FAST_CH; ++c) {
      kp[h][c] = lane < ccnt[h][c] && e[h][c].x >= kth[h];
      km[h] = max(km[h], kp[h][c] ? e[h][c].x : 0u);
    }
  }
  const uint32_t kmax0 = wave_max_dpp(km[0]), kmax1 = wave_max_dpp(km[1]);
  if (m.mode == MODE_GREEDY) {
    // p and q are point masses at the lowest id of each row's largest key.
    uint32_t best0 = NONE, best1 = NONE;
#pragma unroll
    for (int c = 0; c < FAST_CH; ++c) {
      if (kp[0][c] && e[0][c].x == kmax0) best0 = min(best0, e[0][c].y);
      if (kp[1][c] && e[1][c].x == kmax1) best1 = min(best1, e[1][c].y);
    }
    const uint32_t arg0 = wave_min_dpp(best0), arg1 = wave_min_dpp(best1);
    if (lane == 0) {
      if (resid) {
        s.pos_p[i] = (uint32_t)x == arg0 ? 1.0 : 0.0;
        s.pos_q[i] = (uint32_t)x == arg1 ? 1.0 : 0.0;
        s.pos_alpha[i] = arg0 == arg1 ? 1.0 : 0.0;
      }
      s.cand_tok[i] = (int)arg0;
      s.fempty[i] = 0u;
    }
    return;
  }
  // exp((z - zmax) / T) of every kept entry and the rows' normalisers.
  const float invT = 1.0f / m.T;
  float ev[2][FAST_CH];
  double S0 = 0.0, S1 = 0.0;
  {
    const float zmax0 = Key<ET>::value(kmax0), zmax1 = Key<ET>::value(kmax1);
#pragma unroll
    for (int c = 0; c < FAST_CH; ++c) {
      ev[0][c] = 0.0f;
      ev[1][c] = 0.0f;
      if (ccnt[0][c] > 0) ev[0][c] = kp[0][c] ? expf((Key<ET>::value(e[0][c].x) - zmax0) * invT) : 0.0f;
      if (ccnt[1][c] > 0) ev[1][c] = kp[1][c] ? expf((Key<ET>::value(e[1][c].x) - zmax1) * invT) : 0.0f;
      S0 += (double)ev[0][c];
      S1 += (double)ev[1][c];
    }
  }
  S0 = wave_sum_dpp(S0);
  S1 = wave_sum_dpp(S1);
  const double ip = 1.0 / S0, iq = resid ? 1.0 / S1 : 0.0;
  // q at each target entry's id: the draft row's entries go to the
  // wavefront's own LDS range (part p at p * FC * 64, in ascending id), and
  // each target entry searches its part's range (every chunk's search
  // advances one step per round, so their LDS reads overlap).
  float qe[FAST_CH];
#pragma unroll
  for (int c = 0; c < FAST_CH; ++c) qe[c] = 0.0f;
  if (resid) {
    uint2* qs = s.pool + i * (64 * FAST_CH);
#pragma unroll
    for (int c = 0; c < FAST_CH; ++c)
      if (lane < ccnt[1][c]) qs[c * 64 + lane] = make_uint2(e[1][c].y, __float_as_uint(ev[1][c]));
    wave_lds_sync();
    int lo[FAST_CH], hi[FAST_CH], end[FAST_CH];
    int steps = 0;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      int nq = 0;
#pragma unroll
      for (int sub = 0; sub < FC; ++sub) nq += ccnt[1][p * FC + sub];
#pragma unroll
      for (int sub = 0; sub < FC; ++sub) {
        const int c = p * FC + sub;
        lo[c] = p * FC * 64;
        end[c] = hi[c] = lo[c] + nq;
        if (ccnt[0][c] > 0) steps = max(steps, 32 - __clz(nq));   // bit length: enough halvings for nq + 1 outcomes
      }
    }
    for (int st = 0; st < steps; ++st) {
      uint32_t v[NP * FC];
      int mid[NP * FC];
#pragma unroll
      for (int c = 0; c < NP * FC; ++c) {
        mid[c] = (lo[c] + hi[c]) >> 1;
        v[c] = qs[min(mid[c], 64 * FAST_CH - 1)].x;
      }
#pragma unroll
      for (int c = 0; c < NP * FC; ++c) {
        const bool go = lo[c] < hi[c];
        const bool right = v[c] < e[0][c].y;
        lo[c] = go && right ? mid[c] + 1 : lo[c];
        hi[c] = go && !right ? mid[c] : hi[c];
      }
    }
#pragma unroll
    for (int c = 0; c < NP * FC; ++c) {
      const uint2 q = qs[min(lo[c], 64 * FAST_CH - 1)];
      if (lo[c] < end[c] && q.x == e[0][c].y) qe[c] = __uint_as_float(q.y);
    }
  }
  double al = 0.0, px = 0.0, qx = 0.0, zl = 0.0, zp = 0.0;
#pragma unroll
  for (int c = 0; c < FAST_CH; ++c) {
    const double p = (double)ev[0][c] * ip;
    const double q = (double)qe[c] * iq;
    if (kp[0][c]) {
      al += fmin(p, q);
      if (e[0][c].y == (uint32_t)x) px = p;
      zl += resid ? fmax(p - q, 0.0) : p;
      zp += p;
    }
    if (resid && kp[1][c] && e[1][c].y == (uint32_t)x) qx = (double)ev[1][c] * iq;
  }
  double Z = wave_sum_dpp(zl);
  al = wave_sum_dpp(al);
  px = wave_sum_dpp(px);
  qx = wave_sum_dpp(qx);
  zp = wave_sum_dpp(zp);
  const bool fallback = !(Z > 0.0);   // zero residual mass: draw from the target itself
  if (fallback) Z = zp;
  // Inverse CDF in ascending id: chunk by chunk, a prefix scan and a ballot.
  const double target = (double)ures * Z;
  double base = 0.0;
  int tok = -1, lastw = -1, lastk = -1;
#pragma unroll
  for (int c = 0; c < NP * FC; ++c) {
    if (tok < 0 && ccnt[0][c] > 0) {
      const double p = (double)ev[0][c] * ip;
      const double w = !kp[0][c] ? 0.0 : (fallback || !resid) ? p : fmax(p - (double)qe[c] * iq, 0.0);
      const double cv = base + wave_incl_scan_f64(w);
      const unsigned long long hit = __ballot(kp[0][c] && cv > target);
      if (hit) {
        tok = __builtin_amdgcn_readlane((int)e[0][c].y, __ffsll((long long)hit) - 1);
      } else {
        const unsigned long long pw = __ballot(w > 0.0), pk = __ballot(kp[0][c]);
        if (pw) lastw = __builtin_amdgcn_readlane((int)e[0][c].y, 63 - __clzll((long long)pw));
        if (pk) lastk = __builtin_amdgcn_readlane((int)e[0][c].y, 63 - __clzll((long long)pk));
        base = readlane_f64(cv, 63);
      }
    }
  }
  if (tok < 0) tok = lastw >= 0 ? lastw : lastk;   // rounding left no crossing
  if (lane == 0) {
    if (resid) {
      s.pos_p[i] = px;
      s.pos_q[i] = qx;
      s.pos_alpha[i] = al;
    }
    s.cand_tok[i] = tok;
    s.fempty[i] = 0u;
  }
}

// ===========================================================================
// Multi-pass procedure for a whole sequence (unfiltered / top-p / overflow).
// ===========================================================================

// Calls fn(key, index) for every element of a logit row, this thread's share.
template <typename ET, bool VECTOR, class F>
__device__ __forceinline__ void row_for_each(const ET* rp, int V, F fn) {
  constexpr int VEC = Key<ET>::VEC;
  if constexpr (VECTOR) {
    const uint4* vp = reinterpret_cast<const uint4*>(rp);
    const int nv = V / VEC;
    for (int vi = threadIdx.x; vi < nv; vi += NT) {
      const uint4 d = vp[vi];
      const uint32_t w[4] = {d.x, d.y, d.z, d.w};
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
  } else {
    for (int i = threadIdx.x; i < V; i += NT) fn(Key<ET>::load_key(rp, i), i);
  }
}

__device__ __forceinline__ unsigned long long shfl_up_u64(unsigned long long v, int o) {
  const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)v, o, 64);
  const uint32_t hi = (uint32_t)__shfl_up((int)(uint32_t)(v >> 32), o, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// Mass-weighted radix select: the largest key t with mass(key >= t) >= tau,
// over keys >= lo.  Returns (t, mass(key >= t)) in fixed point.
template <typename ET, bool VECTOR>
__device__ __forceinline__ uint32_t dense_topp_select(FinSmem& s, const ET* rp, int V, uint32_t lo, float zmax, float invT,
                                      double fscale, double tau, unsigned long long* mass_out) {
  constexpr int LEVELS = Key<ET>::LEVELS;
  uint32_t prefix = 0, pmask = 0;
  unsigned long long above = 0;
  for (int lvl = 0; lvl < LEVELS; ++lvl) {
    const int shift = 8 * (LEVELS - 1 - lvl);
    for (int i = threadIdx.x; i < 256; i += NT) s.hist.h64[i] = 0ull;
    __syncthreads();
    row_for_each<ET, VECTOR>(rp, V, [&](uint32_t uk, int) {
      if (uk >= lo && (uk & pmask) == prefix) {
        const float e = __expf((Key<ET>::value(uk) - zmax) * invT);
        const unsigned long long f = (unsigned long long)((double)e * fscale);
        if (f) atomicAdd(&s.hist.h64[(uk >> shift) & 255u], f);
      }
    });
    __syncthreads();
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const int top = 255 - 4 * lane;
      const unsigned long long c0 = s.hist.h64[top], c1 = s.hist.h64[top - 1], c2 = s.hist.h64[top - 2],
                               c3 = s.hist.h64[top - 3];
      const unsigned long long sum = c0 + c1 + c2 + c3;
      unsigned long long incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long u = shfl_up_u64(incl, o);
        if (lane >= o) incl += u;
      }
      const unsigned long long excl = incl - sum;
      const double cum0 = (double)(above + excl + c0), cum1 = (double)(above + excl + c0 + c1),
                   cum2 = (double)(above + excl + c0 + c1 + c2), cum3 = (double)(above + incl);
      // Cumulative mass grows bin by bin from the top: the first lane whose
      // last bin reaches tau holds the crossing bin.
      const unsigned long long any = __ballot(cum3 >= tau);
      const int firstlane = any ? __ffsll((long long)any) - 1 : -1;
      if (lane == firstlane) {
        uint32_t d;
        unsigned long long ab;
        if (cum0 >= tau) {
          d = top; ab = above + excl;
        } else if (cum1 >= tau) {
          d = top - 1; ab = above + excl + c0;
        } else if (cum2 >= tau) {
          d = top - 2; ab = above + excl + c0 + c1;
        } else {
          d = top - 3; ab = above + excl + c0 + c1 + c2;
        }
        s.bc[0] = d;
        s.bc[1] = (uint32_t)ab;
        s.bc[2] = (uint32_t)(ab >> 32);
        const unsigned long long at = ab + s.hist.h64[d];
        s.bc[5] = (uint32_t)at;
        s.bc[6] = (uint32_t)(at >> 32);
      }
      if (lane == 0 && any == 0ull) s.bc[0] = NONE;
    }
    __syncthreads();
    const uint32_t d = s.bc[0];
    const unsigned long long ab = ((unsigned long long)s.bc[2] << 32) | s.bc[1];
    const unsigned long long at = ((unsigned long long)s.bc[6] << 32) | s.bc[5];
    __syncthreads();
    if (d == NONE) {
      *mass_out = 0;
      return 0;   // rounding: caller keeps everything
    }
    prefix |= d << shift;
    pmask |= 255u << shift;
    above = ab;
    if (lvl == LEVELS - 1) *mass_out = at;
  }
  return prefix;
}

template <typename ET, bool VECTOR>
__device__ __forceinline__ bool dense_row_stats(const Args& a, FinSmem& s, int b, const Mode& m) {
  constexpr int LEVELS = Key<ET>::LEVELS;
  const int RS = 2 * a.G + 1;
  const double fscale = ldexp(1.0, a.fixbits);
  const int k = a.topk ? a.topk[b] : 0;
  for (int r = 0; r <= 2 * m.g; ++r) {
    const int slot = used_slot(a.G, m.g, r);
    const bool isP = slot <= a.G;
    const ET* rp = row_ptr<ET>(a, b, isP, isP ? slot : slot - a.G - 1);
    uint32_t kmax = 0, bad = 0;
    row_for_each<ET, VECTOR>(rp, a.V, [&](uint32_t uk, int) {
      kmax = max(kmax, uk);
      bad |= key_valid<ET>(uk) ? 0u : 1u;
    });
    bad = block_or_u32(bad, s.red_u);
    kmax = block_max_u32(kmax, s.red_u);
    if (bad || kmax <= Key<ET>::NEG_INF) return false;
    if (m.mode == MODE_GREEDY) {
      uint32_t arg = 0xFFFFFFFFu;
      row_for_each<ET, VECTOR>(rp, a.V, [&](uint32_t uk, int i) {
        if (uk == kmax) arg = min(arg, (uint32_t)i);
      });
      arg = block_min_u32(arg, s.red_u);
      if (threadIdx.x == 0) s.st_arg[r] = arg;
      __syncthreads();
      continue;
    }
    const float zmax = Key<ET>::value(kmax);
    const float invT = 1.0f / m.T;
    uint32_t thr = 1;
    if (k > 0 && k < a.V) {
      thr = block_kth_largest<LEVELS>(
          [&](auto fn) { row_for_each<ET, VECTOR>(rp, a.V, [&](uint32_t uk, int) { fn(uk); }); }, (uint32_t)k,
          s.hist.h32, s.bc);
      if (thr == 0) thr = 1;
    }
    unsigned long long sl = 0;
    row_for_each<ET, VECTOR>(rp, a.V, [&](uint32_t uk, int) {
      if (uk >= thr) sl += (unsigned long long)((double)__expf((Key<ET>::value(uk) - zmax) * invT) * fscale);
    });
    unsigned long long S = block_sum(sl, s.red_u64);
    if (m.tp < 1.0f) {
      uint32_t tstar;
      unsigned long long mass = 0;
      if (m.tp <= 0.0f) {
        tstar = kmax;
        unsigned long long ml = 0;
        row_for_each<ET, VECTOR>(rp, a.V, [&](uint32_t uk, int) {
          if (uk >= tstar) ml += (unsigned long long)((double)__expf((Key<ET>::value(uk) - zmax) * invT) * fscale);
        });
        mass = block_sum(ml, s.red_u64);
      } else {
        tstar = dense_topp_select<ET, VECTOR>(s, rp, a.V, thr, zmax, invT, fscale, (double)m.tp * (double)S, &mass);
      }
      if (tstar != 0 && mass > 0) {
        thr = max(thr, tstar);
        S = mass;
      }
    }
    if (threadIdx.x == 0) {
      s.st_thr[r] = thr;
      s.st_zmax[r] = zmax;
      s.st_S[r] = (double)S / fscale;
    }
    __syncthreads();
  }
  return true;
}

template <typename ET>
__device__ __forceinline__ double dense_prob(uint32_t uk, uint32_t thr, float zmax, float invT, double invS) {
  if (uk < thr) return 0.0;
  return (double)__expf((Key<ET>::value(uk) - zmax) * invT) * invS;
}

template <typename ET, bool VECTOR>
__device__ __forceinline__ void dense_positions(const Args& a, FinSmem& s, int b, const Mode& m) {
  const float invT = m.mode == MODE_GREEDY ? 0.f : 1.0f / m.T;
  for (int i = 0; i < m.g; ++i) {
    const int rp = i, rq = m.g + 1 + i;
    const int x = a.draft[(size_t)b * a.G + i];
    if (m.mode == MODE_GREEDY) {
      if (threadIdx.x == 0) {
        s.pos_p[i] = (uint32_t)x == s.st_arg[rp] ? 1.0 : 0.0;
        s.pos_q[i] = (uint32_t)x == s.st_arg[rq] ? 1.0 : 0.0;
        s.pos_alpha[i] = s.st_arg[rp] == s.st_arg[rq] ? 1.0 : 0.0;
      }
      continue;
    }
    const ET* pp = row_ptr<ET>(a, b, true, i);
    const ET* qp = row_ptr<ET>(a, b, false, i);
    const uint32_t thrA = s.st_thr[rp], thrB = s.st_thr[rq];
    const float zA = s.st_zmax[rp], zB = s.st_zmax[rq];
    const double iA = 1.0 / s.st_S[rp], iB = 1.0 / s.st_S[rq];
    double al = 0.0;
    row_for_each<ET, VECTOR>(pp, a.V, [&](uint32_t uk, int v) {
      const double pv = dense_prob<ET>(uk, thrA, zA, invT, iA);
      if (pv > 0.0) {
        const double qv = dense_prob<ET>(Key<ET>::load_key(qp, v), thrB, zB, invT, iB);
        al += fmin(pv, qv);
      }
    });
    al = block_sum(al, s.red_d);
    if (threadIdx.x == 0) {
      s.pos_p[i] = dense_prob<ET>(Key<ET>::load_key(pp, x), thrA, zA, invT, iA);
      s.pos_q[i] = dense_prob<ET>(Key<ET>::load_key(qp, x), thrB, zB, invT, iB);
      s.pos_alpha[i] = al;
    }
    __syncthreads();
  }
  __syncthreads();
}

template <typename ET, bool VECTOR>
__device__ __forceinline__ int dense_draw(const Args& a, FinSmem& s, int b, const Mode& m, int n, float ures) {
  if (m.mode == MODE_GREEDY) return (int)s.st_arg[n];
  const float invT = 1.0f / m.T;
  const bool resid = n < m.g;
  const int rp = n, rq = m.g + 1 + n;
  const ET* pp = row_ptr<ET>(a, b, true, n);
  const ET* qp = resid ? row_ptr<ET>(a, b, false, n) : nullptr;
  const uint32_t thrA = s.st_thr[rp];
  const float zA = s.st_zmax[rp];
  const double iA = 1.0 / s.st_S[rp];
  uint32_t thrB = 0;
  float zB = 0.f;
  double iB = 0.0;
  if (resid) {
    thrB = s.st_thr[rq];
    zB = s.st_zmax[rq];
    iB = 1.0 / s.st_S[rq];
  }
  const int V = a.V;
  auto weight = [&](int v, bool fallback) -> double {
    const double p = dense_prob<ET>(Key<ET>::load_key(pp, v), thrA, zA, invT, iA);
    if (!resid || fallback) return p;
    const double q = dense_prob<ET>(Key<ET>::load_key(qp, v), thrB, zB, invT, iB);
    return fmax(p - q, 0.0);
  };
  bool fallback = false;
  double zl = 0.0;
  for (int v = threadIdx.x; v < V; v += NT) zl += weight(v, false);
  double Z = block_sum(zl, s.red_d);
  if (!(Z > 0.0)) {
    fallback = true;
    zl = 0.0;
    for (int v = threadIdx.x; v < V; v += NT) zl += weight(v, true);
    Z = block_sum(zl, s.red_d);
  }
  const double target = (double)ures * Z;
  // Ascending vocabulary order: each thread takes 8 consecutive ids per tile.
  constexpr int PER = 8;
  double base = 0.0;
  int lastpos = -1;
  for (int t0 = 0; t0 < V; t0 += NT * PER) {
    const int v0 = t0 + (int)threadIdx.x * PER;
    double w[PER];
    double loc = 0.0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      w[e] = (v0 + e < V) ? weight(v0 + e, fallback) : 0.0;
      loc += w[e];
      if (w[e] > 0.0) lastpos = v0 + e;
    }
    double tot;
    const double ex = block_excl_scan(loc, s.red_d, &tot);
    double c = base + ex;
    uint32_t hit = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      c += w[e];
      if (hit == 0xFFFFFFFFu && v0 + e < V && c > target) hit = (uint32_t)(v0 + e);
    }
    hit = block_min_u32(hit, s.red_u);
    if (hit != 0xFFFFFFFFu) return (int)hit;
    base += tot;
  }
  return (int)block_max_u32((uint32_t)(lastpos + 1), s.red_u) - 1;
}


// ===========================================================================
// The finisher kernel: one workgroup per sequence.
// ===========================================================================
// A dense sequence whose positions the pair kernel has already resolved:
// one wavefront reads the records (lane i holds position i), runs the
// acceptance tests, finds the first rejection by ballot and writes the
// outputs; the other wavefronts of the workgroup leave at once.
__device__ __forceinline__ void finish_from_pairs_wave(const Args& a, int b, const Mode& m) {
  const int lane = threadIdx.x & 63;
  const int G = a.G, g = m.g;
  const float* ub = a.u + (size_t)b * (G + 1);
  const int32_t* xb = a.draft + (size_t)b * G;
  const PosRec* rec = a.pos + (size_t)b * (G + 1);
  PosRec r{0.0, 0.0, 0.0, -1, 0u};
  int32_t xv = 0;
  float uv = 0.5f;
  if (lane < g) {
    r = rec[lane];
    xv = xb[lane];
    uv = ub[lane];
  }
  const PosRec rb = rec[g];
  const float ures = ub[G];
  const uint32_t fl = a.seq_flags[b];
  const int gl = a.gamma_len ? a.gamma_len[b] : G;
  const float lv = a.lenience ? a.lenience[b] : 1.0f;
  bool ok = !(fl & F_BAD) && (a.sampler || (gl >= 1 && gl <= G)) && !(m.tp != m.tp) && lv >= 0.0f && lv <= 1.0f;
  ok = ok && ures >= 0.0f && ures < 1.0f && !rb.bad;
  const bool badl = lane < g && (xv < 0 || xv >= a.V || !(uv >= 0.0f && uv < 1.0f) || r.bad);
  ok = ok && __ballot(badl) == 0ull;
  const bool rej = lane < g && !((double)uv * (double)lv * r.qx < r.px);
  const unsigned long long mask = __ballot(rej);
  const int n = mask ? __ffsll((long long)mask) - 1 : g;
  const int tn = __shfl(r.tok, n < 64 ? n : 0, 64);
  const int tok = n < g ? tn : rb.tok;
  int32_t* ot = a.out_tokens + (size_t)b * (G + 1);
  float* oa = a.out_alpha + (size_t)b * G;
  const float qnan = __int_as_float(0x7FC00000);
  for (int i = lane; i <= G; i += 64) ot[i] = ok ? (i < n ? xv : (i == n ? tok : -1)) : -1;
  if (lane < G) {
    oa[lane] = ok ? (lane < g ? (float)r.alpha : 0.0f) : qnan;
    if (a.out_pq) {
      float* op = a.out_pq + ((size_t)b * G + lane) * 2;
      op[0] = ok ? (lane < g ? (float)r.px : 0.0f) : qnan;
      op[1] = ok ? (lane < g ? (float)r.qx : 0.0f) : qnan;
    }
  }
  if (lane == 0) {
    if (a.out_n) a.out_n[b] = ok ? n : -1;
    a.seq_flags[b] = 0;
    if (b == 0) {   // the pair kernel has finished with the list
      a.dense_count[0] = 0;
      a.dense_count[1] = 0;
      a.dense_count[2] = 0;
      a.dense_count[3] = 0;
    }
  }
}

// Whether the pair kernel left a position of sequence b uncomputed (a row
// it could not take): then the whole sequence is computed from the logits.
// Every wavefront reads the records itself, so the answer is uniform without
// a block barrier.
__device__ __forceinline__ bool pair_redo(const Args& a, int b, int g) {
  const int lane = threadIdx.x & 63;
  const PosRec* rec = a.pos + (size_t)b * (a.G + 1);
  bool r = false;
  for (int i = lane; i <= g; i += 64) r = r || rec[i].bad == REC_REDO;
  return __ballot(r) != 0ull;
}

// FAST: the register path is compiled in (not for the all-dense finisher,
// whose calls have no survivor lists).
template <typename ET, bool VECTOR, bool FAST = true>
__device__ __forceinline__ void finish_sequence(const Args& a, FinSmem& s, int b) {
  bool redo = false;
  {
    const Mode m = seq_mode(a, b);
    if (a.pair && m.mode == MODE_DENSE) {   // block-uniform; no block barrier follows
      redo = pair_redo(a, b, m.g);
      if (!redo) {
        if (threadIdx.x < 64) finish_from_pairs_wave(a, b, m);
        return;
      }
    }
  }
  const int RS = a.RS;
  const int G = a.G;
  const float* ub = a.u + (size_t)b * (G + 1);
  const int32_t* xb = a.draft + (size_t)b * G;
  // Every global load of the opening is issued before any is used: the
  // survivor counts of all slots and the drafts and uniforms of all
  // positions (padding included, masked below), with the parameters.
  const int nslot = RS * a.NP;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // wavefront-uniform
  const int lane = threadIdx.x & 63;
  int32_t craw = 0, xraw = 0;
  float uraw = 0.5f;
  if (nslot <= MAXSEG && (int)threadIdx.x < nslot) craw = a.counts[(size_t)b * nslot + threadIdx.x];
  if ((int)threadIdx.x < G) {
    xraw = xb[threadIdx.x];
    uraw = ub[threadIdx.x];
  }
  const float ubon = ub[G];          // the bonus / residual draw's uniform
  // The first SPEC entries of the first 2 NWAVE (slot, part) lists are
  // fetched in the same round trip as the counts (wavefront w: lists w and
  // w + NWAVE, one entry per lane), before the counts say how many are
  // valid: a top-k list of k <= 64 without ties is no longer, so the pool is
  // then filled from registers.  Every list has SEG slots, so these reads
  // stay in its storage.
  constexpr int SPEC = 64;
  // When the register path can apply (at most FAST_CH parts per row, G <
  // NWAVE), the first 64 entries of every list are fetched position-wise
  // instead: wavefront w holds those of its target row (slot w) and draft
  // row (slot G+1+w, w < G), part p in chunk p * fc, and lane h * NP + p
  // the part list's size.  Both the register path and the LDS list path use
  // them.  Every list has SEG >= 64 * FAST_CH slots, so these reads stay in
  // its storage.
  const bool fastc = FAST && !a.all_dense && nslot <= MAXSEG && a.NP <= FAST_CH && G < NWAVE;
  const bool spec = !a.all_dense && nslot <= MAXSEG && !fastc;
  uint2 sp[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int li = wave + h * NWAVE;
    const uint2* lp = a.lists + ((size_t)b * nslot + li) * SEG;
    sp[h] = spec && li < nslot ? lp[lane] : make_uint2(0u, 0u);
  }
  // f0[h][p]: the first 64 entries of part p of the position's target (h =
  // 0) and draft (h = 1) row; the conditions are wavefront-uniform.
  const uint2* lpw[2];
  uint2 f0[2][FAST_CH];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bool row = fastc && wave <= G && (h == 0 || wave < G);
    lpw[h] = a.lists + list_index(a, b * RS + (row ? (h ? G + 1 + wave : wave) : 0), 0);
#pragma unroll
    for (int p = 0; p < FAST_CH; ++p) f0[h][p] = make_uint2(0u, 0u);
    if (row) {
#pragma unroll
      for (int p = 0; p < FAST_CH; ++p)
        if (p < a.NP) f0[h][p] = lpw[h][(size_t)p * SEG + lane];
    }
  }
  uint32_t fcnt = 0;
  if (fastc && wave <= G && lane < 2 * a.NP) {
    const int h = lane / a.NP, p = lane - h * a.NP;
    if (h == 0 || wave < G) fcnt = (uint32_t)a.counts[(size_t)b * nslot + (h ? G + 1 + wave : wave) * a.NP + p];
  }
  const int xw = fastc && wave < G ? xb[wave] : -1;   // draft of the wavefront's position
  const Mode m = seq_mode(a, b);
  const uint32_t fl = a.seq_flags[b];
  const int R = 2 * m.g + 1;
  const int NS = R * a.NP;          // (row, part) lists of the sequence
  bool ok = m.mode != MODE_INVALID && !(fl & F_BAD);
  const int gl = a.gamma_len ? a.gamma_len[b] : G;
  ok = ok && (a.sampler || (gl >= 1 && gl <= G));
  ok = ok && !(m.tp != m.tp);
  const float lv = a.lenience ? a.lenience[b] : 1.0f;
  ok = ok && lv >= 0.0f && lv <= 1.0f;
  // Without the select launch (every sequence promised dense) there are no
  // survivor lists: a sequence that is not dense after all takes the
  // multi-pass path.
  bool dense = m.mode == MODE_DENSE || (fl & F_DEMOTE) || NS > MAXSEG || a.all_dense;
  const bool from_pairs = a.pair && m.mode == MODE_DENSE && !redo;
  uint32_t badin = 0;
  if ((int)threadIdx.x < m.g)
    badin |= (xraw < 0 || xraw >= a.V || !(uraw >= 0.0f && uraw < 1.0f)) ? 1u : 0u;
  if (threadIdx.x == 0) badin |= !(ubon >= 0.0f && ubon < 1.0f) ? 1u : 0u;
  // The register path: top-k sequences without top-p and argmax sequences,
  // when their lists fit the registers in ascending id (checked in
  // fast_position; otherwise the LDS list path below takes the sequence).
  const bool fastm = fastc && ok && !dense && (m.mode == MODE_GREEDY || (m.mode == MODE_SPARSE && !(m.tp < 1.0f)));
  if constexpr (FAST) {
    const uint32_t fw = __ballot(badin != 0u) ? 1u : 0u;
    if (lane == 0) s.fflag[wave] = fw;
    if (fastm && wave <= m.g) {
      const int x = wave < m.g ? xw : -1;
      switch (a.NP) {
        case 1: fast_position<ET, 1>(s, m, wave, f0, fcnt, lpw[0], lpw[1], x, ubon); break;
        case 2: fast_position<ET, 2>(s, m, wave, f0, fcnt, lpw[0], lpw[1], x, ubon); break;
        case 3: fast_position<ET, 3>(s, m, wave, f0, fcnt, lpw[0], lpw[1], x, ubon); break;
        default: fast_position<ET, 4>(s, m, wave, f0, fcnt, lpw[0], lpw[1], x, ubon); break;
      }
    }
  }
  if ((int)threadIdx.x < G) s.xs[threadIdx.x] = xraw;
  if (nslot <= MAXSEG && (int)threadIdx.x < nslot) s.cslot[threadIdx.x] = (uint32_t)max(craw, 0);
  __syncthreads();
  bool fast_done = false;
  if constexpr (FAST) {
    if (fastm) {
      uint32_t fflags = 0, fpos = 0;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) {
        fflags |= s.fflag[w];
        fpos |= w <= m.g ? s.fempty[w] : 0u;
      }
      fast_done = fflags == 0u && (fpos & 2u) == 0u;   // inputs valid, every list held (block-uniform)
    }
  }
  if (fast_done) {
    if (wave != 0) return;
    // Wavefront 0: the acceptance test, the first rejection, the outputs
    // (thread i < 64 holds draft i and its uniform; G < 64).
    const uint32_t emp = lane <= m.g ? s.fempty[min(lane, NWAVE - 1)] : 0u;
    const bool fok = __ballot(emp != 0u) == 0ull;
    const bool rej = lane < m.g && !((double)uraw * (double)lv * s.pos_q[lane] < s.pos_p[lane]);
    const unsigned long long mask = __ballot(rej);
    const int nn = mask ? __ffsll((long long)mask) - 1 : m.g;
    const int tk = s.cand_tok[nn];
    if (lane <= G) a.out_tokens[(size_t)b * (G + 1) + lane] = fok ? (lane < nn ? xraw : (lane == nn ? tk : -1)) : -1;
    if (lane < G) {
      const float qnan = __int_as_float(0x7FC00000);
      const bool used = lane < m.g;
      a.out_alpha[(size_t)b * G + lane] = fok ? (used ? (float)s.pos_alpha[lane] : 0.0f) : qnan;
      if (a.out_pq) {
        float* op = a.out_pq + ((size_t)b * G + lane) * 2;
        op[0] = fok ? (used ? (float)s.pos_p[lane] : 0.0f) : qnan;
        op[1] = fok ? (used ? (float)s.pos_q[lane] : 0.0f) : qnan;
      }
    }
    if (lane == 0) {
      if (a.out_n) a.out_n[b] = fok ? nn : -1;
      a.seq_flags[b] = 0;
      if (b == 0) {   // the pair kernel has finished with the list
        a.dense_count[0] = 0;
        a.dense_count[1] = 0;
        a.dense_count[2] = 0;
        a.dense_count[3] = 0;
      }
    }
    return;
  }
  uint32_t c = 0, rest = 0;
  if (ok && !dense && (int)threadIdx.x < NS) {
    const int r = threadIdx.x / a.NP, p = threadIdx.x - r * a.NP;
    const int si = used_slot(G, m.g, r) * a.NP + p;
    c = nslot <= MAXSEG ? s.cslot[si] : (uint32_t)max(a.counts[(size_t)b * RS * a.NP + si], 0);
    rest = fastc ? c > 64u : (!spec || si >= 2 * NWAVE || c > (uint32_t)SPEC);
  }
  // The list sizes' exclusive scan and the OR of the input checks and of the
  // lists' needs in one LDS round trip (the barrier after cslot already
  // separates earlier LDS use, and the one after soff below separates later
  // use).
  uint32_t total = 0, excl = 0, flags = 0;
  {
    const uint32_t incl = wave_incl_scan_dpp(c);
    const uint32_t orw = (__ballot(badin != 0u) ? 1u : 0u) | (__ballot(rest != 0u) ? 2u : 0u);
    if (lane == 63) {
      s.red_u[wave] = incl;
      s.red_or[wave] = orw;
    }
    __syncthreads();
    uint32_t base = 0;
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) {
      const uint32_t v = s.red_u[i];
      base += i < wave ? v : 0u;
      total += v;
      flags |= s.red_or[i];
    }
    excl = base + incl - c;
    ok = ok && (flags & 1u) == 0;
  }
  if (ok && !dense) {
    if ((int)threadIdx.x < NS) s.soff[threadIdx.x] = excl;
    if (threadIdx.x == 0) s.soff[NS] = total;
    if (total > (uint32_t)POOL) dense = true;   // does not fit in LDS: multi-pass path
  }
  __syncthreads();
  if (ok && !dense) {
    for (int r = threadIdx.x; r <= R; r += NT) s.off[r] = s.soff[r * a.NP];
    // The entries fetched with the counts go from registers to their pool
    // slots: slot-list li = slot * NP + part is used row r's part (P rows
    // r = slot <= g, Q rows r = slot - G + g for G < slot <= G + g).
    if (spec) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int li = wave + h * NWAVE;
        const int slot = li / a.NP, p = li - slot * a.NP;
        const int r = slot <= m.g ? slot : (slot > G && slot <= G + m.g ? slot - G + m.g : -1);
        if (li < nslot && r >= 0) {
          const uint32_t o = s.soff[r * a.NP + p], n = s.soff[r * a.NP + p + 1] - o;
          if ((uint32_t)lane < n) s.pool[o + lane] = sp[h];
        }
      }
    } else if (fastc) {
      // The register path's first chunks: wavefront w holds those of used
      // rows w (target) and g + 1 + w (draft).
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = h == 0 ? (wave <= m.g ? wave : -1) : (wave < m.g ? m.g + 1 + wave : -1);
        if (r >= 0) {
#pragma unroll
          for (int p = 0; p < FAST_CH; ++p) {
            if (p < a.NP) {
              const uint32_t o = s.soff[r * a.NP + p], n = s.soff[r * a.NP + p + 1] - o;
              if ((uint32_t)lane < n) s.pool[o + lane] = f0[h][p];
            }
          }
        }
      }
    }
    // The rest (lists past the first 2 NWAVE, entries past the first SPEC;
    // with the register path's chunks, entries past the first 64) in one
    // round trip.
    for (uint32_t e = (flags & 2u) ? threadIdx.x : total; e < total; e += NT) {
      int lo = 0, hi = NS;   // list with soff[lo] <= e < soff[lo+1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s.soff[mid] <= e) lo = mid;
        else hi = mid;
      }
      const int r = lo / a.NP, p = lo - r * a.NP;
      const int si = used_slot(G, m.g, r) * a.NP + p;
      const uint32_t j = e - s.soff[lo];
      if (fastc ? j < 64u : (spec && si < 2 * NWAVE && j < (uint32_t)SPEC)) continue;
      s.pool[e] = a.lists[list_index(a, b * RS + used_slot(G, m.g, r), p) + j];
    }
    __syncthreads();
    // A row without a finite logit: every wavefront checks all rows itself
    // (R <= 129 offsets, published by the barrier above), so no block
    // reduction is needed.
    bool empty = false;
    for (int r = lane; r < R; r += 64) empty = empty || s.off[r + 1] == s.off[r];
    ok = __ballot(empty) == 0ull;
    if (ok) {
      for (int r = wave; r < R; r += NWAVE) pool_row_stats<ET>(s, r, m, a.NP);
      __syncthreads();
      // Every position's p(x), q(x), overlap and residual draw (as if the
      // first rejection were there), and the bonus draw, in parallel; the
      // acceptance test then only picks one of the drawn tokens.
      for (int i = wave; i <= m.g; i += NWAVE) {
        int tk;
        if (m.mode != MODE_GREEDY && s.st_sorted[i] && (i == m.g || s.st_sorted[m.g + 1 + i])) {
          tk = wave_position_draw_sorted(s, i, i < m.g ? s.xs[i] : -1, m, ubon);
        } else {
          if (i < m.g) wave_position(s, i, s.xs[i], m);
          tk = pool_draw(s, m, i, ubon);
        }
        if (lane == 0) s.cand_tok[i] = tk;
      }
      __syncthreads();
    }
  } else if (ok && dense && from_pairs) {
    // Per-position results of the pair-resident kernel.
    const PosRec* rec = a.pos + (size_t)b * (G + 1);
    uint32_t badr = 0;
    for (int i = threadIdx.x; i <= m.g; i += NT) {
      const PosRec r = rec[i];
      badr |= r.bad;
      s.cand_tok[i] = r.tok;
      if (i < m.g) {
        s.pos_p[i] = r.px;
        s.pos_q[i] = r.qx;
        s.pos_alpha[i] = r.alpha;
      }
    }
    ok = block_or_u32(badr, s.red_u) == 0;
  } else if (ok && dense) {
    ok = dense_row_stats<ET, VECTOR>(a, s, b, m);
    if (ok) dense_positions<ET, VECTOR>(a, s, b, m);
  }
  int n = 0, tok = -1;
  if (ok) {
    // Acceptance of each draft, then the first rejection via one ballot.
    if (threadIdx.x < 64) {
      const int i = threadIdx.x;
      bool rej = false;
      if (i < m.g) rej = !((double)uraw * (double)lv * s.pos_q[i] < s.pos_p[i]);   // uraw = ub[i]
      const unsigned long long mask = __ballot(rej);
      const int nn = mask ? __ffsll((long long)mask) - 1 : m.g;
      if (i == 0) {
        if (!dense || from_pairs) s.bc[6] = (uint32_t)s.cand_tok[nn];
        s.bc[7] = (uint32_t)nn;
      }
    }
    __syncthreads();
    n = (int)s.bc[7];
    tok = (int)s.bc[6];
    __syncthreads();
    if (dense && !from_pairs) tok = dense_draw<ET, VECTOR>(a, s, b, m, n, ubon);
  }
  int32_t* ot = a.out_tokens + (size_t)b * (G + 1);
  float* oa = a.out_alpha + (size_t)b * G;
  // Thread i < G holds draft i in xraw (G < NT).
  if ((int)threadIdx.x <= G) {
    const int i = threadIdx.x;
    ot[i] = ok ? (i < n ? xraw : (i == n ? tok : -1)) : -1;
  }
  const float qnan = __int_as_float(0x7FC00000);
  for (int i = threadIdx.x; i < G; i += NT) {
    oa[i] = ok ? (i < m.g ? (float)s.pos_alpha[i] : 0.0f) : qnan;
    if (a.out_pq) {
      float* op = a.out_pq + ((size_t)b * G + i) * 2;
      op[0] = ok ? (i < m.g ? (float)s.pos_p[i] : 0.0f) : qnan;
      op[1] = ok ? (i < m.g ? (float)s.pos_q[i] : 0.0f) : qnan;
    }
  }
  if (threadIdx.x == 0) {
    if (a.out_n) a.out_n[b] = ok ? n : -1;
    a.seq_flags[b] = 0;
    if (b == 0) {   // the pair kernel has finished with the list
      a.dense_count[0] = 0;
      a.dense_count[1] = 0;
      a.dense_count[2] = 0;
      a.dense_count[3] = 0;
    }
  }
  (void)lane;
}

// One workgroup per sequence; when every sequence was promised dense, one
// workgroup per NWAVE sequences: each wavefront finishes one pair-resolved
// sequence, and a sequence that is not dense after all is then finished by
// the whole workgroup.
template <typename ET, bool VECTOR>
__global__ __launch_bounds__(NT) void finish_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char fin_smem_raw[];
  FinSmem& s = *reinterpret_cast<FinSmem*>(fin_smem_raw);
  finish_sequence<ET, VECTOR>(a, s, blockIdx.x);
}

// The finisher when every sequence was promised dense: a workgroup per NWAVE
// sequences, each wavefront finishing one pair-resolved sequence; a sequence
// that is not dense after all is then finished by the whole workgroup.  (A
// kernel of its own: the loop around the whole-sequence procedure costs
// registers that the one-sequence finisher should not pay.)
template <typename ET, bool VECTOR>
__global__ __launch_bounds__(NT) void finish_dense_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char fin_smem_raw[];
  FinSmem& s = *reinterpret_cast<FinSmem*>(fin_smem_raw);
  const int wave = threadIdx.x >> 6;
  const int b0 = blockIdx.x * NWAVE;
  uint32_t other = 0;
  if (b0 + wave < a.B) {
    const Mode m = seq_mode(a, b0 + wave);
    if (m.mode == MODE_DENSE && !pair_redo(a, b0 + wave, m.g)) finish_from_pairs_wave(a, b0 + wave, m);
    else other = 1;
  }
  if ((threadIdx.x & 63) == 0) s.red_u[wave] = other;
  __syncthreads();
  uint32_t mask = 0;
  for (int w = 0; w < NWAVE; ++w) mask |= s.red_u[w] << w;
  __syncthreads();   // finish_sequence reuses the LDS
  while (mask) {     // workgroup-uniform
    const int w = __builtin_ctz(mask);
    mask &= mask - 1u;
    finish_sequence<ET, VECTOR, false>(a, s, b0 + w);
    if (mask) __syncthreads();
  }
}

}  // namespace sv
