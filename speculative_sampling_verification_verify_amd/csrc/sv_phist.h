// Dense (sequence, position) pairs with bf16 rows too long to hold in LDS:
// statistics from an exact count histogram of the row's bf16 values.
//
// A bf16 logit takes one of 65536 bit patterns, so a row's exact count per
// value (16-bit counts, two per 32-bit LDS word: 128 KB) fits in one CU's
// LDS.  One streaming pass over a row fills it; a scan of the histogram in
// descending value order then gives, with no further pass over the row:
//   * validity (no NaN or +inf) and the maximum logit,
//   * the top-k threshold (the k-th largest value, ties kept) for large k,
//   * the normaliser S = sum of the weights e(z) = 2^((z - zmax) log2(e) / T),
//     and for top-p the nucleus cut t*: the largest value whose mass at or
//     above reaches top_p * S (ties kept).
// Masses are count(value) * e(value), summed in double in a fixed order.  The processed distribution is
// that of "Fast Inference from Transformers via Speculative Decoding"
// (mtandhj.com summary), "Speculative Sampling: theoretical basis" (the
// sampling adjustments applied to both models).
//
// Per pair: each row is read once for its histogram (rows of up to 131072
// values: 16 16-byte units per thread); then both rows are read again, but
// only in the units whose largest target value can reach the target's
// nucleus, for the overlap
// alpha = sum min(p, q) ("How to choose gamma" on the same summary) and the
// per-(tile, wavefront) sums of the draw weights, the residual max(0, p - q)
// or, at the bonus position, p ("Speculative Decoding: the art of guessing
// well", "Speculative sampling"): elsewhere p = 0, so neither has a term.
// The tile holding the inverse-CDF crossing at u * Z ("Sampling with shared
// noise" on the same page, ascending vocabulary id) is then examined again.
// Row bytes read per pair: 2x the algorithmic bytes for unfiltered rows,
// less the smaller the nucleus (about 1x when it holds a few values).
//
// A row in which more than 65535 elements share one value would overflow its
// 16-bit count; the decoded counts then no longer add up to V.  The pair's
// record then asks the finisher to compute the whole sequence by its
// multi-pass procedure over the logits.
//
// Two kernels run these pairs: pair_hist_kernel, and mixed_hist_kernel for
// calls that also hold top-k / argmax sequences, which streams their select
// units in the same launch (at the end of this file).
#pragma once

#include "sv_pair.h"
#include "sv_wave.h"

namespace sv {

constexpr int PH_NT = 1024;                 // threads per workgroup (one workgroup per CU)
constexpr int PH_NW = PH_NT / 64;
constexpr int PH_UPT = 16;                  // 16-byte units of a row per thread
constexpr int PH_WORDS = 32768;             // histogram words: bf16 key 2j in the low half of word j, 2j+1 high
constexpr int PH_INFLIGHT = 8;              // units of a row in flight per thread while it streams
constexpr int PH_WINFLIGHT = 8;             // list entries in flight per thread in the weights pass
constexpr int PH_MAX_UNITS = PH_NT * PH_UPT;
constexpr int PH_BLKW = 256;                // histogram words per block (four per lane of a wavefront)
constexpr int PH_NBLK = PH_WORDS / PH_BLKW; // 128 blocks
constexpr int PH_BPW = PH_NBLK / PH_NW;     // blocks per wavefront

struct PhSmem {
  uint32_t hist[PH_WORDS];
  uint8_t umax[PH_MAX_UNITS];               // bucket (ph_bucket) of each target unit's largest value
  float uref[PH_UPT / PH_INFLIGHT][PH_NW];  // the floor those buckets start from, per (batch, wavefront)
  double blk[PH_NBLK];                      // per-block sums of f(key, count) from the last ph_sums
  double wpart[PH_NW];                      // per-wavefront totals of the same
  double part[PH_UPT][PH_NW];               // draw-weight sum per (tile, wavefront)
  uint32_t red[5 * PH_NW];
  uint32_t bc[8];
  double bd[2];
  uint32_t next_pair;
  uint32_t spare[64];                       // per-lane targets of the count pass's below-floor atomics
  uint32_t rx[2];                           // thread 0's draft token and its two logits' patterns
};

// Order-preserving 16-bit keys of two bf16 patterns at once (+0 and -0 share
// a key; -inf is 0x0080; NaN and +inf fall outside [0x0080, 0xFF7F]).
typedef unsigned short ph_u16x2 __attribute__((ext_vector_type(2)));
typedef short ph_i16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t ph_keys2(uint32_t w) {
  const ph_u16x2 h = __builtin_bit_cast(ph_u16x2, w);
  // m = 0xFFFF for a negative pattern, else 0: a negative pattern's key is
  // its complement plus one (so -0 meets +0), a positive one's its pattern
  // with the top bit set.
  const ph_u16x2 m = __builtin_bit_cast(ph_u16x2, __builtin_bit_cast(ph_i16x2, w) >> (short)15);
  const ph_u16x2 key = (h ^ (m | (unsigned short)0x8000)) - m;
  return __builtin_bit_cast(uint32_t, key);
}
__device__ __forceinline__ void ph_count(uint32_t* hist, uint32_t key) {
  atomicAdd(&hist[key >> 1], 1u << ((key & 1u) << 4));
}

// The packed key extremes of one 16-byte unit (8 bf16), folded into kmax2 /
// kmin2 (both halves at once).
__device__ __forceinline__ void ph_extremes_unit(const uint4& u, uint32_t& kmax2, uint32_t& kmin2) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t k2 = ph_keys2(w[j]);
    kmax2 = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(ph_u16x2, kmax2),
                                                                   __builtin_bit_cast(ph_u16x2, k2)));
    kmin2 = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(ph_u16x2, kmin2),
                                                                   __builtin_bit_cast(ph_u16x2, k2)));
  }
}
// The same, replacing the unit's patterns by their keys (two per word), so
// the count that follows need not form them again.
__device__ __forceinline__ void ph_keys_extremes_unit(uint4& u, uint32_t& kmax2, uint32_t& kmin2) {
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[j] = ph_keys2(w[j]);
    kmax2 = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(ph_u16x2, kmax2),
                                                                   __builtin_bit_cast(ph_u16x2, w[j])));
    kmin2 = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(ph_u16x2, kmin2),
                                                                   __builtin_bit_cast(ph_u16x2, w[j])));
  }
  u = make_uint4(w[0], w[1], w[2], w[3]);
}
// Counts the keys of a unit (ph_keys_extremes_unit's output) that are at
// least kfloor, with no branch: a key below the floor adds to the lane's own
// spare word instead (no two lanes share one, so those atomics never meet),
// and the wavefront's number of such keys is added to skipped
// (wavefront-uniform).
__device__ __forceinline__ void ph_add_keys(uint32_t* hist, uint32_t* spare, const uint4& kk, uint32_t kfloor,
                                            uint32_t& skipped) {
  const uint32_t w[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t klo = w[j] & 0xFFFFu, khi = w[j] >> 16;
    const bool glo = klo >= kfloor, ghi = khi >= kfloor;
    skipped += (uint32_t)__popcll(__ballot(!glo)) + (uint32_t)__popcll(__ballot(!ghi));
    // Word key >> 1 of each key (bit-field extracts), and the count's half
    // (key & 1) as a shift of 16, formed for both keys at once.
    const uint32_t sh = __builtin_bit_cast(uint32_t, __builtin_bit_cast(ph_u16x2, w[j]) << (unsigned short)4);
    atomicAdd(glo ? &hist[__builtin_amdgcn_ubfe(w[j], 1u, 15u)] : spare, 1u << (sh & 16u));
    atomicAdd(ghi ? &hist[__builtin_amdgcn_ubfe(w[j], 17u, 15u)] : spare, 1u << ((sh >> 16) & 16u));
  }
}
// The largest key of a unit (its max over the 8 elements).
__device__ __forceinline__ uint32_t ph_unit_max(const uint4& u) {
  uint32_t mx = 0u, mn = 0xFFFFFFFFu;
  ph_extremes_unit(u, mx, mn);
  return max(mx & 0xFFFFu, mx >> 16);
}
// Bucket of a value z above a floor zf in steps of 1 / inv: 0 below the
// floor (or for NaN), 1 + floor((z - zf) inv) up to 255.  Non-decreasing in
// z for fixed zf and inv, so a unit whose largest value reaches a threshold
// has a bucket at least the threshold's: comparing buckets never skips a unit
// that holds a value at or above it.  A floor of -inf puts every value in 255.
__device__ __forceinline__ uint32_t ph_bucket(float z, float zf, float inv) {
  if (!(z >= zf)) return 0u;
  const float t = (z - zf) * inv;
  return t >= 254.0f ? 255u : 1u + (uint32_t)t;
}

struct PhFind {
  uint32_t key;    // the key where the running sum first reaches tau (NONE: never)
  double above;    // sum over larger keys
  double at;       // above + the key's own contribution
};

// Sums of per-key contributions f(key, count) (double) over the histogram:
// each block of 256 words (512 keys) is summed by one wavefront, four words
// per lane read at once, blocks that hold no count skipped by a ballot, and
// its sum is kept in s.blk for ph_find.  Blocks outside [b_lo, b_hi] hold no
// counted key and are not read.  Returns the total (the per-wavefront sums
// added in wavefront order) and the decoded counts (block-uniform).
template <class F>
__device__ __forceinline__ double ph_sums(PhSmem& s, F f, int b_lo, int b_hi, uint32_t& count) {
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), l = threadIdx.x & 63;
  const uint4* h4 = reinterpret_cast<const uint4*>(s.hist);
  uint32_t cnt = 0;
  double wsum = 0.0;
  constexpr int HALF = PH_BPW / 2;
#pragma unroll 1
  for (int r0 = 0; r0 < PH_BPW; r0 += HALF) {
    uint4 q[HALF];
#pragma unroll
    for (int r = 0; r < HALF; ++r) {
      const int bk = w + (r0 + r) * PH_NW;
      q[r] = bk >= b_lo && bk <= b_hi ? h4[bk * (PH_BLKW / 4) + l] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int r = 0; r < HALF; ++r) {
      const int bk = w + (r0 + r) * PH_NW;
      double v = 0.0;
      if (__ballot((q[r].x | q[r].y | q[r].z | q[r].w) != 0u)) {
        const uint32_t wd0 = (uint32_t)(bk * PH_BLKW + 4 * l);
        const uint32_t ww[4] = {q[r].x, q[r].y, q[r].z, q[r].w};
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          const uint32_t chi = ww[j] >> 16, clo = ww[j] & 0xFFFFu;
          cnt += chi + clo;
          if (chi) v += f(2u * (wd0 + (uint32_t)j) + 1u, chi);
          if (clo) v += f(2u * (wd0 + (uint32_t)j), clo);
        }
        v = wave_sum_dpp(v);
        wsum += v;
      }
      if (l == 0) s.blk[bk] = v;
    }
  }
  cnt = wave_reduce_dpp_u32(cnt, 0u, [](uint32_t x, uint32_t y) { return x + y; });
  if (l == 0) {
    s.red[3 * PH_NW + w] = cnt;
    s.wpart[w] = wsum;
  }
  __syncthreads();
  count = 0;
  double tot = 0.0;
  for (int x = 0; x < PH_NW; ++x) {
    count += s.red[3 * PH_NW + x];
    tot += s.wpart[x];
  }
  __syncthreads();   // red / wpart are written again by the next call
  return tot;
}

// The largest key at which the running sum of f over descending keys reaches
// tau (> 0), from the block sums of the last ph_sums with the same f.
// Wavefront 0 scans the 128 block sums (two per lane), then, within the
// crossing block, the per-lane sums of its 512 keys (eight per lane), then
// the eight keys of the crossing lane.  Where rounding leaves a level's
// running sum short of tau, its smallest entry is taken.
template <class F>
__device__ __forceinline__ PhFind ph_find(PhSmem& s, F f, double tau) {
  const int l = threadIdx.x & 63;
  if ((threadIdx.x >> 6) == 0) {
    // Lane l: blocks 127 - 2 l and 126 - 2 l (descending keys).
    const double b1 = s.blk[PH_NBLK - 1 - 2 * l], b0 = s.blk[PH_NBLK - 2 - 2 * l];
    const double inc = wave_incl_scan_f64(b1 + b0);
    uint32_t key = NONE;
    double above = 0.0, at = 0.0;
    if (readlane_f64(inc, 63) >= tau) {
      const unsigned long long hit = __ballot(inc >= tau);
      const int cl = __ffsll((long long)hit) - 1;
      double run = readlane_f64(inc - b1 - b0, cl);
      const double c1 = readlane_f64(b1, cl);
      const bool upper = run + c1 >= tau;
      const int cb = upper ? PH_NBLK - 1 - 2 * cl : PH_NBLK - 2 - 2 * cl;
      if (!upper) run += c1;
      // Lane l: words 4 (63 - l) + 3 .. 4 (63 - l) of the block, descending.
      const uint32_t wd0 = (uint32_t)(cb * PH_BLKW + 4 * (63 - l));
      const uint4 q = reinterpret_cast<const uint4*>(s.hist)[cb * (PH_BLKW / 4) + (63 - l)];
      const uint32_t ww[4] = {q.x, q.y, q.z, q.w};
      double ls = 0.0;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        const uint32_t chi = ww[j] >> 16, clo = ww[j] & 0xFFFFu;
        if (chi) ls += f(2u * (wd0 + (uint32_t)j) + 1u, chi);
        if (clo) ls += f(2u * (wd0 + (uint32_t)j), clo);
      }
      const double winc = wave_incl_scan_f64(ls);
      const unsigned long long whit = __ballot(run + winc >= tau);
      const unsigned long long nz = __ballot(ls > 0.0);
      const int wl = whit ? __ffsll((long long)whit) - 1 : (nz ? 63 - __clzll((long long)nz) : 63);
      const double base = run + readlane_f64(winc - ls, wl);
      // Lanes 0..7: the crossing lane's keys in descending order.
      const uint32_t lw0 = (uint32_t)__builtin_amdgcn_readlane((int)wd0, wl);
      double mk = 0.0;
      uint32_t kk = 0u;
      if (l < 8) {
        kk = 2u * (lw0 + 3u - (uint32_t)(l >> 1)) + 1u - (uint32_t)(l & 1);
        const uint32_t word = s.hist[kk >> 1];
        const uint32_t cn = (kk & 1u) ? word >> 16 : word & 0xFFFFu;
        if (cn) mk = f(kk, cn);
      }
      const double kinc = wave_incl_scan_f64(mk);
      const unsigned long long khit = __ballot(l < 8 && base + kinc >= tau);
      const unsigned long long knz = __ballot(mk > 0.0);
      const int kl = khit ? __ffsll((long long)khit) - 1 : (knz ? 63 - __clzll((long long)knz) : 7);
      key = (uint32_t)__builtin_amdgcn_readlane((int)kk, kl);
      at = base + readlane_f64(kinc, kl);
      above = at - readlane_f64(mk, kl);
    }
    if (l == 0) {
      s.bc[0] = key;
      s.bd[0] = above;
      s.bd[1] = at;
    }
  }
  __syncthreads();
  PhFind r;
  r.key = s.bc[0];
  r.above = s.bd[0];
  r.at = s.bd[1];
  __syncthreads();   // bc / bd are written again by the next call
  return r;
}

enum { PH_OK = 0, PH_BAD = 1, PH_OVERFLOW = 2 };

// The row statistics from its histogram.  kmax / kmin: the row's largest and
// smallest keys, kcount_min: the lowest floor any wavefront counted from,
// skipped: elements left out of the histogram (block-uniform).
// Returns PH_BAD for NaN / +inf or a row of only -inf, PH_OVERFLOW when some
// count overflowed.
__device__ __forceinline__ int ph_stats(PhSmem& s, uint32_t kmax, uint32_t kmin, uint32_t kcount_min,
                                        uint32_t skipped, int V, const Mode& m, int k, RowStat& st) {
  using K = Key<uint16_t>;
  if (kmax >= K::POS_INF || kmin < K::NEG_INF || kmax <= K::NEG_INF) return PH_BAD;
  // Counted keys lie in [max(kmin, kcount_min), kmax]: only their segments are scanned.
  const int b_lo = (int)(max(kmin, kcount_min) >> 1) / PH_BLKW, b_hi = (int)(kmax >> 1) / PH_BLKW;
  st.zmax = K::value(kmax);
  st.c = LOG2E_F / m.T;
  st.zthr = -INFINITY;
  const float zmax = st.zmax, c = st.c;
  uint32_t kthr = K::NEG_INF + 1u;   // smallest key that can carry mass
  bool counted = false;
  if (k > 0 && k < V) {
    // Top-k: the k-th largest key (ties kept) from the counts.
    auto count_of = [](uint32_t, uint32_t cn) { return (double)cn; };
    uint32_t n = 0;
    ph_sums(s, count_of, b_lo, b_hi, n);
    if (n + skipped != (uint32_t)V) return PH_OVERFLOW;
    counted = true;
    const PhFind f = ph_find(s, count_of, (double)k);
    if (f.key != NONE && f.key > kthr) kthr = f.key;
  }
  // A key's mass: its count times its weight e = 2^((z - zmax) c).
  auto mass = [&](uint32_t key, uint32_t cn) -> double {
    if (key < kthr) return 0.0;
    return (double)cn * (double)ew(K::value(key), zmax, c);
  };
  if (kthr > K::NEG_INF + 1u) st.zthr = K::value(kthr);
  uint32_t n = 0;
  double S = ph_sums(s, mass, b_lo, b_hi, n);
  if (!counted && n + skipped != (uint32_t)V) return PH_OVERFLOW;
  if (m.tp < 1.0f) {
    if (m.tp <= 0.0f) {
      // Only the largest value (with its ties) survives.
      st.zthr = zmax;
      const uint32_t word = s.hist[kmax >> 1];
      S = (double)((kmax & 1u) ? word >> 16 : word & 0xFFFFu);
    } else {
      // The nucleus: the largest value whose mass at or above reaches top_p S.
      const PhFind f = ph_find(s, mass, (double)m.tp * S);
      if (f.key != NONE && f.at > 0.0) {
        st.zthr = fmaxf(st.zthr, K::value(f.key));
        S = f.at;
      }
    }
  }
  st.sp = (float)(1.0 / S);
  return PH_OK;
}

// Unit j of the calling thread (16-byte unit threadIdx.x + j * PH_NT of the
// row) through the row's buffer descriptor: one 32-bit offset per thread,
// the unit's position in the scalar offset, units past the row read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ph_rsrc(const uint4* row, int NU) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(row), (short)0, NU * 16, BUF_WORD3);
}
template <int AUX>
__device__ __forceinline__ uint4 ph_load(__amdgpu_buffer_rsrc_t r, int j) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)threadIdx.x * 16, j * PH_NT * 16, AUX);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Unit ui of a row (any thread, any unit) through the row's descriptor.
template <int AUX>
__device__ __forceinline__ uint4 ph_load_unit(__amdgpu_buffer_rsrc_t r, int ui) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, ui * 16, 0, AUX);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void ph_clear(PhSmem& s) {
  uint4* h = reinterpret_cast<uint4*>(&s.hist[0]);
  for (int i = threadIdx.x; i < PH_WORDS / 4; i += PH_NT) h[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Block max / min of the packed key extremes (both halves), in one round trip.
__device__ __forceinline__ void ph_extremes(PhSmem& s, uint32_t kmax2, uint32_t kmin2, uint32_t& kmax, uint32_t& kmin) {
  uint32_t mx = max(kmax2 & 0xFFFFu, kmax2 >> 16), mn = min(kmin2 & 0xFFFFu, kmin2 >> 16);
  mx = wave_max_dpp(mx);
  mn = wave_min_dpp(mn);
  if ((threadIdx.x & 63) == 0) {
    s.red[threadIdx.x >> 6] = mx;
    s.red[PH_NW + (threadIdx.x >> 6)] = mn;
  }
  __syncthreads();
  kmax = 0;
  kmin = 0xFFFFu;
  for (int x = 0; x < PH_NW; ++x) {
    kmax = max(kmax, s.red[x]);
    kmin = min(kmin, s.red[PH_NW + x]);
  }
  __syncthreads();
}

// One streaming pass over a row (resource rr, NU units) into the histogram,
// then the row's statistics (ph_stats): the count pass of pair_hist_one.
// With record, each unit's bucket (ph_bucket) of its largest value and the
// floors they start from are kept in s.umax / s.uref for a list of the units
// that can reach the nucleus.  Returns ph_stats' result; ends with a block
// barrier, after which the histogram may be reused.
__device__ __forceinline__ int ph_row_pass(PhSmem& s, __amdgpu_buffer_rsrc_t rr, int NU, int fb, float cT, float binv,
                                           bool filter_k, bool record, int V, const Mode& m, int k, RowStat& st) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  ph_clear(s);
  __syncthreads();
  uint32_t kmax2 = 0u, kmin2 = 0xFFFFFFFFu, skipped = 0, kf_first = 0xFFFFFFFFu;
  for (int j0 = 0; j0 < PH_UPT; j0 += PH_INFLIGHT) {
    uint4 u[PH_INFLIGHT];
#pragma unroll
    for (int r = 0; r < PH_INFLIGHT; ++r) u[r] = ph_load<0>(rr, j0 + r);
    uint32_t umx[PH_INFLIGHT / 2];   // the units' largest keys, two per word
    uint32_t bmin2 = 0xFFFFFFFFu;    // the batch's smallest keys
#pragma unroll
    for (int r = 0; r < PH_INFLIGHT; ++r) {
      const int ui = (j0 + r) * PH_NT + (int)threadIdx.x;
      uint32_t mx = 0u, mn = 0xFFFFFFFFu;
      if (ui < NU) {
        ph_keys_extremes_unit(u[r], mx, mn);
        kmax2 = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(ph_u16x2, kmax2),
                                                                       __builtin_bit_cast(ph_u16x2, mx)));
        bmin2 = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(ph_u16x2, bmin2),
                                                                       __builtin_bit_cast(ph_u16x2, mn)));
      }
      const uint32_t m1 = max(mx & 0xFFFFu, mx >> 16);
      umx[r >> 1] = (r & 1) ? umx[r >> 1] | (m1 << 16) : m1;
    }
    // The floor: the value (fb + 2) / c below the wavefront's running
    // maximum, also the origin of the target units' buckets (in steps of
    // 1/254 of that distance).
    const uint32_t wmax = wave_max_dpp(max(kmax2 & 0xFFFFu, kmax2 >> 16));
    float zf = -INFINITY;
    if (wmax > Key<uint16_t>::NEG_INF && wmax < Key<uint16_t>::POS_INF)
      zf = Key<uint16_t>::value(wmax) - (float)(fb + 2) / cT;
    uint32_t kfloor = 0u;
    if (!filter_k && zf > -INFINITY) {
      // Smallest bf16 key whose value is at least zf.
      const uint32_t bits = __float_as_uint(zf);
      const uint32_t b16 = zf >= 0.0f ? (bits + 0xFFFFu) >> 16 : bits >> 16;
      kfloor = Key<uint16_t>::of_bits(b16);
    }
    if (record) {
      if (lane == 0) s.uref[j0 / PH_INFLIGHT][wave] = zf;
#pragma unroll
      for (int r = 0; r < PH_INFLIGHT; ++r) {
        const int ui = (j0 + r) * PH_NT + (int)threadIdx.x;
        const uint32_t m1 = (r & 1) ? umx[r >> 1] >> 16 : umx[r >> 1] & 0xFFFFu;
        if (ui < NU) s.umax[ui] = (uint8_t)ph_bucket(Key<uint16_t>::value(m1), zf, binv);
      }
    }
    kf_first = min(kf_first, kfloor);
    kmin2 = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(ph_u16x2, kmin2),
                                                                   __builtin_bit_cast(ph_u16x2, bmin2)));
#pragma unroll
    for (int r = 0; r < PH_INFLIGHT; ++r)
      if ((j0 + r) * PH_NT + (int)threadIdx.x < NU) ph_add_keys(s.hist, &s.spare[lane], u[r], kfloor, skipped);
  }
  skipped = (uint32_t)__builtin_amdgcn_readfirstlane((int)skipped);
  if (lane == 0) {
    s.red[2 * PH_NW + wave] = skipped;
    s.red[4 * PH_NW + wave] = kf_first;
  }
  uint32_t kmax, kmin;
  ph_extremes(s, kmax2, kmin2, kmax, kmin);   // its barriers also close the counting
  skipped = 0;
  uint32_t kcount_min = 0xFFFFFFFFu;
  for (int x = 0; x < PH_NW; ++x) {
    skipped += s.red[2 * PH_NW + x];
    kcount_min = min(kcount_min, s.red[4 * PH_NW + x]);
  }
  RowStat r{};
  const int bad = ph_stats(s, kmax, kmin, kcount_min, skipped, V, m, k, r);
  st = r;
  __syncthreads();   // the statistics' last histogram reads before the histogram is reused
  return bad;
}

// One (sequence b, position i) pair by the whole workgroup.  Thread t's
// units of a row are t + j * PH_NT, j < PH_UPT (tile j).
__device__ __forceinline__ void pair_hist_one(const Args& a, int b, int i, PhSmem& s) {
  using T = PT<uint16_t, true>;
  const int G1 = a.G + 1;
  const Mode m = seq_mode(a, b);
  if (m.mode != MODE_DENSE || i > m.g) return;
  const bool resid = i < m.g;
  const int V = a.V;
  const int NU = V / 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = a.topk ? a.topk[b] : 0;
  const uint4* gp = reinterpret_cast<const uint4*>(row_ptr<uint16_t>(a, b, true, i));
  const uint4* gq = resid ? reinterpret_cast<const uint4*>(row_ptr<uint16_t>(a, b, false, i)) : gp;
  const __amdgpu_buffer_rsrc_t rp = ph_rsrc(gp, NU), rq = ph_rsrc(gq, NU);
  PosRec* rec = a.pos + (size_t)b * G1 + i;
  const int fb = a.fixbits;
  const float cT = LOG2E_F / m.T;
  const float binv = 254.0f * cT / (float)(fb + 2);   // buckets per unit of value
  const bool filter_k = k > 0 && k < V;
  int bad = 0;
  // The draft token and the patterns of its two logits, for the record
  // written at the end: fetched now, so their two dependent round trips
  // overlap the other wavefronts' row passes instead of ending the pair.
  if (threadIdx.x == 0) {
    const int x = resid ? a.draft[(size_t)b * a.G + i] : -1;
    uint32_t raw = 0u;
    if (x >= 0 && x < V) {
      const uint16_t* pr = reinterpret_cast<const uint16_t*>(gp);
      const uint16_t* qr = reinterpret_cast<const uint16_t*>(gq);
      raw = (uint32_t)pr[x] | ((uint32_t)qr[x] << 16);
    }
    s.rx[0] = (uint32_t)x;
    s.rx[1] = raw;
  }

  // Row 0, the draft row, then row 1, the target row: one streaming pass
  // each, counting the elements at or above a floor into the histogram.
  // The floor: elements whose weight is below 2^-(fb+2) of the maximum's
  // (fb = 62 - bits(V + 1), at least 44 for the rows taken here) together hold
  // less than V 2^-46 <= 2^-29 of the mass, so they are left out of S and can
  // never be in a nucleus (a float top_p below 1 is at most 1 - 2^-24).  Top-k
  // rows count every element: the k-th may lie anywhere.  Each wavefront takes
  // its floor from its own running maximum, never above the row's.  The target
  // pass also notes the top byte of each unit's largest key.
  RowStat sq{INFINITY, 0.0f, 0.0f, 0.0f}, sp{};
  for (int row = resid ? 0 : 1; row < 2; ++row) {
    RowStat st{};
    bad |= ph_row_pass(s, row == 0 ? rq : rp, NU, fb, cT, binv, filter_k, row == 1, V, m, k, st);
    if (row == 0) sq = st;
    else sp = st;
    if (bad) break;
  }
  if (bad) {
    // Invalid data, or a count that overflowed: the finisher then takes the
    // sequence through its multi-pass procedure (REC_REDO) or reports it
    // invalid.
    if (threadIdx.x == 0) {
      rec->bad = (bad & PH_BAD) ? 1u : REC_REDO;
      rec->tok = -1;
    }
    return;
  }

  // The units read again: those whose largest target value can reach the
  // target's nucleus threshold (elsewhere p = 0, so neither the overlap nor a
  // draw weight has a term), listed in ascending unit order in the
  // histogram's memory, free once both rows' statistics are known.  Every
  // list entry is then one thread's work, so a wavefront computes only units
  // that are needed, however few and however scattered.
  uint16_t* list = reinterpret_cast<uint16_t*>(s.hist);
  uint32_t* lcnt = s.hist + PH_WORDS / 2;   // per-(tile, wavefront) counts, then their offsets
  uint32_t nd_bits = 0;
#pragma unroll 1
  for (int j = 0; j < PH_UPT; ++j) {
    const int ui = j * PH_NT + (int)threadIdx.x;
    const bool nd = ui < NU && (uint32_t)s.umax[ui] >= ph_bucket(sp.zthr, s.uref[j / PH_INFLIGHT][wave], binv);
    const unsigned long long bal = __ballot(nd);
    nd_bits |= nd ? 1u << j : 0u;
    if (lane == 0) lcnt[j * PH_NW + wave] = (uint32_t)__popcll(bal);
  }
  __syncthreads();
  if (wave == 0) {
    // Exclusive prefix of the (tile, wavefront) counts in that order, four per lane.
    uint32_t c4[4], sum4 = 0;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      c4[x] = lcnt[4 * lane + x];
      sum4 += c4[x];
    }
    const uint32_t inc = wave_incl_scan_dpp(sum4);
    uint32_t run = inc - sum4;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      lcnt[4 * lane + x] = run;
      run += c4[x];
    }
    if (lane == 63) s.bc[1] = inc;
  }
  __syncthreads();
  const int nlist = (int)s.bc[1];
#pragma unroll 1
  for (int j = 0; j < PH_UPT; ++j) {
    const bool nd = (nd_bits >> j) & 1u;
    const unsigned long long bal = __ballot(nd);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (nd) list[lcnt[j * PH_NW + wave] + below] = (uint16_t)(j * PH_NT + (int)threadIdx.x);
  }
  __syncthreads();

  // Overlap and per-(chunk, wavefront) draw-weight sums over the list, a
  // chunk being PH_NT consecutive entries: the residual max(0, p - q), or p
  // at the bonus position and when the residual is zero (there the draft's
  // threshold is +inf, so q = 0 everywhere and the same code sums p).
  const int nch = max(1, (nlist + PH_NT - 1) / PH_NT);
  double al = 0.0;
  RowStat sqw = sq;   // the draft's statistics as the draw uses them (q = 0 once the residual is empty)
  auto weights_pass = [&](bool use_q) {
    for (int c0 = 0; c0 < nch; c0 += PH_WINFLIGHT) {
      uint4 up[PH_WINFLIGHT], uq[PH_WINFLIGHT];
      bool nd[PH_WINFLIGHT];
#pragma unroll
      for (int r = 0; r < PH_WINFLIGHT; ++r) {
        const int le = (c0 + r) * PH_NT + (int)threadIdx.x;
        nd[r] = le < nlist;
        up[r] = make_uint4(0u, 0u, 0u, 0u);
        uq[r] = up[r];
        if (nd[r]) {
          const int ui = list[le];
          up[r] = ph_load_unit<BUF_NT>(rp, ui);
          if (use_q) uq[r] = ph_load_unit<BUF_NT>(rq, ui);
        }
      }
#pragma unroll
      for (int r = 0; r < PH_WINFLIGHT; ++r) {
        if (c0 + r >= nch) break;
        float rs = 0.0f, av = 0.0f;
        if (nd[r]) {
          const uint32_t pw[4] = {up[r].x, up[r].y, up[r].z, up[r].w}, qw[4] = {uq[r].x, uq[r].y, uq[r].z, uq[r].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t pr = e & 1 ? pw[e >> 1] >> 16 : pw[e >> 1] & 0xFFFFu;
            const uint32_t qr = e & 1 ? qw[e >> 1] >> 16 : qw[e >> 1] & 0xFFFFu;
            const float pv = pprob(sp, T::val(pr)), qv = pprob(sqw, T::val(qr));
            av += fminf(pv, qv);
            rs += fmaxf(pv - qv, 0.0f);
          }
        }
        al += (double)av;
        const double wsum = wave_sum_dpp((double)rs);
        if (lane == 0) s.part[c0 + r][wave] = wsum;
      }
    }
  };
  weights_pass(resid);
  __syncthreads();
  const double u = (double)a.u[(size_t)b * G1 + a.G];
  auto locate = [&]() {
    if (threadIdx.x < 64) {
      double tt = 0.0;
      if (lane < nch) {
#pragma unroll
        for (int w = 0; w < PH_NW; ++w) tt += s.part[lane][w];
      }
      const double incl = wave_incl_scan_f64(tt);
      const double Z = readlane_f64(incl, 63);
      const double target = u * Z;
      const unsigned long long hit = __ballot(lane < nch && incl > target);
      const int j = hit ? __ffsll((long long)hit) - 1 : nch - 1;
      if (lane == j) {
        s.bc[0] = (uint32_t)j;
        s.bd[0] = incl - tt;
      }
      if (lane == 0) s.bd[1] = Z > 0.0 ? target : -1.0;
    }
    __syncthreads();
  };
  locate();
  bool use_q = resid;
  if (resid && !(s.bd[1] >= 0.0)) {
    // Zero residual mass (p == q after processing): draw from p itself.  The
    // overlap already summed stays (q = 0 adds nothing to it).
    __syncthreads();
    sqw.zthr = INFINITY;
    const double al0 = al;
    weights_pass(false);
    al = al0;
    __syncthreads();
    locate();
    use_q = false;
  }
  const int tj = (int)s.bc[0];
  const double base = s.bd[0], target = s.bd[1];
  // Examine the crossing chunk's units again, in ascending id.
  uint32_t hitpos = 0xFFFFFFFFu, lastpos = 0;
  {
    const int le = tj * PH_NT + (int)threadIdx.x;
    const bool has = le < nlist;
    const int ui = has ? (int)list[le] : 0;
    const uint4 up = ph_load_unit<0>(rp, ui);
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = 0.0f;
    float r = 0.0f;
    const uint4 uq = use_q ? ph_load_unit<0>(rq, ui) : up;
    if (has) {
      T::each(up, [&](int e, uint32_t raw) { w[e] = pprob(sp, T::val(raw)); });
      T::each(uq, [&](int e, uint32_t raw) {
        w[e] = fmaxf(w[e] - pprob(sqw, T::val(raw)), 0.0f);
        r += w[e];
      });
    }
    const double rd = (double)r;
    const double incl = wave_incl_scan_f64(rd);
    double cum = base;
    for (int w2 = 0; w2 < wave; ++w2) cum += s.part[tj][w2];
    cum += incl - rd;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cum += (double)w[e];
      const uint32_t idx = (uint32_t)(ui * 8 + e);
      if (hitpos == 0xFFFFFFFFu && w[e] > 0.0f && cum > target) hitpos = idx;
      if (w[e] > 0.0f) lastpos = idx + 1u;
    }
  }
  hitpos = pb_min<PH_NT>(hitpos, s.red);
  int tok = (int)hitpos;
  if (hitpos == 0xFFFFFFFFu) tok = (int)pb_max<PH_NT>(lastpos, s.red) - 1;   // rounding left no crossing
  if (resid) {
    al = wave_sum_dpp(al);
    __syncthreads();
    if (lane == 0) s.part[0][wave] = al;
    __syncthreads();
    double tot = 0.0;
    for (int w2 = 0; w2 < PH_NW; ++w2) tot += s.part[0][w2];
    al = tot;
  }
  if (threadIdx.x == 0) {
    const int x = (int)s.rx[0];
    double pxv = 0.0, qxv = 0.0;
    if (x >= 0 && x < V) {
      pxv = (double)pprob(sp, T::val(s.rx[1] & 0xFFFFu));
      qxv = (double)pprob(sq, T::val(s.rx[1] >> 16));
    }
    rec->px = pxv;
    rec->qx = qxv;
    rec->alpha = al;
    rec->tok = tok;
    rec->bad = 0u;
  }
}

// The dense pairs, one workgroup per CU, in the order and with the shared
// work counter of the streamed pair variant: workgroup w starts with pair w,
// and a workgroup that has finished takes the next unstarted pair.
__global__ __launch_bounds__(PH_NT) void pair_hist_kernel(Args a) {
  // Static, so the histogram's LDS addresses are constants the count pass
  // need not add.
  __shared__ __align__(16) PhSmem s;
  const int G1 = a.G + 1;
  const uint32_t npairs = (uint32_t)a.B * (uint32_t)G1;
  const bool direct = a.all_dense != 0;
  const uint32_t nf = direct ? npairs : min(a.dense_count[0], npairs);
  const uint32_t nd = direct ? npairs : min(nf + a.dense_count[1], npairs);
  const uint32_t nlead = (uint32_t)a.B * (uint32_t)a.G;
  uint32_t t = blockIdx.x;
  while (t < nd) {
    int pid;
    if (direct) {
      pid = t < nlead ? (int)((t / (uint32_t)a.G) * (uint32_t)G1 + t % (uint32_t)a.G)
                      : (int)((t - nlead) * (uint32_t)G1 + (uint32_t)a.G);
    } else {
      const uint32_t idx = t < nf ? t : npairs - 1u - (t - nf);
      pid = a.dense_list[idx];
    }
    if (pid >= 0 && (uint32_t)pid < npairs) {
      const int b = pid / G1;
      pair_hist_one(a, b, pid - b * G1, s);
    }
    __syncthreads();
    if (threadIdx.x == 0) s.next_pair = gridDim.x + atomicAdd(&a.dense_count[2], 1u);
    __syncthreads();
    t = s.next_pair;
  }
}

// Calls that may hold both dense and streamed (top-k, argmax) sequences on
// this variant: the select units and the dense pairs in one launch, after a
// launch that only lists the dense pairs.  One workgroup per CU first takes
// groups of PH_NW consecutive select units (a wavefront each) from a
// workspace counter, then dense pairs from the pair counter, every one
// claimed.  So the CUs whose groups hold streamed rows (a few, since a
// group covers consecutive rows of one or two sequences) stream them while
// the others start on the pairs, and the pairs' tail no longer waits for a
// separate select launch.  When the listing found no dense pair, every
// wavefront instead takes single units from the counter, so the streamed
// rows spread over all CUs as in the select kernel.  Both counters are
// cleared by the finisher.
__global__ __launch_bounds__(PH_NT) void mixed_hist_kernel(Args a) {
  __shared__ __align__(16) union {
    PhSmem ph;
    WaveSmem w[PH_NW];
  } sm;
  __shared__ uint32_t claim;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const long long units = (long long)a.B * a.RS * a.NP;
  const long long ngroups = (units + PH_NW - 1) / PH_NW;
  const int G1 = a.G + 1;
  const uint32_t npairs = (uint32_t)a.B * (uint32_t)G1;
  const uint32_t nf = min(a.dense_count[0], npairs);
  const uint32_t nd = min(nf + a.dense_count[1], npairs);
  if (nd == 0) {
    for (;;) {
      uint32_t u = 0;
      if ((threadIdx.x & 63) == 0) u = atomicAdd(&a.dense_count[3], 1u);
      u = (uint32_t)__builtin_amdgcn_readlane((int)u, 0);
      if ((long long)u >= units) return;
      select_unit<uint16_t, true>(a, (long long)u, sm.w[wave]);
      __builtin_amdgcn_s_setprio(0);
    }
  }
  for (;;) {
    __syncthreads();   // every wavefront has read the last claim
    if (threadIdx.x == 0) claim = atomicAdd(&a.dense_count[3], 1u);
    __syncthreads();
    const uint32_t g = claim;
    if ((long long)g >= ngroups) break;
    select_unit<uint16_t, true>(a, (long long)g * PH_NW + wave, sm.w[wave]);
    __builtin_amdgcn_s_setprio(0);
  }
  __syncthreads();   // the select units' LDS, and the last claim, are done with
  if (threadIdx.x == 0) claim = atomicAdd(&a.dense_count[2], 1u);
  __syncthreads();
  uint32_t t = claim;
  while (t < nd) {
    const uint32_t idx = t < nf ? t : npairs - 1u - (t - nf);
    const int pid = a.dense_list[idx];
    if (pid >= 0 && (uint32_t)pid < npairs) {
      const int b = pid / G1;
      pair_hist_one(a, b, pid - b * G1, sm.ph);
    }
    __syncthreads();
    if (threadIdx.x == 0) claim = atomicAdd(&a.dense_count[2], 1u);
    __syncthreads();
    t = claim;
  }
}

}  // namespace sv
