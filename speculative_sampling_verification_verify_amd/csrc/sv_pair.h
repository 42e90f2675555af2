// Pair-parallel verify of the dense sequences (temperature > 0 and no top-k
// up to KMAX_SPARSE: unfiltered, large top-k and top-p rows).
//
// One workgroup per (sequence, position i <= gamma_b) owns the target row p_i
// and, for i < gamma_b, the draft row q_i; every row belongs to exactly one
// workgroup.  Rows of up to 64 KB are read from HBM once into LDS and every
// later pass runs on chip (short unfiltered rows stay in the wavefront's
// registers instead: pair_small); longer rows are streamed from global
// memory on each pass (the re-reads of one workgroup's rows hit L2 / MALL).
// Per row:
//   * validity and the maximum logit;
//   * the top-k threshold key (radix select) when KMAX_SPARSE < k < V;
//   * the normaliser and, for top-p, the nucleus cut by a mass-weighted radix
//     select on 64-bit fixed-point masses (independent of summation order);
//     streamed rows first bin the masses by value in the same pass as the
//     normaliser, so only the crossing bin's keys need exact resolution.
// Per pair: p_i(x_i), q_i(x_i), the overlap alpha_i = sum min(p_i, q_i)
// ("Fast Inference from Transformers via Speculative Decoding", mtandhj.com
// summary, "How to choose gamma") and the draw at u from the residual
// max(0, p_i - q_i) (same summary, "Speculative Sampling: theoretical basis"),
// or from p_{gamma_b} at the bonus position ("Speculative Decoding: the art
// of guessing well", "Speculative sampling"), by an inverse CDF in ascending
// vocabulary id ("Sampling with shared noise" on the same page).  The overlap
// pass keeps one residual sum per (tile, wavefront); the crossing tile is
// then found from those sums and only that tile is examined again.  The
// finisher runs the acceptance test and picks the draw at the first
// rejection.
#pragma once

#include <type_traits>

#include "sv_common.h"

namespace sv {

#ifndef SV_PAIR_UNR
#define SV_PAIR_UNR 2      // units in flight per thread on a streamed pass over one row
#endif
#ifndef SV_PAIR_UNR1
#define SV_PAIR_UNR1 2     // units of each row in flight per thread on the first streamed pass
#endif
// Streamed-row workgroups are kept to 64 VGPRs so that two 1024-thread
// workgroups share a CU (8 waves per SIMD): their passes are latency-bound,
// and two resident workgroups beat one with more loads in flight.
constexpr int PAIR_STREAM_WAVES_PER_EU = 8;

constexpr int PAIR_LDS_ROW_MAX = 65536;   // bytes of one row held in LDS
constexpr int PAIR_LDS_UR = 4;            // units per row whose loads a thread issues together (rows in LDS)
constexpr int PAIR_MAXTILE = 64;          // residual tiles (NTP units each) per row
constexpr int PAIR_NBIN = 2048;           // value bins of the streamed nucleus histogram
constexpr int PAIR_NCAP = 2048;           // keys of the crossing bin gathered in LDS
constexpr float LOG2E_F = 1.4426950408889634f;

template <int NTP>
struct PairSmem {
  union {
    unsigned long long h64[256];
    uint32_t h32[512];
  } hist;
  double part[PAIR_MAXTILE][NTP / 64];   // draw-weight sum per (tile, wavefront)
  double red_d[NTP / 64];
  unsigned long long red_u64[NTP / 64];
  uint32_t red_u[3 * (NTP / 64)];
  uint32_t bc[8];
  double bd[2];
  int xd;   // thread 0's draft token of the pair, fetched at its start
};
struct PairStream {   // extra LDS of the streamed variant
  unsigned long long vh[PAIR_NBIN];
  uint32_t keys[PAIR_NCAP];
  uint32_t ncol;
};
struct PairNoStream {};
template <bool LDSR>
using PairExtra = typename std::conditional<LDSR, PairNoStream, PairStream>::type;

// ---- block reductions over NTP threads --------------------------------------
// Each wave reduces in registers, lane 0 of each wave parks the wave's value
// in scr, and every wave then combines the NTP / 64 parked values
// lane-parallel, so all threads hold the same result.
template <int NTP>
__device__ __forceinline__ uint32_t pb_max(uint32_t v, uint32_t* scr) {
  v = wave_max_dpp(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scr[threadIdx.x >> 6] = v;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  return wave_max_dpp(lane < NTP / 64 ? scr[lane] : 0u);
}
// Three maxima in one LDS round trip.
template <int NTP>
__device__ __forceinline__ void pb_max3(uint32_t& a, uint32_t& b, uint32_t& c, uint32_t* scr) {
  constexpr int NW = NTP / 64;
  a = wave_max_dpp(a);
  b = wave_max_dpp(b);
  c = wave_max_dpp(c);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    scr[threadIdx.x >> 6] = a;
    scr[NW + (threadIdx.x >> 6)] = b;
    scr[2 * NW + (threadIdx.x >> 6)] = c;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  a = wave_max_dpp(lane < NW ? scr[lane] : 0u);
  b = wave_max_dpp(lane < NW ? scr[NW + lane] : 0u);
  c = wave_max_dpp(lane < NW ? scr[2 * NW + lane] : 0u);
}
template <int NTP>
__device__ __forceinline__ uint32_t pb_min(uint32_t v, uint32_t* scr) {
  v = wave_min_dpp(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scr[threadIdx.x >> 6] = v;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  return wave_min_dpp(lane < NTP / 64 ? scr[lane] : 0xFFFFFFFFu);
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o, 64);
    v += ((unsigned long long)hi << 32) | lo;
  }
  return v;
}
template <int NTP>
__device__ __forceinline__ unsigned long long pb_sum_u64(unsigned long long v, unsigned long long* scr) {
  v = wave_sum_u64(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scr[threadIdx.x >> 6] = v;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  return wave_sum_u64(lane < NTP / 64 ? scr[lane] : 0ull);
}
template <int NTP>
__device__ __forceinline__ double pb_sum_f64(double v, double* scr) {
  v = wave_sum_dpp(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scr[threadIdx.x >> 6] = v;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  return wave_sum_dpp(lane < NTP / 64 ? scr[lane] : 0.0);
}

// ---- element access -----------------------------------------------------------
// A row is an array of units: 16-byte vectors when the row allows, else
// single elements.  raw = an element's bit pattern (bf16 in the low half).
template <typename ET, bool VECTOR>
struct PT {
  static constexpr int E = VECTOR ? 16 / (int)sizeof(ET) : 1;
  using U = typename std::conditional<VECTOR, uint4, ET>::type;
  template <class F>
  __device__ __forceinline__ static void each(const U& u, F fn) {
    if constexpr (VECTOR) {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      if constexpr (sizeof(ET) == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          fn(2 * j, w[j] & 0xFFFFu);
          fn(2 * j + 1, w[j] >> 16);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) fn(j, w[j]);
      }
    } else if constexpr (sizeof(ET) == 2) {
      fn(0, (uint32_t)u);
    } else {
      fn(0, __float_as_uint(u));
    }
  }
  __device__ __forceinline__ static float val(uint32_t raw) {
    if constexpr (sizeof(ET) == 2) return __uint_as_float(raw << 16);
    else return __uint_as_float(raw);
  }
  __device__ __forceinline__ static uint32_t key(uint32_t raw) { return Key<ET>::of_bits(raw); }
  __device__ __forceinline__ static uint32_t raw_at(const U* row, int idx) {
    const ET* r = reinterpret_cast<const ET*>(row);
    if constexpr (sizeof(ET) == 2) return (uint32_t)r[idx];
    else return __float_as_uint(r[idx]);
  }
};

// Unnormalised weight e(z) = 2^((z - zmax) * c), c = log2(e) / T: one
// instruction sequence wherever a row's weights are formed, so sums, bins
// and probabilities agree element by element.
__device__ __forceinline__ float ew(float z, float zmax, float c) { return __builtin_amdgcn_exp2f((z - zmax) * c); }

// floor(e * 2^fb) as a 64-bit integer (e in [0, 1], fb <= 62): e * 2^fb is
// exact in fp32; its high and low 32-bit halves are split off exactly.
__device__ __forceinline__ unsigned long long fixq(float e, float two_fb, float two_fb32) {
  const float t = e * two_fb;
  const float hi = floorf(e * two_fb32);
  const float lo = fmaf(-hi, 4294967296.0f, t);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}
// Value bin of a weight: 32 bins per binade, bin 0 holding e = 1.  Bins are
// monotone (non-increasing) in the logit, so a bin is a run of adjacent keys.
__device__ __forceinline__ int vbin(float e) { return (int)((0x3F800000u - __float_as_uint(e)) >> 18); }

// Mass-weighted radix select: the largest key t among the fed keys with
// above + mass(fed keys >= t) >= tau; *mass_out = above + mass(fed keys >= t).
// feed(fn) calls fn(key, f) for the calling thread's share (f: fixed-point
// mass).  Returns 0 when the fed mass never reaches tau.
template <int LEVELS, int NTP, class Feed>
__device__ __forceinline__ uint32_t mass_select(Feed feed, double tau, unsigned long long above,
                                                unsigned long long* h64, uint32_t* bc, unsigned long long* mass_out) {
  uint32_t prefix = 0, pmask = 0;
  for (int lvl = 0; lvl < LEVELS; ++lvl) {
    const int shift = 8 * (LEVELS - 1 - lvl);
    for (int i = threadIdx.x; i < 256; i += NTP) h64[i] = 0ull;
    __syncthreads();
    feed([&](uint32_t uk, unsigned long long f) {
      if (f && (uk & pmask) == prefix) atomicAdd(&h64[(uk >> shift) & 255u], f);
    });
    __syncthreads();
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const int top = 255 - 4 * lane;
      const unsigned long long c0 = h64[top], c1 = h64[top - 1], c2 = h64[top - 2], c3 = h64[top - 3];
      const unsigned long long sum = c0 + c1 + c2 + c3;
      unsigned long long incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t ulo = (uint32_t)__shfl_up((int)(uint32_t)incl, o, 64);
        const uint32_t uhi = (uint32_t)__shfl_up((int)(uint32_t)(incl >> 32), o, 64);
        if (lane >= o) incl += ((unsigned long long)uhi << 32) | ulo;
      }
      const unsigned long long excl = incl - sum;
      // Mass grows bin by bin from the top: the first lane whose last bin
      // reaches tau holds the crossing bin.
      const unsigned long long any = __ballot((double)(above + incl) >= tau);
      const int first = any ? __ffsll((long long)any) - 1 : -1;
      if (lane == first) {
        uint32_t d;
        unsigned long long ab;
        if ((double)(above + excl + c0) >= tau) {
          d = top; ab = above + excl;
        } else if ((double)(above + excl + c0 + c1) >= tau) {
          d = top - 1; ab = above + excl + c0;
        } else if ((double)(above + excl + c0 + c1 + c2) >= tau) {
          d = top - 2; ab = above + excl + c0 + c1;
        } else {
          d = top - 3; ab = above + excl + c0 + c1 + c2;
        }
        const unsigned long long at = ab + h64[d];
        bc[0] = d;
        bc[1] = (uint32_t)ab;
        bc[2] = (uint32_t)(ab >> 32);
        bc[3] = (uint32_t)at;
        bc[4] = (uint32_t)(at >> 32);
      }
      if (lane == 0 && any == 0ull) bc[0] = NONE;
    }
    __syncthreads();
    const uint32_t d = bc[0];
    const unsigned long long ab = ((unsigned long long)bc[2] << 32) | bc[1];
    const unsigned long long at = ((unsigned long long)bc[4] << 32) | bc[3];
    __syncthreads();
    if (d == NONE) {
      *mass_out = 0;
      return 0;
    }
    prefix |= d << shift;
    pmask |= 255u << shift;
    above = ab;
    if (lvl == LEVELS - 1) *mass_out = at;
  }
  return prefix;
}

// Processed distribution of one row: p(z) = (z >= zthr) ? e(z) * sp : 0.
// Keys and values order the same way (+0 and -0 share a key), so the value
// test equals the key test key(z) >= thr.
struct RowStat {
  float zthr, zmax, c, sp;
};

template <typename ET>
__device__ __forceinline__ uint32_t key_of_value(float z) {
  if constexpr (sizeof(ET) == 2) return Key<ET>::of_bits(__float_as_uint(z) >> 16);
  else return Key<ET>::of_bits(__float_as_uint(z));
}

template <typename ET>
__device__ __forceinline__ float key_floor_value(uint32_t thr) {
  return thr <= Key<ET>::NEG_INF ? -INFINITY : Key<ET>::value(thr);
}

// Calls fn(unit) for every unit of the calling thread; streamed rows keep
// UNR loads in flight.
template <typename ET, int NTP, bool VECTOR, bool LDSR, class F>
__device__ __forceinline__ void row_units(const typename PT<ET, VECTOR>::U* src, int NU, F fn) {
  using T = PT<ET, VECTOR>;
  constexpr int UNR = LDSR ? 2 : SV_PAIR_UNR;
  int ui = threadIdx.x;
  for (; ui + (UNR - 1) * NTP < NU; ui += UNR * NTP) {
    typename T::U u[UNR];
#pragma unroll
    for (int r = 0; r < UNR; ++r) u[r] = src[ui + r * NTP];
#pragma unroll
    for (int r = 0; r < UNR; ++r) fn(u[r]);
  }
  for (; ui < NU; ui += NTP) fn(src[ui]);
}
// Calls fn(raw) for every element of the calling thread's units.
template <typename ET, int NTP, bool VECTOR, bool LDSR, class F>
__device__ __forceinline__ void row_each(const typename PT<ET, VECTOR>::U* src, int NU, F fn) {
  using T = PT<ET, VECTOR>;
  row_units<ET, NTP, VECTOR, LDSR>(src, NU, [&](const typename T::U& u) {
    T::each(u, [&](int, uint32_t raw) { fn(raw); });
  });
}

// Row statistics.  src: the row (LDS or global), NU units; zmax: its largest
// logit.
template <typename ET, int NTP, bool VECTOR, bool LDSR>
__device__ __forceinline__ RowStat row_stats(const typename PT<ET, VECTOR>::U* src, int NU, float zmax,
                                             const Args& a, const Mode& m, int k, PairSmem<NTP>& s,
                                             PairExtra<LDSR>& ps) {
  using T = PT<ET, VECTOR>;
  constexpr int LEVELS = Key<ET>::LEVELS;
  RowStat st;
  st.zmax = zmax;
  st.c = LOG2E_F / m.T;
  st.zthr = -INFINITY;
  const float c = st.c;
  const int fb = a.fixbits;
  const float two_fb = ldexpf(1.0f, fb), two_fb32 = ldexpf(1.0f, fb - 32);
  auto each = [&](auto fn) { row_each<ET, NTP, VECTOR, LDSR>(src, NU, fn); };
  if (k > 0 && k < a.V) {   // dense sequences reach here only with k > KMAX_SPARSE
    const uint32_t kth = block_kth_largest<LEVELS, NTP>(
        [&](auto fn) { each([&](uint32_t raw) { fn(T::key(raw)); }); }, (uint32_t)k, s.hist.h32, s.bc);
    st.zthr = key_floor_value<ET>(kth ? kth : 1u);
  }
  const float zthr = st.zthr;
  if (!(m.tp < 1.0f)) {
    // No nucleus cut: S = sum of e over the kept elements.
    double sl = 0.0;
    row_units<ET, NTP, VECTOR, LDSR>(src, NU, [&](const typename T::U& u) {
      float us = 0.0f;
      T::each(u, [&](int, uint32_t raw) {
        const float z = T::val(raw);
        us += z >= zthr ? ew(z, zmax, c) : 0.0f;
      });
      sl += (double)us;
    });
    st.sp = (float)(1.0 / pb_sum_f64<NTP>(sl, s.red_d));
    return st;
  }
  if (m.tp <= 0.0f) {
    // Only the maximal logit (with its ties) survives.
    unsigned long long cl = 0;
    each([&](uint32_t raw) { cl += T::val(raw) == zmax ? 1ull : 0ull; });
    const unsigned long long cnt = pb_sum_u64<NTP>(cl, s.red_u64);
    st.zthr = zmax;
    st.sp = (float)(1.0 / (double)cnt);
    return st;
  }
  auto fx = [&](float z) { return fixq(ew(z, zmax, c), two_fb, two_fb32); };
  unsigned long long S, mass = 0;
  uint32_t tstar = 0;
  if constexpr (LDSR) {
    unsigned long long sl = 0;
    each([&](uint32_t raw) {
      const float z = T::val(raw);
      if (z >= zthr) sl += fx(z);
    });
    S = pb_sum_u64<NTP>(sl, s.red_u64);
    tstar = mass_select<LEVELS, NTP>(
        [&](auto fn) {
          each([&](uint32_t raw) {
            const float z = T::val(raw);
            if (z >= zthr) fn(T::key(raw), fx(z));
          });
        },
        (double)m.tp * (double)S, 0ull, s.hist.h64, s.bc, &mass);
  } else {
    // Value-binned masses: one pass gives S and the bin where the nucleus
    // mass is reached.
    for (int i = threadIdx.x; i < PAIR_NBIN; i += NTP) ps.vh[i] = 0ull;
    if (threadIdx.x == 0) ps.ncol = 0;
    __syncthreads();
    each([&](uint32_t raw) {
      const float z = T::val(raw);
      if (z >= zthr) {
        const float e = ew(z, zmax, c);
        const unsigned long long f = fixq(e, two_fb, two_fb32);
        if (f) atomicAdd(&ps.vh[vbin(e)], f);
      }
    });
    __syncthreads();   // publishes vh
    if (threadIdx.x < 64) {
      constexpr int PER = PAIR_NBIN / 64;
      const int lane = threadIdx.x;
      unsigned long long ls = 0;
#pragma unroll 8
      for (int j = 0; j < PER; ++j) ls += ps.vh[lane * PER + j];
      unsigned long long incl = ls;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t ulo = (uint32_t)__shfl_up((int)(uint32_t)incl, o, 64);
        const uint32_t uhi = (uint32_t)__shfl_up((int)(uint32_t)(incl >> 32), o, 64);
        if (lane >= o) incl += ((unsigned long long)uhi << 32) | ulo;
      }
      // Every nonzero mass (e >= 2^-fb >= 2^-62) lands in a bin (bin <= 1984),
      // so the bins' total, lane 63's prefix, is the exact normaliser S.
      const unsigned long long Sw =
          ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(incl >> 32), 63) << 32) |
          (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)incl, 63);
      if (lane == 0) s.red_u64[0] = Sw;
      const double tau = (double)m.tp * (double)Sw;
      const unsigned long long any = __ballot((double)incl >= tau);
      const int first = any ? __ffsll((long long)any) - 1 : 63;
      if (lane == first) {
        unsigned long long ab = incl - ls;
        int cb = lane * PER + PER - 1;
        for (int j = 0; j < PER; ++j) {
          const unsigned long long h = ps.vh[lane * PER + j];
          if ((double)(ab + h) >= tau) {
            cb = lane * PER + j;
            break;
          }
          ab += h;
        }
        // The bin's key range [klo, khi): klo = smallest key whose bin is
        // <= cb, khi the same for cb - 1 (bins fall as keys rise).
        auto first_key_at_most = [&](int bin) {
          uint32_t lo = Key<ET>::NEG_INF, hi = key_of_value<ET>(zmax);   // bin(hi) == 0
          while (lo < hi) {
            const uint32_t mid = lo + (hi - lo) / 2;
            if (vbin(ew(Key<ET>::value(mid), zmax, c)) <= bin) hi = mid;
            else lo = mid + 1;
          }
          return lo;
        };
        const uint32_t klo = first_key_at_most(cb);
        const uint32_t khi = cb > 0 ? first_key_at_most(cb - 1) : Key<ET>::POS_INF;
        s.bc[5] = klo;
        s.bc[6] = khi;
        s.bd[0] = __longlong_as_double((long long)ab);
        s.bd[1] = __longlong_as_double((long long)ps.vh[cb]);
      }
    }
    __syncthreads();
    S = s.red_u64[0];
    const double tau = (double)m.tp * (double)S;
    const uint32_t klo = s.bc[5], khi = s.bc[6];
    const unsigned long long above = (unsigned long long)__double_as_longlong(s.bd[0]);
    const unsigned long long hbin = (unsigned long long)__double_as_longlong(s.bd[1]);
    const float zlo = Key<ET>::value(klo);
    if (khi == klo + 1) {
      // One key in the bin: the nucleus ends with all of its ties.
      tstar = klo;
      mass = above + hbin;
    } else {
      // Gather the crossing bin's keys (a key range: no weights needed).
      const float zhi = khi >= Key<ET>::POS_INF ? INFINITY : Key<ET>::value(khi);
      const float zl = fmaxf(zlo, zthr);
      each([&](uint32_t raw) {
        const float z = T::val(raw);
        if (z >= zl && z < zhi) {
          const uint32_t slot = atomicAdd(&ps.ncol, 1u);
          if (slot < (uint32_t)PAIR_NCAP) ps.keys[slot] = T::key(raw);
        }
      });
      __syncthreads();
      const uint32_t n = ps.ncol;
      if (n <= (uint32_t)PAIR_NCAP) {
        tstar = mass_select<LEVELS, NTP>(
            [&](auto fn) {
              for (uint32_t j = threadIdx.x; j < n; j += NTP) {
                const uint32_t uk = ps.keys[j];
                fn(uk, fx(Key<ET>::value(uk)));
              }
            },
            tau, above, s.hist.h64, s.bc, &mass);
      } else {
        tstar = mass_select<LEVELS, NTP>(
            [&](auto fn) {
              each([&](uint32_t raw) {
                const float z = T::val(raw);
                if (z >= zl && z < zhi) fn(T::key(raw), fx(z));
              });
            },
            tau, above, s.hist.h64, s.bc, &mass);
      }
    }
  }
  if (tstar != 0 && mass > 0) {
    st.zthr = fmaxf(zthr, Key<ET>::value(tstar));
    S = mass;
  }
  st.sp = (float)(ldexp(1.0, fb) / (double)S);
  return st;
}

// Probability of one element under a row's statistics.
__device__ __forceinline__ float pprob(const RowStat& st, float z) {
  return z >= st.zthr ? ew(z, st.zmax, st.c) * st.sp : 0.0f;
}

// A pair of short unfiltered rows (no top-k below V, no top-p; at most
// PAIR_SMALL_CH 16-byte units per lane, one wavefront) with the rows in
// registers: the same record as pair_one, with no LDS and no barrier.  Unit
// u of a row is chunk u / 64 of lane u % 64, so ascending id is (chunk,
// lane, element) order.  Every load is issued at once (an index past the
// row re-reads its last unit, which is then masked).
constexpr int PAIR_SMALL_CH = 4;
// Workgroups per CU of the 64-thread variant when no pair holds rows in LDS
// (its wavefronts per SIMD: five for fp32, four for bf16 rows).
constexpr int PAIR_REGS_WGS_F32 = 20;
constexpr int PAIR_REGS_WGS_BF16 = 16;
template <typename ET>
__device__ __forceinline__ void pair_small(const Args& a, int b, int i, const Mode& m, bool resid) {
  using T = PT<ET, true>;
  using U = typename T::U;
  constexpr int E = T::E;
  constexpr int NR = PAIR_SMALL_CH;
  const int lane = threadIdx.x & 63;
  const int G1 = a.G + 1;
  const int NU = a.V / E;
  const U* gp = reinterpret_cast<const U*>(row_ptr<ET>(a, b, true, i));
  const U* gq = resid ? reinterpret_cast<const U*>(row_ptr<ET>(a, b, false, i)) : gp;
  U up[NR], uq[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int ui = min(r * 64 + lane, NU - 1);
    up[r] = load_nt(gp + ui);
    uq[r] = load_nt(gq + ui);
  }
  const int x = resid ? a.draft[(size_t)b * a.G + i] : -1;
  const double u = (double)a.u[(size_t)b * G1 + a.G];
  PosRec* rec = a.pos + (size_t)b * G1 + i;
  // Validity and the rows' maxima.
  uint32_t bad = 0;
  float zmp = -INFINITY, zmq = -INFINITY;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (r * 64 + lane < NU) {
      T::each(up[r], [&](int, uint32_t raw) {
        const float z = T::val(raw);
        bad |= z < INFINITY ? 0u : 1u;
        zmp = fmaxf(zmp, z);
      });
      if (resid) {
        T::each(uq[r], [&](int, uint32_t raw) {
          const float z = T::val(raw);
          bad |= z < INFINITY ? 0u : 1u;
          zmq = fmaxf(zmq, z);
        });
      }
    }
  }
  const uint32_t kmp = wave_max_dpp(key_of_value<ET>(zmp));
  const uint32_t kmq = wave_max_dpp(key_of_value<ET>(zmq));
  if (__ballot(bad != 0u) != 0ull || kmp <= Key<ET>::NEG_INF || (resid && kmq <= Key<ET>::NEG_INF)) {
    if (lane == 0) {
      rec->bad = 1u;
      rec->tok = -1;
    }
    return;
  }
  const float c = LOG2E_F / m.T;
  const float zp = Key<ET>::value(kmp), zq = resid ? Key<ET>::value(kmq) : 0.0f;
  // Normalisers.
  double lsp = 0.0, lsq = 0.0;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (r * 64 + lane < NU) {
      float fp = 0.0f, fq = 0.0f;
      T::each(up[r], [&](int, uint32_t raw) { fp += ew(T::val(raw), zp, c); });
      if (resid) T::each(uq[r], [&](int, uint32_t raw) { fq += ew(T::val(raw), zq, c); });
      lsp += (double)fp;
      lsq += (double)fq;
    }
  }
  const double Sp = wave_sum_dpp(lsp), Sq = wave_sum_dpp(lsq);
  const RowStat sp{-INFINITY, zp, c, (float)(1.0 / Sp)};
  const RowStat sq = resid ? RowStat{-INFINITY, zq, c, (float)(1.0 / Sq)} : sp;
  // Unfiltered rows: every element is in the support, so a probability needs
  // no threshold test.
  const auto uprob = [](const RowStat& st, float z) { return ew(z, st.zmax, st.c) * st.sp; };
  // Element j of a unit (its bit pattern).
  auto elem = [](const U& v, int j) -> uint32_t {
    const uint32_t w = j < E / 4 * 1 ? v.x : (j < 2 * (E / 4) ? v.y : (j < 3 * (E / 4) ? v.z : v.w));
    if constexpr (sizeof(ET) == 2) return (j & 1) ? (w >> 16) : (w & 0xFFFFu);
    else return w;
  };
  // Overlap, p(x), q(x) and the weight totals.
  double al = 0.0, zl = 0.0, zt = 0.0, px = 0.0, qx = 0.0;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int ui = r * 64 + lane;
    if (ui < NU) {
      float av = 0.0f, wr = 0.0f, pr = 0.0f;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const float pj = uprob(sp, T::val(elem(up[r], j)));
        const float qj = resid ? uprob(sq, T::val(elem(uq[r], j))) : 0.0f;
        av += fminf(pj, qj);
        wr += resid ? fmaxf(pj - qj, 0.0f) : pj;
        pr += pj;
        if (ui * E + j == x) {
          px = (double)pj;
          qx = (double)qj;
        }
      }
      al += (double)av;
      zl += (double)wr;
      zt += (double)pr;
    }
  }
  al = wave_sum_dpp(al);
  double Z = wave_sum_dpp(zl);
  zt = wave_sum_dpp(zt);
  px = wave_sum_dpp(px);
  qx = wave_sum_dpp(qx);
  const bool use_q = resid && Z > 0.0;   // zero residual mass: draw from p itself
  if (resid && !use_q) Z = zt;
  // The inverse CDF in ascending id: chunk by chunk, a prefix scan of the
  // lanes' weight sums, then each lane's own elements in order (weights
  // formed again rather than kept).
  auto weight = [&](const U& vp, const U& vq, int j) -> float {
    const float pj = uprob(sp, T::val(elem(vp, j)));
    return use_q ? fmaxf(pj - uprob(sq, T::val(elem(vq, j))), 0.0f) : pj;
  };
  const double target = u * Z;
  double base = 0.0;
  uint32_t hit = NONE, lastpos = 0u;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (hit == NONE && r * 64 < NU) {
      const int ui = r * 64 + lane;
      const bool in = ui < NU;
      double lw = 0.0;
      if (in) {
#pragma unroll
        for (int j = 0; j < E; ++j) lw += (double)weight(up[r], uq[r], j);
      }
      const double incl = wave_incl_scan_f64(lw);
      double cum = base + (incl - lw);
      uint32_t h = NONE;
      if (in) {
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const float wj = weight(up[r], uq[r], j);
          cum += (double)wj;
          const uint32_t idx = (uint32_t)(ui * E + j);
          if (h == NONE && wj > 0.0f && cum > target) h = idx;
          if (wj > 0.0f) lastpos = idx + 1u;
        }
      }
      hit = wave_min_dpp(h);
      base += readlane_f64(incl, 63);
    }
  }
  const int tok = hit != NONE ? (int)hit : (int)wave_max_dpp(lastpos) - 1;   // rounding left no crossing
  if (lane == 0) {
    rec->px = px;
    rec->qx = qx;
    rec->alpha = resid ? al : 0.0;
    rec->tok = tok;
    rec->bad = 0u;
  }
}

// One (sequence b, position i) pair by the whole workgroup.
template <typename ET, int NTP, bool VECTOR, bool LDSR>
__device__ __forceinline__ void pair_one(const Args& a, int b, int i, PairSmem<NTP>& s, PairExtra<LDSR>& ps,
                                         unsigned char* pair_rows) {
  using T = PT<ET, VECTOR>;
  using U = typename T::U;
  constexpr int E = T::E;
  constexpr int NW = NTP / 64;
  const int G1 = a.G + 1;
  const Mode m = seq_mode(a, b);
  if (m.mode != MODE_DENSE || i > m.g) return;
  const bool resid = i < m.g;
  const int V = a.V;
  const int NU = VECTOR ? V / E : V;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = a.topk ? a.topk[b] : 0;
  const U* gp = reinterpret_cast<const U*>(row_ptr<ET>(a, b, true, i));
  const U* gq = resid ? reinterpret_cast<const U*>(row_ptr<ET>(a, b, false, i)) : gp;

  // Pass 1: maxima and validity (NaN or +inf makes the pair invalid); the
  // LDS variant copies the rows on chip as it goes.  Unfiltered rows also get
  // their normaliser in this pass: each thread keeps a running maximum m and
  // the sum of 2^((z - m) c) over its elements, taken a unit at a time (the
  // unit's maximum first, the sum rescaled once if m grows, then one
  // exponential per element); the block combines the sums at the row
  // maximum.
  const U* P;
  const U* Q;
  const bool online = !(k > 0 && k < V) && !(m.tp < 1.0f);
  if constexpr (NTP == 64 && VECTOR && LDSR) {
    if (online && NU <= PAIR_SMALL_CH * 64) {   // short unfiltered rows: registers only
      pair_small<ET>(a, b, i, m, resid);
      return;
    }
    if (a.pair_regs) {   // no row LDS in this launch: the finisher computes the sequence
      if (threadIdx.x == 0) a.pos[(size_t)b * G1 + i].bad = REC_REDO;
      return;
    }
  }
  // The draft token, for the record written at the end: fetched now, so its
  // round trip overlaps the passes.
  if (threadIdx.x == 0) s.xd = resid ? a.draft[(size_t)b * a.G + i] : -1;
  const float cT = LOG2E_F / m.T;
  float zmp = -INFINITY, zmq = -INFINITY, smp = 0.0f, smq = 0.0f;
  uint32_t bad = 0;
  auto scan_unit = [&](const U& u, float& zm, float& sm) {
    float um = -INFINITY;
    T::each(u, [&](int, uint32_t raw) {
      const float z = T::val(raw);
      bad |= z < INFINITY ? 0u : 1u;
      um = fmaxf(um, z);
    });
    if (online) {
      // Terms relative to the new running maximum (0 while every element
      // seen is -inf, whose terms are then 0).
      const float mn = fmaxf(zm, um);
      const float base = mn > -INFINITY ? mn : 0.0f;
      float acc = sm * __builtin_amdgcn_exp2f((zm - base) * cT);
      T::each(u, [&](int, uint32_t raw) { acc += __builtin_amdgcn_exp2f((T::val(raw) - base) * cT); });
      sm = acc;
    }
    zm = fmaxf(zm, um);
  };
  if constexpr (LDSR) {
    // Every thread issues the loads of up to PAIR_LDS_UR units of each row
    // before it examines any: unconditional loads (an index past the row
    // reads its last unit, which is then skipped) stay in flight together.
    const int nup = (NU * (int)sizeof(U) + 15) / 16 * 16 / (int)sizeof(U);
    U* lp = reinterpret_cast<U*>(pair_rows);
    U* lq = lp + nup;
    for (int u0 = 0; u0 < NU; u0 += PAIR_LDS_UR * NTP) {
      U pu[PAIR_LDS_UR], qu[PAIR_LDS_UR];
#pragma unroll
      for (int r = 0; r < PAIR_LDS_UR; ++r) {
        const int ui = min(u0 + r * NTP + (int)threadIdx.x, NU - 1);
        if constexpr (VECTOR) {
          pu[r] = load_nt(gp + ui);
          qu[r] = load_nt(gq + ui);
        } else {
          pu[r] = gp[ui];
          qu[r] = gq[ui];
        }
      }
#pragma unroll
      for (int r = 0; r < PAIR_LDS_UR; ++r) {
        const int ui = u0 + r * NTP + (int)threadIdx.x;
        if (ui < NU) {
          lp[ui] = pu[r];
          scan_unit(pu[r], zmp, smp);
          if (resid) {
            lq[ui] = qu[r];
            scan_unit(qu[r], zmq, smq);
          }
        }
      }
    }
    P = lp;
    Q = lq;
  } else {
    constexpr int U1 = SV_PAIR_UNR1;
    int ui = threadIdx.x;
    for (; ui + (U1 - 1) * NTP < NU; ui += U1 * NTP) {
      U pu[U1], qu[U1];
#pragma unroll
      for (int r = 0; r < U1; ++r) {
        pu[r] = gp[ui + r * NTP];
        if (resid) qu[r] = gq[ui + r * NTP];
      }
#pragma unroll
      for (int r = 0; r < U1; ++r) {
        scan_unit(pu[r], zmp, smp);
        if (resid) scan_unit(qu[r], zmq, smq);
      }
    }
    for (; ui < NU; ui += NTP) {
      scan_unit(gp[ui], zmp, smp);
      if (resid) scan_unit(gq[ui], zmq, smq);
    }
    P = gp;
    Q = gq;
  }
  // Order-preserving keys of the maxima (a max key of 0 marks no finite logit).
  uint32_t kmp = Key<ET>::of_bits(__float_as_uint(zmp)), kmq = Key<ET>::of_bits(__float_as_uint(zmq));
  if constexpr (sizeof(ET) == 2) {
    kmp = Key<ET>::of_bits(__float_as_uint(zmp) >> 16);
    kmq = Key<ET>::of_bits(__float_as_uint(zmq) >> 16);
  }
  pb_max3<NTP>(kmp, kmq, bad, s.red_u);   // its barriers also publish the LDS rows
  PosRec* rec = a.pos + (size_t)b * G1 + i;
  if (bad || kmp <= Key<ET>::NEG_INF || (resid && kmq <= Key<ET>::NEG_INF)) {
    if (threadIdx.x == 0) {
      rec->bad = 1u;
      rec->tok = -1;
    }
    return;
  }
  RowStat sp, sq;
  if (online) {
    // The threads' sums at the row maxima (a thread that saw no finite
    // logit holds 0), summed over the block in double.
    const float zp = Key<ET>::value(kmp), zq = resid ? Key<ET>::value(kmq) : 0.0f;
    const double vp = wave_sum_dpp((double)(smp * __builtin_amdgcn_exp2f((zmp - zp) * cT)));
    const double vq = resid ? wave_sum_dpp((double)(smq * __builtin_amdgcn_exp2f((zmq - zq) * cT))) : 0.0;
    if (lane == 0) {
      s.part[0][wave] = vp;
      s.part[1][wave] = vq;
    }
    __syncthreads();
    double Sp = 0.0, Sq = 0.0;
    for (int w2 = 0; w2 < NW; ++w2) {
      Sp += s.part[0][w2];
      Sq += s.part[1][w2];
    }
    __syncthreads();   // the weights pass reuses s.part
    sp = RowStat{-INFINITY, zp, cT, (float)(1.0 / Sp)};
    sq = resid ? RowStat{-INFINITY, zq, cT, (float)(1.0 / Sq)} : sp;
  } else {
    sp = row_stats<ET, NTP, VECTOR, LDSR>(P, NU, Key<ET>::value(kmp), a, m, k, s, ps);
    sq = sp;
    if (resid) sq = row_stats<ET, NTP, VECTOR, LDSR>(Q, NU, Key<ET>::value(kmq), a, m, k, s, ps);
  }

  // Overlap and per-(tile, wavefront) sums of the draw weights: the residual
  // max(0, p - q), or p at the bonus position and when the residual is zero.
  // Streamed rows load the next tile while the current one is summed.
  const int ntile = (NU + NTP - 1) / NTP;
  double al = 0.0;
  // unf: unfiltered rows (every element in the support), whose probability
  // needs no threshold test.
  auto weights_pass = [&](bool use_q, auto unf) {
    const auto prob = [&](const RowStat& st, float z) {
      if constexpr (decltype(unf)::value) return ew(z, st.zmax, st.c) * st.sp;
      else return pprob(st, z);
    };
    int ui = threadIdx.x;
    U np{}, nq{};
    if (ui < NU) {
      np = P[ui];
      if (use_q) nq = Q[ui];
    }
    for (int t = 0; t < ntile; ++t, ui += NTP) {
      const U up = np, uq = nq;
      if (ui + NTP < NU) {
        np = P[ui + NTP];
        if (use_q) nq = Q[ui + NTP];
      }
      float r = 0.0f, av = 0.0f;
      if (ui < NU) {
        if (use_q) {
          float pv[E];
          T::each(up, [&](int j, uint32_t raw) { pv[j] = prob(sp, T::val(raw)); });
          T::each(uq, [&](int j, uint32_t raw) {
            const float qv = prob(sq, T::val(raw));
            av += fminf(pv[j], qv);
            r += fmaxf(pv[j] - qv, 0.0f);
          });
        } else {
          T::each(up, [&](int, uint32_t raw) { r += prob(sp, T::val(raw)); });
        }
      }
      al += (double)av;
      const double w = wave_sum_dpp((double)r);
      if (lane == 0) s.part[t][wave] = w;
    }
  };
  if (online)
    weights_pass(resid, std::true_type{});
  else
    weights_pass(resid, std::false_type{});
  __syncthreads();
  // The crossing tile: lane t of wavefront 0 holds tile t's total.
  const double u = (double)a.u[(size_t)b * G1 + a.G];
  auto locate = [&]() {
    if (threadIdx.x < 64) {
      double tt = 0.0;
      if (lane < ntile) {
#pragma unroll
        for (int w = 0; w < NW; ++w) tt += s.part[lane][w];
      }
      const double incl = wave_incl_scan_f64(tt);
      const double Z = readlane_f64(incl, 63);
      const double target = u * Z;
      const unsigned long long hit = __ballot(lane < ntile && incl > target);
      const int j = hit ? __ffsll((long long)hit) - 1 : ntile - 1;
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
    // Zero residual mass (p == q after processing): draw from p itself.
    __syncthreads();
    if (online)
      weights_pass(false, std::true_type{});
    else
      weights_pass(false, std::false_type{});
    __syncthreads();
    locate();
    use_q = false;
  }
  const int tj = (int)s.bc[0];
  const double base = s.bd[0], target = s.bd[1];
  // Examine the crossing tile again, in ascending id.
  uint32_t hitpos = 0xFFFFFFFFu, lastpos = 0;
  {
    const int ui = tj * NTP + (int)threadIdx.x;
    float w[E];
#pragma unroll
    for (int j = 0; j < E; ++j) w[j] = 0.0f;
    float r = 0.0f;
    if (ui < NU) {
      const U up = P[ui];
      if (use_q) {
        const U uq = Q[ui];
        T::each(up, [&](int j, uint32_t raw) { w[j] = pprob(sp, T::val(raw)); });
        T::each(uq, [&](int j, uint32_t raw) {
          w[j] = fmaxf(w[j] - pprob(sq, T::val(raw)), 0.0f);
          r += w[j];
        });
      } else {
        T::each(up, [&](int j, uint32_t raw) {
          w[j] = pprob(sp, T::val(raw));
          r += w[j];
        });
      }
    }
    const double rd = (double)r;
    const double incl = wave_incl_scan_f64(rd);
    double cum = base;
    for (int w2 = 0; w2 < wave; ++w2) cum += s.part[tj][w2];
    cum += incl - rd;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      cum += (double)w[j];
      const uint32_t idx = (uint32_t)(ui * E + j);
      if (hitpos == 0xFFFFFFFFu && w[j] > 0.0f && cum > target) hitpos = idx;
      if (w[j] > 0.0f) lastpos = idx + 1u;
    }
  }
  hitpos = pb_min<NTP>(hitpos, s.red_u);
  int tok = (int)hitpos;
  if (hitpos == 0xFFFFFFFFu) tok = (int)pb_max<NTP>(lastpos, s.red_u) - 1;   // rounding left no crossing
  if (resid) al = pb_sum_f64<NTP>(al, s.red_d);
  if (threadIdx.x == 0) {
    const int x = s.xd;
    double px = 0.0, qx = 0.0;
    if (x >= 0 && x < V) {
      px = (double)pprob(sp, T::val(T::raw_at(P, x)));
      qx = (double)pprob(sq, T::val(T::raw_at(Q, x)));
    }
    rec->px = px;
    rec->qx = qx;
    rec->alpha = al;
    rec->tok = tok;
    rec->bad = 0u;
  }
}

// The dense pairs listed by the select kernel's extra workgroups, run by a
// grid sized to what the chip holds at once; workgroup w starts with pair w.
// Streamed pairs are long and few: a workgroup that has finished one takes
// the next unstarted pair from a shared counter, so the pairs left over after
// the first round go to the workgroups that finished first (the list puts the
// cheaper bonus positions last).  Pairs held in LDS are short and many, and a
// counter taken after each would serialise thousands of atomics on one
// address: those workgroups step through the list by the grid size.  When no
// sequence is dense every workgroup reads the counts once and leaves.  When
// the caller has promised that every sequence is dense there is no list (and
// no select launch): the pairs are taken in a fixed order instead.  The
// 64-thread variant keeps PAIR_REGS_WGS_* / 4 wavefronts per SIMD, which
// bounds the registers of its register-only path.
template <typename ET, int NTP, bool VECTOR, bool LDSR>
__global__ __launch_bounds__(NTP) __attribute__((amdgpu_waves_per_eu(
    LDSR ? (NTP == 64 ? (sizeof(ET) == 4 ? PAIR_REGS_WGS_F32 : PAIR_REGS_WGS_BF16) / 4 : 1) : PAIR_STREAM_WAVES_PER_EU)))
void pair_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char pair_rows[];
  __shared__ PairSmem<NTP> s;
  __shared__ PairExtra<LDSR> ps;
  __shared__ uint32_t next_pair;
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
      // No list: positions 0..G-1 of every sequence in order, then position G
      // of every sequence (the bonus position of a full-length draft), so the
      // cheaper pairs still come last; pair_one skips padding positions and
      // sequences that are not dense.
      pid = t < nlead ? (int)((t / (uint32_t)a.G) * (uint32_t)G1 + t % (uint32_t)a.G)
                      : (int)((t - nlead) * (uint32_t)G1 + (uint32_t)a.G);
    } else {
      const uint32_t idx = t < nf ? t : npairs - 1u - (t - nf);
      pid = a.dense_list[idx];
    }
    if (pid >= 0 && (uint32_t)pid < npairs) {   // else never written by this call's listing
      const int b = pid / G1;
      pair_one<ET, NTP, VECTOR, LDSR>(a, b, pid - b * G1, s, ps, pair_rows);
    }
    __syncthreads();   // the next pair reuses the LDS
    if constexpr (LDSR) {
      t += gridDim.x;
    } else {
      if (threadIdx.x == 0) next_pair = gridDim.x + atomicAdd(&a.dense_count[2], 1u);
      __syncthreads();
      t = next_pair;
    }
  }
}

}  // namespace sv
