// Pair-parallel verify of the dense sequences (temperature > 0 and no top-k
// up to KMAX_SPARSE: unfiltered, large top-k and top-p rows).
//
// One workgroup per (sequence, position i <= gamma_b) owns the target row p_i
// and, for i < gamma_b, the draft row q_i; every row belongs to exactly one
// workgroup.  Rows of up to 64 KB are read from HBM once into LDS and every
// later pass runs on chip; longer rows are streamed from global memory on
// each pass (the re-reads of one workgroup's rows hit L2 / MALL).  Per row:
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

constexpr int PAIR_LDS_ROW_MAX = 65536;   // bytes of one row held in LDS
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

// e * 2^fb truncated to an integer (e in [0, 1]; 0 below 2^-fb).
__device__ __forceinline__ unsigned long long fixq(float e, int fb) {
  const uint32_t b = __float_as_uint(e);
  const int sh = (int)(b >> 23) - 150 + fb;
  const unsigned long long man = (unsigned long long)((b & 0x7FFFFFu) | 0x800000u);
  if (sh >= 0) return man << sh;
  return sh > -24 ? man >> (-sh) : 0ull;
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

// Processed distribution of one row: p(z) = (key(z) >= thr) ? e(z) * sp : 0.
struct RowStat {
  uint32_t thr;
  float zmax, c, sp;
};

// Row statistics.  src: the row (LDS or global), NU units; kmax: its largest key.
template <typename ET, int NTP, bool VECTOR, bool LDSR>
__device__ __forceinline__ RowStat row_stats(const typename PT<ET, VECTOR>::U* src, int NU, uint32_t kmax,
                                             const Args& a, const Mode& m, int k, PairSmem<NTP>& s,
                                             PairExtra<LDSR>& ps) {
  using T = PT<ET, VECTOR>;
  constexpr int LEVELS = Key<ET>::LEVELS;
  RowStat st;
  st.zmax = Key<ET>::value(kmax);
  st.c = LOG2E_F / m.T;
  st.thr = 1;
  const float zmax = st.zmax, c = st.c;
  const int fb = a.fixbits;
  // fn(key, raw) over the calling thread's elements.
  auto row_each = [&](auto fn) {
    for (int ui = threadIdx.x; ui < NU; ui += NTP) {
      const typename T::U u = src[ui];
      T::each(u, [&](int, uint32_t raw) { fn(T::key(raw), raw); });
    }
  };
  if (k > KMAX_SPARSE && k < a.V) {
    const uint32_t kth = block_kth_largest<LEVELS, NTP>(
        [&](auto fn) { row_each([&](uint32_t uk, uint32_t) { fn(uk); }); }, (uint32_t)k, s.hist.h32, s.bc);
    st.thr = kth ? kth : 1u;
  }
  const uint32_t thr0 = st.thr;
  if (!(m.tp < 1.0f)) {
    // No nucleus cut: S = sum of e over the kept keys.
    double sl = 0.0;
    row_each([&](uint32_t uk, uint32_t raw) {
      if (uk >= thr0) sl += (double)ew(T::val(raw), zmax, c);
    });
    st.sp = (float)(1.0 / pb_sum_f64<NTP>(sl, s.red_d));
    return st;
  }
  if (m.tp <= 0.0f) {
    // Only the maximal logit (with its ties) survives.
    unsigned long long cl = 0;
    row_each([&](uint32_t uk, uint32_t) { cl += uk == kmax ? 1ull : 0ull; });
    const unsigned long long cnt = pb_sum_u64<NTP>(cl, s.red_u64);
    st.thr = kmax;
    st.sp = (float)(1.0 / (double)cnt);
    return st;
  }
  const double fscale = ldexp(1.0, fb);
  unsigned long long S, mass = 0;
  uint32_t tstar = 0;
  if constexpr (LDSR) {
    unsigned long long sl = 0;
    row_each([&](uint32_t uk, uint32_t raw) {
      if (uk >= thr0) sl += fixq(ew(T::val(raw), zmax, c), fb);
    });
    S = pb_sum_u64<NTP>(sl, s.red_u64);
    tstar = mass_select<LEVELS, NTP>(
        [&](auto fn) {
          row_each([&](uint32_t uk, uint32_t raw) {
            if (uk >= thr0) fn(uk, fixq(ew(T::val(raw), zmax, c), fb));
          });
        },
        (double)m.tp * (double)S, 0ull, s.hist.h64, s.bc, &mass);
  } else {
    // Value-binned masses: one pass gives S and the bin where the nucleus
    // mass is reached.
    for (int i = threadIdx.x; i < PAIR_NBIN; i += NTP) ps.vh[i] = 0ull;
    if (threadIdx.x == 0) ps.ncol = 0;
    __syncthreads();
    unsigned long long sl = 0;
    row_each([&](uint32_t uk, uint32_t raw) {
      if (uk >= thr0) {
        const float e = ew(T::val(raw), zmax, c);
        const unsigned long long f = fixq(e, fb);
        if (f) {
          sl += f;
          atomicAdd(&ps.vh[vbin(e)], f);
        }
      }
    });
    S = pb_sum_u64<NTP>(sl, s.red_u64);   // its barriers also publish vh
    const double tau = (double)m.tp * (double)S;
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
        s.bc[5] = (uint32_t)cb;
        s.bc[6] = (uint32_t)ab;
        s.bc[7] = (uint32_t)(ab >> 32);
      }
    }
    __syncthreads();
    const int cbin = (int)s.bc[5];
    const unsigned long long above = ((unsigned long long)s.bc[7] << 32) | s.bc[6];
    // Gather the crossing bin's keys.
    row_each([&](uint32_t uk, uint32_t raw) {
      if (uk >= thr0 && vbin(ew(T::val(raw), zmax, c)) == cbin) {
        const uint32_t slot = atomicAdd(&ps.ncol, 1u);
        if (slot < (uint32_t)PAIR_NCAP) ps.keys[slot] = uk;
      }
    });
    __syncthreads();
    const uint32_t n = ps.ncol;
    if (n <= (uint32_t)PAIR_NCAP) {
      tstar = mass_select<LEVELS, NTP>(
          [&](auto fn) {
            for (uint32_t j = threadIdx.x; j < n; j += NTP) {
              const uint32_t uk = ps.keys[j];
              fn(uk, fixq(ew(Key<ET>::value(uk), zmax, c), fb));
            }
          },
          tau, above, s.hist.h64, s.bc, &mass);
    } else {
      tstar = mass_select<LEVELS, NTP>(
          [&](auto fn) {
            row_each([&](uint32_t uk, uint32_t raw) {
              if (uk >= thr0) {
                const float e = ew(T::val(raw), zmax, c);
                if (vbin(e) == cbin) fn(uk, fixq(e, fb));
              }
            });
          },
          tau, above, s.hist.h64, s.bc, &mass);
    }
  }
  if (tstar != 0 && mass > 0) {
    st.thr = max(st.thr, tstar);
    S = mass;
  }
  st.sp = (float)(fscale / (double)S);
  return st;
}

// Probability of one element under a row's statistics.
template <typename ET, bool VECTOR>
__device__ __forceinline__ float pprob(const RowStat& st, uint32_t raw) {
  using T = PT<ET, VECTOR>;
  return T::key(raw) >= st.thr ? ew(T::val(raw), st.zmax, st.c) * st.sp : 0.0f;
}

template <typename ET, int NTP, bool VECTOR, bool LDSR>
__global__ __launch_bounds__(NTP) void pair_kernel(Args a) {
  using T = PT<ET, VECTOR>;
  using U = typename T::U;
  constexpr int E = T::E;
  constexpr int NW = NTP / 64;
  extern __shared__ __align__(16) unsigned char pair_rows[];
  __shared__ PairSmem<NTP> s;
  __shared__ PairExtra<LDSR> ps;
  const int G1 = a.G + 1;
  const int b = blockIdx.x / G1, i = blockIdx.x - (blockIdx.x / G1) * G1;
  const Mode m = seq_mode(a, b);
  if (m.mode != MODE_DENSE || i > m.g) return;
  const bool resid = i < m.g;
  const int V = a.V;
  const int NU = VECTOR ? V / E : V;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = a.topk ? a.topk[b] : 0;
  const U* gp = reinterpret_cast<const U*>(row_ptr<ET>(a, b, true, i));
  const U* gq = resid ? reinterpret_cast<const U*>(row_ptr<ET>(a, b, false, i)) : gp;

  // Pass 1: maxima and validity (LDS variant: the rows are copied on chip).
  const U* P;
  const U* Q;
  uint32_t kmp = 0, kmq = 0, bad = 0;
  auto scan_unit = [&](const U& u, uint32_t& km) {
    T::each(u, [&](int, uint32_t raw) {
      const uint32_t uk = T::key(raw);
      km = max(km, uk);
      bad |= key_valid<ET>(uk) ? 0u : 1u;
    });
  };
  if constexpr (LDSR) {
    const int nup = (NU * (int)sizeof(U) + 15) / 16 * 16 / (int)sizeof(U);
    U* lp = reinterpret_cast<U*>(pair_rows);
    U* lq = lp + nup;
    for (int ui = threadIdx.x; ui < NU; ui += NTP) {
      U up, uq;
      if constexpr (VECTOR) {
        up = load_nt(gp + ui);
        if (resid) uq = load_nt(gq + ui);
      } else {
        up = gp[ui];
        if (resid) uq = gq[ui];
      }
      lp[ui] = up;
      scan_unit(up, kmp);
      if (resid) {
        lq[ui] = uq;
        scan_unit(uq, kmq);
      }
    }
    P = lp;
    Q = lq;
  } else {
    for (int ui = threadIdx.x; ui < NU; ui += NTP) {
      scan_unit(gp[ui], kmp);
      if (resid) scan_unit(gq[ui], kmq);
    }
    P = gp;
    Q = gq;
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
  const RowStat sp = row_stats<ET, NTP, VECTOR, LDSR>(P, NU, kmp, a, m, k, s, ps);
  RowStat sq = sp;
  if (resid) sq = row_stats<ET, NTP, VECTOR, LDSR>(Q, NU, kmq, a, m, k, s, ps);

  // Overlap and per-(tile, wavefront) sums of the draw weights: the residual
  // max(0, p - q), or p at the bonus position and when the residual is zero.
  const int ntile = (NU + NTP - 1) / NTP;
  double al = 0.0;
  auto weights_pass = [&](bool use_q) {
    for (int t = 0; t < ntile; ++t) {
      const int ui = t * NTP + (int)threadIdx.x;
      float r = 0.0f, av = 0.0f;
      if (ui < NU) {
        const U up = P[ui];
        if (use_q) {
          const U uq = Q[ui];
          float pv[E];
          T::each(up, [&](int j, uint32_t raw) { pv[j] = pprob<ET, VECTOR>(sp, raw); });
          T::each(uq, [&](int j, uint32_t raw) {
            const float qv = pprob<ET, VECTOR>(sq, raw);
            av += fminf(pv[j], qv);
            r += fmaxf(pv[j] - qv, 0.0f);
          });
        } else {
          T::each(up, [&](int, uint32_t raw) { r += pprob<ET, VECTOR>(sp, raw); });
        }
      }
      al += (double)av;
      const double w = wave_sum_dpp((double)r);
      if (lane == 0) s.part[t][wave] = w;
    }
  };
  weights_pass(resid);
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
    weights_pass(false);
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
        T::each(up, [&](int j, uint32_t raw) { w[j] = pprob<ET, VECTOR>(sp, raw); });
        T::each(uq, [&](int j, uint32_t raw) {
          const float qv = pprob<ET, VECTOR>(sq, raw);
          w[j] = fmaxf(w[j] - qv, 0.0f);
          r += w[j];
        });
      } else {
        T::each(up, [&](int j, uint32_t raw) {
          w[j] = pprob<ET, VECTOR>(sp, raw);
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
    const int x = resid ? a.draft[(size_t)b * a.G + i] : -1;
    double px = 0.0, qx = 0.0;
    if (x >= 0 && x < V) {
      px = (double)pprob<ET, VECTOR>(sp, T::raw_at(P, x));
      qx = (double)pprob<ET, VECTOR>(sq, T::raw_at(Q, x));
    }
    rec->px = px;
    rec->qx = qx;
    rec->alpha = al;
    rec->tok = tok;
    rec->bad = 0u;
  }
}

}  // namespace sv
