// Verify with shared Gumbel noise ("Speculative Decoding: the art of guessing
// well", section "Sampling with shared noise"): the drafter proposed
// x_k = argmax_i(log q_k(i) + g_k,i) with the same noise vectors g_k that the
// target uses here.  The target's own sample at position k is
// t_k = argmax_i(log p_k(i) + g_k,i); the verify keeps the longest prefix with
// x_k == t_k and appends t at the first disagreement (t after the last draft
// when all agree).  Exact matching, like greedy decoding.
//
// log p_k(i) = z_i / T - log S on the processed support, so the argmax needs
// only the support and z_i + T g_i (the factor T > 0 keeps the argmax); the
// score is formed in float32 as fl(z + fl(T * g)) with no fused multiply-add,
// and ties go to the lowest id.  T = 0 is argmax of z (noise unused).
//
// gumbel_list_kernel: argmax and top-k sequences from the streaming
// select's survivor lists, one workgroup per sequence (a wavefront per row
// in registers, or the rows' kept sets in LDS); with the no-dense promise it
// is the call's last launch and also takes the other sequences and the
// outputs.
// gumbel_kernel: one workgroup per (sequence, position) of the dense and
// demoted sequences.  Unfiltered rows take one pass over the logits and the
// noise (validity, and the argmax of the score); top-k rows first find the
// k-th largest key (block radix select), top-p rows the nucleus threshold
// (the pair kernel's row statistics), then the argmax pass runs over the
// support.
// gumbel_finish_kernel: one wavefront per sequence: the first disagreement
// by one ballot and find-first-set, and the outputs.
#pragma once

#include "sv_pair.h"
#include "sv_phist.h"
#include "sv_finish.h"

namespace sv {

constexpr int GUMBEL_NT = 512;
constexpr int32_t GUMBEL_BAD_ROW = -2;
constexpr int32_t GUMBEL_REDO = -3;   // gumbel_hist_kernel left the row to gumbel_kernel

// Order-preserving 32-bit key of a float score (larger float -> larger key;
// every non-NaN float maps above 0, so 0 means "no candidate").
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Position j of sequence b by the whole workgroup (NTP threads): the
// target's sample, the lowest-id argmax of the score over the processed
// support, or GUMBEL_BAD_ROW (invalid parameters, NaN / +inf among the
// logits or the support's noise, no finite logit).  The result is
// workgroup-uniform.
template <typename ET, int NTP, bool VECTOR>
__device__ __forceinline__ int32_t gumbel_row_block(const Args& a, PairSmem<NTP>& s, PairStream& ps, int b, int j) {
  using T = PT<ET, VECTOR>;
  using U = typename T::U;
  constexpr int E = T::E;
  constexpr int LEVELS = Key<ET>::LEVELS;
  const int G1 = a.G + 1;
  const int gl = a.gamma_len ? a.gamma_len[b] : a.G;
  const int g = min(max(gl, 1), a.G);
  const float Tv = a.temp[b];
  const int k = a.topk ? a.topk[b] : 0;
  const float tp = a.topp ? a.topp[b] : 1.0f;
  if (!(Tv >= 0.0f) || tp != tp) return GUMBEL_BAD_ROW;   // the finisher rejects the sequence
  const int V = a.V;
  const int NU = VECTOR ? V / E : V;
  const U* gp = reinterpret_cast<const U*>(row_ptr<ET>(a, b, true, j));
  const float* gn = a.noise + ((size_t)b * G1 + j) * (size_t)V;
  const bool use_noise = Tv > 0.0f;
  const bool filtered = use_noise && ((k > 0 && k < V) || tp < 1.0f);

  // Support threshold: keep z >= zthr.
  float zthr = -INFINITY;
  uint32_t bad = 0;
  if (filtered) {
    // Validity and the maximum (the threshold passes need it).
    uint32_t km = 0;
    row_each<ET, NTP, VECTOR, false>(gp, NU, [&](uint32_t raw) {
      const float z = T::val(raw);
      bad |= z < INFINITY ? 0u : 1u;
      km = max(km, T::key(raw));
    });
    uint32_t dummy = 0;
    pb_max3<NTP>(km, bad, dummy, s.red_u);
    if (bad || km <= Key<ET>::NEG_INF) return GUMBEL_BAD_ROW;
    if (tp < 1.0f) {
      Mode m;
      m.g = g;
      m.mode = MODE_DENSE;
      m.k = 0;
      m.T = Tv;
      m.tp = tp;
      PairExtra<false>& pe = ps;
      zthr = row_stats<ET, NTP, VECTOR, false>(gp, NU, Key<ET>::value(km), a, m, k, s, pe).zthr;
    } else {
      const uint32_t kth = block_kth_largest<LEVELS, NTP>(
          [&](auto fn) { row_each<ET, NTP, VECTOR, false>(gp, NU, [&](uint32_t raw) { fn(T::key(raw)); }); },
          (uint32_t)k, s.hist.h32, s.bc);
      zthr = key_floor_value<ET>(kth ? kth : 1u);
    }
  }

  // The argmax pass: the lowest id with the largest score over the support.
  uint32_t bkey = 0, bidx = NONE, kmax = 0;
  auto consider = [&](uint32_t raw, float noise, uint32_t idx) {
#pragma clang fp contract(off)
    // Two roundings, as the score's definition says: no fused multiply-add.
    const float z = T::val(raw);
    bad |= z < INFINITY ? 0u : 1u;
    kmax = max(kmax, T::key(raw));
    if (z >= zthr) {
      if (use_noise) bad |= fabsf(noise) < INFINITY ? 0u : 1u;   // noise on the support only
      const float tg = Tv * noise;
      const float sc = use_noise ? z + tg : z;
      const uint32_t sk = score_key(sc);
      if (sc == sc && sk > bkey) {        // strictly greater: the first of equals in id order stays
        bkey = sk;
        bidx = idx;
      }
    }
  };
  for (int ui = threadIdx.x; ui < NU; ui += NTP) {
    const U u = gp[ui];
    if constexpr (VECTOR) {
      float nv[E];
      if (use_noise) {
        const float4* np4 = reinterpret_cast<const float4*>(gn + (size_t)ui * E);
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
          const float4 f = np4[q];
          nv[4 * q] = f.x;
          nv[4 * q + 1] = f.y;
          nv[4 * q + 2] = f.z;
          nv[4 * q + 3] = f.w;
        }
      } else {
#pragma unroll
        for (int q = 0; q < E; ++q) nv[q] = 0.0f;
      }
      T::each(u, [&](int e, uint32_t raw) { consider(raw, nv[e], (uint32_t)(ui * E + e)); });
    } else {
      const float nz = use_noise ? gn[ui] : 0.0f;
      T::each(u, [&](int, uint32_t raw) { consider(raw, nz, (uint32_t)ui); });
    }
  }
  const uint32_t mykey = bkey;
  pb_max3<NTP>(bkey, bad, kmax, s.red_u);     // block-wide maxima
  const uint32_t win = pb_min<NTP>(bkey != 0u && mykey == bkey ? bidx : NONE, s.red_u);
  return (bad || kmax <= Key<ET>::NEG_INF || win == NONE) ? GUMBEL_BAD_ROW : (int32_t)win;
}

// Rows that gumbel_hist_kernel takes (when the call launches it, a.ghist):
// position j <= gamma_b of a sequence outside the list path with T > 0 and a
// filter (top-k below V, or top-p), whose support the exact histogram gives.
__device__ __forceinline__ bool gumbel_hist_takes(const Args& a, int b, int j) {
  if (!a.ghist) return false;
  const Mode sm = seq_mode(a, b);
  if (j > sm.g) return false;
  // Under a.gmix the rows are taken while the select still runs, before any
  // demotion is known: a demoted top-k sequence then goes to gumbel_kernel.
  if ((sm.mode == MODE_GREEDY || sm.mode == MODE_SPARSE) && (a.gmix || !(a.seq_flags[b] & F_DEMOTE)) && !a.all_dense)
    return false;
  const int k = a.topk ? a.topk[b] : 0;
  return sm.T > 0.0f && sm.tp == sm.tp && ((k > 0 && k < a.V) || sm.tp < 1.0f);
}

// Position j of sequence b, a filtered bf16 row of at most PH_MAX_UNITS
// 16-byte units, by the whole workgroup: the row's support from its exact
// value histogram (one pass over the logits: the k-th largest value for
// top-k, then the nucleus cut for top-p, as the verify's histogram kernel
// finds them), then the lowest-id argmax of fl(z + fl(T g)) over the
// support, reading logits and noise only in the units whose largest value
// reaches the support's threshold.  Returns the sample, GUMBEL_BAD_ROW, or
// GUMBEL_REDO when a 16-bit count overflowed (gumbel_kernel then takes the
// row).  Workgroup-uniform.
__device__ __forceinline__ int32_t gumbel_hist_row(const Args& a, PhSmem& s, int b, int j) {
  using T = PT<uint16_t, true>;
  const int G1 = a.G + 1;
  const int V = a.V, NU = V / 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const Mode sm = seq_mode(a, b);
  Mode m = sm;
  m.mode = MODE_DENSE;
  const int k = a.topk ? a.topk[b] : 0;
  const uint4* gp = reinterpret_cast<const uint4*>(row_ptr<uint16_t>(a, b, true, j));
  const __amdgpu_buffer_rsrc_t rp = ph_rsrc(gp, NU);
  const float cT = LOG2E_F / m.T;
  const float binv = 254.0f * cT / (float)(a.fixbits + 2);
  RowStat st{};
  const int bad = ph_row_pass(s, rp, NU, a.fixbits, cT, binv, k > 0 && k < V, true, V, m, k, st);
  if (bad) return (bad & PH_BAD) ? GUMBEL_BAD_ROW : GUMBEL_REDO;
  // The units that can hold an element of the support, in ascending order,
  // in the histogram's memory (as the verify's histogram kernel lists them).
  uint16_t* list = reinterpret_cast<uint16_t*>(s.hist);
  uint32_t* lcnt = s.hist + PH_WORDS / 2;
  uint32_t nd_bits = 0;
#pragma unroll 1
  for (int jj = 0; jj < PH_UPT; ++jj) {
    const int ui = jj * PH_NT + (int)threadIdx.x;
    const bool nd = ui < NU && (uint32_t)s.umax[ui] >= ph_bucket(st.zthr, s.uref[jj / PH_INFLIGHT][wave], binv);
    const unsigned long long bal = __ballot(nd);
    nd_bits |= nd ? 1u << jj : 0u;
    if (lane == 0) lcnt[jj * PH_NW + wave] = (uint32_t)__popcll(bal);
  }
  __syncthreads();
  if (wave == 0) {
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
  for (int jj = 0; jj < PH_UPT; ++jj) {
    const bool nd = (nd_bits >> jj) & 1u;
    const unsigned long long bal = __ballot(nd);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (nd) list[lcnt[jj * PH_NW + wave] + below] = (uint16_t)(jj * PH_NT + (int)threadIdx.x);
  }
  __syncthreads();
  // The argmax over the listed units: strictly greater keeps the first of
  // equal scores in this thread's (ascending) order; the block takes the
  // lowest id among the maxima.
  const float* gn = a.noise + ((size_t)b * G1 + j) * (size_t)V;
  const float Tv = m.T, zthr = st.zthr;
  uint32_t bkey = 0, bidx = NONE, badn = 0;
  for (int le = threadIdx.x; le < nlist; le += PH_NT) {
    const int ui = list[le];
    const uint4 u = ph_load_unit<BUF_NT>(rp, ui);
    const float4* np4 = reinterpret_cast<const float4*>(gn + (size_t)ui * 8);
    const float4 n0 = np4[0], n1 = np4[1];
    const float nv[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
    T::each(u, [&](int e, uint32_t raw) {
#pragma clang fp contract(off)
      const float z = T::val(raw);
      if (z >= zthr) {
        badn |= fabsf(nv[e]) < INFINITY ? 0u : 1u;   // noise on the support only
        const float tg = Tv * nv[e];
        const float sc = z + tg;
        const uint32_t sk = score_key(sc);
        if (sc == sc && sk > bkey) {
          bkey = sk;
          bidx = (uint32_t)(ui * 8 + e);
        }
      }
    });
  }
  const uint32_t mykey = bkey;
  uint32_t dummy = 0;
  pb_max3<PH_NT>(bkey, badn, dummy, s.red);
  const uint32_t win = pb_min<PH_NT>(bkey != 0u && mykey == bkey ? bidx : NONE, s.red);
  return (badn || win == NONE) ? GUMBEL_BAD_ROW : (int32_t)win;
}

// The rows gumbel_hist_takes, one workgroup per CU: workgroup w starts with
// row w (sequence-major order) and then takes the next unstarted row from a
// workspace counter (cleared by gumbel_finish_kernel); other rows are
// skipped.
__global__ __launch_bounds__(PH_NT) void gumbel_hist_kernel(Args a) {
  __shared__ __align__(16) PhSmem s;   // static, as in pair_hist_kernel
  const int G1 = a.G + 1;
  const uint32_t nrows = (uint32_t)a.B * (uint32_t)G1;
  uint32_t t = blockIdx.x;
  while (t < nrows) {
    const int b = (int)(t / (uint32_t)G1), j = (int)(t - (uint32_t)b * (uint32_t)G1);
    if (gumbel_hist_takes(a, b, j)) {   // workgroup-uniform
      const int32_t tok = gumbel_hist_row(a, s, b, j);
      if (threadIdx.x == 0) a.out_target[(size_t)b * G1 + j] = tok;
    }
    __syncthreads();
    if (threadIdx.x == 0) s.next_pair = gridDim.x + atomicAdd(&a.dense_count[2], 1u);
    __syncthreads();
    t = s.next_pair;
  }
}

// The select units and the histogram rows of a shared-noise call in one
// launch (a.gmix), in the manner of mixed_hist_kernel: one workgroup per CU
// first takes groups of PH_NW consecutive select units (a wavefront each),
// then the rows gumbel_hist_takes, every one claimed from the row counter.
// A call in which no sequence is dense (found by each workgroup from the
// sampling settings) has its units taken one per wavefront instead, spread
// over all CUs.  Both counters are cleared by gumbel_finish_kernel.
__global__ __launch_bounds__(PH_NT) void gumbel_mixed_kernel(Args a) {
  __shared__ __align__(16) union {
    PhSmem ph;
    WaveSmem w[PH_NW];
  } sm;
  __shared__ uint32_t claim;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const long long units = (long long)a.B * a.RS * a.NP;
  const long long ngroups = (units + PH_NW - 1) / PH_NW;
  int dense = 0;
  for (int b = threadIdx.x; b < a.B; b += PH_NT) {
    const int md = seq_mode(a, b).mode;
    dense |= md != MODE_GREEDY && md != MODE_SPARSE ? 1 : 0;
  }
  if (!__syncthreads_or(dense)) {
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
  const int G1 = a.G + 1;
  const uint32_t nrows = (uint32_t)a.B * (uint32_t)G1;
  __syncthreads();   // the select units' LDS, and the last claim, are done with
  if (threadIdx.x == 0) claim = atomicAdd(&a.dense_count[2], 1u);
  __syncthreads();
  uint32_t t = claim;
  while (t < nrows) {
    const int b = (int)(t / (uint32_t)G1), j = (int)(t - (uint32_t)b * (uint32_t)G1);
    if (gumbel_hist_takes(a, b, j)) {   // workgroup-uniform
      const int32_t tok = gumbel_hist_row(a, sm.ph, b, j);
      if (threadIdx.x == 0) a.out_target[(size_t)b * G1 + j] = tok;
    }
    __syncthreads();
    if (threadIdx.x == 0) claim = atomicAdd(&a.dense_count[2], 1u);
    __syncthreads();
    t = claim;
  }
}

template <typename ET, int NTP, bool VECTOR>
__global__ __launch_bounds__(NTP) void gumbel_kernel(Args a) {
  __shared__ PairSmem<NTP> s;
  __shared__ PairStream ps;
  const int G1 = a.G + 1;
  const int b = blockIdx.x / G1, j = blockIdx.x - (blockIdx.x / G1) * G1;
  const int gl = a.gamma_len ? a.gamma_len[b] : a.G;
  const int g = min(max(gl, 1), a.G);
  if (j > g) return;                          // padding: the finisher writes it
  {
    // Argmax and top-k sequences belong to the list path unless their lists
    // were demoted (overflow) by the select or the list kernel, or there is
    // no list path in this call (every sequence promised dense).
    const Mode sm = seq_mode(a, b);
    if ((sm.mode == MODE_GREEDY || sm.mode == MODE_SPARSE) && !(a.seq_flags[b] & F_DEMOTE) && !a.all_dense) return;
  }
  // Rows the histogram kernel took (unless a count overflowed there).
  if (gumbel_hist_takes(a, b, j) && a.out_target[(size_t)b * G1 + j] != GUMBEL_REDO) return;
  const int32_t tok = gumbel_row_block<ET, NTP, VECTOR>(a, s, ps, b, j);
  if (threadIdx.x == 0) a.out_target[(size_t)b * G1 + j] = tok;
}

// Chunks of 64 list entries the list kernel's register path holds per row
// (a row of NP <= GUMBEL_CH parts keeps GUMBEL_CH / NP chunks of each part).
constexpr int GUMBEL_CH = 8;
static_assert(64 * GUMBEL_CH <= SEG, "a row part's register chunks stay inside its list segment");

// Register path of the list kernel: row r of a top-k (top-p off) or argmax
// sequence by one wavefront, from its survivor lists in registers (rows of
// NP parts; chunk c is part c / FC, entries (c % FC) * 64 + lane, FC =
// GUMBEL_CH / NP; f0[p] holds part p's first chunk, loaded by the caller, the
// others are loaded here when the part's size (cnt, lane p) reaches them; lp
// is the row's part-0 list).  The kept set is the k-th largest key of the
// union of the parts and everything above (all listed keys for one part),
// and the result is the lowest-id argmax of fl(z + fl(T * g)) over it, as on
// the LDS path.  Sets *fits = false (and returns nothing) when a part list
// does not fit the registers.
template <typename ET, int NP>
__device__ __forceinline__ int32_t gumbel_row_fast(const Args& a, FinSmem& s, const Mode& m, int b, int r,
                                                   const uint2 (&f0)[GUMBEL_CH], uint32_t cnt, const uint2* lp,
                                                   bool* fits) {
  constexpr int CH = GUMBEL_CH;
  constexpr int FC = CH / NP;
  const int lane = threadIdx.x & 63;
  int ccnt[CH];
  uint32_t total = 0;
  bool ok = true;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const uint32_t pc = (uint32_t)__builtin_amdgcn_readlane((int)cnt, p);
    total += pc;
    ok = ok && pc <= (uint32_t)(64 * FC);
#pragma unroll
    for (int sub = 0; sub < FC; ++sub) ccnt[p * FC + sub] = (int)min(pc - min(pc, (uint32_t)(sub * 64)), 64u);
  }
#pragma unroll
  for (int c = NP * FC; c < CH; ++c) ccnt[c] = 0;
  *fits = ok;
  if (!ok) return GUMBEL_BAD_ROW;
  if (total == 0u) return GUMBEL_BAD_ROW;   // no finite logit
  uint2 e[CH];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    e[p * FC] = f0[p];
#pragma unroll
    for (int sub = 1; sub < FC; ++sub)
      e[p * FC + sub] = ccnt[p * FC + sub] > 0 ? lp[(size_t)p * SEG + sub * 64 + lane] : make_uint2(0u, 0u);
  }
#pragma unroll
  for (int c = NP * FC; c < CH; ++c) e[c] = make_uint2(0u, 0u);
  if (m.mode == MODE_GREEDY) {
    uint32_t km = 0u;
#pragma unroll
    for (int c = 0; c < CH; ++c) km = max(km, lane < ccnt[c] ? e[c].x : 0u);
    const uint32_t kmax = wave_max_dpp(km);
    uint32_t best = NONE;
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (lane < ccnt[c] && e[c].x == kmax) best = min(best, e[c].y);
    return (int32_t)wave_min_dpp(best);
  }
  uint32_t kth = 0u;
  if (NP > 1 && total > m.k) {
    kth = wave_kth<Key<ET>::LEVELS>(
        [&](auto fn) {
#pragma unroll
          for (int c = 0; c < NP * FC; ++c)
            if (lane < ccnt[c]) fn(e[c].x);
        },
        m.k, s.whist[threadIdx.x >> 6]);
  }
  // The noise at the kept ids, then the lowest-id argmax of the score.
  const float* gn = a.noise + ((size_t)b * (a.G + 1) + r) * (size_t)a.V;
  float nz[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) nz[c] = lane < ccnt[c] && e[c].x >= kth ? gn[e[c].y] : 0.0f;
  uint32_t bkey = 0u, bid = NONE, bad = 0u;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
#pragma clang fp contract(off)
    if (lane < ccnt[c] && e[c].x >= kth) {
      bad |= fabsf(nz[c]) < INFINITY ? 0u : 1u;
      const float tg = m.T * nz[c];
      const float sc = Key<ET>::value(e[c].x) + tg;
      const uint32_t sk = score_key(sc);
      if (sc == sc && (sk > bkey || (sk == bkey && e[c].y < bid))) {
        bkey = sk;
        bid = e[c].y;
      }
    }
  }
  const uint32_t best = wave_max_dpp(bkey);
  const uint32_t id = wave_min_dpp(bkey == best && best != 0u ? bid : NONE);
  return (__ballot(bad != 0u) != 0ull || id == NONE) ? GUMBEL_BAD_ROW : (int32_t)id;
}

// The first disagreement and the outputs of sequence b, by one wavefront:
// validity (parameters, drafts, every row's sample), the first position
// whose draft differs from the target's sample (one ballot, find-first-set),
// then the tokens, n and the per-position samples (-1 past gamma_b or for an
// invalid sequence).  target(j) is row j's sample for j <= gamma_b.
template <class TG>
__device__ __forceinline__ void gumbel_finish_wave(const Args& a, int b, TG target) {
  const int lane = threadIdx.x & 63;
  const int G = a.G, G1 = G + 1;
  const int gl = a.gamma_len ? a.gamma_len[b] : G;
  const float Tv = a.temp[b];
  const float tp = a.topp ? a.topp[b] : 1.0f;
  const int g = min(max(gl, 1), G);
  int32_t* tgt = a.out_target + (size_t)b * G1;
  const int32_t* xb = a.draft + (size_t)b * G;
  uint32_t badl = ((a.sampler || (gl >= 1 && gl <= G)) && Tv >= 0.0f && tp == tp) ? 0u : 1u;
  for (int jj = lane; jj <= g; jj += 64) badl |= target(jj) < 0 ? 1u : 0u;
  bool mism = false;
  if (lane < g) {
    const int x = xb[lane];
    badl |= (x < 0 || x >= a.V) ? 1u : 0u;
    mism = x != target(lane);
  }
  const bool ok = __ballot(badl != 0u) == 0ull;
  const unsigned long long mask = __ballot(mism);
  const int n = mask ? __ffsll((long long)mask) - 1 : g;
  const int32_t tok = ok ? target(n) : -1;
  int32_t* ot = a.out_tokens + (size_t)b * G1;
  for (int jj = lane; jj <= G; jj += 64) {
    ot[jj] = ok ? (jj < n ? xb[jj] : (jj == n ? tok : -1)) : -1;
    if (!ok || jj > g) tgt[jj] = -1;
  }
  if (lane == 0) {
    if (a.out_n) a.out_n[b] = ok ? n : -1;
    a.seq_flags[b] = 0;
  }
}

// The list kernel's LDS: the LDS list path's, or (calls it finishes) the
// whole-workgroup row path's.
template <int NTP>
constexpr size_t gumbel_pair_stream_offset() {
  return (sizeof(PairSmem<NTP>) + 15) / 16 * 16;
}
constexpr size_t gumbel_list_smem_bytes() {
  return sizeof(FinSmem) > gumbel_pair_stream_offset<NT>() + sizeof(PairStream)
             ? sizeof(FinSmem)
             : gumbel_pair_stream_offset<NT>() + sizeof(PairStream);
}

// Argmax and top-k (<= KMAX_SPARSE) sequences from the streaming select's
// survivor lists: one workgroup per sequence.  Every row's kept set (the
// union of its part lists cut to the k-th largest, then to the nucleus when
// top_p < 1) is built in LDS as by the verify's finisher; one wavefront per
// row then takes the lowest-id argmax of fl(z + fl(T * g)) over it, reading
// the noise only at the kept ids.  Sequences whose lists do not fit are
// marked demoted and left to gumbel_kernel, which runs next.  Top-k
// sequences without top-p and argmax sequences whose part lists fit in
// registers take the register path first: wavefront r takes row r
// (gumbel_row_fast), with no block barrier unless some row does not fit,
// which sends the whole sequence to the LDS path.
//
// With a.gfuse (calls promised to hold no dense sequence) this launch is
// the last of the call: dense, invalid and demoted sequences get their rows
// from the whole workgroup here (gumbel_row_block, one row after another),
// and every sequence is finished here (gumbel_finish_wave).  So it is with
// a.gmix, where gumbel_mixed_kernel has already sampled the histogram rows:
// those samples are taken as they are, unless a count overflowed there.
template <typename ET, bool VECTOR>
__global__ __launch_bounds__(NT) void gumbel_list_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char gl_smem[];
  FinSmem& s = *reinterpret_cast<FinSmem*>(gl_smem);
  __shared__ int32_t ftok[SV_MAX_GAMMA + 1];   // a.gfuse: every row's sample
  const int b = blockIdx.x;
  const int G = a.G, RS = a.RS, V = a.V;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // wavefront-uniform
  const int lane = threadIdx.x & 63;
  // The register path's lists, fetched with the parameters: wavefront w <= G
  // takes row w's first 64 entries of each part (parts <= GUMBEL_CH), and
  // lane p the part's list size.  Every list has SEG >= 64 * GUMBEL_CH slots.
  const bool fastc = a.NP <= GUMBEL_CH && G < NWAVE && wave <= G;
  uint2 f0[GUMBEL_CH];
  uint32_t fcnt = 0;
  const uint2* lpw = a.lists + list_index(a, b * RS + (fastc ? wave : 0), 0);
#pragma unroll
  for (int p = 0; p < GUMBEL_CH; ++p) f0[p] = make_uint2(0u, 0u);
  if (fastc) {
#pragma unroll
    for (int p = 0; p < GUMBEL_CH; ++p)
      if (p < a.NP) f0[p] = lpw[(size_t)p * SEG + lane];
    if (lane < a.NP) fcnt = (uint32_t)a.counts[((size_t)b * RS + wave) * a.NP + lane];
  }
  const Mode m = seq_mode(a, b);
  const uint32_t fl = a.seq_flags[b];
  const bool fuse = a.gfuse != 0 || a.gmix != 0;
  const int R = m.g + 1;
  const int NS = R * a.NP;
  int32_t* tgt = a.out_target + (size_t)b * (G + 1);
  // Where the sequence's rows come from (block-uniform).
  enum { ROWS_LIST, ROWS_BLOCK, ROWS_BAD };
  int src = ROWS_LIST;
  if (m.mode != MODE_GREEDY && m.mode != MODE_SPARSE) src = ROWS_BLOCK;
  else if (fl & F_DEMOTE) src = ROWS_BLOCK;
  else if (fl & F_BAD) src = ROWS_BAD;
  else if (NS > MAXSEG) {
    if (!fuse && threadIdx.x == 0) a.seq_flags[b] = fl | F_DEMOTE;
    src = ROWS_BLOCK;
  }
  if (src == ROWS_BLOCK && !fuse) return;   // gumbel_kernel takes it
  if (src == ROWS_BAD) {
    for (int j = threadIdx.x; j < R; j += NT) {
      tgt[j] = GUMBEL_BAD_ROW;
      ftok[j] = GUMBEL_BAD_ROW;
    }
  }
  bool listed = false;   // every row's sample found from the lists (block-uniform)
  if (src == ROWS_LIST && a.NP <= GUMBEL_CH && G < NWAVE && (m.mode == MODE_GREEDY || !(m.tp < 1.0f))) {
    bool fits = true;
    if (wave < R) {
      int32_t tok;
      switch (a.NP) {
        case 1: tok = gumbel_row_fast<ET, 1>(a, s, m, b, wave, f0, fcnt, lpw, &fits); break;
        case 2: tok = gumbel_row_fast<ET, 2>(a, s, m, b, wave, f0, fcnt, lpw, &fits); break;
        case 3: tok = gumbel_row_fast<ET, 3>(a, s, m, b, wave, f0, fcnt, lpw, &fits); break;
        case 4: tok = gumbel_row_fast<ET, 4>(a, s, m, b, wave, f0, fcnt, lpw, &fits); break;
        case 5: tok = gumbel_row_fast<ET, 5>(a, s, m, b, wave, f0, fcnt, lpw, &fits); break;
        case 6: tok = gumbel_row_fast<ET, 6>(a, s, m, b, wave, f0, fcnt, lpw, &fits); break;
        case 7: tok = gumbel_row_fast<ET, 7>(a, s, m, b, wave, f0, fcnt, lpw, &fits); break;
        default: tok = gumbel_row_fast<ET, 8>(a, s, m, b, wave, f0, fcnt, lpw, &fits); break;
      }
      if (fits && lane == 0) {
        tgt[wave] = tok;
        ftok[wave] = tok;
      }
    }
    if (lane == 0) s.fflag[wave] = fits ? 0u : 1u;
    __syncthreads();
    uint32_t any = 0;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) any |= s.fflag[w];
    listed = any == 0u;
    __syncthreads();   // the LDS path below reuses the memory
  }
  if (src == ROWS_LIST && !listed) {
    uint32_t c = 0;
    if ((int)threadIdx.x < NS) c = (uint32_t)max(a.counts[(size_t)b * RS * a.NP + threadIdx.x], 0);
    uint32_t total = 0;
    const uint32_t excl = block_excl_scan(c, s.red_u, &total);
    if (total > (uint32_t)POOL) {   // does not fit in LDS
      if (!fuse) {
        if (threadIdx.x == 0) a.seq_flags[b] = fl | F_DEMOTE;
        return;
      }
      src = ROWS_BLOCK;
    } else {
      if ((int)threadIdx.x < NS) s.soff[threadIdx.x] = excl;
      if (threadIdx.x == 0) s.soff[NS] = total;
      __syncthreads();
      for (int r = threadIdx.x; r <= R; r += NT) s.off[r] = s.soff[r * a.NP];
      for (uint32_t e = threadIdx.x; e < total; e += NT) {
        int lo = 0, hi = NS;   // list with soff[lo] <= e < soff[lo+1]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s.soff[mid] <= e) lo = mid;
          else hi = mid;
        }
        const int r = lo / a.NP, p = lo - r * a.NP;
        s.pool[e] = a.lists[list_index(a, b * RS + r, p) + (e - s.soff[lo])];
      }
      __syncthreads();
      for (int r = wave; r < R; r += NWAVE) {
        if (s.off[r + 1] > s.off[r]) pool_row_stats<ET>(s, r, m, a.NP);
      }
      __syncthreads();
      for (int r = wave; r < R; r += NWAVE) {
        int32_t tok;
        if (s.off[r + 1] == s.off[r]) {
          tok = GUMBEL_BAD_ROW;   // no finite logit
        } else if (m.mode == MODE_GREEDY) {
          tok = (int32_t)s.st_arg[r];
        } else {
          const int o = (int)s.off[r], n = (int)s.st_cnt[r];
          const float* gn = a.noise + ((size_t)b * (G + 1) + r) * (size_t)V;
          uint32_t bkey = 0, bid = NONE, bad = 0;
          for (int j = lane; j < n; j += 64) {
#pragma clang fp contract(off)
            const uint2 e = s.pool[o + j];
            const float nz = gn[e.y];
            bad |= fabsf(nz) < INFINITY ? 0u : 1u;
            const float tg = m.T * nz;
            const float sc = Key<ET>::value(e.x) + tg;
            const uint32_t sk = score_key(sc);
            if (sc == sc && (sk > bkey || (sk == bkey && e.y < bid))) {
              bkey = sk;
              bid = e.y;
            }
          }
          const uint32_t best = wave_max_dpp(bkey);
          const uint32_t id = wave_min_dpp(bkey == best && best != 0u ? bid : NONE);
          bad = __ballot(bad != 0u) ? 1u : 0u;
          tok = (bad || id == NONE) ? GUMBEL_BAD_ROW : (int32_t)id;
        }
        if (lane == 0) {
          tgt[r] = tok;
          ftok[r] = tok;
        }
      }
    }
  }
  if (!fuse) return;
  if (src == ROWS_BLOCK) {
    // The workgroup takes the rows one after another; under a.gmix the rows
    // gumbel_mixed_kernel sampled are first taken as they are, all at once.
    constexpr int32_t NEED = INT32_MIN;
    __syncthreads();   // the LDS above is free
    for (int j = threadIdx.x; j < R; j += NT)
      ftok[j] = a.gmix && gumbel_hist_takes(a, b, j) && tgt[j] != GUMBEL_REDO ? tgt[j] : NEED;
    __syncthreads();
    PairSmem<NT>& ps_s = *reinterpret_cast<PairSmem<NT>*>(gl_smem);
    PairStream& ps_x = *reinterpret_cast<PairStream*>(gl_smem + gumbel_pair_stream_offset<NT>());
    for (int j = 0; j < R; ++j) {
      if (ftok[j] != NEED) continue;   // block-uniform
      const int32_t tok = gumbel_row_block<ET, NT, VECTOR>(a, ps_s, ps_x, b, j);
      if (threadIdx.x == 0) {
        tgt[j] = tok;
        ftok[j] = tok;
      }
      __syncthreads();   // the next row reuses the LDS, and ftok[j] is published
    }
  }
  __syncthreads();   // publishes ftok
  if (wave == 0) gumbel_finish_wave(a, b, [&](int j) { return ftok[j]; });
  if (b == 0 && threadIdx.x == 0 && a.gmix) {   // gumbel_mixed_kernel's counters
    a.dense_count[2] = 0;
    a.dense_count[3] = 0;
  }
}

// One wavefront per sequence: validity, the first disagreement between the
// drafts and the target's samples (one ballot, find-first-set), outputs.
__global__ __launch_bounds__(256) void gumbel_finish_kernel(Args a) {
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.x * 4 + wave;
  if (b >= a.B) return;
  if (b == 0 && threadIdx.x == 0 && a.ghist) {   // the histogram rows' counter, the select groups' counter
    a.dense_count[2] = 0;
    a.dense_count[3] = 0;
  }
  const int32_t* tgt = a.out_target + (size_t)b * (a.G + 1);
  gumbel_finish_wave(a, b, [&](int j) { return tgt[j]; });
}

}  // namespace sv
