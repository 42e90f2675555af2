// Multi-candidate verify: K-SEQ at every node of the candidate tree, then
// the SpecTr walk ("SpecTr: Fast Speculative Decoding via Optimal Transport",
// mtandhj.com, sections "K-SEQ", "Residual distribution", "SpecTr").  That
// page names the draft p and the target q; here p is the target and q the
// draft:
//   a_rho(x) = min(1, p(x) / (rho q(x))),  m_rho(x) = min(q(x), p(x) / rho),
//   beta(rho) = sum_x m_rho(x),  P_A = 1 - (1 - beta)^k,
//   rho* = the smallest rho in [1, k] with rho beta(rho) >= 1 - (1 - beta(rho))^k,
//   residual weights max(0, p(x) - (P_A / beta) m_rho*(x)) (p itself when beta = 0
//   or when they sum to zero).
// The k candidates of a node are tested in order with u[0..k-1] (accept iff
// u_i < a); if all are rejected the output is the inverse-CDF draw over
// ascending id from the residual at u[k].
//
// kseq_node_kernel: one workgroup per (depth j, candidate c, sequence).  The
// node of depth j holds the candidates whose first j tokens equal candidate
// c's; only the lowest-numbered member of that class (the representative)
// computes it.  Its rows are P[b][c][j] (target after that prefix) and
// Q[b][c][j] (draft); depth L is the bonus node, a draw from P[b][c][L] at
// u[L][0].  Rows of up to 64 KB are held in LDS, longer rows are read from
// global memory on each pass.  rho* comes from one pass that bins the ratios
// p / q with their masses (g is exact at every bin boundary), then one pass
// that lists the elements of the bracket bin, then bracket steps on that
// list alone (g(rho) is non-decreasing in rho); a bracket too full for the
// list takes further listing passes.
// A call runs the node kernel twice.  The first launch (kphase 1) computes
// the nodes of classes of two or more candidates and defers the others: a
// single-candidate node is needed only if the walk reaches it, and from
// there on the walk follows that one candidate.  A first walk finds, per
// sequence, the first deferred node it reaches; the second launch (kphase 2)
// computes that candidate's nodes from that depth to L, at most L + 1 per
// sequence instead of every single-candidate node of the tree.
// spectr_walk_kernel: one wavefront per sequence (candidates and node outputs
// staged in LDS) follows the output through the nodes: at depth j the node of
// the current class gives Y; the class shrinks, by a ballot over the
// candidates, to those whose j-th token is Y; the round ends at the first
// depth whose output is no candidate, or with the bonus node after depth L.
#pragma once

#include "sv_pair.h"

namespace sv {

constexpr int KSEQ_NT = 1024;
constexpr int KSEQ_MAXK = 64;
constexpr int KSEQ_NPT = 8;       // points of the rho* bracket evaluated per pass
constexpr int KSEQ_PASSES = 24;   // bracket steps (over the rows: (KSEQ_NPT + 1)-fold, on the list: 65-fold)
constexpr int KSEQ_NG = 1536;     // listed elements of the bracket (LDS)
constexpr int KSEQ_NB = 768;      // ratio bins of the first pass (share the list's LDS)
constexpr int KSEQ_UR = 4;        // units per row whose loads a thread issues together on the first pass
constexpr int32_t KSEQ_BAD = -2;
constexpr int32_t KSEQ_DEFER = -3;   // a single-candidate node left for the pending-chain launch

// x^n for 0 <= n <= 64 by repeated squaring (a few dependent multiplies
// instead of a general power's logarithm and exponential).
__device__ __forceinline__ double ipow(double x, int n) {
  double r = 1.0;
  while (n) {
    if (n & 1) r *= x;
    x *= x;
    n >>= 1;
  }
  return r;
}

// Inverse-CDF draw over ascending id from per-element weights w(idx, rawp,
// rawq) >= 0 (block-wide).  Tiles of NTP units: one pass leaves per-(tile,
// wavefront) sums, wavefront 0 finds the crossing tile, and only that tile is
// read again.  Returns the token, or -1 when the weights sum to zero.
template <typename ET, int NTP, bool VECTOR, class W>
__device__ __forceinline__ int block_draw(const typename PT<ET, VECTOR>::U* P, const typename PT<ET, VECTOR>::U* Q,
                                          int NU, double u, W wfn, PairSmem<NTP>& s) {
  using T = PT<ET, VECTOR>;
  using U = typename T::U;
  constexpr int E = T::E;
  constexpr int NW = NTP / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ntile = (NU + NTP - 1) / NTP;
  auto unit_weights = [&](int ui, float* w) {
    const U up = P[ui], uq = Q[ui];
    uint32_t rq[E];
    T::each(uq, [&](int e, uint32_t raw) { rq[e] = raw; });
    T::each(up, [&](int e, uint32_t raw) { w[e] = wfn(ui * E + e, raw, rq[e]); });
  };
  __syncthreads();
  for (int t = 0; t < ntile; ++t) {
    const int ui = t * NTP + (int)threadIdx.x;
    float r = 0.0f;
    if (ui < NU) {
      float w[E];
      unit_weights(ui, w);
#pragma unroll
      for (int e = 0; e < E; ++e) r += w[e];
    }
    const double ws = wave_sum_dpp((double)r);
    if (lane == 0) s.part[t][wave] = ws;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    double tt = 0.0;
    if (lane < ntile) {
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) tt += s.part[lane][w2];
    }
    const double incl = wave_incl_scan_f64(tt);
    const double Z = readlane_f64(incl, 63);
    const double target = u * Z;
    const unsigned long long hit = __ballot(lane < ntile && incl > target);
    const int jt = hit ? __ffsll((long long)hit) - 1 : ntile - 1;
    if (lane == jt) {
      s.bc[0] = (uint32_t)jt;
      s.bd[0] = incl - tt;
    }
    if (lane == 0) s.bd[1] = Z > 0.0 ? target : -1.0;
  }
  __syncthreads();
  const int tj = (int)s.bc[0];
  const double base = s.bd[0], target = s.bd[1];
  __syncthreads();
  if (!(target >= 0.0)) return -1;
  uint32_t hitpos = 0xFFFFFFFFu, lastpos = 0;
  {
    const int ui = tj * NTP + (int)threadIdx.x;
    float w[E];
#pragma unroll
    for (int e = 0; e < E; ++e) w[e] = 0.0f;
    float r = 0.0f;
    if (ui < NU) {
      unit_weights(ui, w);
#pragma unroll
      for (int e = 0; e < E; ++e) r += w[e];
    }
    const double rd = (double)r;
    const double incl = wave_incl_scan_f64(rd);
    double cum = base;
    for (int w2 = 0; w2 < wave; ++w2) cum += s.part[tj][w2];
    cum += incl - rd;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      cum += (double)w[e];
      const uint32_t idx = (uint32_t)(ui * E + e);
      if (hitpos == 0xFFFFFFFFu && w[e] > 0.0f && cum > target) hitpos = idx;
      if (w[e] > 0.0f) lastpos = idx + 1u;
    }
  }
  hitpos = pb_min<NTP>(hitpos, s.red_u);
  if (hitpos != 0xFFFFFFFFu) return (int)hitpos;
  return (int)pb_max<NTP>(lastpos, s.red_u) - 1;   // rounding left no crossing
}

template <typename ET, int NTP, bool VECTOR, bool LDSR>
__global__ __launch_bounds__(NTP) void kseq_node_kernel(Args a) {
  using T = PT<ET, VECTOR>;
  using U = typename T::U;
  constexpr int E = T::E;
  extern __shared__ __align__(16) unsigned char kseq_rows[];
  __shared__ PairSmem<NTP> s;
  __shared__ PairExtra<LDSR> ps;
  __shared__ int32_t cands[KSEQ_MAXK];
  __shared__ uint32_t kcount;
  __shared__ int32_t result;
  __shared__ double gred[NTP / 64][KSEQ_NPT];
  __shared__ double rr[KSEQ_NPT], gg[KSEQ_NPT], bb[KSEQ_NPT];
  __shared__ double brk[3];   // lo, hi, beta(hi)
  __shared__ union {
    struct {
      float p[KSEQ_NG], q[KSEQ_NG];   // listed (p, q) of the bracket's elements
    } l;
    struct {
      double p[KSEQ_NB], q[KSEQ_NB];  // the first pass's p and q mass per ratio bin
    } h;
  } gx;
  __shared__ int32_t bins_root;       // the first bin boundary with g >= 0 (KSEQ_NB: none below k)
  __shared__ uint32_t gcount;
  __shared__ double gout[2];  // p and q mass of the elements above the listing bracket
  const int K = a.K, L = a.L, L1 = L + 1;
  // Grid order (depth, candidate, sequence): the shallow nodes, where
  // candidates still share prefixes and the rho* search runs, start first
  // and the cheap deep and bonus nodes fill in behind them.  The sequence
  // varies fastest, so the workgroups dealt round-robin to the chip's
  // partitions mix sequences rather than candidate numbers (the lowest
  // candidate of a class is its representative, so a candidate-major deal
  // would pile the work on one partition).
  int j, c, b;
  if (a.kphase == 2) {
    // One workgroup per (depth, sequence): the node of depth j on the chain
    // of the candidate at whose single-candidate node the first walk stopped
    // (out_n[b] = c (L + 1) + j0 between the launches), for every j >= j0.
    j = blockIdx.x / a.B;
    b = blockIdx.x - j * a.B;
    const int32_t pend = a.out_n[b];
    if (pend < 0) return;
    c = pend / L1;
    if (j < pend - c * L1) return;
  } else {
    j = blockIdx.x / (a.B * K);
    const int rem = blockIdx.x - j * a.B * K;
    c = rem / a.B;
    b = rem - (rem / a.B) * a.B;
  }
  int32_t* outp = a.node_tok + ((size_t)b * K + c) * L1 + j;
  const int32_t* cb = a.cand + (size_t)b * K * L;
  // The node's class: candidates whose first j tokens equal candidate c's.
  if (threadIdx.x < 64) {
    const int t = threadIdx.x;
    bool same = false;
    if (t < K) {
      same = true;
      for (int jj = 0; jj < j; ++jj) same = same && cb[t * L + jj] == cb[c * L + jj];
    }
    const unsigned long long m = __ballot(same);
    const int rep = __ffsll((long long)m) - 1;
    if (t == 0) kcount = rep == c ? (uint32_t)__popcll(m) : 0u;
    if (same && j < L) cands[__popcll(m & ((1ull << t) - 1ull))] = cb[t * L + j];
  }
  __syncthreads();
  const int k = (int)kcount;
  if (k == 0) {   // another member of the class computes this node
    if (threadIdx.x == 0) *outp = -1;
    return;
  }
  if (k == 1 && a.kphase == 1) {   // computed later if the walk reaches it
    if (threadIdx.x == 0) *outp = KSEQ_DEFER;
    return;
  }
  const float Tv = a.temp[b];
  const int kk = a.topk ? a.topk[b] : 0;
  const float tp = a.topp ? a.topp[b] : 1.0f;
  if (!(Tv >= 0.0f) || tp != tp) {
    if (threadIdx.x == 0) *outp = KSEQ_BAD;
    return;
  }
  const bool bonus = j == L;
  const int V = a.V;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int NU = VECTOR ? V / E : V;
  const U* gp = reinterpret_cast<const U*>(reinterpret_cast<const ET*>(a.p) + (((size_t)b * K + c) * L1 + j) * (size_t)V);
  const U* gq = bonus ? gp : reinterpret_cast<const U*>(reinterpret_cast<const ET*>(a.q) + (((size_t)b * K + c) * L + j) * (size_t)V);
  const float* uj = a.u + ((size_t)b * L1 + j) * (K + 1);

  // Pass 1: validity, maxima and (for T = 0) the lowest-id argmax of each
  // row; rows of up to 64 KB are copied to LDS on the way.  Unfiltered rows
  // at T > 0 also get their normaliser in this pass: each thread keeps a
  // running maximum m and the sum of 2^((z - m) c) over its elements,
  // rescaled when m grows (one exponential per element: 2^(-|z - m| c) is the
  // new term or the rescale factor), and the block combines the sums at the
  // row maximum.  Each thread issues the loads of up to KSEQ_UR units per row
  // before it examines any of them.
  const U* P;
  const U* Q;
  const bool greedy = Tv == 0.0f;
  const bool online = !greedy && !(kk > 0 && kk < V) && !(tp < 1.0f);
  const float cT = greedy ? 1.0f : LOG2E_F / Tv;
  uint32_t bad = 0, kmp = 0, kmq = 0, ip = NONE, iq = NONE;
  float mp = -INFINITY, smp = 0.0f, mq = -INFINITY, smq = 0.0f;
  // The lowest-id argmax is tracked on keys at T = 0 only; otherwise the
  // running maximum is a float and its key is taken once per thread.
  auto scan = [&](const U& u, int ui, uint32_t& km, uint32_t& im, float& mo, float& so) {
    T::each(u, [&](int e, uint32_t raw) {
      const float z = T::val(raw);
      bad |= z < INFINITY ? 0u : 1u;
      if (greedy) {
        const uint32_t kz = T::key(raw);
        if (kz > km) {
          km = kz;
          im = (uint32_t)(ui * E + e);
        }
      } else if (online) {
        const float d = (z - mo) * cT;
        const float ex = z > -INFINITY ? __builtin_amdgcn_exp2f(-fabsf(d)) : 0.0f;
        so = d > 0.0f ? fmaf(so, ex, 1.0f) : so + ex;
        mo = fmaxf(mo, z);
      } else {
        mo = fmaxf(mo, z);
      }
    });
  };
  {
    U* lp = reinterpret_cast<U*>(kseq_rows);
    U* lq = lp;
    if constexpr (LDSR) lq = lp + (NU * (int)sizeof(U) + 15) / 16 * 16 / (int)sizeof(U);
    for (int u0 = 0; u0 < NU; u0 += KSEQ_UR * NTP) {
      U pu[KSEQ_UR], qu[KSEQ_UR];
      // Unconditional loads (an index past the row reads its last unit, which
      // is then skipped) keep all of them in flight together.
#pragma unroll
      for (int r = 0; r < KSEQ_UR; ++r) {
        const int ui = min(u0 + r * NTP + (int)threadIdx.x, NU - 1);
        pu[r] = gp[ui];
        qu[r] = gq[ui];
      }
#pragma unroll
      for (int r = 0; r < KSEQ_UR; ++r) {
        const int ui = u0 + r * NTP + (int)threadIdx.x;
        if (ui < NU) {
          if constexpr (LDSR) lp[ui] = pu[r];
          scan(pu[r], ui, kmp, ip, mp, smp);
          if (!bonus) {
            if constexpr (LDSR) lq[ui] = qu[r];
            scan(qu[r], ui, kmq, iq, mq, smq);
          }
        }
      }
    }
    if constexpr (LDSR) {
      P = lp;
      Q = bonus ? lp : lq;
    } else {
      P = gp;
      Q = gq;
    }
  }
  if (!greedy) {   // NaN never enters the float maxima (it marks the row bad)
    kmp = key_of_value<ET>(mp);
    kmq = bonus ? 0u : key_of_value<ET>(mq);
  }
  const uint32_t my_kmp = kmp, my_kmq = kmq;
  pb_max3<NTP>(kmp, kmq, bad, s.red_u);   // its barriers also publish the LDS rows
  if (bad || kmp <= Key<ET>::NEG_INF || (!bonus && kmq <= Key<ET>::NEG_INF)) {
    if (threadIdx.x == 0) *outp = KSEQ_BAD;
    return;
  }
  uint32_t argp = 0, argq = 0;
  if (greedy) {
    argp = pb_min<NTP>(my_kmp == kmp ? ip : NONE, s.red_u);
    argq = bonus ? 0u : pb_min<NTP>(my_kmq == kmq ? iq : NONE, s.red_u);
  }
  Mode m;
  m.g = 1;
  m.mode = MODE_DENSE;
  m.k = 0;
  m.T = greedy ? 1.0f : Tv;
  m.tp = tp;
  RowStat sp{}, sq{};
  if (online) {
    // The threads' sums at the row maxima (a thread that saw no finite
    // logit holds 0), summed over the block in double.
    const float zmp = Key<ET>::value(kmp), zmq = bonus ? 0.0f : Key<ET>::value(kmq);
    const double vp = wave_sum_dpp((double)(smp * __builtin_amdgcn_exp2f((mp - zmp) * cT)));
    const double vq = bonus ? 0.0 : wave_sum_dpp((double)(smq * __builtin_amdgcn_exp2f((mq - zmq) * cT)));
    if (lane == 0) {
      s.part[0][wave] = vp;
      s.part[1][wave] = vq;
    }
    __syncthreads();
    double Sp = 0.0, Sq = 0.0;
    for (int w2 = 0; w2 < NTP / 64; ++w2) {
      Sp += s.part[0][w2];
      Sq += s.part[1][w2];
    }
    sp = RowStat{-INFINITY, zmp, cT, (float)(1.0 / Sp)};
    sq = bonus ? sp : RowStat{-INFINITY, zmq, cT, (float)(1.0 / Sq)};
  } else if (!greedy) {
    sp = row_stats<ET, NTP, VECTOR, LDSR>(P, NU, Key<ET>::value(kmp), a, m, kk, s, ps);
    if (!bonus) sq = row_stats<ET, NTP, VECTOR, LDSR>(Q, NU, Key<ET>::value(kmq), a, m, kk, s, ps);
  }
  auto prob_p = [&](uint32_t idx, uint32_t raw) -> float {
    return greedy ? (idx == argp ? 1.0f : 0.0f) : pprob(sp, T::val(raw));
  };
  auto prob_q = [&](uint32_t idx, uint32_t raw) -> float {
    return greedy ? (idx == argq ? 1.0f : 0.0f) : pprob(sq, T::val(raw));
  };

  if (bonus) {
    const int tok = block_draw<ET, NTP, VECTOR>(
        P, Q, NU, (double)uj[0], [&](uint32_t idx, uint32_t rp, uint32_t) { return prob_p(idx, rp); }, s);
    if (threadIdx.x == 0) *outp = tok;
    return;
  }

  // The root condition rho beta(rho) >= 1 - (1 - beta(rho))^k is evaluated
  // without cancellation: with D(rho) = sum_x max(0, p(x) - rho q(x)) =
  // 1 - rho beta(rho), it reads (1 - beta)^k >= D, and beta = (1 - D) / rho.
  // For large k, (1 - beta)^k drops below the rounding of rho beta - 1 near
  // the root, whereas D is a sum of non-negative terms that is exactly 0 once
  // every element is saturated (rho q >= p).  g(rho) = (1 - beta)^k - D at
  // the KSEQ_NPT values rr[] in one pass over the rows (per-thread float
  // sums, block sums in double); results in gg[], bb[] (beta).
  // With gather set, the pass also splits the elements by their ratio
  // r = p / q against the current bracket [glo, ghi]: r >= ghi contributes
  // p - rho q for every rho in the bracket (p summed into gout[0], q into
  // gout[1]), r <= glo contributes 0, and the elements in between are listed
  // in LDS (up to KSEQ_NG; gcount counts them all).
  auto g_multi = [&](bool gather, float glo, float ghi) {
    float rf[KSEQ_NPT], acc[KSEQ_NPT];
#pragma unroll
    for (int m2 = 0; m2 < KSEQ_NPT; ++m2) {
      rf[m2] = (float)rr[m2];
      acc[m2] = 0.0f;
    }
    float ao = 0.0f, bo = 0.0f;
    bool glive = gather;   // wavefront-uniform: cleared once the list has overflowed
    for (int ui = threadIdx.x; ui < NU; ui += NTP) {
      const U up = P[ui], uq = Q[ui];
      uint32_t rq[E];
      T::each(uq, [&](int e, uint32_t raw) { rq[e] = raw; });
      uint32_t inm = 0;   // bit e: element e of the unit lies inside the bracket
      T::each(up, [&](int e, uint32_t raw) {
        const uint32_t idx = (uint32_t)(ui * E + e);
        const float pv = prob_p(idx, raw), qv = prob_q(idx, rq[e]);
#pragma unroll
        for (int m2 = 0; m2 < KSEQ_NPT; ++m2) acc[m2] += fmaxf(fmaf(-rf[m2], qv, pv), 0.0f);
        if (gather) {
          const bool above = pv >= qv * ghi, below = !above && pv <= qv * glo;
          ao += above ? pv : 0.0f;
          bo += above ? qv : 0.0f;
          inm |= (!above && !below) ? (1u << e) : 0u;
        }
      });
      if (glive) {
        // One LDS atomic per unit and wavefront: the lanes' counts (<= E <= 8)
        // are prefix-summed bit by bit over ballots.
        const uint32_t cnt = (uint32_t)__popc(inm);
        const unsigned long long below_lane = (1ull << lane) - 1ull;
        uint32_t pre = 0, tot = 0;
#pragma unroll
        for (int bit = 0; bit < 4; ++bit) {
          const unsigned long long bl = __ballot((cnt >> bit) & 1u);
          pre += (uint32_t)__popcll(bl & below_lane) << bit;
          tot += (uint32_t)__popcll(bl) << bit;
        }
        if (tot) {
          const int leader = __ffsll((long long)__ballot(true)) - 1;
          uint32_t base = 0;
          if (lane == leader) base = atomicAdd(&gcount, tot);
          base = (uint32_t)__shfl((int)base, leader, 64);
          uint32_t slot = base + pre;
          while (inm) {   // the listed elements again (few once the bracket is narrow)
            const int e = __builtin_ctz(inm);
            inm &= inm - 1u;
            if (slot < (uint32_t)KSEQ_NG) {
              uint32_t rp = 0, rqe = 0;
              T::each(up, [&](int e2, uint32_t raw) { rp = e2 == e ? raw : rp; });
              T::each(uq, [&](int e2, uint32_t raw) { rqe = e2 == e ? raw : rqe; });
              const uint32_t idx = (uint32_t)(ui * E + e);
              gx.l.p[slot] = prob_p(idx, rp);
              gx.l.q[slot] = prob_q(idx, rqe);
            }
            ++slot;
          }
          if (base + tot > (uint32_t)KSEQ_NG) glive = false;
        }
      }
    }
#pragma unroll
    for (int m2 = 0; m2 < KSEQ_NPT; ++m2) {
      const double w = wave_sum_dpp((double)acc[m2]);
      if (lane == 0) gred[wave][m2] = w;
    }
    if (gather) {
      const double wa = wave_sum_dpp((double)ao), wb = wave_sum_dpp((double)bo);
      if (lane == 0) {
        s.part[0][wave] = wa;
        s.part[1][wave] = wb;
      }
    }
    __syncthreads();
    if (threadIdx.x < KSEQ_NPT) {
      const int m2 = threadIdx.x;
      double dsum = 0.0;
      for (int w2 = 0; w2 < NTP / 64; ++w2) dsum += gred[w2][m2];
      const double bsum = (1.0 - dsum) / rr[m2];
      bb[m2] = bsum;
      gg[m2] = ipow(1.0 - bsum, k) - dsum;
    }
    if (gather && threadIdx.x == 64) {
      double sa = 0.0, sb = 0.0;
      for (int w2 = 0; w2 < NTP / 64; ++w2) {
        sa += s.part[0][w2];
        sb += s.part[1][w2];
      }
      gout[0] = sa;
      gout[1] = sb;
    }
    __syncthreads();
  };
  // One step on the listed elements: 64 points spread over the bracket, one
  // per lane; wavefront w sums the lane's terms over list entries w, w + 16,
  // ...; wavefront 0 adds the constant parts, evaluates g and narrows the
  // bracket to the first sub-interval where g turns non-negative.
  auto g_list = [&]() {
    const double lo = brk[0], hi = brk[1];
    const double rm = lo + (hi - lo) * (double)(lane + 1) / 65.0;
    const float rmf = (float)rm;
    const uint32_t n = min(gcount, (uint32_t)KSEQ_NG);
    float acc = 0.0f;
    for (uint32_t jl = (uint32_t)wave; jl < n; jl += NTP / 64) acc += fmaxf(fmaf(-rmf, gx.l.q[jl], gx.l.p[jl]), 0.0f);
    s.part[lane][wave] = (double)acc;
    __syncthreads();
    if (threadIdx.x < 64) {
      double dsum = fmax(gout[0] - rm * gout[1], 0.0);
      for (int w2 = 0; w2 < NTP / 64; ++w2) dsum += s.part[lane][w2];
      const double bsum = (1.0 - dsum) / rm;
      const double g = ipow(1.0 - bsum, k) - dsum;
      const unsigned long long up = __ballot(g >= 0.0);
      const int f = up ? __ffsll((long long)up) - 1 : 64;
      if (lane == f) {
        brk[1] = rm;
        brk[2] = bsum;
      }
      if (f > 0 && lane == f - 1) brk[0] = rm;
    }
    __syncthreads();
  };
  // rho*: the smallest root of the non-decreasing g on [1, k].  With one
  // candidate g(1) = beta - (1 - (1 - beta)) = 0, so rho* = 1, the acceptance
  // is min(1, p / q) and the residual max(0, p - q): beta is never needed
  // (P_A / beta = 1 stands for it).  Otherwise the first pass tries rho = 1
  // and spreads the other points up to k; later passes over the rows split
  // the bracket (lo: g < 0, hi: g >= 0) into KSEQ_NPT + 1 parts and list the
  // elements whose ratio lies inside it; once the list holds all of them,
  // the remaining steps run on the list alone.
  // The bracket in one pass: the elements with 1 < r = p / q < k go to
  // KSEQ_NB bins of log_k r (bin i: r in [rho_i, rho_{i+1}), rho_i =
  // k^(i / KSEQ_NB)), their p and q summed per bin (double LDS atomics); the
  // elements with r >= k (q = 0 included) are summed per thread.  Elements
  // with r <= 1 add nothing to D for rho >= 1.  Then D(rho_i) = sum over the
  // bins at or above i and the r >= k part of (p - rho_i q), exact at every
  // boundary up to the rounding of the bin assignment (an element within a
  // rounding of rho_i adds about 0 either way), and wavefront 0 evaluates g
  // at all KSEQ_NB boundaries.  The root lies at or below the first boundary
  // i* with g >= 0; the bracket [rho_{i*-2}, rho_{i*}] keeps one bin below in
  // case rounding put g(rho_{i*-1}) on the wrong side.  Sets brk and
  // bins_root (0: g(1) >= 0, so rho* = 1, with beta(1) in brk[2]).
  auto g_bins = [&]() {
    for (int i = threadIdx.x; i < KSEQ_NB; i += NTP) {
      gx.h.p[i] = 0.0;
      gx.h.q[i] = 0.0;
    }
    __syncthreads();
    const float fk = (float)k;
    const float sc = (float)KSEQ_NB / __log2f(fk);
    float ao = 0.0f, bo = 0.0f;
    for (int ui = threadIdx.x; ui < NU; ui += NTP) {
      const U up = P[ui], uq = Q[ui];
      uint32_t rq[E];
      T::each(uq, [&](int e, uint32_t raw) { rq[e] = raw; });
      T::each(up, [&](int e, uint32_t raw) {
        const uint32_t idx = (uint32_t)(ui * E + e);
        const float pv = prob_p(idx, raw), qv = prob_q(idx, rq[e]);
        if (pv > qv) {
          if (qv * fk <= pv) {
            ao += pv;
            bo += qv;
          } else {
            const int bi = min(KSEQ_NB - 1, max(0, (int)(__log2f(pv / qv) * sc)));
            atomicAdd(&gx.h.p[bi], (double)pv);
            atomicAdd(&gx.h.q[bi], (double)qv);
          }
        }
      });
    }
    const double wa = wave_sum_dpp((double)ao), wb = wave_sum_dpp((double)bo);
    if (lane == 0) {
      s.part[0][wave] = wa;
      s.part[1][wave] = wb;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      double A = 0.0, Bq = 0.0;
      for (int w2 = 0; w2 < NTP / 64; ++w2) {
        A += s.part[0][w2];
        Bq += s.part[1][w2];
      }
      constexpr int BPL = KSEQ_NB / 64;   // lane l: bins BPL l .. BPL l + BPL - 1
      double lp = 0.0, lq = 0.0;
      for (int t = 0; t < BPL; ++t) {
        lp += gx.h.p[BPL * lane + t];
        lq += gx.h.q[BPL * lane + t];
      }
      const double ip = wave_incl_scan_f64(lp), iq = wave_incl_scan_f64(lq);
      double SP = A + (readlane_f64(ip, 63) - ip), SQ = Bq + (readlane_f64(iq, 63) - iq);
      const double lk = log2((double)k);
      int first = BPL;
      double bfirst = 0.0;
      for (int t = BPL - 1; t >= 0; --t) {   // boundaries from the lane's top down, while g >= 0
        const int i = BPL * lane + t;
        SP += gx.h.p[i];
        SQ += gx.h.q[i];
        const double rho_i = exp2(lk * (double)i / KSEQ_NB);
        const double D = fmax(SP - rho_i * SQ, 0.0);
        const double be = (1.0 - D) / rho_i;
        if (!(ipow(1.0 - be, k) - D >= 0.0)) break;
        first = t;
        bfirst = be;
      }
      const unsigned long long has = __ballot(first < BPL);
      const int hl = has ? __ffsll((long long)has) - 1 : 0;
      const int rf = __builtin_amdgcn_readlane(first, hl);
      const double rb = readlane_f64(bfirst, hl);
      if (lane == 0) {
        const int root = has ? BPL * hl + rf : KSEQ_NB;
        bins_root = root;
        brk[0] = exp2(lk * (double)max(root - 2, 0) / KSEQ_NB);
        brk[1] = root >= KSEQ_NB ? (double)k : exp2(lk * (double)root / KSEQ_NB);
        brk[2] = has ? rb : (1.0 - fmax(A - (double)k * Bq, 0.0)) / (double)k;   // beta(k) when none below k
      }
    }
    __syncthreads();
  };
  double rho = 1.0, beta = 1.0;
  if (k > 1) {
    g_bins();
    beta = brk[2];
  }
  if (k > 1 && bins_root > 0) {
    bool listed = false;
    for (int pass = 0; pass < KSEQ_PASSES; ++pass) {
      const double lo = brk[0], hi = brk[1];
      if (!(hi - lo > 1e-15 * hi)) break;          // uniform: every thread reads the same brk
      if (listed) {
        g_list();
        continue;
      }
      __syncthreads();
      if (threadIdx.x < KSEQ_NPT) rr[threadIdx.x] = lo + (hi - lo) * (threadIdx.x + 1) / (KSEQ_NPT + 1);
      if (threadIdx.x == 0) gcount = 0;
      __syncthreads();
      g_multi(true, (float)lo, (float)hi);
      listed = gcount <= (uint32_t)KSEQ_NG;
      if (threadIdx.x == 0) {
        double nlo = lo;
        for (int m2 = 0; m2 < KSEQ_NPT; ++m2) {
          if (gg[m2] >= 0.0) {
            brk[1] = rr[m2];
            brk[2] = bb[m2];
            break;
          }
          nlo = rr[m2];
        }
        brk[0] = nlo;
      }
      __syncthreads();
    }
    rho = brk[1];
    beta = brk[2];
  }
  const double pacc = 1.0 - ipow(1.0 - beta, k);

  // The candidates in order.
  if (threadIdx.x == 0) {
    int y = -1;
    for (int i = 0; i < k; ++i) {
      const int x = cands[i];
      if (x < 0 || x >= V) {
        y = KSEQ_BAD;
        break;
      }
      const double px = (double)prob_p((uint32_t)x, T::raw_at(P, x));
      const double qx = (double)prob_q((uint32_t)x, T::raw_at(Q, x));
      double acc;
      if (qx == 0.0) acc = px > 0.0 ? 1.0 : 0.0;
      else acc = qx * rho <= px ? 1.0 : px / (rho * qx);
      if ((double)uj[i] < acc) {
        y = x;
        break;
      }
    }
    result = y;
  }
  __syncthreads();
  int tok = result;
  if (tok == -1) {
    const float scale = beta > 0.0 ? (float)(pacc / beta) : 0.0f;
    const float inv = (float)(1.0 / rho);
    tok = block_draw<ET, NTP, VECTOR>(
        P, Q, NU, (double)uj[k],
        [&](uint32_t idx, uint32_t rp, uint32_t rq) {
          const float pv = prob_p(idx, rp);
          if (!(beta > 0.0)) return pv;
          return fmaxf(pv - scale * fminf(prob_q(idx, rq), pv * inv), 0.0f);
        },
        s);
    if (tok < 0)   // residual weights summed to zero: draw from the target
      tok = block_draw<ET, NTP, VECTOR>(
          P, Q, NU, (double)uj[k], [&](uint32_t idx, uint32_t rp, uint32_t) { return prob_p(idx, rp); }, s);
  }
  if (threadIdx.x == 0) *outp = tok;
}

// One wavefront per sequence: the walk through the nodes.  The lanes first
// check the candidates and uniforms and stage the candidates and node
// outputs in LDS with coalesced loads; the walk then takes one ballot per
// depth (lane c tests candidate c against the node's output).
__global__ __launch_bounds__(64) void spectr_walk_kernel(Args a) {
  __shared__ int32_t cs[SV_MAX_CANDIDATES * SV_MAX_GAMMA];
  __shared__ int32_t ns[SV_MAX_CANDIDATES * (SV_MAX_GAMMA + 1)];
  __shared__ int32_t ys[SV_MAX_GAMMA + 1];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int K = a.K, L = a.L, L1 = L + 1, V = a.V;
  const float Tv = a.temp[b];
  const float tp = a.topp ? a.topp[b] : 1.0f;
  const int32_t* cb = a.cand + (size_t)b * K * L;
  const float* ub = a.u + (size_t)b * L1 * (K + 1);
  const int32_t* nt = a.node_tok + (size_t)b * K * L1;
  bool lane_ok = true;
  for (int i = lane; i < K * L; i += 64) {
    const int32_t v = cb[i];
    cs[i] = v;
    lane_ok = lane_ok && v >= 0 && v < V;
  }
  for (int i = lane; i < K * L1; i += 64) ns[i] = nt[i];
  for (int i = lane; i < L1 * (K + 1); i += 64) {
    const float u = ub[i];
    lane_ok = lane_ok && u >= 0.0f && u < 1.0f;
  }
  bool ok = Tv >= 0.0f && tp == tp && __ballot(!lane_ok) == 0ull;
  __syncthreads();
  unsigned long long alive = K >= 64 ? ~0ull : ((1ull << K) - 1ull);
  int n = L;
  // After the first node launch (kphase 1): stop at the first deferred node
  // the walk reaches and leave its chain, c (L + 1) + j, in out_n[b] for the
  // second node launch (-1: none).
  const bool first = a.kphase == 1;
  int32_t pend = -1;
  for (int j = 0; j < L && ok; ++j) {
    const int rep = __ffsll((long long)alive) - 1;
    const int y = ns[rep * L1 + j];
    if (first && y == KSEQ_DEFER) {
      pend = rep * L1 + j;
      break;
    }
    if (y < 0) {
      ok = false;
      break;
    }
    if (lane == 0) ys[j] = y;
    const unsigned long long next = __ballot(lane < K && ((alive >> lane) & 1ull) && cs[lane * L + j] == y);
    if (!next) {
      n = j;
      break;
    }
    alive = next;
  }
  if (ok && n == L && pend < 0) {
    const int rep = __ffsll((long long)alive) - 1;
    const int y = ns[rep * L1 + L];
    if (first && y == KSEQ_DEFER) pend = rep * L1 + L;
    else if (y < 0) ok = false;
    else if (lane == 0) ys[L] = y;
  }
  if (first) {
    if (lane == 0) a.out_n[b] = ok ? pend : -1;
    return;
  }
  __syncthreads();
  int32_t* ot = a.out_tokens + (size_t)b * L1;
  for (int j = lane; j < L1; j += 64) ot[j] = ok && j <= n ? ys[j] : -1;
  if (lane == 0) a.out_n[b] = ok ? n : -1;
}

}  // namespace sv
