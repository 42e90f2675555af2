// Dense pairs of unfiltered rows (T > 0, no top-k, no top-p) split over
// several workgroups: each (sequence, position) pair's rows are cut into S
// chunks, and three launches exchange per-chunk records through the
// workspace, so that a pair no longer waits on one CU:
//   split_stats_kernel   one workgroup per (pair, chunk): validity, the
//                        chunk maxima of both rows, and the sums of
//                        2^((z - m) c) at those maxima (one running maximum and
//                        sum per thread, one exponential per element);
//   split_weights_kernel the same grid (so each chunk is read again from the
//                        L2 of the XCD that read it first): the row maxima and
//                        normalisers from the pair's S records, then the
//                        chunk's overlap sum min(p, q), its residual (or, at
//                        the bonus position, target) weight sum and its target
//                        mass;
//   split_draw_kernel    one workgroup per pair: the crossing chunk of the
//                        inverse CDF at u Z in ascending id ("Sampling with
//                        shared noise", "Speculative Decoding: the art of
//                        guessing well"), then that chunk's tiles, and the
//                        pair's record (p(x), q(x), alpha, the token drawn as
//                        if the first rejection were here), as pair_kernel
//                        writes it.
// The processed distributions are those of "Fast Inference from Transformers
// via Speculative Decoding" (mtandhj.com summary), "Speculative Sampling:
// theoretical basis"; the residual max(0, p - q) and the bonus draw from p
// follow "Speculative Decoding: the art of guessing well", "Speculative
// sampling"; alpha = sum min(p, q), mtandhj summary, "How to choose gamma".
// A pair whose sequence has top-k or top-p after all (the caller's hint was
// wrong) is left to the finisher's multi-pass procedure (REC_REDO).
#pragma once

#include "sv_pair.h"

namespace sv {

constexpr int SPL_NT = 256;      // threads per workgroup of the three kernels
constexpr int SPL_NW = SPL_NT / 64;
constexpr int SPL_MAXS = 32;     // chunks per pair at most
constexpr int SPL_MIN_UNITS = 2 * SPL_NT;   // units of a row per chunk at least
constexpr int SPL_UR = 4;        // units per row a thread loads together in the first pass
constexpr int SPL_MAXTILE = 4;   // SPL_NT-unit tiles per chunk at most (the draw holds them in registers)

struct ChunkRec {
  float mp, mq;     // chunk maxima of the target and draft rows (-inf: none finite)
  double sp, sq;    // sums of 2^((z - m) c) over the chunk at those maxima
  double w;         // residual (bonus: target) weight sum of the chunk
  double al;        // overlap sum of the chunk
  double pz;        // target mass of the chunk (the draw when the residual is empty)
  uint32_t bad;     // NaN or +inf in the chunk
  uint32_t pad;
};

// The pair handled by workgroup-group t (the dense list's order, or the fixed
// order when every sequence was promised dense); -1 when t is past the list.
__device__ __forceinline__ int split_pair_id(const Args& a, uint32_t t) {
  const int G1 = a.G + 1;
  const uint32_t npairs = (uint32_t)a.B * (uint32_t)G1;
  const bool direct = a.all_dense != 0;
  const uint32_t nf = direct ? npairs : min(a.dense_count[0], npairs);
  const uint32_t nd = direct ? npairs : min(nf + a.dense_count[1], npairs);
  if (t >= nd) return -1;
  if (direct) {
    const uint32_t nlead = (uint32_t)a.B * (uint32_t)a.G;
    return t < nlead ? (int)((t / (uint32_t)a.G) * (uint32_t)G1 + t % (uint32_t)a.G)
                     : (int)((t - nlead) * (uint32_t)G1 + (uint32_t)a.G);
  }
  const uint32_t idx = t < nf ? t : npairs - 1u - (t - nf);
  const int pid = a.dense_list[idx];
  return pid >= 0 && (uint32_t)pid < npairs ? pid : -1;
}

// Unfiltered: no top-k below V and no top-p below 1.
__device__ __forceinline__ bool split_unfiltered(const Args& a, int b, const Mode& m) {
  const int k = a.topk ? a.topk[b] : 0;
  return !(k > 0 && k < a.V) && !(m.tp < 1.0f);
}

// Units [u0, u1) of chunk c of a row of NU units in S chunks.
__device__ __forceinline__ void split_range(int NU, int S, int c, int& u0, int& u1) {
  const int cu = (NU + S - 1) / S;
  u0 = min(NU, c * cu);
  u1 = min(NU, u0 + cu);
}

__device__ __forceinline__ float split_wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// The row statistics of a pair from its S (<= 64) chunk records: lane c
// reads record c and every wavefront combines them itself (block-uniform
// result, no barrier).  False when a chunk is invalid or a row has no
// finite value.
__device__ __forceinline__ bool split_combine(const ChunkRec* recs, int S, bool resid, float cT, RowStat& sp,
                                              RowStat& sq) {
  const int lane = threadIdx.x & 63;
  float mp = -INFINITY, mq = -INFINITY;
  double spc = 0.0, sqc = 0.0;
  uint32_t bad = 0;
  if (lane < S) {
    mp = recs[lane].mp;
    mq = recs[lane].mq;
    spc = recs[lane].sp;
    sqc = recs[lane].sq;
    bad = recs[lane].bad;
  }
  const float Mp = split_wave_max(mp), Mq = split_wave_max(mq);
  if (__ballot(bad != 0u) || !(Mp > -INFINITY) || (resid && !(Mq > -INFINITY))) return false;
  const double Sp = wave_sum_dpp(mp > -INFINITY ? spc * (double)__builtin_amdgcn_exp2f((mp - Mp) * cT) : 0.0);
  const double Sq =
      wave_sum_dpp(resid && mq > -INFINITY ? sqc * (double)__builtin_amdgcn_exp2f((mq - Mq) * cT) : 0.0);
  sp = RowStat{-INFINITY, Mp, cT, (float)(1.0 / Sp)};
  sq = resid ? RowStat{-INFINITY, Mq, cT, (float)(1.0 / Sq)} : sp;
  return true;
}

// Pass 1 over one chunk of both rows.
template <typename ET, bool VECTOR>
__global__ __launch_bounds__(SPL_NT) void split_stats_kernel(Args a) {
  using T = PT<ET, VECTOR>;
  using U = typename T::U;
  __shared__ float fm[2][SPL_NW];
  __shared__ double dm[2][SPL_NW];
  __shared__ uint32_t bm[SPL_NW];
  const int S = a.split_s;
  const int c = (int)(blockIdx.x % (unsigned)S);
  const int pid = split_pair_id(a, blockIdx.x / (unsigned)S);
  if (pid < 0) return;
  const int G1 = a.G + 1;
  const int b = pid / G1, i = pid - b * G1;
  const int NU = VECTOR ? a.V / T::E : a.V;
  // The chunk's first loads go out before the sequence's parameters arrive:
  // target row i <= G and draft row i < G exist for every pair id.
  const U* gp = reinterpret_cast<const U*>(row_ptr<ET>(a, b, true, i));
  const U* gq = i < a.G ? reinterpret_cast<const U*>(row_ptr<ET>(a, b, false, i)) : gp;
  int u0, u1;
  split_range(NU, S, c, u0, u1);
  U pu0[SPL_UR], qu0[SPL_UR];
#pragma unroll
  for (int r = 0; r < SPL_UR; ++r) {
    const int ui = max(0, min(u0 + r * SPL_NT + (int)threadIdx.x, u1 - 1));
    pu0[r] = gp[ui];
    qu0[r] = gq[ui];
  }
  const Mode m = seq_mode(a, b);
  if (m.mode != MODE_DENSE || i > m.g || !split_unfiltered(a, b, m)) return;
  const bool resid = i < m.g;
  const float cT = LOG2E_F / m.T;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float zmp = -INFINITY, zmq = -INFINITY, smp = 0.0f, smq = 0.0f;
  uint32_t bad = 0;
  // A running maximum and the sum of 2^((z - m) c), rescaled when m grows:
  // 2^(-|z - m| c) is the new term or the rescale factor.
  auto scan_unit = [&](const U& u, float& zm, float& sm) {
    T::each(u, [&](int, uint32_t raw) {
      const float z = T::val(raw);
      bad |= z < INFINITY ? 0u : 1u;
      const float d = (z - zm) * cT;
      const float ex = z > -INFINITY ? __builtin_amdgcn_exp2f(-fabsf(d)) : 0.0f;
      sm = d > 0.0f ? fmaf(sm, ex, 1.0f) : sm + ex;
      zm = fmaxf(zm, z);
    });
  };
  // Past the chunk: its last unit, skipped.  Ordinary loads, so that the
  // second pass finds the chunk in L2.
  for (int v0 = u0; v0 < u1; v0 += SPL_UR * SPL_NT) {
    U pu[SPL_UR], qu[SPL_UR];
#pragma unroll
    for (int r = 0; r < SPL_UR; ++r) {
      if (v0 == u0) {
        pu[r] = pu0[r];
        qu[r] = qu0[r];
      } else {
        const int ui = min(v0 + r * SPL_NT + (int)threadIdx.x, u1 - 1);
        pu[r] = gp[ui];
        qu[r] = gq[ui];
      }
    }
#pragma unroll
    for (int r = 0; r < SPL_UR; ++r) {
      if (v0 + r * SPL_NT + (int)threadIdx.x < u1) {
        scan_unit(pu[r], zmp, smp);
        if (resid) scan_unit(qu[r], zmq, smq);
      }
    }
  }
  // Block maxima, then the threads' sums at them (a thread without a finite
  // value holds 0).
  float wp = zmp, wq = zmq;
  for (int o = 32; o > 0; o >>= 1) {
    wp = fmaxf(wp, __shfl_xor(wp, o, 64));
    wq = fmaxf(wq, __shfl_xor(wq, o, 64));
  }
  const uint32_t wb = __ballot(bad != 0u) ? 1u : 0u;
  if (lane == 0) {
    fm[0][wave] = wp;
    fm[1][wave] = wq;
    bm[wave] = wb;
  }
  __syncthreads();
  float Mp = -INFINITY, Mq = -INFINITY;
  uint32_t anybad = 0;
  for (int w2 = 0; w2 < SPL_NW; ++w2) {
    Mp = fmaxf(Mp, fm[0][w2]);
    Mq = fmaxf(Mq, fm[1][w2]);
    anybad |= bm[w2];
  }
  const double vp = wave_sum_dpp(zmp > -INFINITY ? (double)(smp * __builtin_amdgcn_exp2f((zmp - Mp) * cT)) : 0.0);
  const double vq =
      wave_sum_dpp(resid && zmq > -INFINITY ? (double)(smq * __builtin_amdgcn_exp2f((zmq - Mq) * cT)) : 0.0);
  if (lane == 0) {
    dm[0][wave] = vp;
    dm[1][wave] = vq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double Sp = 0.0, Sq = 0.0;
    for (int w2 = 0; w2 < SPL_NW; ++w2) {
      Sp += dm[0][w2];
      Sq += dm[1][w2];
    }
    ChunkRec* r = a.chunks + (size_t)pid * S + c;
    r->mp = Mp;
    r->mq = resid ? Mq : -INFINITY;
    r->sp = Sp;
    r->sq = Sq;
    r->bad = anybad;
  }
}

// Pass 2 over one chunk: its overlap, residual (bonus: target) weight and
// target mass under the pair's statistics.
template <typename ET, bool VECTOR>
__global__ __launch_bounds__(SPL_NT) void split_weights_kernel(Args a) {
  using T = PT<ET, VECTOR>;
  using U = typename T::U;
  constexpr int E = T::E;
  __shared__ double dm[3][SPL_NW];
  const int S = a.split_s;
  const int c = (int)(blockIdx.x % (unsigned)S);
  const int pid = split_pair_id(a, blockIdx.x / (unsigned)S);
  if (pid < 0) return;
  const int G1 = a.G + 1;
  const int b = pid / G1, i = pid - b * G1;
  const int NU = VECTOR ? a.V / E : a.V;
  // As in the first pass, the chunk's first loads precede the parameters.
  const U* gp = reinterpret_cast<const U*>(row_ptr<ET>(a, b, true, i));
  const U* gq = i < a.G ? reinterpret_cast<const U*>(row_ptr<ET>(a, b, false, i)) : gp;
  int u0, u1;
  split_range(NU, S, c, u0, u1);
  U pu0[SPL_UR], qu0[SPL_UR];
#pragma unroll
  for (int r = 0; r < SPL_UR; ++r) {
    const int ui = max(0, min(u0 + r * SPL_NT + (int)threadIdx.x, u1 - 1));
    pu0[r] = gp[ui];
    qu0[r] = gq[ui];
  }
  const Mode m = seq_mode(a, b);
  if (m.mode != MODE_DENSE || i > m.g || !split_unfiltered(a, b, m)) return;
  const bool resid = i < m.g;
  RowStat sp, sq;
  ChunkRec* recs = a.chunks + (size_t)pid * S;
  if (!split_combine(recs, S, resid, LOG2E_F / m.T, sp, sq)) return;   // the draw kernel reports it
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float w = 0.0f, av = 0.0f, pz = 0.0f;
  for (int v0 = u0; v0 < u1; v0 += SPL_UR * SPL_NT) {
    U pu[SPL_UR], qu[SPL_UR];
#pragma unroll
    for (int r = 0; r < SPL_UR; ++r) {
      if (v0 == u0) {
        pu[r] = pu0[r];
        qu[r] = qu0[r];
      } else {
        const int ui = min(v0 + r * SPL_NT + (int)threadIdx.x, u1 - 1);
        pu[r] = gp[ui];
        qu[r] = gq[ui];
      }
    }
#pragma unroll
    for (int r = 0; r < SPL_UR; ++r) {
      if (v0 + r * SPL_NT + (int)threadIdx.x < u1) {
        float pv[E];
        T::each(pu[r], [&](int j, uint32_t raw) {
          pv[j] = pprob(sp, T::val(raw));
          pz += pv[j];
        });
        if (resid) {
          T::each(qu[r], [&](int j, uint32_t raw) {
            const float qv = pprob(sq, T::val(raw));
            av += fminf(pv[j], qv);
            w += fmaxf(pv[j] - qv, 0.0f);
          });
        } else {
#pragma unroll
          for (int j = 0; j < E; ++j) w += pv[j];
        }
      }
    }
  }
  const double ws = wave_sum_dpp((double)w), as = wave_sum_dpp((double)av), ps = wave_sum_dpp((double)pz);
  if (lane == 0) {
    dm[0][wave] = ws;
    dm[1][wave] = as;
    dm[2][wave] = ps;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double W = 0.0, A = 0.0, P = 0.0;
    for (int w2 = 0; w2 < SPL_NW; ++w2) {
      W += dm[0][w2];
      A += dm[1][w2];
      P += dm[2][w2];
    }
    recs[c].w = W;
    recs[c].al = A;
    recs[c].pz = P;
  }
}

// One workgroup per pair: the crossing chunk, the draw inside it, the record.
template <typename ET, bool VECTOR>
__global__ __launch_bounds__(SPL_NT) void split_draw_kernel(Args a) {
  using T = PT<ET, VECTOR>;
  using U = typename T::U;
  constexpr int E = T::E;
  __shared__ double part[SPL_MAXTILE][SPL_NW];
  __shared__ uint32_t red[3 * SPL_NW];
  __shared__ uint32_t bc[2];
  __shared__ double bd[2];
  const int S = a.split_s;
  const int pid = split_pair_id(a, blockIdx.x);
  if (pid < 0) return;
  const int G1 = a.G + 1;
  const int b = pid / G1, i = pid - b * G1;
  const Mode m = seq_mode(a, b);
  if (m.mode != MODE_DENSE || i > m.g) return;
  PosRec* rec = a.pos + (size_t)b * G1 + i;
  if (!split_unfiltered(a, b, m)) {   // top-k or top-p after all: the finisher's multi-pass procedure
    if (threadIdx.x == 0) {
      rec->bad = REC_REDO;
      rec->tok = -1;
    }
    return;
  }
  const bool resid = i < m.g;
  const ChunkRec* recs = a.chunks + (size_t)pid * S;
  RowStat sp, sq;
  if (!split_combine(recs, S, resid, LOG2E_F / m.T, sp, sq)) {
    if (threadIdx.x == 0) {
      rec->bad = 1u;
      rec->tok = -1;
    }
    return;
  }
  const int NU = VECTOR ? a.V / E : a.V;
  const U* gp = reinterpret_cast<const U*>(row_ptr<ET>(a, b, true, i));
  const U* gq = resid ? reinterpret_cast<const U*>(row_ptr<ET>(a, b, false, i)) : gp;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // The chunks' weights in order (lane c: chunk c); a zero residual draws
  // from p itself.  The crossing chunk is the first whose inclusive sum
  // passes u Z; where rounding leaves none, the last chunk that holds weight.
  double wl = 0.0, pzl = 0.0, all = 0.0;
  if (lane < S) {
    wl = recs[lane].w;
    pzl = recs[lane].pz;
    all = recs[lane].al;
  }
  const double al = wave_sum_dpp(all);
  const bool use_q = resid && wave_sum_dpp(wl) > 0.0;
  const double wc = use_q || !resid ? wl : pzl;
  const double incl = wave_incl_scan_f64(wc);
  const double Z = readlane_f64(incl, 63);
  const double target = (double)a.u[(size_t)b * G1 + a.G] * Z;
  const unsigned long long hit = __ballot(lane < S && incl > target);
  const unsigned long long pos = __ballot(lane < S && wc > 0.0);
  const int cc = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : S - 1);
  const double base = readlane_f64(incl - wc, cc);
  int u0, u1;
  split_range(NU, S, cc, u0, u1);
  // The crossing chunk, at most SPL_MAXTILE tiles of SPL_NT units (the host
  // sizes the chunks so), read once: thread t holds units u0 + r SPL_NT + t
  // and their weights; per-(tile, wavefront) sums, the crossing tile, then
  // its elements in ascending id from the same registers.
  const int ntile = min((u1 - u0 + SPL_NT - 1) / SPL_NT, SPL_MAXTILE);
  U up[SPL_MAXTILE], uq[SPL_MAXTILE];
#pragma unroll
  for (int r = 0; r < SPL_MAXTILE; ++r) {
    const int ui = max(0, min(u0 + r * SPL_NT + (int)threadIdx.x, u1 - 1));
    up[r] = gp[ui];
    uq[r] = gq[ui];
  }
  float wv[SPL_MAXTILE][E];
#pragma unroll
  for (int r = 0; r < SPL_MAXTILE; ++r) {
    const bool in = r < ntile && u0 + r * SPL_NT + (int)threadIdx.x < u1;
    T::each(up[r], [&](int j, uint32_t raw) { wv[r][j] = in ? pprob(sp, T::val(raw)) : 0.0f; });
    if (use_q) T::each(uq[r], [&](int j, uint32_t raw) { wv[r][j] = fmaxf(wv[r][j] - pprob(sq, T::val(raw)), 0.0f); });
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < E; ++j) t += wv[r][j];
    const double ws = wave_sum_dpp((double)t);
    if (lane == 0) part[r][wave] = ws;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    double tt = 0.0;
    if (lane < ntile)
      for (int w2 = 0; w2 < SPL_NW; ++w2) tt += part[lane][w2];
    const double incl = base + wave_incl_scan_f64(tt);
    const unsigned long long hit = __ballot(lane < ntile && incl > target);
    const int j = hit ? __ffsll((long long)hit) - 1 : ntile - 1;
    if (lane == j) {
      bc[0] = (uint32_t)j;
      bd[0] = incl - tt;
    }
  }
  __syncthreads();
  const int tj = (int)bc[0];
  uint32_t hitpos = 0xFFFFFFFFu, lastpos = 0;
  {
    const int ui = u0 + tj * SPL_NT + (int)threadIdx.x;
    float w[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      float v = 0.0f;
#pragma unroll
      for (int r = 0; r < SPL_MAXTILE; ++r) v = r == tj ? wv[r][j] : v;
      w[j] = v;
    }
    float r = 0.0f;
#pragma unroll
    for (int j = 0; j < E; ++j) r += w[j];
    const double rd = (double)r;
    const double incl = wave_incl_scan_f64(rd);
    double cum = bd[0];
    for (int w2 = 0; w2 < wave; ++w2) cum += part[tj][w2];
    cum += incl - rd;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      cum += (double)w[j];
      const uint32_t idx = (uint32_t)(ui * E + j);
      if (hitpos == 0xFFFFFFFFu && w[j] > 0.0f && cum > target) hitpos = idx;
      if (w[j] > 0.0f) lastpos = idx + 1u;
    }
  }
  hitpos = pb_min<SPL_NT>(hitpos, red);
  int tok = (int)hitpos;
  if (hitpos == 0xFFFFFFFFu) tok = (int)pb_max<SPL_NT>(lastpos, red) - 1;   // rounding left no crossing
  if (threadIdx.x == 0) {
    const int x = resid ? a.draft[(size_t)b * a.G + i] : -1;
    double px = 0.0, qx = 0.0;
    if (x >= 0 && x < a.V) {
      px = (double)pprob(sp, T::val(T::raw_at(gp, x)));
      qx = (double)pprob(sq, T::val(T::raw_at(gq, x)));
    }
    rec->px = px;
    rec->qx = qx;
    rec->alpha = resid ? al : 0.0;
    rec->tok = tok;
    rec->bad = 0u;
  }
}

}  // namespace sv
