// Batched speculative-sampling verify step for MI355X (gfx950): kernels and
// the C ABI.
//
// A call is three launches on the caller's stream:
//   1. select_kernel -- one wavefront per (logit row, row part) of every
//      top-k / argmax sequence: streams the part once from HBM with 16-byte
//      non-temporal loads and writes its exact kept set (top-k survivors,
//      ties included) to the workspace; a few extra workgroups list the
//      (sequence, position) pairs of the dense sequences.  See sv_wave.h.
//   2. pair_kernel -- one workgroup per listed dense pair (unfiltered, large
//      top-k and top-p sequences): normalisers, nucleus cut, p(x), q(x),
//      overlap and the draw as if the first rejection were at that position.
//      See sv_pair.h.
//   3. finish_kernel -- one workgroup per sequence: for top-k / argmax
//      sequences, merges the part lists of every row and computes the
//      normalisers, top-p cut, p(x), q(x), overlap, the first rejection (one
//      wavefront ballot) and the residual / bonus draw from the lists; for
//      dense sequences it takes the pair kernel's per-position results (or,
//      for rows beyond the pair kernel's limits, runs a multi-pass procedure
//      over the logits).  See sv_finish.h.
// A caller that promises that every sequence is dense skips launch 1 (the
// pair kernel then takes the pairs in a fixed order), and launch 3 becomes
// finish_dense_kernel, one workgroup per 16 sequences.  When the dense pairs
// take the histogram variant (bf16 rows of 32K-131K values) and no hint is
// given, launch 1 only lists the pairs and launch 2 is mixed_hist_kernel,
// which streams the select units as well (see sv_phist.h).
//
// Definitions followed (page titles and sections): the acceptance rule and
// the residual, "Fast Inference from Transformers via Speculative Decoding"
// (mtandhj.com summary), "Speculative Sampling: theoretical basis"; the
// first-rejection count, the Leviathan review (dongryeollee1), Algorithm 1;
// the bonus token via a zero draft distribution after the last draft,
// "Speculative Decoding: the art of guessing well", "Speculative sampling";
// the inverse-CDF draw, same page, "Sampling with shared noise"; the overlap
// alpha = sum min(p, q), mtandhj summary, "How to choose gamma".

#include "sv_wave.h"
#include "sv_pair.h"
#include "sv_phist.h"
#include "sv_split.h"
#include "sv_finish.h"
#include "sv_gumbel.h"
#include "sv_kseq.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

namespace sv {

__global__ void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
static bool sizes_ok(int B, int G, int V) {
  return B >= 0 && G >= 1 && G <= SV_MAX_GAMMA && V >= 1 && V <= SV_MAX_VOCAB;
}

struct Plan {
  int NP;     // parts per logit row
  int PL;     // part length in elements
  int split;  // 1 when NP comes from the small-call rule below
};

// Parts per row: about SV_UNIT_TARGET (row, part) units, with at least
// SV_MIN_STEPS steps per part.  A part costs a fixed start (certifying the
// first bound) and end (exact select, list write) besides its stream, and
// every part's kept set goes to the finisher's pool, so parts stay long:
// measured at B = 64, V = 128256, gamma = 4, top-k 50, 3 parts per row
// (1728 units) beat 6 and 7 (55 against 59-60 us per call); the shared-noise
// verify at the same shapes (320 rows) was fastest at 6 parts (1920 units).
// RS: logit rows per sequence in the list layout (2G+1 for the verify, G+1
// for the shared-noise verify, whose draft rows are not inputs).
#ifndef SV_UNIT_TARGET
#define SV_UNIT_TARGET 2048
#endif
#ifndef SV_MIN_STEPS
#define SV_MIN_STEPS 2
#endif
// Calls of up to this many units at SV_SPLIT_PARTS parts per row get that many: the
// plan counts every row of the call, but where some sequences are dense (run
// by the pair kernel) only the others' rows are streamed here, and with one
// part each those few rows would take one wavefront apiece from end to end.
#ifndef SV_SPLIT_MAX_UNITS
#define SV_SPLIT_MAX_UNITS 4608
#endif
#ifndef SV_SPLIT_PARTS
#define SV_SPLIT_PARTS 2
#endif
static Plan plan(int B, int RS, int V, int dtype) {
  const int vec = dtype == SV_BF16 ? 8 : 4;
  const int step = 64 * WVPL * vec;
  const long long R = (long long)B * RS;
  long long np = R > 0 ? SV_UNIT_TARGET / R : 1;
  np = np < 1 ? 1 : np;
  int split = 0;
  if (np == 1 && SV_SPLIT_PARTS * R <= SV_SPLIT_MAX_UNITS) {
    np = SV_SPLIT_PARTS;
    split = 1;
  }
  np = np > MAXNP ? MAXNP : np;
  const long long by_len = V / ((long long)SV_MIN_STEPS * step);
  if (np > by_len) np = by_len < 1 ? 1 : by_len;
  Plan p;
  int pl = (int)((V + np - 1) / np);
  pl = (pl + vec - 1) / vec * vec;
  p.PL = pl;
  p.NP = (V + pl - 1) / pl;
  p.split = split && p.NP > 1;
  return p;
}

// Dense (unfiltered / large top-k / top-p) sequences run the pair kernel:
// rows of up to 4 / 16 / 64 KB are held in LDS by 64 / 256 / 1024-thread
// workgroups; longer rows are streamed by 1024-thread workgroups as long as
// the residual pass fits its tile table.  Returns the workgroup size (0: the
// finisher's multi-pass procedure handles dense rows) and sets *lds_bytes to
// the dynamic LDS of the launch.
static int pair_variant(int V, int dtype, bool vector_ok, size_t* lds_bytes) {
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  const size_t row = ((size_t)V * es + 15) / 16 * 16;
  *lds_bytes = 2 * row;
  if (row <= 4096) return 64;
  if (row <= 16384) return 256;
  if (row <= (size_t)PAIR_LDS_ROW_MAX) return 1024;
  *lds_bytes = 0;
  const size_t units = vector_ok ? (size_t)V * es / 16 : (size_t)V;
  return units <= (size_t)1024 * PAIR_MAXTILE ? -1024 : 0;   // negative: streamed rows
}

// Resident workgroups of each pair-kernel shape across the chip (256 CUs):
// the pair kernel's grid, which walks the dense-pair list.
#ifndef SV_PAIR_STREAM_WGS
#define SV_PAIR_STREAM_WGS 512
#endif
static int pair_grid_cap(int variant) {
  switch (variant) {
    case 64: return 256 * 16;
    case 256: return 256 * 4;
    case 1024: return 256;        // 128 KB of rows in LDS: one per CU
    default: return SV_PAIR_STREAM_WGS;   // streamed rows
  }
}

// Chunks per dense pair for the split kernels (1: no split).  Three launches
// cost about 30 us however small, so the split is for rows longer than the
// 64 KB that one workgroup holds in LDS (a pair then takes one CU 60-70 us)
// and calls of at most SV_SPLIT_MAX_PAIRS pairs (at most two rounds of one
// workgroup per CU): B = 1..8, gamma 4, V = 128256 went from 72-73 to
// 32-38 us per call, while B = 32, gamma 5, V = 32000 (rows in LDS) went from
// 27.4 to 33.9 us.  Enough pairs times chunks to give every CU about four
// workgroups, at most SPL_MAXS, each chunk at least SPL_MIN_UNITS 16-byte
// units of a row and at most the SPL_MAXTILE tiles of SPL_NT units that the
// draw kernel holds in registers.
#ifndef SV_SPLIT_TARGET_WGS
#define SV_SPLIT_TARGET_WGS 1024
#endif
#ifndef SV_SPLIT_MAX_PAIRS
#define SV_SPLIT_MAX_PAIRS 512
#endif
static int split_chunks(int B, int G, int V, int dtype) {
  const long long npairs = (long long)B * (G + 1);
  if (npairs <= 0 || npairs > SV_SPLIT_MAX_PAIRS) return 1;
  const long long row = (long long)V * (dtype == SV_BF16 ? 2 : 4);
  if (row <= PAIR_LDS_ROW_MAX) return 1;
  const long long units = row / 16;
  long long s = (SV_SPLIT_TARGET_WGS + npairs - 1) / npairs;
  if (s > SPL_MAXS) s = SPL_MAXS;
  if (s > units / SPL_MIN_UNITS) s = units / SPL_MIN_UNITS;
  if (s < 2) return 1;
  while (s < SPL_MAXS && (units + s - 1) / s > (long long)SPL_MAXTILE * SPL_NT) ++s;
  if ((units + s - 1) / s > (long long)SPL_MAXTILE * SPL_NT || (units + s - 1) / s < SPL_MIN_UNITS) return 1;
  return (int)s;
}

struct Layout {
  size_t seq_flags_off, dense_count_off, counters_bytes, pos_off, dense_list_off, counts_off, lists_off, chunks_off,
      total;
};

// S: chunks per dense pair (split_chunks), for the verify's layout; 0 elsewhere.
static Layout layout(int B, int G, int RS, const Plan& p, int S = 0) {
  Layout L;
  const size_t R = (size_t)B * RS;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  L.seq_flags_off = 0;
  L.dense_count_off = (size_t)B * 4;
  L.counters_bytes = up(L.dense_count_off + 4 * 4);
  L.pos_off = L.counters_bytes;
  L.dense_list_off = up(L.pos_off + (size_t)B * (G + 1) * sizeof(PosRec));
  L.counts_off = up(L.dense_list_off + (size_t)B * (G + 1) * 4);
  L.lists_off = up(L.counts_off + R * p.NP * 4);
  L.chunks_off = up(L.lists_off + R * p.NP * SEG * sizeof(uint2));
  L.total = L.chunks_off + (S > 1 ? (size_t)B * (G + 1) * S * sizeof(ChunkRec) : 0);
  return L;
}

static thread_local char g_errbuf[256];
// Timing hook: events recorded around one kernel of every call.
static thread_local hipEvent_t g_stage_begin = nullptr, g_stage_end = nullptr;
static thread_local int g_stage_kernel = SV_KERNEL_SELECT;

static hipError_t stage_mark(int kernel, bool begin, hipStream_t st) {
  if (kernel != g_stage_kernel) return hipSuccess;
  hipEvent_t ev = begin ? g_stage_begin : g_stage_end;
  return ev ? hipEventRecord(ev, st) : hipSuccess;
}

// Dynamic-LDS limits of every kernel that takes dynamic LDS, raised once per
// device to the largest size any call can launch with, so that the limit in
// force never depends on the order of calls or on the calling thread.  The
// set-up runs under a mutex with the device current; a failed set-up is
// retried by the next call.
constexpr int SV_MAX_DEVICES = 64;
static std::mutex g_setup_mu;
static bool g_setup_done[SV_MAX_DEVICES];

template <typename ET, bool VECTOR>
static hipError_t set_lds_limits() {
  const int fin = (int)sizeof(FinSmem);
  const int pair_max = 2 * PAIR_LDS_ROW_MAX;   // both rows of a pair, or a K-SEQ node's two rows
  struct {
    const void* fn;
    int bytes;
  } const lim[] = {
      {reinterpret_cast<const void*>(&finish_kernel<ET, VECTOR>), fin},
      {reinterpret_cast<const void*>(&finish_dense_kernel<ET, VECTOR>), fin},
      {reinterpret_cast<const void*>(&pair_kernel<ET, 64, VECTOR, true>), 2 * 4096},
      {reinterpret_cast<const void*>(&pair_kernel<ET, 256, VECTOR, true>), 2 * 16384},
      {reinterpret_cast<const void*>(&pair_kernel<ET, 1024, VECTOR, true>), pair_max},
      {reinterpret_cast<const void*>(&kseq_node_kernel<ET, KSEQ_NT, VECTOR, true>), pair_max},
  };
  for (const auto& l : lim) {
    const hipError_t e = hipFuncSetAttribute(l.fn, hipFuncAttributeMaxDynamicSharedMemorySize, l.bytes);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static hipError_t device_setup() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SV_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_setup_mu);
  if (g_setup_done[dev]) return hipSuccess;
  if ((e = set_lds_limits<uint16_t, true>()) != hipSuccess) return e;
  if ((e = set_lds_limits<uint16_t, false>()) != hipSuccess) return e;
  if ((e = set_lds_limits<float, true>()) != hipSuccess) return e;
  if ((e = set_lds_limits<float, false>()) != hipSuccess) return e;
  {
    const void* gk[4] = {reinterpret_cast<const void*>(&gumbel_list_kernel<uint16_t, true>),
                         reinterpret_cast<const void*>(&gumbel_list_kernel<uint16_t, false>),
                         reinterpret_cast<const void*>(&gumbel_list_kernel<float, true>),
                         reinterpret_cast<const void*>(&gumbel_list_kernel<float, false>)};
    for (const void* f : gk) {
      e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)gumbel_list_smem_bytes());
      if (e != hipSuccess) return e;
    }
  }
  g_setup_done[dev] = true;
  return hipSuccess;
}

// The mixed launches (select units inside the histogram kernels' launch, for
// calls that hold both kinds of sequence) are on unless built with
// -DSV_MIXED=0, which restores the separate select launch for comparison.
#ifndef SV_MIXED
#define SV_MIXED 1
#endif
template <typename ET, bool VECTOR>
static hipError_t launch_pair(const Args& a, long long grid, size_t fin_lds, hipStream_t st) {
  hipError_t e = device_setup();
  if (e != hipSuccess) return e;
  // Dense pairs on the histogram variant beside streamed rows: the select
  // units run inside the pair launch (mixed_hist_kernel), and the select
  // launch only lists the dense pairs.
  bool mixed = false;
  if constexpr (VECTOR && sizeof(ET) == 2) {
    if (SV_MIXED && a.pair && a.split_s <= 1 && !a.all_dense) {
      size_t plds = 0;
      mixed = pair_variant(a.V, SV_BF16, true, &plds) == -1024 && (long long)a.V / 8 <= PH_MAX_UNITS;
    }
  }
  if ((e = stage_mark(SV_KERNEL_SELECT, true, st)) != hipSuccess) return e;
  if (!a.all_dense) {
    if (mixed) {
      Args al = a;
      al.sel_blocks = 0;
      hipLaunchKernelGGL((select_kernel<ET, VECTOR>), dim3((unsigned)(grid - a.sel_blocks)), dim3(K1_NT), 0, st, al);
    } else {
      hipLaunchKernelGGL((select_kernel<ET, VECTOR>), dim3((unsigned)grid), dim3(K1_NT), 0, st, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((e = stage_mark(SV_KERNEL_SELECT, false, st)) != hipSuccess) return e;
  if (mixed) {
    if ((e = stage_mark(SV_KERNEL_PAIR, true, st)) != hipSuccess) return e;
    hipLaunchKernelGGL(mixed_hist_kernel, dim3(256), dim3(PH_NT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = stage_mark(SV_KERNEL_PAIR, false, st)) != hipSuccess) return e;
  } else if (a.pair && a.split_s > 1) {
    const long long npairs = (long long)a.B * (a.G + 1);
    const dim3 g1((unsigned)(npairs * a.split_s));
    if ((e = stage_mark(SV_KERNEL_PAIR, true, st)) != hipSuccess) return e;
    hipLaunchKernelGGL((split_stats_kernel<ET, VECTOR>), g1, dim3(SPL_NT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((split_weights_kernel<ET, VECTOR>), g1, dim3(SPL_NT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((split_draw_kernel<ET, VECTOR>), dim3((unsigned)npairs), dim3(SPL_NT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = stage_mark(SV_KERNEL_PAIR, false, st)) != hipSuccess) return e;
  } else if (a.pair) {
    size_t plds = 0;
    int pv = pair_variant(a.V, sizeof(ET) == 2 ? SV_BF16 : SV_FP32, VECTOR, &plds);
    if (pv != 64 && pv != 256 && pv != 1024 && pv != -1024) return hipErrorInvalidValue;
    const long long npairs = (long long)a.B * (a.G + 1);
    // bf16 rows streamed from memory, up to PH_MAX_UNITS 16-byte units: the
    // histogram variant, one workgroup per CU.
    const bool hist = pv == -1024 && sizeof(ET) == 2 && VECTOR && (long long)a.V / 8 <= PH_MAX_UNITS;
    long long cap = hist ? 256 : pair_grid_cap(pv);
    if (pv == 64 && a.pair_regs) {   // rows in registers: no row LDS, more workgroups per CU
      plds = 0;
      cap = 256LL * (sizeof(ET) == 4 ? PAIR_REGS_WGS_F32 : PAIR_REGS_WGS_BF16);
    }
    const dim3 grid((unsigned)(npairs < cap ? npairs : cap));
    if ((e = stage_mark(SV_KERNEL_PAIR, true, st)) != hipSuccess) return e;
    if (hist) pv = 0;
    switch (pv) {
      case 0: hipLaunchKernelGGL(pair_hist_kernel, grid, dim3(PH_NT), 0, st, a); break;
      case 64: hipLaunchKernelGGL((pair_kernel<ET, 64, VECTOR, true>), grid, dim3(64), plds, st, a); break;
      case 256: hipLaunchKernelGGL((pair_kernel<ET, 256, VECTOR, true>), grid, dim3(256), plds, st, a); break;
      case 1024: hipLaunchKernelGGL((pair_kernel<ET, 1024, VECTOR, true>), grid, dim3(1024), plds, st, a); break;
      default: hipLaunchKernelGGL((pair_kernel<ET, 1024, VECTOR, false>), grid, dim3(1024), 0, st, a); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if ((e = stage_mark(SV_KERNEL_PAIR, false, st)) != hipSuccess) return e;
  }
  if ((e = stage_mark(SV_KERNEL_FINISH, true, st)) != hipSuccess) return e;
  if (a.all_dense)
    hipLaunchKernelGGL((finish_dense_kernel<ET, VECTOR>), dim3((unsigned)(((long long)a.B + NWAVE - 1) / NWAVE)),
                       dim3(NT), fin_lds, st, a);
  else
    hipLaunchKernelGGL((finish_kernel<ET, VECTOR>), dim3((unsigned)a.B), dim3(NT), fin_lds, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return stage_mark(SV_KERNEL_FINISH, false, st);
}

// Workspace size and preparation for B sequences of G drafts (G == 0: rows
// to sample).
// The verify's layout (RS = 2G + 1) holds the split kernels' chunk records.
static int layout_chunks(int B, int G, int V, int dtype, int RS) {
  return RS == 2 * G + 1 ? split_chunks(B, G, V, dtype) : 0;
}

static size_t ws_bytes(int B, int G, int V, int dtype, int RS) {
  if (B < 0 || G < 0 || G > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB) return 0;
  if (dtype != SV_BF16 && dtype != SV_FP32) return 0;
  if (B == 0) return 256;
  return layout(B, G, RS, plan(B, RS, V, dtype), layout_chunks(B, G, V, dtype, RS)).total;
}

static int ws_init(void* workspace, size_t workspace_bytes, int B, int G, int V, int dtype, int RS, void* stream) {
  const size_t need = ws_bytes(B, G, V, dtype, RS);
  if (need == 0) return SV_ERR_ARG;
  if (!workspace || workspace_bytes < need) return SV_ERR_WORKSPACE;
  if (B == 0) return SV_OK;
  const Layout L = layout(B, G, RS, plan(B, RS, V, dtype), layout_chunks(B, G, V, dtype, RS));
  const size_t n = L.counters_bytes / 4;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024)), dim3(256), 0,
                     (hipStream_t)stream, (uint32_t*)workspace, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_errbuf, sizeof g_errbuf, "HIP error: %s", hipGetErrorString(e));
    return SV_ERR_HIP;
  }
  return SV_OK;
}

// Pointer, alignment and hint checks of the verify entry points (sizes are
// checked by the callers).
static int check_verify_args(const void* p_logits, const void* q_logits, int dtype, const int32_t* draft_tokens,
                             const float* uniforms, const float* temperature, int hints, const int32_t* out_tokens,
                             const int32_t* out_n_accepted, const float* out_alpha, int sampler) {
  if (hints & ~(SV_HINT_NO_DENSE | SV_HINT_ALL_DENSE | SV_HINT_UNFILTERED)) return SV_ERR_ARG;
  if ((hints & SV_HINT_NO_DENSE) && (hints & SV_HINT_ALL_DENSE)) return SV_ERR_ARG;
  if (!p_logits || !uniforms || !temperature || !out_tokens) return SV_ERR_ARG;
  if (!sampler && (!q_logits || !draft_tokens || !out_n_accepted || !out_alpha)) return SV_ERR_ARG;
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  if (((uintptr_t)p_logits % es) || (q_logits && ((uintptr_t)q_logits % es))) return SV_ERR_ARG;
  return SV_OK;
}

// The verify launch sequence.  sampler == 1: G == 0, every "sequence" is one
// row drawn from its processed distribution at u[b] (the bonus draw), with no
// drafts, no draft logits and no n output.
static int run_verify(const void* p_logits, const void* q_logits, int dtype, const int32_t* draft_tokens,
                      const int32_t* gamma_len, const float* uniforms, const float* temperature,
                      const int32_t* top_k, const float* top_p, const float* lenience, int hints, int B,
                      int gamma_max, int V, int32_t* out_tokens, int32_t* out_n_accepted, float* out_alpha,
                      float* out_pq, void* workspace, size_t workspace_bytes, void* stream, int sampler) {
  const int rc = check_verify_args(p_logits, q_logits, dtype, draft_tokens, uniforms, temperature, hints,
                                   out_tokens, out_n_accepted, out_alpha, sampler);
  if (rc != SV_OK) return rc;
  const int RS = 2 * gamma_max + 1;
  const size_t need = ws_bytes(B, gamma_max, V, dtype, RS);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % 256)) return SV_ERR_WORKSPACE;
  const Plan pl = plan(B, RS, V, dtype);
  const long long rows = (long long)B * RS;
  const long long units = rows * pl.NP;
  const long long sel_grid = (units + K1_WAVES - 1) / K1_WAVES;
  const long long list_grid = ((long long)B + K1_NT - 1) / K1_NT;
  const long long grid = sel_grid + list_grid;
  if (grid > 0x7FFFFFFFLL || units > 0x7FFFFFFFLL) return SV_ERR_UNSUPPORTED;
  const int vec = dtype == SV_BF16 ? 8 : 4;
  const bool vector_ok = (V % vec == 0) && ((uintptr_t)p_logits % 16 == 0) &&
                         (!q_logits || (uintptr_t)q_logits % 16 == 0);
  int vb = 0;
  while ((1LL << vb) < (long long)V + 1) ++vb;
  const Layout Lw = layout(B, gamma_max, RS, pl, layout_chunks(B, gamma_max, V, dtype, RS));
  char* ws = (char*)workspace;
  Args a;
  memset(&a, 0, sizeof a);
  a.RS = RS;
  a.p = p_logits;
  a.q = q_logits;
  a.draft = draft_tokens;
  a.gamma_len = sampler ? nullptr : gamma_len;
  a.u = uniforms;
  a.temp = temperature;
  a.topk = top_k;
  a.topp = top_p;
  a.lenience = lenience;
  a.sampler = sampler;
  a.B = B;
  a.G = gamma_max;
  a.V = V;
  a.NP = pl.NP;
  a.split = pl.split;
  a.PL = pl.PL;
  a.fixbits = 62 - vb;
  a.out_tokens = out_tokens;
  a.out_n = out_n_accepted;
  a.out_alpha = out_alpha;
  a.out_pq = out_pq;
  a.seq_flags = reinterpret_cast<uint32_t*>(ws + Lw.seq_flags_off);
  a.counts = reinterpret_cast<int32_t*>(ws + Lw.counts_off);
  a.pos = reinterpret_cast<PosRec*>(ws + Lw.pos_off);
  a.dense_count = reinterpret_cast<uint32_t*>(ws + Lw.dense_count_off);
  a.dense_list = reinterpret_cast<int32_t*>(ws + Lw.dense_list_off);
  size_t pair_lds = 0;
  a.pair = pair_variant(V, dtype, vector_ok, &pair_lds) != 0 && (long long)B * (gamma_max + 1) <= 0x7FFFFFFFLL ? 1 : 0;
  // The caller's promise that no sequence is dense saves the pair launch; a
  // dense sequence under that hint still gets its exact result from the
  // finisher's multi-pass path.
  if (hints & SV_HINT_NO_DENSE) a.pair = 0;
  // The promise that every sequence is dense saves the select launch (whose
  // only work would be the listing); it needs the pair kernel for this V.
  if ((hints & SV_HINT_ALL_DENSE) && a.pair && !sampler) a.all_dense = 1;
  // Without the pair kernel the dense sequences go to the finisher whole and
  // nothing is listed.
  // Few pairs of unfiltered rows (the caller's promise): each pair is split
  // over several workgroups.
  const int S = layout_chunks(B, gamma_max, V, dtype, RS);
  size_t pair_lds_unused = 0;
  a.split_s = (hints & SV_HINT_UNFILTERED) && a.pair && !sampler && vector_ok && S > 1 ? S : 0;
  // Short unfiltered rows (the same promise) need no LDS copy: the 64-thread
  // pair kernel then holds them in registers, and more of its workgroups fit
  // on a CU.
  a.pair_regs = (hints & SV_HINT_UNFILTERED) && a.pair && !sampler && vector_ok && a.split_s <= 1 &&
                pair_variant(V, dtype, true, &pair_lds_unused) == 64 ? 1 : 0;
  a.chunks = reinterpret_cast<ChunkRec*>(ws + Lw.chunks_off);
  a.sel_blocks = a.pair ? sel_grid : grid;
  a.lists = reinterpret_cast<uint2*>(ws + Lw.lists_off);
  hipStream_t st = (hipStream_t)stream;
  const size_t fin_lds = sizeof(FinSmem);
  hipError_t e = hipSuccess;
  if (dtype == SV_BF16) {
    e = vector_ok ? launch_pair<uint16_t, true>(a, grid, fin_lds, st) : launch_pair<uint16_t, false>(a, grid, fin_lds, st);
  } else {
    e = vector_ok ? launch_pair<float, true>(a, grid, fin_lds, st) : launch_pair<float, false>(a, grid, fin_lds, st);
  }
  if (e != hipSuccess) {
    snprintf(g_errbuf, sizeof g_errbuf, "HIP error: %s", hipGetErrorString(e));
    return SV_ERR_HIP;
  }
  return SV_OK;
}

}  // namespace sv

using namespace sv;

extern "C" size_t spec_verify_workspace_bytes(int B, int gamma_max, int V, int dtype) {
  if (!sizes_ok(B, gamma_max, V)) return 0;
  return ws_bytes(B, gamma_max, V, dtype, 2 * gamma_max + 1);
}

extern "C" int spec_verify_workspace_init(void* workspace, size_t workspace_bytes, int B, int gamma_max, int V,
                                          int dtype, void* stream) {
  if (!sizes_ok(B, gamma_max, V)) return SV_ERR_ARG;
  return ws_init(workspace, workspace_bytes, B, gamma_max, V, dtype, 2 * gamma_max + 1, stream);
}

extern "C" int spec_verify_ex(const void* p_logits, const void* q_logits, int dtype, const int32_t* draft_tokens,
                              const int32_t* gamma_len, const float* uniforms, const float* temperature,
                              const int32_t* top_k, const float* top_p, const float* lenience, int hints, int B,
                              int gamma_max, int V, int32_t* out_tokens, int32_t* out_n_accepted, float* out_alpha,
                              float* out_pq, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != SV_BF16 && dtype != SV_FP32) return SV_ERR_UNSUPPORTED;
  if (gamma_max > SV_MAX_GAMMA || V > SV_MAX_VOCAB) return SV_ERR_UNSUPPORTED;
  if (!sizes_ok(B, gamma_max, V)) return SV_ERR_ARG;
  if (B == 0) return SV_OK;
  return run_verify(p_logits, q_logits, dtype, draft_tokens, gamma_len, uniforms, temperature, top_k, top_p, lenience,
                    hints, B, gamma_max, V, out_tokens, out_n_accepted, out_alpha, out_pq, workspace, workspace_bytes,
                    stream, 0);
}

extern "C" int spec_verify(const void* p_logits, const void* q_logits, int dtype, const int32_t* draft_tokens,
                           const int32_t* gamma_len, const float* uniforms, const float* temperature,
                           const int32_t* top_k, const float* top_p, int B, int gamma_max, int V,
                           int32_t* out_tokens, int32_t* out_n_accepted, float* out_alpha, float* out_pq,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return spec_verify_ex(p_logits, q_logits, dtype, draft_tokens, gamma_len, uniforms, temperature, top_k, top_p,
                        nullptr, 0, B, gamma_max, V, out_tokens, out_n_accepted, out_alpha, out_pq, workspace,
                        workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// spec_verify_ex without a workspace argument, for callers that cannot
// allocate device memory.  Its workspace is the file-scope array below: one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol);
// it uses the device address that hipGetSymbolAddress returned for the
// current device.
// ---------------------------------------------------------------------------
namespace sv {

static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[SV_MAX_DEVICES];

// The current device's copy of `scratch` (looked up once per device, with
// that device current).
static hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SV_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace sv

extern "C" int spec_verify_noalloc(const void* p_logits, const void* q_logits, int dtype,
                                   const int32_t* draft_tokens, const int32_t* gamma_len, const float* uniforms,
                                   const float* temperature, const int32_t* top_k, const float* top_p,
                                   const float* lenience, int hints, int B, int gamma_max, int V, int32_t* out_tokens,
                                   int32_t* out_n_accepted, float* out_alpha, float* out_pq, void* stream) {
  if (dtype != SV_BF16 && dtype != SV_FP32) return SV_ERR_UNSUPPORTED;
  if (gamma_max > SV_MAX_GAMMA || V > SV_MAX_VOCAB) return SV_ERR_UNSUPPORTED;
  if (!sizes_ok(B, gamma_max, V)) return SV_ERR_ARG;
  if (B == 0) return SV_OK;
  int rc = check_verify_args(p_logits, q_logits, dtype, draft_tokens, uniforms, temperature, hints, out_tokens,
                             out_n_accepted, out_alpha, 0);
  if (rc != SV_OK) return rc;
  const int RS = 2 * gamma_max + 1;
  const size_t need = ws_bytes(B, gamma_max, V, dtype, RS);
  if (need == 0 || need > (size_t)SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_SCRATCH;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) {
    snprintf(g_errbuf, sizeof g_errbuf, "HIP error: %s", hipGetErrorString(e));
    return SV_ERR_HIP;
  }
  // The array keeps whatever the last call on this GPU left in it, and the
  // counters' offsets depend on the sizes: clear them on every call (a fill
  // kernel on the stream, as the workspace preparation does).
  rc = ws_init(ws, SV_NOALLOC_SCRATCH_BYTES, B, gamma_max, V, dtype, RS, stream);
  if (rc != SV_OK) return rc;
  return run_verify(p_logits, q_logits, dtype, draft_tokens, gamma_len, uniforms, temperature, top_k, top_p, lenience,
                    hints, B, gamma_max, V, out_tokens, out_n_accepted, out_alpha, out_pq, ws,
                    SV_NOALLOC_SCRATCH_BYTES, stream, 0);
}

extern "C" size_t spec_sample_workspace_bytes(int R, int V, int dtype) { return ws_bytes(R, 0, V, dtype, 1); }

extern "C" int spec_sample_workspace_init(void* workspace, size_t workspace_bytes, int R, int V, int dtype,
                                          void* stream) {
  return ws_init(workspace, workspace_bytes, R, 0, V, dtype, 1, stream);
}

extern "C" size_t spec_verify_gumbel_workspace_bytes(int B, int gamma_max, int V, int dtype) {
  if (B < 0 || gamma_max < 0) return 0;
  return ws_bytes(B, gamma_max, V, dtype, gamma_max + 1);
}

extern "C" int spec_verify_gumbel_workspace_init(void* workspace, size_t workspace_bytes, int B, int gamma_max, int V,
                                                 int dtype, void* stream) {
  if (B < 0 || gamma_max < 0) return SV_ERR_ARG;
  return ws_init(workspace, workspace_bytes, B, gamma_max, V, dtype, gamma_max + 1, stream);
}

extern "C" int spec_sample(const void* logits, int dtype, const float* uniforms, const float* temperature,
                           const int32_t* top_k, const float* top_p, int R, int V, int32_t* out_tokens,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != SV_BF16 && dtype != SV_FP32) return SV_ERR_UNSUPPORTED;
  if (V > SV_MAX_VOCAB) return SV_ERR_UNSUPPORTED;
  if (R < 0 || V < 1) return SV_ERR_ARG;
  if (R == 0) return SV_OK;
  return run_verify(logits, nullptr, dtype, nullptr, nullptr, uniforms, temperature, top_k, top_p, nullptr, 0, R, 0,
                    V, out_tokens, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream, 1);
}

namespace sv {

template <typename ET, bool VECTOR>
static hipError_t launch_gumbel(const Args& a, long long sel_grid, hipStream_t st) {
  hipError_t e = device_setup();
  if (e != hipSuccess) return e;
  // 1. Streaming select over the target rows of argmax / top-k sequences
  //    (with a.gmix, in one launch with the histogram rows).
  if (a.gmix) {
    if ((e = stage_mark(SV_KERNEL_GUMBEL, true, st)) != hipSuccess) return e;
    hipLaunchKernelGGL(gumbel_mixed_kernel, dim3(256), dim3(PH_NT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = stage_mark(SV_KERNEL_GUMBEL, false, st)) != hipSuccess) return e;
  } else {
    if ((e = stage_mark(SV_KERNEL_SELECT, true, st)) != hipSuccess) return e;
    if (!a.all_dense) {
      hipLaunchKernelGGL((select_kernel<ET, VECTOR>), dim3((unsigned)sel_grid), dim3(K1_NT), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = stage_mark(SV_KERNEL_SELECT, false, st)) != hipSuccess) return e;
  }
  // 2. Their per-position argmax from the survivor lists (with a.gfuse or
  //    a.gmix, every sequence's rows and its outputs: the call ends here).
  if (!a.all_dense) {
    hipLaunchKernelGGL((gumbel_list_kernel<ET, VECTOR>), dim3((unsigned)a.B), dim3(NT), gumbel_list_smem_bytes(), st,
                       a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.gfuse || a.gmix) return hipSuccess;
  }
  // 3. Dense and demoted sequences: filtered bf16 rows of 32K-131K values by
  //    the histogram kernel (one workgroup per CU), the rest one workgroup
  //    per (sequence, position).
  if (!a.gmix && (e = stage_mark(SV_KERNEL_GUMBEL, true, st)) != hipSuccess) return e;
  if (a.ghist && !a.gmix) {
    const long long nrows = (long long)a.B * (a.G + 1);
    hipLaunchKernelGGL(gumbel_hist_kernel, dim3((unsigned)(nrows < 256 ? nrows : 256)), dim3(PH_NT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((gumbel_kernel<ET, GUMBEL_NT, VECTOR>), dim3((unsigned)((long long)a.B * (a.G + 1))),
                     dim3(GUMBEL_NT), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!a.gmix && (e = stage_mark(SV_KERNEL_GUMBEL, false, st)) != hipSuccess) return e;
  // 4. The first disagreement and the outputs.
  hipLaunchKernelGGL(gumbel_finish_kernel, dim3((unsigned)((a.B + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// The shared-noise launch sequence.  sampler == 1: G == 0, each "sequence"
// is one row whose Gumbel-max sample is written to out_tokens (which is also
// the per-row scratch), no drafts, no n output.
static int run_gumbel(const void* p_logits, int dtype, const float* noise, const int32_t* draft_tokens,
                      const int32_t* gamma_len, const float* temperature, const int32_t* top_k, const float* top_p,
                      int B, int gamma_max, int V, int32_t* out_tokens, int32_t* out_n_accepted, int32_t* out_target,
                      void* workspace, size_t workspace_bytes, void* stream, int sampler, int hints) {
  if (hints & ~(SV_HINT_NO_DENSE | SV_HINT_ALL_DENSE)) return SV_ERR_ARG;
  if ((hints & SV_HINT_NO_DENSE) && (hints & SV_HINT_ALL_DENSE)) return SV_ERR_ARG;
  if (!p_logits || !noise || !temperature || !out_tokens || !out_target) return SV_ERR_ARG;
  if (!sampler && (!draft_tokens || !out_n_accepted)) return SV_ERR_ARG;
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  if (((uintptr_t)p_logits % es) || ((uintptr_t)noise % 4)) return SV_ERR_ARG;
  const int RS = gamma_max + 1;
  const size_t need = ws_bytes(B, gamma_max, V, dtype, RS);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % 256)) return SV_ERR_WORKSPACE;
  if ((long long)B * RS > 0x7FFFFFFFLL) return SV_ERR_UNSUPPORTED;
  const Plan pl = plan(B, RS, V, dtype);
  const long long units = (long long)B * RS * pl.NP;
  const long long sel_grid = (units + K1_WAVES - 1) / K1_WAVES;
  if (sel_grid > 0x7FFFFFFFLL) return SV_ERR_UNSUPPORTED;
  const int vec = dtype == SV_BF16 ? 8 : 4;
  const bool vector_ok = (V % vec == 0) && ((uintptr_t)p_logits % 16 == 0) && ((uintptr_t)noise % 16 == 0);
  int vb = 0;
  while ((1LL << vb) < (long long)V + 1) ++vb;
  const Layout Lw = layout(B, gamma_max, RS, pl, layout_chunks(B, gamma_max, V, dtype, RS));
  char* ws = (char*)workspace;
  Args a;
  memset(&a, 0, sizeof a);
  a.RS = RS;
  a.p = p_logits;
  a.draft = draft_tokens;
  a.gamma_len = sampler ? nullptr : gamma_len;
  a.sampler = sampler;
  a.temp = temperature;
  a.topk = top_k;
  a.topp = top_p;
  a.B = B;
  a.G = gamma_max;
  a.V = V;
  a.NP = pl.NP;
  a.split = pl.split;
  a.PL = pl.PL;
  a.fixbits = 62 - vb;
  a.out_tokens = out_tokens;
  a.out_n = out_n_accepted;
  a.noise = noise;
  a.out_target = out_target;
  a.seq_flags = reinterpret_cast<uint32_t*>(ws + Lw.seq_flags_off);
  a.counts = reinterpret_cast<int32_t*>(ws + Lw.counts_off);
  a.lists = reinterpret_cast<uint2*>(ws + Lw.lists_off);
  a.sel_blocks = sel_grid;   // no dense-pair listing here
  // The promise that every sequence is dense saves the select and list
  // launches; the per-(sequence, position) kernel then takes every sequence.
  a.all_dense = (hints & SV_HINT_ALL_DENSE) && !sampler ? 1 : 0;
  // The promise that no sequence is dense lets the list kernel finish the
  // call: it takes the rare dense, invalid or demoted sequence itself.
  a.gfuse = (hints & SV_HINT_NO_DENSE) && !sampler ? 1 : 0;
  // Filtered bf16 rows too long for one pass over the row to give their
  // support cheaply: the exact histogram kernel.
  a.ghist = !a.gfuse && dtype == SV_BF16 && vector_ok && V > 32768 && V / 8 <= PH_MAX_UNITS ? 1 : 0;
  // With a list path beside it, the select units run in the histogram rows'
  // launch, and the list kernel then finishes the call.
  a.gmix = SV_MIXED && a.ghist && !a.all_dense && !sampler ? 1 : 0;
  a.dense_count = reinterpret_cast<uint32_t*>(ws + Lw.dense_count_off);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (dtype == SV_BF16)
    e = vector_ok ? launch_gumbel<uint16_t, true>(a, sel_grid, st) : launch_gumbel<uint16_t, false>(a, sel_grid, st);
  else
    e = vector_ok ? launch_gumbel<float, true>(a, sel_grid, st) : launch_gumbel<float, false>(a, sel_grid, st);
  if (e != hipSuccess) {
    snprintf(g_errbuf, sizeof g_errbuf, "HIP error: %s", hipGetErrorString(e));
    return SV_ERR_HIP;
  }
  return SV_OK;
}

}  // namespace sv

using namespace sv;

extern "C" int spec_verify_gumbel(const void* p_logits, int dtype, const float* noise, const int32_t* draft_tokens,
                                  const int32_t* gamma_len, const float* temperature, const int32_t* top_k,
                                  const float* top_p, int B, int gamma_max, int V, int32_t* out_tokens,
                                  int32_t* out_n_accepted, int32_t* out_target, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (dtype != SV_BF16 && dtype != SV_FP32) return SV_ERR_UNSUPPORTED;
  if (gamma_max > SV_MAX_GAMMA || V > SV_MAX_VOCAB) return SV_ERR_UNSUPPORTED;
  if (!sizes_ok(B, gamma_max, V)) return SV_ERR_ARG;
  if (B == 0) return SV_OK;
  return run_gumbel(p_logits, dtype, noise, draft_tokens, gamma_len, temperature, top_k, top_p, B, gamma_max, V,
                    out_tokens, out_n_accepted, out_target, workspace, workspace_bytes, stream, 0, 0);
}

extern "C" int spec_verify_gumbel_ex(const void* p_logits, int dtype, const float* noise, const int32_t* draft_tokens,
                                     const int32_t* gamma_len, const float* temperature, const int32_t* top_k,
                                     const float* top_p, int hints, int B, int gamma_max, int V, int32_t* out_tokens,
                                     int32_t* out_n_accepted, int32_t* out_target, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (hints & ~(SV_HINT_NO_DENSE | SV_HINT_ALL_DENSE)) return SV_ERR_ARG;
  if ((hints & SV_HINT_NO_DENSE) && (hints & SV_HINT_ALL_DENSE)) return SV_ERR_ARG;
  if (dtype != SV_BF16 && dtype != SV_FP32) return SV_ERR_UNSUPPORTED;
  if (gamma_max > SV_MAX_GAMMA || V > SV_MAX_VOCAB) return SV_ERR_UNSUPPORTED;
  if (!sizes_ok(B, gamma_max, V)) return SV_ERR_ARG;
  if (B == 0) return SV_OK;
  return run_gumbel(p_logits, dtype, noise, draft_tokens, gamma_len, temperature, top_k, top_p, B, gamma_max, V,
                    out_tokens, out_n_accepted, out_target, workspace, workspace_bytes, stream, 0, hints);
}

extern "C" int spec_sample_gumbel(const void* logits, int dtype, const float* noise, const float* temperature,
                                  const int32_t* top_k, const float* top_p, int R, int V, int32_t* out_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != SV_BF16 && dtype != SV_FP32) return SV_ERR_UNSUPPORTED;
  if (V > SV_MAX_VOCAB) return SV_ERR_UNSUPPORTED;
  if (R < 0 || V < 1) return SV_ERR_ARG;
  if (R == 0) return SV_OK;
  return run_gumbel(logits, dtype, noise, nullptr, nullptr, temperature, top_k, top_p, R, 0, V, out_tokens, nullptr,
                    out_tokens, workspace, workspace_bytes, stream, 1, 0);
}

namespace sv {

template <typename ET, bool VECTOR>
static hipError_t launch_spectr(const Args& a, bool ldsr, size_t lds, hipStream_t st) {
  hipError_t e = device_setup();
  if (e != hipSuccess) return e;
  // 1. The nodes of classes of two or more candidates (the rho* searches);
  //    single-candidate nodes are deferred.  2. A walk that stops at the
  //    first deferred node it reaches and records that candidate's chain.
  //    3. The recorded chains' nodes, from that depth to L: the only
  //    single-candidate nodes the round can use.  4. The walk.
  auto nodes = [&](const Args& an, long long n) {
    const dim3 grid((unsigned)n);
    if (ldsr) hipLaunchKernelGGL((kseq_node_kernel<ET, KSEQ_NT, VECTOR, true>), grid, dim3(KSEQ_NT), lds, st, an);
    else hipLaunchKernelGGL((kseq_node_kernel<ET, KSEQ_NT, VECTOR, false>), grid, dim3(KSEQ_NT), 0, st, an);
    return hipGetLastError();
  };
  Args a1 = a, a2 = a;
  a1.kphase = 1;
  a2.kphase = 2;
  if ((e = stage_mark(SV_KERNEL_KSEQ, true, st)) != hipSuccess) return e;
  if ((e = nodes(a1, (long long)a.B * a.K * (a.L + 1))) != hipSuccess) return e;
  if ((e = stage_mark(SV_KERNEL_KSEQ, false, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(spectr_walk_kernel, dim3((unsigned)a.B), dim3(64), 0, st, a1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = nodes(a2, (long long)a.B * (a.L + 1))) != hipSuccess) return e;
  hipLaunchKernelGGL(spectr_walk_kernel, dim3((unsigned)a.B), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace sv

extern "C" int spec_verify_spectr(const void* p_logits, const void* q_logits, int dtype, const int32_t* candidates,
                                  const float* uniforms, const float* temperature, const int32_t* top_k,
                                  const float* top_p, int B, int K, int L, int V, int32_t* out_tokens,
                                  int32_t* out_n, int32_t* out_node_tokens, void* stream) {
  if (dtype != SV_BF16 && dtype != SV_FP32) return SV_ERR_UNSUPPORTED;
  if (K > SV_MAX_CANDIDATES || L > SV_MAX_GAMMA || V > SV_MAX_VOCAB) return SV_ERR_UNSUPPORTED;
  if (B < 0 || K < 1 || L < 1 || V < 1) return SV_ERR_ARG;
  if (B == 0) return SV_OK;
  if (!p_logits || !q_logits || !candidates || !uniforms || !temperature || !out_tokens || !out_n || !out_node_tokens)
    return SV_ERR_ARG;
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  if (((uintptr_t)p_logits % es) || ((uintptr_t)q_logits % es)) return SV_ERR_ARG;
  if ((long long)B * K * (L + 1) > 0x7FFFFFFFLL) return SV_ERR_UNSUPPORTED;
  const int vec = dtype == SV_BF16 ? 8 : 4;
  const bool vector_ok = (V % vec == 0) && ((uintptr_t)p_logits % 16 == 0) && ((uintptr_t)q_logits % 16 == 0);
  const size_t row = ((size_t)V * es + 15) / 16 * 16;
  const bool ldsr = row <= (size_t)PAIR_LDS_ROW_MAX;
  const size_t units = vector_ok ? (size_t)V * es / 16 : (size_t)V;
  if (!ldsr && units > (size_t)KSEQ_NT * PAIR_MAXTILE) return SV_ERR_UNSUPPORTED;
  int vb = 0;
  while ((1LL << vb) < (long long)V + 1) ++vb;
  Args a;
  memset(&a, 0, sizeof a);
  a.p = p_logits;
  a.q = q_logits;
  a.cand = candidates;
  a.u = uniforms;
  a.temp = temperature;
  a.topk = top_k;
  a.topp = top_p;
  a.B = B;
  a.K = K;
  a.L = L;
  a.V = V;
  a.fixbits = 62 - vb;
  a.out_tokens = out_tokens;
  a.out_n = out_n;
  a.node_tok = out_node_tokens;
  hipStream_t st = (hipStream_t)stream;
  const size_t lds = ldsr ? 2 * row : 0;
  hipError_t e;
  if (dtype == SV_BF16)
    e = vector_ok ? launch_spectr<uint16_t, true>(a, ldsr, lds, st) : launch_spectr<uint16_t, false>(a, ldsr, lds, st);
  else
    e = vector_ok ? launch_spectr<float, true>(a, ldsr, lds, st) : launch_spectr<float, false>(a, ldsr, lds, st);
  if (e != hipSuccess) {
    snprintf(g_errbuf, sizeof g_errbuf, "HIP error: %s", hipGetErrorString(e));
    return SV_ERR_HIP;
  }
  return SV_OK;
}

extern "C" const char* spec_verify_strerror(int code) {
  switch (code) {
    case SV_OK: return "ok";
    case SV_ERR_ARG: return "invalid argument (null pointer, size out of range or misaligned pointer)";
    case SV_ERR_UNSUPPORTED: return "unsupported dtype or size";
    case SV_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case SV_ERR_SCRATCH:
      return "the call needs more workspace than the allocation-free entry point's fixed buffer "
             "(SV_NOALLOC_SCRATCH_BYTES) holds; use spec_verify_ex with a caller workspace";
    case SV_ERR_HIP: return g_errbuf[0] ? g_errbuf : "HIP error";
    default: return "unknown error code";
  }
}

extern "C" int spec_verify_version(void) { return 11; }

extern "C" int spec_verify_set_stage_events(int kernel, void* begin, void* end) {
  if (kernel < SV_KERNEL_SELECT || kernel > SV_KERNEL_KSEQ) return SV_ERR_ARG;
  g_stage_kernel = kernel;
  g_stage_begin = (hipEvent_t)begin;
  g_stage_end = (hipEvent_t)end;
  return SV_OK;
}

// ---------------------------------------------------------------------------
// Throughput analytics (host code; no GPU).
// ---------------------------------------------------------------------------
extern "C" double spec_verify_expected_tokens(double alpha, int gamma) {
  if (!(alpha >= 0.0 && alpha <= 1.0) || gamma < 0) return NAN;
  if (alpha == 1.0) return (double)(gamma + 1);
  return (1.0 - pow(alpha, gamma + 1)) / (1.0 - alpha);
}

extern "C" double spec_verify_speedup(double alpha, int gamma, double c) {
  if (!(c >= 0.0)) return NAN;
  return spec_verify_expected_tokens(alpha, gamma) / ((double)gamma * c + 1.0);
}

extern "C" double spec_verify_operations(double alpha, int gamma, double c_hat) {
  if (!(c_hat >= 0.0)) return NAN;
  return ((double)gamma * c_hat + gamma + 1.0) / spec_verify_expected_tokens(alpha, gamma);
}

extern "C" int spec_verify_optimal_gamma(double alpha, double c, int gamma_max) {
  if (!(alpha >= 0.0 && alpha <= 1.0) || !(c >= 0.0) || gamma_max < 1) return -1;
  int best = 1;
  double best_s = -1.0;
  for (int g = 1; g <= gamma_max; ++g) {
    const double sp = spec_verify_speedup(alpha, g, c);
    if (sp > best_s) {
      best_s = sp;
      best = g;
    }
  }
  return best;
}

extern "C" double spec_verify_acceptance_length(const double* alpha, int gamma) {
  if (gamma < 0 || (gamma > 0 && !alpha)) return NAN;
  double tau = 1.0, run = 1.0;
  for (int k = 0; k < gamma; ++k) {
    if (!(alpha[k] >= 0.0 && alpha[k] <= 1.0)) return NAN;
    run *= alpha[k];
    tau += run;
  }
  return tau;
}
