// Shared definitions of the verify kernels: call arguments, per-sequence
// mode, row addressing and workspace records.
#pragma once

#include "sv_device.h"
#include "spec_verify.h"

namespace sv {

enum { MODE_INVALID = 0, MODE_GREEDY = 1, MODE_SPARSE = 2, MODE_DENSE = 3 };

constexpr int SEG = 1024;          // survivor slots per (logit row, row part) in the workspace
constexpr int MAXNP = 16;          // parts per logit row
constexpr int POOL = 4096;         // survivor entries of one sequence held in the finisher's LDS

// Sequence flags (workspace, one word per sequence).
constexpr uint32_t F_BAD = 1u;     // NaN or +inf among the logits
constexpr uint32_t F_DEMOTE = 2u;  // survivor lists unusable: recompute from the logits

// Result of the pair-resident kernel for one (sequence, position) (workspace).
struct PosRec {
  double px, qx, alpha;   // p_i(x_i), q_i(x_i), overlap (position < gamma_b)
  int32_t tok;            // draw if the first rejection is here (bonus draw at gamma_b)
  uint32_t bad;           // 1: a row of the pair has NaN / +inf or no finite logit; REC_REDO: not
                          // computed, the finisher computes the sequence from the logits
};
constexpr uint32_t REC_REDO = 2u;

struct ChunkRec;   // per-(pair, chunk) record of the split dense-pair kernels (sv_split.h)

struct Args {
  const void* p;
  const void* q;
  const int32_t* draft;
  const int32_t* gamma_len;
  const float* u;
  const float* temp;
  const int32_t* topk;
  const float* topp;
  int B, G, V;
  int RS;             // logit rows per sequence in the list layout: 2G+1 (verify), G+1 (shared noise)
  int NP;             // parts per logit row (streaming select)
  int PL;             // part length in elements (a multiple of the vector width)
  int fixbits;        // fixed-point fraction bits for mass sums
  int32_t* out_tokens;
  int32_t* out_n;
  float* out_alpha;
  float* out_pq;
  uint32_t* seq_flags;    // [B]     F_* bits, set by the select, cleared by the finisher
  int32_t* counts;        // [R][NP] survivors per (row, part)
  uint2* lists;           // [R][NP][SEG] (key, vocabulary id)
  PosRec* pos;            // [B][G+1] pair-resident results
  uint32_t* dense_count;  // [4]: draft pairs listed from the front of dense_list, bonus positions listed
                          // from its back, the pair kernel's work queue, the mixed kernel's select
                          // groups; cleared by the finisher
  int32_t* dense_list;    // [B * (G+1)] pair ids b * (G+1) + i of the dense sequences
  long long sel_blocks;   // workgroups of the select kernel that stream rows; the rest list dense pairs
  int pair;               // 1 when the pair-resident kernel runs for the dense sequences
  int split;              // 1 when NP > 1 only because the call is small: a top-k sequence whose
                          // part lists might overflow the finisher's pool streams rows whole
  int split_s;            // chunks per dense pair when the split kernels run (0: pair_kernel)
  int pair_regs;          // 1: the 64-thread pair kernel holds no rows in LDS (the caller promised
                          // unfiltered rows); a pair that is not unfiltered gets REC_REDO
  ChunkRec* chunks;       // [B * (G+1)][split_s] per-chunk records of the split kernels
  int all_dense;          // 1: no select launch; the pair kernel takes every (sequence, position) in
                          // order and the finisher runs non-dense sequences by its multi-pass path
  const float* lenience;  // [B] or null (1): q(x) is multiplied by it in the acceptance test
  int sampler;            // 1: G == 0 and each "sequence" is one row to sample (no drafts)
  int K, L;               // multi-candidate verify: candidate sequences and their length
  int ghist;              // shared-noise verify: gumbel_hist_kernel runs (filtered bf16 rows of 32K-131K values)
  int gfuse;              // shared-noise verify: the list kernel takes every sequence and finishes it
                          // (no per-(sequence, position) or finish launch follows)
  int gmix;               // shared-noise verify with ghist: gumbel_mixed_kernel streams the select
                          // units and takes the histogram rows (never a top-k or argmax sequence's);
                          // the list kernel then finishes the call
  int kphase;             // multi-candidate verify: 0 every node; 1 nodes of classes of two or more
                          // (single-candidate nodes deferred); 2 the pending chains' nodes
  const int32_t* cand;    // multi-candidate verify: [B][K][L] candidate tokens
  int32_t* node_tok;      // multi-candidate verify: [B][K][L+1] output at each prefix node
  const float* noise;     // shared-noise verify: [B][G+1][V] Gumbel noise
  int32_t* out_target;    // shared-noise verify: [B][G+1] the target's sample per position
};

struct Mode {
  int g;        // rows used by this sequence: clamp(gamma_b, 1, G) drafts
  int mode;
  uint32_t k;   // effective top-k of the streaming select (1 for argmax)
  float T;
  float tp;
};

// The processing mode is a pure function of the sequence's own parameters,
// so every kernel derives the same answer.
__device__ __forceinline__ Mode seq_mode(const Args& a, int b) {
  Mode m;
  const int gl = a.gamma_len ? a.gamma_len[b] : a.G;
  m.g = min(max(gl, 1), a.G);
  m.T = a.temp[b];
  const int k = a.topk ? a.topk[b] : 0;
  m.tp = a.topp ? a.topp[b] : 1.0f;
  m.k = 0;
  if (!(m.T >= 0.0f)) {
    m.mode = MODE_INVALID;
  } else if (m.T == 0.0f) {
    m.mode = MODE_GREEDY;
    m.k = 1;
  } else if (k > 0 && k < a.V && k <= KMAX_SPARSE) {
    m.mode = MODE_SPARSE;
    m.k = (uint32_t)k;
  } else {
    m.mode = MODE_DENSE;
  }
  return m;
}

template <typename ET>
__device__ __forceinline__ const ET* row_ptr(const Args& a, int b, bool isP, int pos) {
  if (isP) return reinterpret_cast<const ET*>(a.p) + ((size_t)b * (a.G + 1) + pos) * (size_t)a.V;
  return reinterpret_cast<const ET*>(a.q) + ((size_t)b * a.G + pos) * (size_t)a.V;
}

// Row slots of sequence b: slot s in [0, G] is target position s, slot
// G+1+i is draft position i.  `r` enumerates the used rows: 0..g are the
// target positions, g+1..2g the draft positions.
__device__ __forceinline__ int used_slot(int G, int g, int r) { return r <= g ? r : G + 1 + (r - g - 1); }

__device__ __forceinline__ size_t list_index(const Args& a, int rowid, int part) {
  return ((size_t)rowid * a.NP + part) * SEG;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource word 3 for untyped loads on gfx9-family GPUs, and the
// cache-policy bits of a non-temporal (streaming) load.
constexpr int BUF_WORD3 = 0x00020000;
constexpr int BUF_NT = 2;

__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace sv
