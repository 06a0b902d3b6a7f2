// Internal declarations shared by the HIP translation units of libspava.
//
// Work decomposition of one layer (all virtual hosts on one GPU):
//   * a "unit" is one workgroup's tile of query rows together with the list
//     of key segments those rows attend to;
//   * the kinds of unit follow the method's row types: anchor tokens,
//     context tokens of host h, and the query block's partials (partial 0 =
//     anchor + query block, partial h+1 = block h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spava.h"

namespace spava {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kKeyTile = 64;      // keys per attention tile
constexpr int kRowsPerWave = 32;  // query rows per wave (MFMA 32x32 column block)

enum UnitKind : int {
  kAnchor = 0,    // anchor tokens, causal over the anchor
  kContext = 1,   // context tokens of host h
  kQueryHead = 2, // query partial 0: anchor + query block (causal)
  kQueryBlock = 3,// query partial h+1: block h in full
};

inline __host__ __device__ int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline __host__ __device__ int round_up(int a, int b) { return ceil_div(a, b) * b; }

// Everything an attention launch needs (passed by value as the kernel argument).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* kp;
  const void* vp;
  void* o;
  float* lse;
  float* o_part;
  float* lse_part;
  float* stats;        // float32 scoring: [V][Hkv][nq*G] log2-domain row LSE
  int N, Hq, Hkv, G, D, la, V, L, nq, lp;
  long q_st, q_sh;     // element strides of q between tokens and between heads
  long kv_st, kv_sh;   // the same for k and v
  float scale;         // softmax scale
  float scale_log2;    // scale * log2(e)
  // Unit ranges, in launch order (see unit_decode):
  int n_ctx_units_per_host;  // ceil(L/BM) * Hq
  int n_q_units;             // ceil(nq*G/BM) * Hkv, per query partial
  int n_anchor_units;        // ceil(la/BM) * Hq
  int n_ctx_first;           // hosts whose context units precede the query-block partials
  int rows_per_unit;         // BM
  int f32;                   // 1: float32 elements, 0: bf16
  int score_ctx;             // scoring rows: 0 = the query block, 1 = each block's own tokens
  int score_from_partials;   // 1: row LSEs of the query scoring come from lse_part
  int xcd_chunk;             // units per XCD chunk (see xcd_unit)
  int unit_lo, unit_hi;      // units [unit_lo, unit_hi) of the launch order run in this launch
};

struct Unit {
  int kind;
  int host;      // kContext / kQueryBlock
  int head;      // query head (single-head units)
  int group;     // KV head
  int tile;      // row tile index inside the unit's row space
};

// Launch order of units (longest rows first, roughly):
//   context units of hosts V-1 down to V-n_ctx_first (later row tiles first,
//   heads fastest), the query-block partials of blocks 0..V-1, the context
//   units of the remaining hosts (down to 0), query partial 0, anchor units.
// n_ctx_first puts the query-block partials (all of length L) after the
// hosts whose every context unit is at least that long.  Query-row units are
// KV-group-major so that units sharing K/V are adjacent.
__device__ inline Unit unit_decode(const AttnArgs& a, int b) {
  Unit u;
  u.host = 0;
  u.head = 0;
  u.group = 0;
  u.tile = 0;
  const int bm = a.rows_per_unit;
  const int qt = a.n_q_units / a.Hkv;  // query row tiles per KV group
  const int nctx = a.V * a.n_ctx_units_per_host;
  const int nqb = a.V * a.n_q_units;
  const int n1 = a.n_ctx_first * a.n_ctx_units_per_host;
  if (b < n1 || (b >= n1 + nqb && b < nctx + nqb)) {
    const int c = b < n1 ? b : b - nqb;   // index among the context units
    u.kind = kContext;
    u.host = a.V - 1 - c / a.n_ctx_units_per_host;
    int r = c % a.n_ctx_units_per_host;
    int ntile = ceil_div(a.L, bm);
    u.head = r % a.Hq;
    u.tile = ntile - 1 - r / a.Hq;
    u.group = u.head / a.G;
    return u;
  }
  if (b < n1 + nqb) {
    b -= n1;
    u.kind = kQueryBlock;
    u.host = b / a.n_q_units;
    int r = b % a.n_q_units;
    u.group = r / qt;
    u.tile = r % qt;
    return u;
  }
  b -= nctx + nqb;
  if (b < a.n_q_units) {
    u.kind = kQueryHead;
    u.group = b / qt;
    u.tile = b % qt;
    return u;
  }
  b -= a.n_q_units;
  u.kind = kAnchor;
  int ntile = ceil_div(a.la, bm);
  u.head = b % a.Hq;
  u.tile = ntile - 1 - b / a.Hq;
  u.group = u.head / a.G;
  return u;
}

__host__ __device__ inline int attn_total_units(const AttnArgs& a) {
  return a.V * a.n_ctx_units_per_host + a.V * a.n_q_units + a.n_q_units + a.n_anchor_units;
}

// Phases of the attention (launch order above): the units that read no
// passing block -- context rows of host 0, the query partials, the anchor --
// are the tail of the order; the context rows of hosts 1..V-1 are its head.
// Running the first phase before the selection lets the selection reuse the
// query partials' row LSEs (Figure 5 ordering).
enum AttnPhase : int { kPhaseAll = 0, kPhaseLocal = 1, kPhasePassing = 2 };
// The phases need the order with every context host first (n_ctx_first = V).
__host__ __device__ inline void attn_phase_units(const AttnArgs& a, int phase, int* lo, int* hi) {
  const int split = (a.V - 1) * a.n_ctx_units_per_host;
  *lo = phase == kPhaseLocal ? split : 0;
  *hi = phase == kPhasePassing ? split : attn_total_units(a);
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8), and each XCD has its own L2 and dispatches only its own
// workgroups.  Units are therefore dealt to XCDs in chunks of `chunk`
// consecutive units (units that read the same K/V tiles), keeping the launch
// order within each XCD.  Round r of 8 chunks starts at XCD r % 8: with
// units ordered longest first, a fixed start would give XCD 0 the longest
// chunk of every round and make it finish last.  The grid is padded to a
// multiple of 8 * chunk; padding workgroups map past the last unit.
constexpr int kXcds = 8;
__host__ __device__ inline int xcd_grid(int n_units, int chunk) {
  return round_up(n_units, kXcds * chunk);
}
__device__ inline int xcd_unit(int b, int chunk) {
  const int x = b % kXcds;
  const int s = b / kXcds;
  const int r = s / chunk;
  return (r * kXcds + (x + r) % kXcds) * chunk + s % chunk;
}

// A run of keys that a unit's rows attend to.
struct Seg {
  int kind;        // 0: rows of k (token-major, stride Hkv*D); 1: rows of kp
  long k_off;      // element offset of key 0 of the segment in k or kp
  long k_stride;   // elements between consecutive keys
  long v_off;      // element offset of key 0 in v or vp
  long v_stride;
  int len;         // number of keys
  int causal;      // 1: key token (tok0 + j) must be <= query token
  int tok0;
};

// Key segments of a unit (at most 3).  Returns the count.
__device__ inline int unit_segments(const AttnArgs& a, const Unit& u, Seg* s) {
  const int g = u.group;
  int n = 0;
  auto main_seg = [&](int tok0, int len, int causal) {
    Seg x;
    x.kind = 0;
    x.k_off = (long)tok0 * a.kv_st + (long)g * a.kv_sh;
    x.k_stride = a.kv_st;
    x.v_off = x.k_off;
    x.v_stride = a.kv_st;
    x.len = len;
    x.causal = causal;
    x.tok0 = tok0;
    s[n++] = x;
  };
  switch (u.kind) {
    case kAnchor:
      main_seg(0, a.la, 1);
      break;
    case kContext: {
      if (a.la > 0) main_seg(0, a.la, 0);
      if (u.host > 0 && a.lp > 0) {
        Seg x;
        x.kind = 1;
        x.k_off = (long)g * a.V * a.lp * a.D;
        x.k_stride = a.D;
        x.v_off = x.k_off;
        x.v_stride = a.D;
        x.len = u.host * a.lp;
        x.causal = 0;
        x.tok0 = 0;
        s[n++] = x;
      }
      const int b0 = a.la + u.host * a.L;
      main_seg(b0, a.L, 1);
      break;
    }
    case kQueryHead: {
      if (a.la > 0) main_seg(0, a.la, 0);
      main_seg(a.la + a.V * a.L, a.nq, 1);
      break;
    }
    case kQueryBlock:
      main_seg(a.la + u.host * a.L, a.L, 0);
      break;
  }
  return n;
}

// Row r of a unit's row space -> (token, query head, valid).
// Single-head units: rows are consecutive tokens of one head.
// Query units pack the G heads of a KV group: r = (a - g*G) * nq + i.
struct RowId {
  int tok, head, valid;
};
__device__ inline RowId unit_row(const AttnArgs& a, const Unit& u, int r) {
  RowId x;
  if (u.kind == kAnchor || u.kind == kContext) {
    const int base = (u.kind == kAnchor) ? 0 : a.la + u.host * a.L;
    const int n = (u.kind == kAnchor) ? a.la : a.L;
    x.valid = r < n;
    x.tok = base + (x.valid ? r : n - 1);
    x.head = u.head;
  } else {
    const int R = a.nq * a.G;
    x.valid = r < R;
    const int rr = x.valid ? r : R - 1;
    x.tok = a.la + a.V * a.L + rr % a.nq;
    x.head = u.group * a.G + rr / a.nq;
  }
  return x;
}

// Rows of the block scoring for block h: the query block's tokens (query
// selector) or block h's own tokens, each attending causally over the
// block's keys (context selector).  Row r of KV head g is token
// tok0 + r % ntok of query head g * G + r / ntok; R = ntok * G rows.
struct ScoreRows {
  int tok0, ntok, R;
};
__host__ __device__ inline ScoreRows score_rows(const AttnArgs& a, int h) {
  ScoreRows s;
  s.tok0 = a.score_ctx ? a.la + h * a.L : a.la + a.V * a.L;
  s.ntok = a.score_ctx ? a.L : a.nq;
  s.R = s.ntok * a.G;
  return s;
}

// ---- launchers (host), defined in the .hip files ----
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s);
int attn_bf16_rows_per_unit();   // query rows per workgroup of the bf16 kernel
// bf16 scoring (row statistics over key chunks, then column sums); ws holds
// score_bf16_ws_bytes(a) bytes.
hipError_t launch_score_bf16(const AttnArgs& a, void* ws, float* scores, hipStream_t s);
size_t score_bf16_ws_bytes(const AttnArgs& a);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);
hipError_t launch_rowstat_f32(const AttnArgs& a, hipStream_t s);
hipError_t launch_colsum_f32(const AttnArgs& a, float* scores, hipStream_t s);
hipError_t launch_topk(const float* scores, int32_t* idx, int n_lists, int L, int lp, hipStream_t s);
hipError_t launch_overlap(const int32_t* idx_a, const int32_t* idx_b, int32_t* counts, int n_lists,
                          int lp, hipStream_t s);
// kv_st_bytes, kv_sh_bytes: byte strides of k and v between tokens and heads.
hipError_t launch_gather(const void* k, const void* v, const int32_t* idx, void* kp, void* vp,
                         int la, int V, int L, int Hkv, int lp, int row_bytes, long kv_st_bytes,
                         long kv_sh_bytes, hipStream_t s);
hipError_t launch_merge(int P, int R, int H, int D, const float* o_part, const float* lse_part,
                        void* o, long o_row_stride, float* lse, long lse_head_stride,
                        int out_bf16, hipStream_t s);

}  // namespace spava
