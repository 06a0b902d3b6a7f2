// Fused approximate-attention forward for bf16 inputs on gfx950 (CDNA4).
//
// Work unit: 256 query rows, one workgroup of 8 waves = 4 SIMD pairs.  Pair
// s owns rows [64s, 64s+64) as two 32-column MFMA blocks and splits the work
// between its two waves, which share one SIMD:
//   softmax wave (wave s):   S = K Q^T on the matrix cores, then the masks,
//                            row maxima, exponentials and row sums;
//   output wave (wave 4+s):  O += V P on the matrix cores, and the tile copies.
// The softmax wave's vector work then issues while the output wave's MFMAs
// occupy the matrix core (a single wave can only slip a few vector
// instructions under its own MFMAs), and every K or V fragment read from
// LDS still feeds two MFMAs (64 rows per wave).
//
// Iteration i (one workgroup barrier each):
//   softmax wave:  S(i) = K(i) Q^T || P(i-1) = exp2(S(i-1) - m), written to
//                  LDS with its rescale factor; row maxima of S(i); then the
//                  first fragments of K(i+1), complete since the barrier
//   output wave:   copies of V(i-1) and K(i+2); O = O*alpha(i-2) + V(i-2) P(i-2)
// LDS: a 2-slot V ring at address 0 (so every V read is a lane offset plus an
// immediate), a 3-slot K ring (both filled by buffer_load_dwordx4 ... lds
// straight from memory) and a double-buffered P exchange.
//   K tile   [64 keys][D]   row-major, read as the MFMA A operand of S^T
//   V tile   [64 keys][D]   row-major; gfx950's transposing LDS reads
//                           (ds_read_b64_tr_b16) give the MFMA A operand of
//                           O^T = V^T P^T, 8 consecutive keys of one channel
//                           per lane, with no transposed copy of V anywhere
//   P tile   [2][4][64 lanes][8 bf16]  already in the B-operand layout
// K and V rows are XOR-swizzled in 16-byte slots, each with the swizzle that
// keeps its reads free of bank conflicts (K: the 16 rows of one ds_read_b128
// phase; V: the 8 rows x 4 chunks of one transposing read).  Every copy
// addresses memory
// inside its tensor: tiles past the end of the walk re-read a tile already
// visited, K and V rows past a run's end read its last row, and both are
// masked (their probabilities are 0).
//
// Math: S^T = K Q^T puts one query column per lane, so a row's softmax
// statistics live in one lane pair (l, l^32) of the softmax wave.  K-tile rows
// are read in a permuted order (bits 2 and 3 of the row index swapped) so that
// the S^T accumulators already have the B-operand layout of O^T += V^T P^T
// with keys in natural order.  Probabilities are taken against a stale
// running maximum as long as they stay within [0, 2^8] (exact after
// normalisation, since O and the row sum share the reference); a lane's sum
// over its keys of a tile bounds every term, so the common path needs no row
// maxima.  When a tile breaks the bound, its row maxima become the reference,
// the row sums are rescaled, the tile's probabilities are recomputed, and the
// output wave rescales O just before adding them.
#include "lds_dma.h"

namespace spava {
namespace {

constexpr int kPairs = 4;                   // SIMD pairs
constexpr int kWaves = 2 * kPairs;          // softmax waves 0-3, output waves 4-7
constexpr int kWaveRows = 64;               // two 32-column MFMA blocks
constexpr int kBM = kPairs * kWaveRows;     // rows per workgroup (unit)
constexpr int kBN = kKeyTile;               // keys per tile
constexpr int kThreads = kWaves * 64;
constexpr int kKSlots = 3;                  // K ring: K(t) in slot t % 3
constexpr int kVSlots = 2;                  // V ring: V(t) in slot t % 2
constexpr int kPBytes = 2 * 4 * 64 * 16;    // P tile of one pair (64 rows x 64 keys, bf16)
constexpr float kGrowLog2 = 8.0f;

template <int D>
struct Geo {
  static constexpr int NC = D / 16;                   // 16-wide d chunks (K steps of S)
  static constexpr int NDB = D / 32;                  // 32-row d blocks of O^T
  static constexpr int KRB = D * 2;                   // bytes per K or V row
  static constexpr int KBYTES = kBN * KRB;            // K tile; a V tile is the same
  static constexpr int KINST = KBYTES / 1024 / kPairs;   // copy instructions per output wave and tile
};

// The unit's key runs as scalar fields (selected by value, never by a
// dynamic index, so that they stay in scalar registers).
struct SegRun {
  const uint16_t* k;   // key 0 of the run (K or passing K rows)
  const uint16_t* v;   // its V row (V and K share their layout and strides)
  int kstride;         // elements between consecutive keys
  int len;             // keys
  int causal;          // 1: key token tok0 + j must be <= the query token
  int tok0;
  int nt;              // 64-key tiles this unit visits
};

__device__ __forceinline__ SegRun empty_run() {
  SegRun r;
  r.k = nullptr;
  r.v = nullptr;
  r.kstride = 0;
  r.len = 0;
  r.causal = 0;
  r.tok0 = 0;
  r.nt = 0;
  return r;
}

// A run of consecutive tokens of K/V head g: tokens [tok0, tok0+len).
__device__ __forceinline__ SegRun main_run(const AttnArgs& a, int g, int tok0, int len, int causal) {
  SegRun r;
  const long off = (long)tok0 * a.kv_st + (long)g * a.kv_sh;
  r.k = (const uint16_t*)a.k + off;
  r.v = (const uint16_t*)a.v + off;
  r.kstride = (int)a.kv_st;
  r.len = len;
  r.causal = causal;
  r.tok0 = tok0;
  r.nt = 0;
  return r;
}

// Key runs of a unit in three fixed slots (an absent run has len 0):
//   anchor unit:        [anchor causal]
//   context unit (h):   [anchor] [passing blocks 0..h-1] [own block causal]
//   query partial 0:    [anchor] [query block causal]
//   query partial h+1:  [block h]
__device__ __forceinline__ void unit_runs(const AttnArgs& a, const Unit& u, SegRun& r0, SegRun& r1,
                                          SegRun& r2) {
  const int g = u.group;
  r0 = empty_run();
  r1 = empty_run();
  r2 = empty_run();
  switch (u.kind) {
    case kAnchor:
      r0 = main_run(a, g, 0, a.la, 1);
      break;
    case kContext:
      r0 = main_run(a, g, 0, a.la, 0);
      if (u.host > 0 && a.lp > 0) {
        const long off = (long)g * a.V * a.lp * a.D;
        r1.k = (const uint16_t*)a.kp + off;
        r1.v = (const uint16_t*)a.vp + off;
        r1.kstride = a.D;
        r1.len = u.host * a.lp;
      }
      r2 = main_run(a, g, a.la + u.host * a.L, a.L, 1);
      break;
    case kQueryHead:
      r0 = main_run(a, g, 0, a.la, 0);
      r1 = main_run(a, g, a.la + a.V * a.L, a.nq, 1);
      break;
    default:  // kQueryBlock
      r0 = main_run(a, g, a.la + u.host * a.L, a.L, 0);
      break;
  }
}

// Selection on values (never on field lvalues, which would turn into a
// select of addresses and keep the runs in scratch memory).
template <typename T>
__device__ __forceinline__ T pick3(T x0, T x1, T x2, int i) {
  return i == 0 ? x0 : (i == 1 ? x1 : x2);
}
__device__ __forceinline__ SegRun sel(SegRun a0, SegRun a1, SegRun a2, int i) {
  SegRun r;
  r.k = pick3(a0.k, a1.k, a2.k, i);
  r.v = pick3(a0.v, a1.v, a2.v, i);
  r.kstride = pick3(a0.kstride, a1.kstride, a2.kstride, i);
  r.len = pick3(a0.len, a1.len, a2.len, i);
  r.causal = pick3(a0.causal, a1.causal, a2.causal, i);
  r.tok0 = pick3(a0.tok0, a1.tok0, a2.tok0, i);
  r.nt = pick3(a0.nt, a1.nt, a2.nt, i);
  return r;
}

// Wave-uniform values made visibly uniform (scalar registers, no waterfall
// loops around the buffer descriptors built from them).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const uint16_t* uni(const uint16_t* p) {
  const unsigned long long v = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return (const uint16_t*)(((unsigned long long)hi << 32) | lo);
}

struct Runs {
  SegRun r0, r1, r2;
  int T;   // tiles in the walk
};

// Tile i of the unit's walk -> its run and first key.  Past the end of the
// walk the run is empty (len 0): its copies read nothing and every logit of
// the tile is masked.
struct TileRef {
  SegRun run;
  int kb0;
};
__device__ __forceinline__ TileRef tile_ref(const Runs& R, int i) {
  const int n0 = R.r0.nt, n1 = R.r1.nt;
  const int s = (i >= n0) + (i >= n0 + n1);
  const int t = i - (s >= 1 ? n0 : 0) - (s >= 2 ? n1 : 0);
  const bool live = i < R.T;
  TileRef r;
  r.run = sel(R.r0, R.r1, R.r2, s);
  r.run.k = uni(r.run.k);
  r.run.v = uni(r.run.v);
  r.run.kstride = uni(r.run.kstride);
  r.run.len = uni(live ? r.run.len : 0);
  r.run.causal = uni(live ? r.run.causal : 0);
  r.run.tok0 = uni(r.run.tok0);
  r.kb0 = uni(live ? t * kBN : 0);
  return r;
}

// Per-lane parts of the copy addresses (K and V tiles alike).  A copy
// instruction moves 1 KB: R rows of the tile (R = 4 for 256-byte rows, 8 for
// 128-byte rows), lane l writing 16 bytes at LDS slot l % (16 / (R / 4)) of
// row l / (64 / R).  The XOR swizzle of that row splits into a lane part and
// a part set by the copy index j: the source chunk is lane_chunk ^ (4 * j')
// with j' = j for 4-row copies and j & 1 for 8-row copies.
struct LaneCopy {
  int kq, kx16;   // row within the copy, lane chunk * 16
};
template <int D>
__device__ __forceinline__ LaneCopy lane_copy(int lane) {
  LaneCopy c;
  if constexpr (D == 128) {            // 4 rows of 16 chunks: chunk = slot ^ (row & 15)
    c.kq = lane >> 4;
    c.kx16 = ((lane & 15) ^ c.kq) << 4;
  } else {                             // 8 rows of 8 chunks: chunk = slot ^ ((row >> 1) & 7)
    c.kq = lane >> 3;
    c.kx16 = ((lane & 7) ^ (lane >> 4)) << 4;
  }
  return c;
}

// A cursor walking one operand's tiles through the unit's runs, in scalar
// registers: moving to the next tile is an add and a subtract, and the run
// table is only consulted when a run ends.  Every copy addresses memory
// inside its tensor: K rows past a run's end are read as the run's last row
// (their logits are masked), and past the walk the cursor keeps pointing at a
// tile it has already visited (or the unit's first run).
struct Cursor {
  unsigned long long addr;  // first key row of the tile (K or V)
  int rem;                  // bytes the copy may read from addr (0: nothing)
  int stride2;              // bytes between keys (below 2^24: a row offset is one 24-bit multiply)
  int left;                 // tiles left in the current run, this one included
  int s;                    // current run; 3 = past the walk
  int rows;                 // rows of the run from this tile on (0 past the walk)
};

// Enter run s (or the first later run that has tiles) at its first tile.
template <int D, bool IS_K>
__device__ __forceinline__ void cursor_enter(Cursor& c, const Runs& R, int s) {
  while (s < 3 && pick3(R.r0.nt, R.r1.nt, R.r2.nt, s) == 0) ++s;
  c.s = s;
  if (s >= 3) {          // past the walk: the cursor stays on its last tile
    c.rem = 0;
    c.rows = 0;
    c.left = 1;
    return;
  }
  const SegRun r = sel(R.r0, R.r1, R.r2, s);
  c.left = uni(r.nt);
  c.addr = (unsigned long long)uni(IS_K ? r.k : r.v);
  c.stride2 = uni(r.kstride) * 2;
  c.rows = uni(r.len);
  c.rem = c.rows * c.stride2;
}

// Start a cursor at the unit's first run (the address stays valid even when
// the walk is empty).
template <int D, bool IS_K>
__device__ __forceinline__ void cursor_start(Cursor& c, const Runs& R) {
  c.addr = (unsigned long long)(IS_K ? uni(R.r0.k) : uni(R.r0.v));
  c.stride2 = uni(R.r0.kstride) * 2;
  cursor_enter<D, IS_K>(c, R, 0);
}

template <int D, bool IS_K>
__device__ __forceinline__ void cursor_next(Cursor& c, const Runs& R) {
  if (c.left > 1) {
    --c.left;
    c.addr += (unsigned long long)(kBN * c.stride2);
    c.rem -= kBN * c.stride2;
    c.rows -= kBN;
  } else {
    cursor_enter<D, IS_K>(c, R, c.s + 1);
  }
}

__device__ __forceinline__ u32x4 cursor_rsrc(const Cursor& c) {
  u32x4 r;
  r.x = (unsigned)c.addr;
  r.y = (unsigned)(c.addr >> 32) & 0xffffu;
  r.z = (unsigned)c.rem;
  r.w = 0x00020000u;
  return r;
}

// Copy instruction j (of Geo::KINST) of this wave's share of the K or V tile
// at the cursor; the lane's tile row is clamped to the run's last row.
template <int D>
__device__ __forceinline__ void copy_k(const Cursor& c, const LaneCopy& lc, int j, const char* kbuf,
                                       int wave) {
  using G = Geo<D>;
  constexpr int R = 1024 / G::KRB;            // rows per copy
  const int blk = wave * G::KINST + j;
  const int jx = (R == 4 ? j : (j & 1)) * 64;
  const int last = max(0, min(kBN, c.rows) - 1);
  const int row = min(blk * R + lc.kq, last);
  copy16_to_lds(cursor_rsrc(c), 0u, __umul24((unsigned)row, (unsigned)c.stride2) + (unsigned)(lc.kx16 ^ jx),
                (unsigned)(unsigned long long)(kbuf + blk * 1024));
}

// V tiles are only read by transposing reads, each of which takes 4 chunks
// of 8 rows (4 r0 + a and 4 r0 + 8 + a, a < 4) with each half of the wave
// on one group of 4 rows.  Their rows therefore take their own swizzle, one
// that puts every half-wave's 16 slots on 16 distinct bank groups (no
// conflict): 256-byte rows store chunk c of row r at slot c ^ g(r) with
// g = ((r & 3) << 2) | ((r >> 2) & 3); 128-byte rows, two to a bank line,
// at slot c ^ (4 ((r >> 1) & 1)).  Both depend on r % 16 only, as the K
// swizzle does.  (The K swizzle would put 4 resp. 2 of a half-wave's slots
// on one bank group.)
template <int RB>
__device__ __forceinline__ int swz_v(int r, int c) {
  if constexpr (RB == 256) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  else return c ^ (((r >> 1) & 1) << 2);
}

// Copy instruction j (of Geo::KINST) of this wave's share of the V tile at
// the cursor, rows swizzled by swz_v; the lane's tile row is clamped to the
// run's last row.  A copy fills LDS block blk = wave * KINST + j, lane l
// writing its 16 bytes at slot l % S of row l / S (S slots per row), so the
// lane reads the source chunk that swz_v puts there.
template <int D>
__device__ __forceinline__ void copy_v(const Cursor& c, const LaneCopy& lc, int j, const char* vbuf, int wave) {
  using G = Geo<D>;
  constexpr int R = 1024 / G::KRB;            // rows per copy
  constexpr int S = G::KRB / 16;              // slots per row
  const int blk = wave * G::KINST + j;
  const int last = max(0, min(kBN, c.rows) - 1);
  const int r = blk * R + lc.kq;              // tile row this lane fills
  const int chunk = swz_v<G::KRB>(r, threadIdx.x & (S - 1));   // swz_v is its own inverse in c
  copy16_to_lds(cursor_rsrc(c), 0u, __umul24((unsigned)min(r, last), (unsigned)c.stride2) + (unsigned)(chunk * 16),
                (unsigned)(unsigned long long)(vbuf + blk * 1024));
}

template <int D>
__device__ __forceinline__ void issue_v(const Cursor& c, const LaneCopy& lc, char* vbuf, int wave) {
#pragma unroll
  for (int j = 0; j < Geo<D>::KINST; ++j) copy_v<D>(c, lc, j, vbuf, wave);
}

// The whole of this wave's share of one tile's copies at once (prologue).
template <int D>
__device__ __forceinline__ void issue_k(const Cursor& c, const LaneCopy& lc, char* kbuf, int wave) {
#pragma unroll
  for (int j = 0; j < Geo<D>::KINST; ++j) copy_k<D>(c, lc, j, kbuf, wave);
}


// Scores of one tile per (query block, 32-key half), and the bf16
// probabilities of one tile per (query block, 16-key chunk).
struct Scores {
  f32x16 s[2][2];
};
struct Probs {
  bf16x8 p[2][4];
};

// Softmax wave: constants and running statistics of its 64 rows.
template <int D>
struct SoftCtx {
  bf16x8 qf[2][D / 16];  // Q^T fragments (B operand) per query block
  int koff[D / 16];      // LDS byte offsets of this lane's K fragments
  int qtok[2];           // this lane's query token per block
  float sl2;             // softmax scale * log2(e)
  int lane, hi;
};
struct SoftState {
  float m[2];       // running max per query block, exp2 domain (scaled logits)
  float l[2];       // this lane's partial row sums (its 16 keys of every 32)
};

// LDS byte offset of P chunk (qb, kc) for a lane: the output wave reads the
// softmax wave's B-operand registers back with the same lane mapping.
__device__ __forceinline__ int p_off(int qb, int kc, int lane) { return ((qb * 4 + kc) * 64 + lane) * 16; }

// Probabilities of S(i-1) against the running maxima, straight to LDS;
// returns (per lane) whether any of them may exceed 2^8 (row sum above it, or
// not finite) or the row has no reference yet.
template <int D>
__device__ __forceinline__ bool soft_probs(const Scores& sp, char* pwrite, const SoftCtx<D>& cx,
                                           const SoftState& st, float (&acc)[2]) {
  bool grow = false;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float m_use = (st.m[qb] == -INFINITY) ? 0.0f : st.m[qb];
    float a = 0.0f;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sp.s[qb][kc >> 1][8 * (kc & 1) + e], cx.sl2, -m_use));
        a += p;
        pb[e] = (__bf16)p;
      }
      *(bf16x8*)(pwrite + p_off(qb, kc, cx.lane)) = pb;
    }
    acc[qb] = a;
    grow |= !(a <= 256.0f) || st.m[qb] == -INFINITY;
  }
  return grow;
}

// One softmax-wave iteration.  kread holds K(i); P(i-1) and the factor that
// moves O from the previous maximum to the one P(i-1) is computed against go
// to pwrite, awrite, fwrite.  MASK applies the visibility limits of S(i).
//
// The maximum is only looked at when the probabilities of a tile could leave
// [0, 2^8]: a lane's sum of its 32 probabilities bounds each of them, so the
// common path needs no row maxima at all.  Then (rarely) the row maxima of
// S(i-1) move the reference, the row sums are rescaled, P(i-1) is recomputed
// and written again, and the output wave rescales O before adding it.
// LIVE = false is iteration T of a T-tile walk: S(T) would be read by nobody,
// so it is not computed (no K reads, no MFMAs); it is left at -inf.
// HEAD = 1 is iteration 0: there is no P(-1), only S(0) is computed.  HEAD = 2
// is iteration 1: no row has a reference yet, so P(0) is computed once,
// against S(0)'s own row maxima, instead of speculatively and again.
// ring carries the first K fragments from one iteration to the next: K(i+1)
// is complete from the barrier of iteration i on (the output waves wait for
// all of their copies before it), so iteration i reads K(i+1)'s first
// fragments after its own MFMAs, and iteration i+1's first MFMAs need not
// wait for LDS after its barrier.  Iteration 0 reads its own.
struct KSlots {
  const char* cur;   // K(i)
  const char* nxt;   // K(i+1)
};
template <int D, bool MASK, bool LIVE = true, int HEAD = 0>
__device__ __forceinline__ void soft_iter(int i, const Runs& run, KSlots ks, bf16x8 (&ring)[4],
                                          char* __restrict__ pwrite, float* __restrict__ awrite,
                                          int* __restrict__ fwrite, const SoftCtx<D>& cx, SoftState& st,
                                          const Scores& s_prev, Scores& s_new) {
  using G = Geo<D>;
  constexpr int NC = G::NC;
  constexpr int KRB = G::KRB;
  constexpr int NA = 2 * NC;   // K fragments (h2, c)
  constexpr int RING = 4;
  asm volatile("" : "+s"(i));
  __syncthreads();
  // Fragment n = (d chunk c, key half h2) with h2 fastest: the four
  // accumulators (qb, h2) alternate, so no MFMA waits on the one before.
  const char* const kread = ks.cur;
  auto kfrag = [&](int n) {
    return *(const bf16x8*)(kread + cx.koff[n / 2] + (n % 2) * 32 * KRB);
  };
  // S(i) = K(i) Q^T, fragments RING reads ahead of their MFMAs, with the
  // probabilities P(i-1) = exp2(S(i-1) * sl2 - m) computed in even chunks
  // between the MFMA pairs: the softmax wave's vector work then issues while
  // the matrix core runs this wave's or the output wave's MFMAs, instead of
  // after all of them.
  constexpr int PPC = 64 / NA;   // probabilities per fragment step
  float mu[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) mu[qb] = (st.m[qb] == -INFINITY) ? 0.0f : st.m[qb];
  float acc[2] = {0.0f, 0.0f};
  bf16x8 pb;
  if (LIVE && HEAD == 1) {
#pragma unroll
    for (int n = 0; n < RING; ++n) ring[n] = kfrag(n);
  }
#pragma unroll
  for (int n = 0; n < NA; ++n) {
    const int h2 = n % 2, c = n / 2;
    if (LIVE) {
      const bf16x8 af = ring[n % RING];
      if (n + RING < NA) ring[n % RING] = kfrag(n + RING);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        s_new.s[qb][h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            af, cx.qf[qb][c], c == 0 ? f32x16{} : s_new.s[qb][h2], 0, 0, 0);
    }
    if (HEAD == 0) {
#pragma unroll
      for (int t = 0; t < PPC; ++t) {
        const int idx = n * PPC + t;
        const int qb = idx >> 5, kc = (idx >> 3) & 3, e = idx & 7;
        const float p = __builtin_amdgcn_exp2f(fmaf(s_prev.s[qb][kc >> 1][8 * (kc & 1) + e], cx.sl2, -mu[qb]));
        acc[qb] += p;
        pb[e] = (__bf16)p;
        if (e == 7) *(bf16x8*)(pwrite + p_off(qb, kc, cx.lane)) = pb;
      }
    }
  }
  if (LIVE) {   // K(i+1)'s first fragments for the next iteration
#pragma unroll
    for (int n = 0; n < RING; ++n) ring[n] = *(const bf16x8*)(ks.nxt + cx.koff[n / 2] + (n % 2) * 32 * KRB);
  }
  if (HEAD != 1) {
    bool grow = HEAD == 2;
    if (HEAD == 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) grow |= !(acc[qb] <= 256.0f) || st.m[qb] == -INFINITY;
    }
    int moved = 0;
    float alpha[2] = {1.0f, 1.0f};
    if (__any(grow)) {
      moved = 1;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float x;
        asm volatile("v_mov_b32 %0, 0xff800000" : "=v"(x));   // -inf, computed only here
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int e = 0; e < 16; ++e) x = fmaxf(x, s_prev.s[qb][h2][e]);
        const float mp = fmaxf(x, __shfl_xor(x, 32)) * cx.sl2;
        const float m_new = fmaxf(st.m[qb], mp);
        alpha[qb] = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(st.m[qb] - m_new);
        st.m[qb] = m_new;
        st.l[qb] *= alpha[qb];
      }
      soft_probs<D>(s_prev, pwrite, cx, st, acc);
    }
    st.l[0] += acc[0];   // float32 row sums: the LSE output needs them to ~1e-6
    st.l[1] += acc[1];
    if (cx.hi == 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) awrite[qb * 32 + (cx.lane & 31)] = alpha[qb];
    }
    if (cx.lane == 0) *fwrite = moved;
  }

  if (!LIVE) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 16; ++e) s_new.s[qb][h2][e] = -INFINITY;
  }
  // Visibility of S(i): keys past the run's end, or in a causal run past the
  // row's token, get -inf.
  if (MASK && LIVE) {
    const TileRef tr = tile_ref(run, i);
    const SegRun& sr = tr.run;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      int lim = sr.len - tr.kb0;            // tile-local key j is visible iff j < lim
      if (sr.causal) lim = min(lim, cx.qtok[qb] - sr.tok0 - tr.kb0 + 1);
      const int lim1 = lim - 1 - 8 * cx.hi;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = 32 * h2 + (e & 7) + 16 * (e >> 3);
          if (lim1 < j) s_new.s[qb][h2][e] = -INFINITY;
        }
    }
  }
}

// One transposing LDS read (gfx950 ds_read_b64_tr_b16).  Each lane gives
// the address of 8 bytes (four 16-bit elements); within each group of 16
// lanes, lane i receives element i % 4 of the 8 bytes addressed by lane
// 4k + i / 4 of its group as its element k (k = 0..3).
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(const_cast<char*>(p)));
}

// Output wave: constants of its 64 rows and its share of the tile copies.
template <int D>
struct OutCtx {
  int voff[2][D / 32];   // LDS byte offsets of this lane's two transposing reads per 32-channel block
  LaneCopy lc;           // per-lane parts of the tile copy addresses
  int w;                 // index among the output waves (its share of each copy)
  int lane;
};

// LDS byte offsets, for 16-key chunk 0 of a row-major V tile, of lane l's two
// transposing reads of channel block db: together they give lane l the A
// operand of O^T += V^T P^T, channel 32 db + l % 32 at keys 8 (l / 32) + 0..7.
// Lane l = 16 G + i addresses row 8 (G / 2) + 4 t + i / 4 (read t = 0, 1),
// channels 32 db + 16 (G % 2) + 4 (i % 4) .. + 3, so lane i of the group
// receives channel 32 db + 16 (G % 2) + i at the four keys of read t.  Rows
// are swizzled in 16-byte slots as the copies wrote them (swz_v); the
// swizzle of row 16 c + r equals that of row r, so chunk c adds c * 16 rows.
template <int D>
__device__ __forceinline__ void v_read_offsets(int lane, int (&voff)[2][D / 32]) {
  constexpr int KRB = 2 * D;
  const int G = lane >> 4, i = lane & 15;
  const int rbase = 8 * (G >> 1) + (i >> 2);
  const int cbase = 16 * (G & 1) + 4 * (i & 3);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int r = 4 * t + rbase;
      const int col = 32 * db + cbase;
      voff[t][db] = r * KRB + swz_v<KRB>(r, col >> 3) * 16 + (col & 7) * 2;
    }
}

// One output-wave iteration: copies of V(i-1) (to vload; empty for i = 0)
// and K(i+2) (to kload), then O = O * alpha(i-2) + V(i-2) P(i-2) from vread,
// pread, aread, fread.  Once all of this wave's copies have landed (V(i-2),
// K(i) and K(i+1), issued an iteration or more ago), the barrier publishes
// them: the softmax waves read K(i+1)'s first fragments before the next one.
template <int D>
__device__ __forceinline__ void out_iter(int i, const Runs& run, const char* __restrict__ vread,
                                         const char* __restrict__ pread, const float* __restrict__ aread,
                                         const int* __restrict__ fread, char* __restrict__ kload,
                                         char* __restrict__ vload, const OutCtx<D>& cx,
                                         f32x16 (&o)[2][D / 32], Cursor& kc, Cursor& vc) {
  using G = Geo<D>;
  constexpr int NDB = G::NDB;
  asm volatile("" : "+s"(i));
  wait_vm<0>();
  __syncthreads();
  constexpr int NB = 4 * NDB;   // V^T fragments (16-key chunk, 32-channel block)
  constexpr int RING = 4;
  if (i >= 2) {
    // The rescale flag, P(i-2) and the first V^T fragments are all in
    // flight before the flag is looked at.
    const int moved = *fread;
    auto vfrag = [&](int n) {
      const char* base = vread + (n / NDB) * 16 * G::KRB;
      union {
        s16x4 h[2];
        bf16x8 v;
      } f;
      f.h[0] = lds_read_tr16(base + cx.voff[0][n % NDB]);
      f.h[1] = lds_read_tr16(base + cx.voff[1][n % NDB]);
      return f.v;
    };
    bf16x8 pf[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) pf[qb][ch] = *(const bf16x8*)(pread + p_off(qb, ch, cx.lane));
    bf16x8 ring[RING];
#pragma unroll
    for (int n = 0; n < RING; ++n) ring[n] = vfrag(n);
    if (__builtin_amdgcn_readfirstlane(moved)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float alpha = aread[qb * 32 + (cx.lane & 31)];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[qb][db][e] *= alpha;
      }
    }
    // O += V(i-2) P(i-2) through the fragment ring.
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const bf16x8 vf = ring[n % RING];
      if (n + RING < NB) ring[n % RING] = vfrag(n + RING);
      const int ch = n / NDB, db = n % NDB;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][ch], o[qb][db], 0, 0, 0);
      // The tile copies go out one per MFMA pair: V(i-1), then K(i+2).
      if (n >= 1 && n < 1 + G::KINST) copy_v<D>(vc, cx.lc, n - 1, vload, cx.w);
      if (n == G::KINST) cursor_next<D, false>(vc, run);
      if (n >= 1 + G::KINST && n < 1 + 2 * G::KINST) copy_k<D>(kc, cx.lc, n - 1 - G::KINST, kload, cx.w);
      if (n == 2 * G::KINST) cursor_next<D, true>(kc, run);
    }
  } else {
    // Nothing to add yet; V(-1) is empty.
    if (i == 0) {
      Cursor none = vc;
      none.rem = 0;
      issue_v<D>(none, cx.lc, vload, cx.w);
    } else {
      issue_v<D>(vc, cx.lc, vload, cx.w);
      cursor_next<D, false>(vc, run);
    }
    issue_k<D>(kc, cx.lc, kload, cx.w);
    cursor_next<D, true>(kc, run);
  }
}

// Leading tiles of the walk that no row of the workgroup sees partly: the
// softmax waves run them without masks.  gmin is the workgroup's smallest
// query token.
__device__ __forceinline__ int unmasked_prefix(const Runs& R, int gmin) {
  int base = 0;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const SegRun r = s == 0 ? R.r0 : (s == 1 ? R.r1 : R.r2);
    int nf = r.len / kBN;                              // whole tiles of the run
    if (r.causal) nf = min(nf, max(0, (gmin - r.tok0 + 1) / kBN));
    nf = min(nf, r.nt);
    if (nf < r.nt) return base + nf;
    base += r.nt;
  }
  return base;
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(AttnArgs a) {
  using G = Geo<D>;
  constexpr int NC = G::NC;
  constexpr int NDB = G::NDB;
  constexpr int KRB = G::KRB;
  // One LDS block laid out by hand with the V ring at address 0: a V read is
  // then its lane's offset plus an immediate (slot, 16-key chunk), which the
  // 16-bit offset field of an LDS read holds, so the output wave spends no
  // vector instruction on V addresses.
  constexpr int kOffK = kVSlots * G::KBYTES;
  constexpr int kOffP = kOffK + kKSlots * G::KBYTES;
  constexpr int kOffA = kOffP + 2 * kPairs * kPBytes;
  constexpr int kOffF = kOffA + 2 * kPairs * 64 * (int)sizeof(float);
  constexpr int kOffL = kOffF + 2 * kPairs * (int)sizeof(int);
  constexpr int kLdsBytes = kOffL + kPairs * 64 * (int)sizeof(float);
  static_assert(kVSlots * G::KBYTES <= 65536, "V reads take their slot and chunk as an immediate");
  static_assert(kOffP % 1024 == 0 && kOffK % 1024 == 0, "tiles stay 1 KB aligned");
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  char* const sV = smem;
  char* const sK = smem + kOffK;
  char* const sP = smem + kOffP;
  float* const sAlpha = (float*)(smem + kOffA);
  int* const sFlag = (int*)(smem + kOffF);
  float* const sL = (float*)(smem + kOffL);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & (kPairs - 1);
  const bool soft = wave < kPairs;
  const int hi = lane >> 5;
  const int col = lane & 31;

  const int b = a.unit_lo + xcd_unit(blockIdx.x, a.xcd_chunk);
  if (b >= a.unit_hi) return;
  const Unit u = unit_decode(a, b);
  Runs run;
  unit_runs(a, u, run.r0, run.r1, run.r2);

  // This lane's query row in each of the pair's two 32-column blocks.
  RowId row[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) row[qb] = unit_row(a, u, u.tile * kBM + pair * kWaveRows + 32 * qb + col);

  // Token range of the workgroup (tile count, mask-free prefix), from the
  // unit's row range: rows r of a context or anchor unit are tokens base + r;
  // query rows r are tokens q0 + r % nq.
  int gmin, gmax;
  {
    const int r_lo = u.tile * kBM;
    if (u.kind == kAnchor || u.kind == kContext) {
      const int base = (u.kind == kAnchor) ? 0 : a.la + u.host * a.L;
      const int n = (u.kind == kAnchor) ? a.la : a.L;
      gmin = base + r_lo;
      gmax = base + min(n, r_lo + kBM) - 1;
    } else {
      const int q0 = a.la + a.V * a.L;
      const int r_hi = min(a.nq * a.G, r_lo + kBM) - 1;
      const bool wraps = r_hi - r_lo + 1 >= a.nq || r_lo % a.nq > r_hi % a.nq;
      gmin = q0 + (wraps ? 0 : r_lo % a.nq);
      gmax = q0 + (wraps ? a.nq - 1 : r_hi % a.nq);
    }
    gmin = uni(gmin);
    gmax = uni(gmax);
  }
  auto tiles = [&](SegRun& x) {
    int n = x.len;
    if (x.causal) n = min(n, gmax - x.tok0 + 1);
    x.nt = uni(n > 0 ? ceil_div(n, kBN) : 0);
  };
  tiles(run.r0);
  tiles(run.r1);
  tiles(run.r2);
  run.T = run.r0.nt + run.r1.nt + run.r2.nt;
  const int n_iter = run.T + 2;   // iteration T+1 adds the last P V

  if (soft) {
    SoftCtx<D> cx;
    cx.lane = lane;
    cx.hi = hi;
    cx.sl2 = a.scale_log2;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      cx.qtok[qb] = row[qb].tok;
      const uint16_t* qp = (const uint16_t*)a.q + (long)row[qb].tok * a.q_st + (long)row[qb].head * a.q_sh + 8 * hi;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        cx.qf[qb][c] = *(const bf16x8*)(qp + 16 * c);
        if (!row[qb].valid) {
#pragma unroll
          for (int e = 0; e < 8; ++e) cx.qf[qb][c][e] = (__bf16)0.0f;
        }
      }
    }
    const int krow = perm_row(col);               // + 32 per 32-key half
#pragma unroll
    for (int c = 0; c < NC; ++c) cx.koff[c] = krow * KRB + swz<KRB>(krow, 2 * c + hi) * 16;

    SoftState st;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      st.m[qb] = -INFINITY;
      st.l[qb] = 0.0f;
    }
    Scores sA, sB;   // S(-1) = -inf: no probabilities
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 16; ++e) sA.s[qb][h2][e] = -INFINITY;

    // Slots of iteration i: K(i) in i % 3; P(i-1) and its factor in buffer
    // (i-1) % 2 (even and odd iterations are unrolled with fixed buffers).
    int k3 = 0;   // i % 3
    bf16x8 kring[4];
    auto knext = [&]() {
      KSlots r;
      r.cur = sK + k3 * G::KBYTES;
      k3 = (k3 == kKSlots - 1) ? 0 : k3 + 1;
      r.nxt = sK + k3 * G::KBYTES;
      return r;
    };
    char* const p0 = sP + pair * kPBytes;
    char* const p1 = sP + (kPairs + pair) * kPBytes;
    float* const a0 = sAlpha + pair * 64;
    float* const a1 = sAlpha + (kPairs + pair) * 64;
    int* const f0 = sFlag + pair;
    int* const f1 = sFlag + kPairs + pair;
    const int n_plain = min(unmasked_prefix(run, gmin), n_iter) & ~1;
    // Iterations 0 and 1: S(0) alone, then S(1) with P(0) against S(0)'s
    // maxima (a walk of one tile makes iteration 1 its last, dead one).
    if (n_plain >= 2) {
      soft_iter<D, false, true, 1>(0, run, knext(), kring, p1, a1, f1, cx, st, sA, sB);
      soft_iter<D, false, true, 2>(1, run, knext(), kring, p0, a0, f0, cx, st, sB, sA);
    } else {
      soft_iter<D, true, true, 1>(0, run, knext(), kring, p1, a1, f1, cx, st, sA, sB);
      if (run.T >= 2)
        soft_iter<D, true, true, 2>(1, run, knext(), kring, p0, a0, f0, cx, st, sB, sA);
      else
        soft_iter<D, true, false, 2>(1, run, knext(), kring, p0, a0, f0, cx, st, sB, sA);
    }
    for (int i = 2; i < n_plain; i += 2) {
      soft_iter<D, false>(i, run, knext(), kring, p1, a1, f1, cx, st, sA, sB);
      soft_iter<D, false>(i + 1, run, knext(), kring, p0, a0, f0, cx, st, sB, sA);
    }
    for (int i = max(2, n_plain); i < run.T; i += 2) {
      soft_iter<D, true>(i, run, knext(), kring, p1, a1, f1, cx, st, sA, sB);
      if (i + 1 >= run.T) break;
      soft_iter<D, true>(i + 1, run, knext(), kring, p0, a0, f0, cx, st, sB, sA);
    }
    // Iteration T computes P(T-1) only; in iteration T+1 (the output wave's
    // last P V) this wave has nothing left that is read, so it only meets the
    // barrier.
    if (run.T >= 2) {
      if ((run.T & 1) == 0)
        soft_iter<D, true, false>(run.T, run, knext(), kring, p1, a1, f1, cx, st, sA, sB);
      else
        soft_iter<D, true, false>(run.T, run, knext(), kring, p0, a0, f0, cx, st, sB, sA);
    }
    __syncthreads();
    // Row sums to the output wave; LSE out.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float lt = st.l[qb] + __shfl_xor(st.l[qb], 32);
      if (hi == 0) sL[pair * 64 + qb * 32 + col] = lt;
      if (hi != 0 || !row[qb].valid) continue;
      const float lse_nat = (lt > 0.0f) ? (st.m[qb] + __log2f(lt)) * 0.69314718055994530942f : -INFINITY;
      if (u.kind == kAnchor || u.kind == kContext) {
        a.lse[(long)row[qb].head * a.N + row[qb].tok] = lse_nat;
      } else {
        const int p = (u.kind == kQueryHead) ? 0 : u.host + 1;
        const int qi = row[qb].tok - (a.la + a.V * a.L);
        a.lse_part[((long)p * a.Hq + row[qb].head) * a.nq + qi] = lse_nat;
      }
    }
    __syncthreads();
  } else {
    OutCtx<D> cx;
    cx.lane = lane;
    cx.w = wave - kPairs;
    cx.lc = lane_copy<D>(lane);
    v_read_offsets<D>(lane, cx.voff);
    f32x16 o[2][NDB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[qb][db][e] = 0.0f;

    // K(0) and K(1) ahead of iteration 0; the cursors then stand at K(2) and V(0).
    Cursor kc, vc;
    cursor_start<D, true>(kc, run);
    cursor_start<D, false>(vc, run);
    issue_k<D>(kc, cx.lc, sK, cx.w);
    cursor_next<D, true>(kc, run);
    issue_k<D>(kc, cx.lc, sK + G::KBYTES, cx.w);
    cursor_next<D, true>(kc, run);

    // Iteration i: copies of V(i-1) into slot (i+1) % 2 and of K(i+2) into
    // slot (i+2) % 3; reads V(i-2) from slot i % 2 and P(i-2) from buffer i % 2.
    int k3 = 2;   // (i + 2) % 3
    char* const v0 = sV;
    char* const v1 = sV + G::KBYTES;
    const char* const p0 = sP + pair * kPBytes;
    const char* const p1 = sP + (kPairs + pair) * kPBytes;
    const float* const a0 = sAlpha + pair * 64;
    const float* const a1 = sAlpha + (kPairs + pair) * 64;
    const int* const f0 = sFlag + pair;
    const int* const f1 = sFlag + kPairs + pair;
    for (int i = 0; i < n_iter; i += 2) {
      out_iter<D>(i, run, v0, p0, a0, f0, sK + k3 * G::KBYTES, v1, cx, o, kc, vc);
      k3 = (k3 == kKSlots - 1) ? 0 : k3 + 1;
      if (i + 1 >= n_iter) break;
      out_iter<D>(i + 1, run, v1, p1, a1, f1, sK + k3 * G::KBYTES, v0, cx, o, kc, vc);
      k3 = (k3 == kKSlots - 1) ? 0 : k3 + 1;
    }
    wait_vm<0>();
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (!row[qb].valid) continue;
      const float lt = sL[pair * 64 + qb * 32 + col];
      const float inv = (lt > 0.0f) ? 1.0f / lt : 0.0f;
      if (u.kind == kAnchor || u.kind == kContext) {
        uint16_t* op = (uint16_t*)a.o + ((long)row[qb].tok * a.Hq + row[qb].head) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * db + 8 * g4 + 4 * hi;
            union { __bf16 h[4]; uint2 u; } pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) pk.h[e] = (__bf16)(o[qb][db][4 * g4 + e] * inv);
            *(uint2*)(op + d0) = pk.u;
          }
      } else {
        const int p = (u.kind == kQueryHead) ? 0 : u.host + 1;
        const int qi = row[qb].tok - (a.la + a.V * a.L);
        float* op = a.o_part + (((long)p * a.nq + qi) * a.Hq + row[qb].head) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * db + 8 * g4 + 4 * hi;
            float4 w;
            w.x = o[qb][db][4 * g4 + 0] * inv;
            w.y = o[qb][db][4 * g4 + 1] * inv;
            w.z = o[qb][db][4 * g4 + 2] * inv;
            w.w = o[qb][db][4 * g4 + 3] * inv;
            *(float4*)(op + d0) = w;
          }
      }
    }
  }
}

}  // namespace

int attn_bf16_rows_per_unit() { return kBM; }

hipError_t launch_attn_bf16(const AttnArgs& a_in, hipStream_t s) {
  AttnArgs a = a_in;
  const int n = a.unit_hi - a.unit_lo;
  if (n <= 0) return hipSuccess;
  // XCD chunks of G units: the query heads of one KV head (one row tile)
  // share an L2.  Chunks of all Hq heads were 2-10 % slower: fewer, larger
  // chunks leave the XCDs unevenly loaded near the end of the launch.
  a.xcd_chunk = a.G;
  const dim3 grid(xcd_grid(n, a.xcd_chunk));
  if (a.D == 128)
    hipLaunchKernelGGL((attn_bf16_kernel<128>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<64>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace spava
