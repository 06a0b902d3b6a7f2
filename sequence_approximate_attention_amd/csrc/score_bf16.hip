// Block scoring for bf16 inputs on gfx950 (CDNA4).
//
// The selection rule (Figure 5 caption of the Spava page: the query rows'
// Q K^(h)T estimate how important block h's keys are; "What carries the
// argument" in the APB-V review: keys ranked by query-to-context attention
// scores) needs, for block h and KV head g, the column sums over the query
// rows r = (token i, head a in g) of softmax_j(q_r . k_j * scale) over the
// block's L keys.  Two MFMA passes over the block:
//
//   rowstat_chunk_kernel: each query row's running (max, sum) of
//     exp2(s * scale * log2 e) over one key chunk of the block (512 keys, or
//     L/16 for longer blocks).  A workgroup
//     is 4 waves x 64 rows; the chunk is walked in 64-key tiles that
//     buffer_load_dwordx4 ... lds copies into a 4-slot LDS ring, three tiles
//     ahead.  Splitting the block into chunks gives the GPU enough
//     workgroups; the partial (max, sum) pairs are combined by the next pass.
//
// CTX = true gives the context-driven selector (APB-V review, Referee Report,
// major comment 1): the rows are block h's own tokens, each attending
// causally over the block's keys (key j visible to token t iff j <= t); key
// chunks above a workgroup's last token and row chunks below its first key
// are skipped.
//
//   colsum_kernel: combines each row's chunk partials into its log2-domain
//     log-sum-exp, then for 256 (query rows) or 384 (context selector) keys
//     sums exp2(s - lse) over the rows of its row split.  Each of 4 waves
//     keeps its 64 or 96 keys' fragments in registers; they walk the split's 32-row
//     chunks, whose Q tiles are copied into a 3-slot LDS ring, two chunks
//     ahead.  Large grids run such 4-wave workgroups two or three to a CU;
//     small ones pair two of them in one workgroup on alternate chunks, their
//     totals added at the end.  Column sums accumulate per chunk in float32, across
//     chunks in float64, in a fixed order (deterministic).  The query rows
//     form one split (the sums go straight to the scores); the context
//     selector splits each head's tokens into ranges of at least 1024, each
//     workgroup starting at its first key's token, and colsum_reduce_kernel
//     adds the splits' float partials in split order.
#include "lds_dma.h"

namespace spava {
namespace {

constexpr int kBN = kKeyTile;

// ---------------------------------------------------------------------------
// Row statistics over key chunks.

constexpr int kRsWaves = 4;
constexpr int kRsWaveRows = 64;                  // two 32-column MFMA blocks
constexpr int kRsBM = kRsWaves * kRsWaveRows;    // rows per workgroup
constexpr int kRsThreads = kRsWaves * 64;
constexpr int kRsSlots = 4;                      // K tile ring
constexpr int kTilesPerChunk = 8;                // 512 keys per chunk (at least)

template <int D>
struct RsGeo {
  static constexpr int NC = D / 16;              // 16-wide d chunks
  static constexpr int KRB = 2 * D;              // bytes per K row
  static constexpr int KBYTES = kBN * KRB;       // K tile
  static constexpr int RPI = 1024 / KRB;         // K rows per copy instruction
  static constexpr int KINST = KBYTES / 1024 / kRsWaves;
};

// Element offset of scoring row r of KV head g (see score_rows).
__device__ __forceinline__ long q_row_elem(const AttnArgs& a, const ScoreRows& sr, int g, int r) {
  const int tok = sr.tok0 + r % sr.ntok;
  const int head = g * a.G + r / sr.ntok;
  return (long)tok * a.q_st + (long)head * a.q_sh;
}

// Largest block-local token among the rows [r_lo, r_hi] (inclusive) of the
// context selector's row order.
__device__ __forceinline__ int last_token(int r_lo, int r_hi, int ntok) {
  return (r_lo / ntok != r_hi / ntok) ? ntok - 1 : r_hi % ntok;
}

// This wave's share of the copy of tile t of the chunk into kbuf.  Every lane
// addresses a key of the block: rows past the block's end read its last key
// (their logits are masked), and past the chunk's last tile (t >= nt, a slot
// that is never read) the copy re-reads the chunk's first tile, so every
// iteration issues the same number of copies.
template <int D>
__device__ __forceinline__ void rs_issue(const u32x4& rs_blk, int kstride2, int L, int t0, int t, int nt,
                                         char* kbuf, int wave, int lane) {
  using G = RsGeo<D>;
  const int tt = t0 + (t < nt ? t : 0);          // tile of the block
  const int q = lane / (G::KRB / 16);            // row within the copy
  const int slot = lane % (G::KRB / 16);
#pragma unroll
  for (int j = 0; j < G::KINST; ++j) {
    const int blk = wave * G::KINST + j;
    const int row = blk * G::RPI + q;            // tile row
    const int chunk = swz<G::KRB>(row, slot);    // source 16-byte chunk stored at this slot
    const int key = min(tt * kBN + row, L - 1);
    copy16_to_lds(rs_blk, 0u, (unsigned)(key * kstride2 + chunk * 16),
                  (unsigned)(unsigned long long)(kbuf + blk * 1024));
  }
}

template <int D, bool CTX>
__global__ __launch_bounds__(kRsThreads, 2) void rowstat_chunk_kernel(AttnArgs a, int KC, int TPC, int RT,
                                                                       float2* __restrict__ part) {
  using G = RsGeo<D>;
  constexpr int NC = G::NC;
  constexpr int KRB = G::KRB;
  __shared__ __attribute__((aligned(1024))) char sK[kRsSlots * G::KBYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  const int col = lane & 31;
  const int VH = a.V * a.Hkv;

  // Unit b = ((h * Hkv + g) * KC + kc) * RT + rt: the row tiles of one key
  // chunk are consecutive (and dealt to one XCD).
  const int n_units = VH * KC * RT;
  const int b = xcd_unit(blockIdx.x, RT);
  if (b >= n_units) return;
  // Context selector: row tiles of later tokens see more keys; they start first.
  const int rt = CTX ? RT - 1 - b % RT : b % RT;
  const int kc = (b / RT) % KC;
  const int hg = b / (RT * KC);
  const int h = hg / a.Hkv;
  const int g = hg % a.Hkv;
  const ScoreRows sr = score_rows(a, h);
  const int R = sr.R;

  // This lane's two scoring rows (one per 32-column block).
  int r[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) r[qb] = rt * kRsBM + wave * kRsWaveRows + 32 * qb + col;

  // The chunk's tiles [t0, t0 + nt) of block h; keys past the block's end
  // are masked.
  const int T = ceil_div(a.L, kBN);
  const int t0 = kc * TPC;
  int nt = min(T, t0 + TPC) - t0;
  int lim_row[2] = {a.L, a.L};   // block-local keys visible to this lane's rows: [0, lim_row)
  if (CTX) {
    // Tiles past the workgroup's last token hold no visible key.
    const int r_lo = rt * kRsBM;
    const int r_hi = min(R, r_lo + kRsBM) - 1;
    nt = max(0, min(nt, ceil_div(last_token(r_lo, r_hi, sr.ntok) + 1, kBN) - t0));
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) lim_row[qb] = (r[qb] < R) ? r[qb] % sr.ntok + 1 : 0;
    if (nt == 0) {   // the whole chunk lies above the diagonal: an empty partial
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        if (hi == 0 && r[qb] < R) part[((long)kc * VH + hg) * R + r[qb]] = make_float2(-INFINITY, 0.0f);
      return;
    }
  }

  bf16x8 qf[2][NC];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const bool valid = r[qb] < R;
    const uint16_t* qp = (const uint16_t*)a.q + q_row_elem(a, sr, g, valid ? r[qb] : 0) + 8 * hi;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[qb][c] = *(const bf16x8*)(qp + 16 * c);
      if (!valid) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qb][c][e] = (__bf16)0.0f;
      }
    }
  }

  const int kstride2 = (int)a.kv_st * 2;
  const uint16_t* kblk = (const uint16_t*)a.k + (long)(a.la + h * a.L) * a.kv_st + (long)g * a.kv_sh;
  const u32x4 rs_blk = make_rsrc(kblk, (unsigned)a.L * (unsigned)kstride2);

  // The compiler's own wait bookkeeping does not see the LDS copies: settle
  // the Q loads here so that no full wait lands inside the tile loop.
  wait_vm<0>();

  const int krow = perm_row(col);
  int koff[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) koff[c] = krow * KRB + swz<KRB>(krow, 2 * c + hi) * 16;

  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.0f, 0.0f};
  const float sl2 = a.scale_log2;
#pragma unroll
  for (int t = 0; t < kRsSlots - 1; ++t) rs_issue<D>(rs_blk, kstride2, a.L, t0, t, nt, sK + t * G::KBYTES, wave, lane);

  for (int t = 0; t < nt; ++t) {
    wait_vm<(kRsSlots - 2) * G::KINST>();   // tile t has landed (this wave's part)
    __syncthreads();                          // ... everyone's; slot of t-1 is free
    const int tn = t + kRsSlots - 1;
    rs_issue<D>(rs_blk, kstride2, a.L, t0, tn, nt, sK + (tn % kRsSlots) * G::KBYTES, wave, lane);
    const char* kt = sK + (t % kRsSlots) * G::KBYTES;

    f32x16 s[2][2];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const bf16x8 af = *(const bf16x8*)(kt + koff[c] + h2 * 32 * KRB);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s[qb][h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[qb][c], c == 0 ? f32x16{} : s[qb][h2], 0, 0, 0);
      }
    // Tile-local key j is visible to a row iff j < lim (past the block's end,
    // and for the context selector past the row's own token, it is masked).
    int lim[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) lim[qb] = min(a.L, lim_row[qb]) - (t0 + t) * kBN;
    if (__any(lim[0] < kBN || lim[1] < kBN)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int j = 32 * h2 + (e & 7) + 8 * hi + 16 * (e >> 3);
            if (j >= lim[qb]) s[qb][h2][e] = -INFINITY;
          }
    }
    // The sums are taken against the running reference m as long as no term
    // can exceed 2^8 (a lane's sum of its 32 terms bounds each of them), so
    // the common tile needs no row maximum; otherwise (and while a row has
    // no reference yet) the tile's maxima move m and the sum is taken again.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float m_use = (m[qb] == -INFINITY) ? 0.0f : m[qb];
      float psum = 0.0f;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 16; ++e) psum += __builtin_amdgcn_exp2f(fmaf(s[qb][h2][e], sl2, -m_use));
      if (__any(!(psum <= 256.0f) || m[qb] == -INFINITY)) {
        float mx = -INFINITY;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[qb][h2][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
        const float m_new = fmaxf(m[qb], mx);
        l[qb] *= (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m[qb] - m_new);
        m[qb] = m_new;
        const float m_use2 = (m_new == -INFINITY) ? 0.0f : m_new;
        psum = 0.0f;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int e = 0; e < 16; ++e) psum += __builtin_amdgcn_exp2f(fmaf(s[qb][h2][e], sl2, -m_use2));
      }
      l[qb] += psum;
    }
  }
  wait_vm<0>();   // no copy may still be landing in LDS when the workgroup ends
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    if (hi == 0 && r[qb] < R) part[((long)kc * VH + hg) * R + r[qb]] = make_float2(m[qb], lt);
  }
}

// ---------------------------------------------------------------------------
// Column sums.

// A workgroup is one or two halves of 4 waves over the same keys; the halves
// take alternate 32-row chunks and add their totals at the end.  One half per
// workgroup lets three workgroups (query rows, 155 VGPRs) or two (context
// selector) share a CU independently, so one's exponentials overlap another's
// MFMAs; two halves keep 8 waves per CU when the grid is too small for that.
constexpr int kCsWavesPerHalf = 4;
constexpr int kCsKbQuery = 2;                    // 32-key blocks per wave: query rows
constexpr int kCsKbCtx = 3;                      // ... context selector
constexpr int kCsSingleGrid = 1024;              // query rows: one half per workgroup from this grid size on
constexpr int kCsRows = 32;                      // rows per chunk
constexpr int kCsSlots = 3;                      // Q tile ring per half
constexpr int kCsLseRows = 4096;                 // rows of the LSE table per pass
constexpr int kMaxKeyChunks = 16;                // key chunks per block (past 8192 keys, chunks grow)

template <int D>
struct CsGeo {
  static constexpr int NC = D / 16;
  static constexpr int QRB = 2 * D;                          // bytes per Q row
  static constexpr int QBYTES = kCsRows * QRB;               // Q tile of one chunk
  static constexpr int RPI = 1024 / QRB;                     // rows per copy instruction
  static constexpr int QINST = QBYTES / 1024 / kCsWavesPerHalf;
};

// This wave's share of the copy of the scoring rows [r0, r0 + 32) into qbuf
// (rs_q covers the rows' tokens from tok0 on).  Row r is token r % ntok of
// head g * G + r / ntok (one division per chunk, then each lane steps from
// r0); rows at or past R read row 0, a real row whose probabilities the +inf
// LSE of those rows zeroes.
template <int D>
__device__ __forceinline__ void cs_issue(const AttnArgs& a, const u32x4& rs_q, int ntok, int g, int r0, int R,
                                         char* qbuf, int w4, int lane) {
  using G = CsGeo<D>;
  const int q = lane / (G::QRB / 16);
  const int slot = lane % (G::QRB / 16);
  const int i0 = r0 % ntok;
  const int a0 = r0 / ntok;
#pragma unroll
  for (int j = 0; j < G::QINST; ++j) {
    const int blk = w4 * G::QINST + j;
    const int row = blk * G::RPI + q;   // row within the chunk
    int tok = i0 + row, head = a0;
    if (ntok >= kCsRows) {              // at most one step to the next head
      const bool wrap = tok >= ntok;
      tok -= wrap ? ntok : 0;
      head += wrap ? 1 : 0;
    } else {
      while (tok >= ntok) {             // at most 32 / ntok + 1 steps
        tok -= ntok;
        ++head;
      }
    }
    if (r0 + row >= R) {
      tok = 0;
      head = 0;
    }
    const int chunk = swz<G::QRB>(row, slot);
    copy16_to_lds(rs_q, 0u, (unsigned)(((long)tok * a.q_st + (long)(g * a.G + head) * a.q_sh) * 2 + chunk * 16),
                  (unsigned)(unsigned long long)(qbuf + blk * 1024));
  }
}

template <int D, bool CTX, int KB, int HALVES>
__global__ __launch_bounds__(HALVES * kCsWavesPerHalf * 64, HALVES == 2 ? 1 : (CTX ? 2 : 3)) void colsum_kernel(AttnArgs a, int KC,
                                                               const float2* __restrict__ part,
                                                               float* __restrict__ scores,
                                                               float* __restrict__ cpart, int splits_per_head,
                                                               int split_rows) {
  using G = CsGeo<D>;
  constexpr int NC = G::NC;
  constexpr int QRB = G::QRB;
  constexpr int kThreads = HALVES * kCsWavesPerHalf * 64;
  __shared__ __attribute__((aligned(1024))) char sQ[HALVES * kCsSlots * G::QBYTES];
  __shared__ __attribute__((aligned(16))) float sLse[kCsLseRows];
  __shared__ double sAcc[HALVES == 2 ? kCsWavesPerHalf * KB * 64 : 1];   // second half's totals
  constexpr int kKeys = kCsWavesPerHalf * 32 * KB;   // keys per workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave / kCsWavesPerHalf;
  const int w4 = wave % kCsWavesPerHalf;
  const int hi = lane >> 5;
  const int col = lane & 31;
  const int hg = blockIdx.y;   // h * Hkv + g
  const int h = hg / a.Hkv;
  const int g = hg % a.Hkv;
  const ScoreRows sr = score_rows(a, h);
  const int R = sr.R;
  const int VH = a.V * a.Hkv;
  const long kstr = a.kv_st;
  const int kw0 = blockIdx.x * kKeys;   // the workgroup's first key
  const int key0 = kw0 + w4 * 32 * KB;
  // Rows [r_begin, r_end) of this workgroup's split.  Context selector: a
  // range of one head's tokens, starting no earlier than token kw0 (earlier
  // tokens see none of the workgroup's keys).
  int r_begin, r_end;
  if (CTX) {
    const int head = blockIdx.z / splits_per_head;
    const int ts = blockIdx.z % splits_per_head;
    r_begin = head * sr.ntok + max(ts * split_rows, kw0);
    r_end = head * sr.ntok + min(sr.ntok, (ts + 1) * split_rows);
  } else {
    r_begin = blockIdx.z * split_rows;
    r_end = min(R, r_begin + split_rows);
  }
  const uint16_t* kbase = (const uint16_t*)a.k + (long)(a.la + h * a.L) * kstr + (long)g * a.kv_sh;

  // This wave's 32 * KB keys as B-operand fragments (K^T: 16 channels x 32 keys).
  bf16x8 kf[KB][NC];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int j = min(key0 + 32 * kb + col, a.L - 1);
    const uint16_t* kr = kbase + (long)j * kstr + 8 * hi;
#pragma unroll
    for (int c = 0; c < NC; ++c) kf[kb][c] = *(const bf16x8*)(kr + 16 * c);
  }
  wait_vm<0>();   // as in the row statistics: no compiler wait inside the chunk loop

  // Q rows of the scoring tokens: the range ends at the last one's last head.
  const u32x4 rs_q = make_rsrc((const uint16_t*)a.q + (long)sr.tok0 * a.q_st,
                               (unsigned)(((long)(sr.ntok - 1) * a.q_st + (long)(a.Hq - 1) * a.q_sh + D) * 2));
  char* const myq = sQ + half * kCsSlots * G::QBYTES;
  const float sl2 = a.scale_log2;
  double acc[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) acc[kb] = 0.0;

  for (int rb = r_begin; rb < r_end; rb += kCsLseRows) {
    const int nrows = min(kCsLseRows, r_end - rb);
    const int nch = ceil_div(nrows, kCsRows);
    const int nj = ceil_div(nch, HALVES);   // chunks per half (the last may be empty)
    __syncthreads();                           // previous pass done with sLse
    // Q tiles of this half's first chunks (chunk c = HALVES * j + half) ...
#pragma unroll
    for (int j = 0; j < kCsSlots - 1; ++j) {
      const int c = HALVES * j + half;
      cs_issue<D>(a, rs_q, sr.ntok, g, c < nch ? rb + c * kCsRows : R, R, myq + j * G::QBYTES, w4, lane);
    }
    // ... while the row LSEs are combined from the chunk partials:
    // lse = M + log2(sum_k l_k 2^(m_k - M)) (or the query partial's LSE in
    // log2 units); rows past r_end get +inf (weight 0).
    // All of a row's partials are loaded at once (KC <= kMaxKeyChunks).
    for (int i = tid; i < nch * kCsRows; i += kThreads) {
      const int rr = rb + i;
      float lse = INFINITY;
      if (!CTX && a.score_from_partials) {
        // The query partial over block h already holds this row's
        // natural-log LSE over the block's keys (Figure 5 ordering).
        if (rr < r_end)
          lse = a.lse_part[((long)(h + 1) * a.Hq + g * a.G + rr / sr.ntok) * a.nq + rr % sr.ntok] *
                1.44269504088896340736f;
      } else if (rr < r_end) {
        float2 pk[kMaxKeyChunks];
#pragma unroll
        for (int k = 0; k < kMaxKeyChunks; ++k)
          pk[k] = (k < KC) ? part[((long)k * VH + hg) * R + rr] : make_float2(-INFINITY, 0.0f);
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < kMaxKeyChunks; ++k) M = fmaxf(M, pk[k].x);
        float lt = 0.0f;
#pragma unroll
        for (int k = 0; k < kMaxKeyChunks; ++k)
          if (pk[k].y > 0.0f) lt += pk[k].y * __builtin_amdgcn_exp2f(pk[k].x - M);
        if (lt > 0.0f) lse = M + __log2f(lt);
      }
      sLse[i] = lse;
    }
    for (int j = 0; j < nj; ++j) {
      wait_vm<G::QINST>();   // chunk j of this half has landed (this wave's part)
      __syncthreads();       // ... everyone's, and the LSE table; slot of j-1 is free
      {
        const int jn = j + kCsSlots - 1;
        const int cn = HALVES * jn + half;
        cs_issue<D>(a, rs_q, sr.ntok, g, (jn < nj && cn < nch) ? rb + cn * kCsRows : R, R,
                    myq + (jn % kCsSlots) * G::QBYTES, w4, lane);
      }
      const int c = HALVES * j + half;
      if (c >= nch) continue;
      // Context selector: the chunk's tokens t see keys j <= t only.  A
      // split lies within one head, so the chunk's tokens are t_first + m
      // (rows at or past r_end have weight 0 whatever the mask says).
      const int r_lo = rb + c * kCsRows;
      int t_first = 0;           // block-local token of the chunk's first row
      bool need_mask = false;
      if (CTX) {
        t_first = r_lo % sr.ntok;
        if (t_first + kCsRows - 1 < key0) continue;   // none of this wave's keys is visible
        need_mask = t_first < key0 + 32 * KB - 1;
      }
      const char* qt = myq + (j % kCsSlots) * G::QBYTES;
      // LSE of this lane's accumulator rows m = 8 * (i / 4) + 4 * hi + i % 4.
      f32x4 lz[4];
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) lz[gi] = *(const f32x4*)(sLse + c * kCsRows + 8 * gi + 4 * hi);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f32x16 s;
#pragma unroll
        for (int c16 = 0; c16 < NC; ++c16) {
          const bf16x8 qa = *(const bf16x8*)(qt + col * QRB + swz<QRB>(col, 2 * c16 + hi) * 16);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kb][c16], c16 == 0 ? f32x16{} : s, 0, 0, 0);
        }
        float pz = 0.0f;
        if (need_mask) {
          const int jk = key0 + 32 * kb + col;     // this lane's key
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int t = t_first + 8 * (i >> 2) + 4 * hi + (i & 3);
            const float p = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, -lz[i >> 2][i & 3]));
            pz += (jk <= t) ? p : 0.0f;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) pz += __builtin_amdgcn_exp2f(fmaf(s[i], sl2, -lz[i >> 2][i & 3]));
        }
        acc[kb] += (double)pz;
      }
    }
    wait_vm<0>();
  }

  // Column totals: the lane pair (l, l^32) holds the two row halves of a
  // key's accumulator rows; a second workgroup half's totals are added to
  // the first's in a fixed order.
  double tot[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) tot[kb] = acc[kb] + __shfl_xor(acc[kb], 32);
  if (HALVES == 2) {
    __syncthreads();
    if (half == 1) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sAcc[(w4 * KB + kb) * 64 + lane] = tot[kb];
    }
    __syncthreads();
    if (half == 0) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) tot[kb] += sAcc[(w4 * KB + kb) * 64 + lane];
    }
  }
  if (half == 0 && hi == 0) {
    float* out = gridDim.z == 1 ? scores + (long)hg * a.L : cpart + ((long)blockIdx.z * VH + hg) * a.L;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int j = key0 + 32 * kb + col;
      if (j < a.L) out[j] = (float)tot[kb];
    }
  }
}

// Scores of n = V * Hkv * L keys from the S row splits' partial sums, added
// in split order.
__global__ __launch_bounds__(256) void colsum_reduce_kernel(const float* __restrict__ cpart,
                                                            float* __restrict__ scores, int S, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  double acc = 0.0;
  for (int z = 0; z < S; ++z) acc += (double)cpart[(long)z * n + i];
  scores[i] = (float)acc;
}

// Row splits of the column sums: the query rows form one split; the context
// selector cuts each head's L tokens into at most 8 ranges of at least 1024
// tokens (a multiple of the 32-row chunk).
struct ColSplits {
  int per_head, rows, total;
};
ColSplits col_splits(const AttnArgs& a) {
  const ScoreRows sr = score_rows(a, 0);
  ColSplits c;
  if (!a.score_ctx) {
    c.per_head = 1;
    c.rows = max(sr.R, 1);
    c.total = 1;
  } else {
    c.rows = max(1024, ceil_div(ceil_div(sr.ntok, 8), kCsRows) * kCsRows);
    c.per_head = ceil_div(sr.ntok, c.rows);
    c.total = c.per_head * a.G;
  }
  return c;
}

// Key tiles per chunk of the row statistics.  Query rows: chunks of 512 keys,
// but at most kMaxKeyChunks per block (longer blocks get proportionally longer
// chunks), so that the few query rows still fill the GPU.  Context selector:
// the block's tokens give enough row tiles; one chunk holds every key, so
// each row tile's Q is read once.
int tiles_per_chunk(const AttnArgs& a) {
  const int T = ceil_div(a.L, kBN);
  if (a.score_ctx) return T;
  return max(kTilesPerChunk, ceil_div(T, kMaxKeyChunks));
}
int key_chunks(const AttnArgs& a) { return ceil_div(ceil_div(a.L, kBN), tiles_per_chunk(a)); }

size_t part_bytes(const AttnArgs& a) {
  const size_t bytes = (size_t)key_chunks(a) * a.V * a.Hkv * score_rows(a, 0).R * sizeof(float2);
  return (bytes + 255) / 256 * 256;
}

}  // namespace

template <bool CTX, int KB, int HALVES>
void launch_colsum(const AttnArgs& a, int KC, const float2* part, float* scores, float* cpart, const ColSplits& cs,
                   hipStream_t s) {
  const dim3 grid(ceil_div(a.L, kCsWavesPerHalf * 32 * KB), a.V * a.Hkv, cs.total);
  const dim3 block(HALVES * kCsWavesPerHalf * 64);
  if (a.D == 128)
    hipLaunchKernelGGL((colsum_kernel<128, CTX, KB, HALVES>), grid, block, 0, s, a, KC, part, scores, cpart,
                       cs.per_head, cs.rows);
  else
    hipLaunchKernelGGL((colsum_kernel<64, CTX, KB, HALVES>), grid, block, 0, s, a, KC, part, scores, cpart,
                       cs.per_head, cs.rows);
}

template <bool CTX>
hipError_t launch_score_bf16_mode(const AttnArgs& a, void* ws, float* scores, hipStream_t s) {
  // Scoring from the query partials passes no workspace: it reads no chunk
  // partials and its single row split writes the scores directly.
  float2* part = (float2*)ws;
  float* cpart = ws ? (float*)((char*)ws + part_bytes(a)) : nullptr;
  const int R = score_rows(a, 0).R;
  const int VH = a.V * a.Hkv;
  const int KC = key_chunks(a);
  const int TPC = tiles_per_chunk(a);
  if (R > 0 && !(a.score_from_partials && !CTX)) {
    const int RT = ceil_div(R, kRsBM);
    const int n = VH * KC * RT;
    const dim3 grid(xcd_grid(n, RT));
    if (a.D == 128)
      hipLaunchKernelGGL((rowstat_chunk_kernel<128, CTX>), grid, dim3(kRsThreads), 0, s, a, KC, TPC, RT, part);
    else
      hipLaunchKernelGGL((rowstat_chunk_kernel<64, CTX>), grid, dim3(kRsThreads), 0, s, a, KC, TPC, RT, part);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const ColSplits cs = col_splits(a);
  // The context selector's grid holds every head's token splits (thousands
  // of workgroups at 32K tokens); the query rows take single-half workgroups
  // when there are at least four per CU, else two halves.
  if constexpr (CTX) {
    launch_colsum<true, kCsKbCtx, 1>(a, KC, part, scores, cpart, cs, s);
  } else {
    if (ceil_div(a.L, kCsWavesPerHalf * 32 * kCsKbQuery) * VH * cs.total >= kCsSingleGrid)
      launch_colsum<false, kCsKbQuery, 1>(a, KC, part, scores, cpart, cs, s);
    else
      launch_colsum<false, kCsKbQuery, 2>(a, KC, part, scores, cpart, cs, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || cs.total == 1) return e;
  const long n = (long)VH * a.L;
  hipLaunchKernelGGL(colsum_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, cpart, scores,
                     cs.total, n);
  return hipGetLastError();
}

hipError_t launch_score_bf16(const AttnArgs& a, void* ws, float* scores, hipStream_t s) {
  return a.score_ctx ? launch_score_bf16_mode<true>(a, ws, scores, s)
                     : launch_score_bf16_mode<false>(a, ws, scores, s);
}

// The (max, sum) partials of every scoring row and key chunk, then (several
// row splits) the splits' column sums.
size_t score_bf16_ws_bytes(const AttnArgs& a) {
  const ColSplits cs = col_splits(a);
  return part_bytes(a) + (cs.total > 1 ? (size_t)cs.total * a.V * a.Hkv * a.L * sizeof(float) : 0);
}

}  // namespace spava
