// Fused approximate-attention forward for bf16 inputs on gfx950 (CDNA4).
//
// One workgroup = 4 waves = one unit of 128 query rows (32 per wave); two
// workgroups share a CU (<= 256 registers per lane), so one workgroup's
// softmax overlaps the other's matrix work.  The unit's key segments
// (anchor / passing blocks / own block / query block, see unit_segments) are
// walked in 64-key tiles that global_load_lds_dwordx4 copies straight into
// double-buffered LDS (one barrier per tile):
//   K tile   [64 keys][D]   row-major, read as the MFMA A operand
//   V^T tile [D][64 keys]   key-contiguous, read as the MFMA A operand
// LDS rows are XOR-swizzled in 16-byte slots so that the 16 rows one
// ds_read_b128 phase touches fall in distinct banks.
//
// Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so every lane
// owns one query column: the softmax row statistics live in one lane pair
// (l, l^32) and rescaling O^T is lane-uniform.  P^T leaves the accumulator
// registers directly as the B operand of O^T += V^T P^T: the A-operand rows
// of the K tile are read in a permuted order (bits 2 and 3 of the row index
// swapped), which makes the S^T accumulator layout equal to the B-operand
// layout with keys in natural order.
//
// The running maximum is only moved (and O^T rescaled) when a row's maximum
// grows by more than 2^8 in the exp2 domain; otherwise probabilities are
// taken against the stale maximum (at most 256, exact in the final
// normalisation since O and the row sum share the same reference).
//
// STATS = true: no V and no PV; each row's log2-domain log-sum-exp over the
// block is written for the block scoring (Figure 5 caption of the Spava
// page: Q_qr K^(h)T estimates KV importance).
#include "spava_common.h"

namespace spava {
namespace {

constexpr int kBM = 128;   // rows per workgroup
constexpr int kBN = kKeyTile;
constexpr int kThreads = 256;
constexpr float kGrowLog2 = 8.0f;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int perm_row(int m) {  // swap bits 2 and 3
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ int wave_reduce_min(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_reduce_max(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// 16-byte slot of chunk c in a swizzled LDS row r of RB bytes.
template <int RB>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (RB == 256) return c ^ (r & 15);
  else return c ^ ((r >> 1) & 7);
}

template <int D>
struct Geo {
  static constexpr int KRB = D * 2;                  // bytes per K row
  static constexpr int KBYTES = kBN * KRB;           // K tile
  static constexpr int VBYTES = D * kBN * 2;         // V^T tile (rows of 64 keys = 128 B)
  static constexpr int KINST = KBYTES / 1024 / 4;    // K load instructions per wave
  static constexpr int VINST = VBYTES / 1024 / 4;
};

// The unit's key segments as scalar fields (selected by value, never by a
// dynamic index, so that they stay in scalar registers).
struct SegRun {
  const uint16_t* k;   // key 0 of the segment (K or passing K rows)
  const uint16_t* vt;  // key 0 in the V^T row of channel 0
  int kstride;         // elements between consecutive keys
  int vrow;            // elements between consecutive V^T channel rows
  int len;             // keys
  int causal;          // 1: key token tok0 + j must be <= the query token
  int tok0;
  int nt;              // 64-key tiles this unit visits
};

__device__ __forceinline__ SegRun empty_run() {
  SegRun r;
  r.k = nullptr;
  r.vt = nullptr;
  r.kstride = 0;
  r.vrow = 0;
  r.len = 0;
  r.causal = 0;
  r.tok0 = 0;
  r.nt = 0;
  return r;
}

// A run of consecutive tokens of K/V head g: tokens [tok0, tok0+len), whose
// V^T copy starts at key offset vkey of the main V^T row.
__device__ __forceinline__ SegRun main_run(const AttnArgs& a, int g, int tok0, int len, int vkey,
                                           int causal) {
  SegRun r;
  r.k = (const uint16_t*)a.k + ((long)tok0 * a.Hkv + g) * a.D;
  r.vt = a.vt + (long)g * a.D * a.vl.main_len + vkey;
  r.kstride = a.Hkv * a.D;
  r.vrow = a.vl.main_len;
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
//   query partial h+1 / statistics over block h: [block h]
__device__ __forceinline__ void unit_runs(const AttnArgs& a, const Unit& u, SegRun* r) {
  const int g = u.group;
  r[0] = empty_run();
  r[1] = empty_run();
  r[2] = empty_run();
  switch (u.kind) {
    case kAnchor:
      r[0] = main_run(a, g, 0, a.la, 0, 1);
      break;
    case kContext:
      r[0] = main_run(a, g, 0, a.la, 0, 0);
      if (u.host > 0 && a.lp > 0) {
        r[1].k = (const uint16_t*)a.kp + (long)g * a.V * a.lp * a.D;
        r[1].vt = a.vpt + (long)g * a.D * a.vl.pass_len;
        r[1].kstride = a.D;
        r[1].vrow = a.vl.pass_len;
        r[1].len = u.host * a.lp;
      }
      r[2] = main_run(a, g, a.la + u.host * a.L, a.L, a.vl.off_block0 + u.host * a.vl.pad_block, 1);
      break;
    case kQueryHead:
      r[0] = main_run(a, g, 0, a.la, 0, 0);
      r[1] = main_run(a, g, a.la + a.V * a.L, a.nq, a.vl.off_query, 1);
      break;
    default:  // kQueryBlock, kStats
      r[0] = main_run(a, g, a.la + u.host * a.L, a.L, a.vl.off_block0 + u.host * a.vl.pad_block, 0);
      break;
  }
}

__device__ __forceinline__ SegRun sel(const SegRun& a0, const SegRun& a1, const SegRun& a2, int i) {
  SegRun r;
  r.k = i == 0 ? a0.k : (i == 1 ? a1.k : a2.k);
  r.vt = i == 0 ? a0.vt : (i == 1 ? a1.vt : a2.vt);
  r.kstride = i == 0 ? a0.kstride : (i == 1 ? a1.kstride : a2.kstride);
  r.vrow = i == 0 ? a0.vrow : (i == 1 ? a1.vrow : a2.vrow);
  r.len = i == 0 ? a0.len : (i == 1 ? a1.len : a2.len);
  r.causal = i == 0 ? a0.causal : (i == 1 ? a1.causal : a2.causal);
  r.tok0 = i == 0 ? a0.tok0 : (i == 1 ? a1.tok0 : a2.tok0);
  r.nt = i == 0 ? a0.nt : (i == 1 ? a1.nt : a2.nt);
  return r;
}

// Raw buffer descriptor (gfx9 family: word 3 = 0x00020000) over `bytes`
// bytes from `base`; loads at offsets past the range return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Issue this wave's share of the direct-to-LDS loads of tile t of run sr.
// The K descriptor starts at the tile and ends at the segment's last key,
// so rows past the segment read as zero (their logits are masked).
template <int D, bool STATS>
__device__ __forceinline__ void issue_tile(const SegRun& sr, int t, char* __restrict__ kbuf,
                                           char* __restrict__ vbuf, int wave, int lane) {
  using G = Geo<D>;
  constexpr int KRB = G::KRB;
  constexpr int KRPI = 1024 / KRB;   // K rows per load instruction
  constexpr int KCPR = KRB / 16;     // 16-byte chunks per K row
  const int kb0 = t * kBN;
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(sr.k + (long)kb0 * sr.kstride, (unsigned)(sr.len - kb0) * sr.kstride * 2u);
#pragma unroll
  for (int j = 0; j < G::KINST; ++j) {
    const int blk = wave * G::KINST + j;
    const int row = blk * KRPI + lane / KCPR;
    const int c = swz<KRB>(row, lane % KCPR);      // involution: slot <-> chunk
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kbuf + blk * 1024), 16,
                                             (row * sr.kstride + c * 8) * 2, 0, 0, 0);
  }
  if (!STATS) {
    const __amdgpu_buffer_rsrc_t vrs =
        make_rsrc(sr.vt + kb0, (unsigned)((D - 1) * sr.vrow + kBN) * 2u);
#pragma unroll
    for (int j = 0; j < G::VINST; ++j) {
      const int blk = wave * G::VINST + j;
      const int row = blk * 8 + lane / 8;
      const int c = swz<128>(row, lane % 8);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(vbuf + blk * 1024), 16,
                                               (row * sr.vrow + c * 8) * 2, 0, 0, 0);
    }
  }
}

template <int D>
struct RowState {
  f32x16 o[D / 32];
  float m;   // running max, exp2 domain (scaled logits)
  float l;   // this lane's partial row sum (its 16 keys of every 32)
};

// One key tile: prefetch the next tile into the other buffers, then
// S^T = K Q^T, mask, online softmax, O^T += V^T P^T from the current ones.
// The buffers are distinct restrict pointers so that reads of the current
// tile need not wait for the in-flight copies of the next one.
template <int D, bool STATS>
__device__ __forceinline__ void tile_step(
    const char* __restrict__ kcur, const char* __restrict__ vcur, char* __restrict__ knext,
    char* __restrict__ vnext, bool issue, const SegRun& nrun, int nt, const SegRun& cur, int ct,
    const bf16x8* qf, const int* koff, const int* voff, RowState<D>& st, float sl2, int row_tok,
    int wmin, int wmax, int wave, int lane, int hi) {
  constexpr int NC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int KRB = Geo<D>::KRB;
  if (issue) issue_tile<D, STATS>(nrun, nt, knext, vnext, wave, lane);
  const int kb0 = ct * kBN;
  if (cur.causal && cur.tok0 + kb0 > wmax) return;   // every key is in this wave's future

  f32x16 sacc[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[h2][e] = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8 af = *(const bf16x8*)(kcur + koff[c] + h2 * 32 * KRB);
      sacc[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[c], sacc[h2], 0, 0, 0);
    }
  }
  const bool need_mask = (kb0 + kBN > cur.len) || (cur.causal && cur.tok0 + kb0 + kBN - 1 > wmin);
  if (need_mask) {
    // Tile-local key j is visible iff j < lim.
    int lim = cur.len - kb0;
    if (cur.causal) lim = min(lim, row_tok - cur.tok0 - kb0 + 1);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = 32 * h2 + (e & 7) + 8 * hi + 16 * (e >> 3);
        if (j >= lim) sacc[h2][e] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[h2][e]);
  mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
  const bool grow = mx > st.m + kGrowLog2;
  if (__any(grow)) {
    const float m_new = fmaxf(st.m, mx);
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);   // m = -inf -> 0
    st.m = m_new;
    st.l *= alpha;
    if (!STATS) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) st.o[db][e] *= alpha;
    }
  }
  const float m_use = (st.m == -INFINITY) ? 0.0f : st.m;
  float psum = 0.0f;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[h2][e], sl2, -m_use));
      sacc[h2][e] = p;
      psum += p;
    }
  st.l += psum;   // float32 row sums: the LSE output needs them to ~1e-6
  if (STATS) return;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    const int h2 = kc >> 1;
    const int base = 8 * (kc & 1);
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sacc[h2][base + e];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16x8 vf = *(const bf16x8*)(vcur + voff[kc] + db * 32 * 128);
      st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, st.o[db], 0, 0, 0);
    }
  }
}

template <int D, bool STATS>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(AttnArgs a) {
  using G = Geo<D>;
  constexpr int NC = D / 16;   // 16-wide d chunks (MFMA K steps of S)
  constexpr int NDB = D / 32;  // 32-row d blocks of O^T
  constexpr int KRB = G::KRB;
  __shared__ __attribute__((aligned(1024))) char sK0[G::KBYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[G::KBYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[STATS ? 16 : G::VBYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[STATS ? 16 : G::VBYTES];
  __shared__ int sTok[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 5;
  const int col = lane & 31;

  const int n_units = attn_total_units(a);
  const int b = xcd_unit(blockIdx.x, a.xcd_chunk);
  if (b >= n_units) return;
  const Unit u = unit_decode(a, b);
  SegRun run[3];
  unit_runs(a, u, run);

  const int r = u.tile * kBM + wave * kRowsPerWave + col;
  const RowId row = unit_row(a, u, r);

  // Q^T fragments (B operand): lane holds its query's d = 16c + 8*hi .. +7.
  bf16x8 qf[NC];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((long)row.tok * a.Hq + row.head) * D + 8 * hi;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[c] = *(const bf16x8*)(qp + 16 * c);
      if (!row.valid) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[c][e] = (__bf16)0.0f;
      }
    }
  }

  // Token range of this wave (masking, skipping) and of the workgroup (tile count).
  const int wmin = wave_reduce_min(row.valid ? row.tok : 0x7fffffff);
  const int wmax = wave_reduce_max(row.valid ? row.tok : -1);
  if (lane == 0) sTok[wave] = wmax;
  __syncthreads();
  const int gmax = max(max(sTok[0], sTok[1]), max(sTok[2], sTok[3]));

#pragma unroll
  for (int s = 0; s < 3; ++s) {
    int n = run[s].len;
    if (run[s].causal) n = min(n, gmax - run[s].tok0 + 1);
    run[s].nt = n > 0 ? ceil_div(n, kBN) : 0;
  }
  const int T = run[0].nt + run[1].nt + run[2].nt;

  // Per-lane LDS byte offsets of the A-operand fragments.
  const int krow = perm_row(col);                 // + 32 per 32-key half
  int koff[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) koff[c] = krow * KRB + swz<KRB>(krow, 2 * c + hi) * 16;
  int voff[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) voff[kc] = col * 128 + swz<128>(col, 2 * kc + hi) * 16;

  RowState<D> st;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[db][e] = 0.0f;
  st.m = -INFINITY;
  st.l = 0.0f;
  const float sl2 = a.scale_log2;

  // Tile i -> (run, tile): runs are visited in order, skipping empty ones.
  auto locate = [&](int i, int& s, int& t) {
    const int n0 = run[0].nt, n1 = run[1].nt;
    s = (i >= n0) + (i >= n0 + n1);
    t = i - (s >= 1 ? n0 : 0) - (s >= 2 ? n1 : 0);
  };
  if (T > 0) {
    int s0, t0;
    locate(0, s0, t0);
    issue_tile<D, STATS>(sel(run[0], run[1], run[2], s0), t0, sK0, sV0, wave, lane);
  }
  for (int i = 0; i < T; i += 2) {
    int s, t, sn, tn;
    locate(i, s, t);
    locate(i + 1, sn, tn);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    tile_step<D, STATS>(sK0, sV0, sK1, sV1, i + 1 < T, sel(run[0], run[1], run[2], sn), tn,
                        sel(run[0], run[1], run[2], s), t, qf, koff, voff, st, sl2, row.tok, wmin,
                        wmax, wave, lane, hi);
    if (i + 1 >= T) break;
    int s2, t2;
    locate(i + 2, s2, t2);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    tile_step<D, STATS>(sK1, sV1, sK0, sV0, i + 2 < T, sel(run[0], run[1], run[2], s2), t2,
                        sel(run[0], run[1], run[2], sn), tn, qf, koff, voff, st, sl2, row.tok,
                        wmin, wmax, wave, lane, hi);
  }

  // Epilogue.
  const float lt = st.l + __shfl_xor(st.l, 32);
  const float lse2 = (lt > 0.0f) ? st.m + __log2f(lt) : -INFINITY;
  if (STATS) {
    if (hi == 0 && row.valid) {
      const int R = a.nq * a.G;
      a.stats[((long)u.host * a.Hkv + u.group) * R + r] = lse2;
    }
    return;
  }
  if (!row.valid) return;
  const float inv = (lt > 0.0f) ? 1.0f / lt : 0.0f;
  const float lse_nat = lse2 * 0.69314718055994530942f;
  if (u.kind == kAnchor || u.kind == kContext) {
    uint16_t* op = (uint16_t*)a.o + ((long)row.tok * a.Hq + row.head) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hi;
        union { __bf16 h[4]; uint2 u; } pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk.h[e] = (__bf16)(st.o[db][4 * g4 + e] * inv);
        *(uint2*)(op + d0) = pk.u;
      }
    if (hi == 0) a.lse[(long)row.head * a.N + row.tok] = lse_nat;
  } else {
    const int p = (u.kind == kQueryHead) ? 0 : u.host + 1;
    const int i = row.tok - (a.la + a.V * a.L);
    float* op = a.o_part + (((long)p * a.nq + i) * a.Hq + row.head) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hi;
        float4 w;
        w.x = st.o[db][4 * g4 + 0] * inv;
        w.y = st.o[db][4 * g4 + 1] * inv;
        w.z = st.o[db][4 * g4 + 2] * inv;
        w.w = st.o[db][4 * g4 + 3] * inv;
        *(float4*)(op + d0) = w;
      }
    if (hi == 0) a.lse_part[((long)p * a.Hq + row.head) * a.nq + i] = lse_nat;
  }
}

}  // namespace

int attn_bf16_rows_per_unit() { return kBM; }

hipError_t launch_attn_bf16(const AttnArgs& a_in, hipStream_t s) {
  AttnArgs a = a_in;
  const int n = attn_total_units(a);
  if (n == 0) return hipSuccess;
  a.xcd_chunk = a.stats_only ? max(1, a.n_q_units / a.Hkv) : a.Hq;
  const dim3 grid(xcd_grid(n, a.xcd_chunk));
  if (a.D == 128) {
    if (a.stats_only)
      hipLaunchKernelGGL((attn_bf16_kernel<128, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<128, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (a.stats_only)
      hipLaunchKernelGGL((attn_bf16_kernel<64, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<64, false>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace spava
