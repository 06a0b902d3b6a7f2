// Row statistics of the block scoring for bf16 inputs on gfx950 (CDNA4):
// for every query row r = (i, a) of KV group g and every block h, the
// log2-domain log-sum-exp of its scaled logits over the block's L keys
// (Spava page, Figure 5 caption: the query rows' Q K^(h)T estimate how
// important block h's keys are; the column sums that rank them need each
// row's softmax normaliser over the block).
//
// One workgroup = 4 waves = 128 query rows (32 per wave), two workgroups per
// CU.  The block is walked in 64-key tiles that buffer_load_dwordx4 ... lds
// copies straight into double-buffered LDS (one barrier per tile), stored
// row-major and XOR-swizzled in 16-byte slots so that the 16 rows one
// ds_read_b128 phase touches fall in distinct banks.  S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 puts one query column per lane, so a row's
// statistics live in one lane pair (l, l^32).  The running maximum only
// moves when a row's maximum grows by more than 2^8 in the exp2 domain; the
// final log makes the stale reference exact.
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

// 16-byte slot of chunk c in a swizzled LDS row r of RB bytes.
template <int RB>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (RB == 256) return c ^ (r & 15);
  else return c ^ ((r >> 1) & 7);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// This wave's share of the direct-to-LDS copy of K tile t of the block
// (keys past the block's end read as zero; their logits are masked).
template <int D>
__device__ __forceinline__ void issue_tile(const uint16_t* kblk, int kstride, int len, int t,
                                           char* __restrict__ kbuf, int wave, int lane) {
  constexpr int KRB = 2 * D;
  constexpr int KINST = kBN * KRB / 1024 / 4;
  constexpr int KRPI = 1024 / KRB;
  constexpr int KCPR = KRB / 16;
  const int kb0 = t * kBN;
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(kblk + (long)kb0 * kstride, (unsigned)(len - kb0) * kstride * 2u);
#pragma unroll
  for (int j = 0; j < KINST; ++j) {
    const int blk = wave * KINST + j;
    const int row = blk * KRPI + lane / KCPR;
    const int c = swz<KRB>(row, lane % KCPR);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kbuf + blk * 1024), 16,
                                             (row * kstride + c * 8) * 2, 0, 0, 0);
  }
}

// One tile: prefetch the next one into the other buffer, then S^T = K Q^T,
// mask the block's tail, fold the tile into (m, l).
template <int D>
__device__ __forceinline__ void tile_step(const char* __restrict__ kcur, char* __restrict__ knext,
                                          bool issue, const uint16_t* kblk, int kstride, int len,
                                          int t, const bf16x8* qf, const int* koff, float& m,
                                          float& l, float sl2, int wave, int lane, int hi) {
  constexpr int NC = D / 16;
  constexpr int KRB = 2 * D;
  if (issue) issue_tile<D>(kblk, kstride, len, t + 1, knext, wave, lane);
  const int kb0 = t * kBN;
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
  if (kb0 + kBN > len) {
    const int lim = len - kb0;   // tile-local key j is in the block iff j < lim
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
  if (__any(mx > m + kGrowLog2)) {
    const float m_new = fmaxf(m, mx);
    l *= (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
  }
  const float m_use = (m == -INFINITY) ? 0.0f : m;
  float psum = 0.0f;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int e = 0; e < 16; ++e) psum += __builtin_amdgcn_exp2f(fmaf(sacc[h2][e], sl2, -m_use));
  l += psum;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void rowstat_bf16_kernel(AttnArgs a) {
  constexpr int NC = D / 16;
  constexpr int KRB = 2 * D;
  __shared__ __attribute__((aligned(1024))) char sK0[kBN * KRB];
  __shared__ __attribute__((aligned(1024))) char sK1[kBN * KRB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 5;
  const int col = lane & 31;

  const int n_units = attn_total_units(a);
  const int b = xcd_unit(blockIdx.x, a.xcd_chunk);
  if (b >= n_units) return;
  const Unit u = unit_decode(a, b);   // kStats: (host, group, row tile)
  const int r = u.tile * kBM + wave * kRowsPerWave + col;
  const RowId row = unit_row(a, u, r);

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
  const uint16_t* kblk = (const uint16_t*)a.k + ((long)(a.la + u.host * a.L) * a.Hkv + u.group) * D;
  const int kstride = a.Hkv * D;
  const int len = a.L;
  const int T = ceil_div(len, kBN);

  const int krow = perm_row(col);
  int koff[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) koff[c] = krow * KRB + swz<KRB>(krow, 2 * c + hi) * 16;

  float m = -INFINITY, l = 0.0f;
  const float sl2 = a.scale_log2;
  if (T > 0) issue_tile<D>(kblk, kstride, len, 0, sK0, wave, lane);
  for (int t = 0; t < T; t += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    tile_step<D>(sK0, sK1, t + 1 < T, kblk, kstride, len, t, qf, koff, m, l, sl2, wave, lane, hi);
    if (t + 1 >= T) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    tile_step<D>(sK1, sK0, t + 2 < T, kblk, kstride, len, t + 1, qf, koff, m, l, sl2, wave, lane, hi);
  }
  const float lt = l + __shfl_xor(l, 32);
  if (hi == 0 && row.valid) {
    const int R = a.nq * a.G;
    a.stats[((long)u.host * a.Hkv + u.group) * R + r] = (lt > 0.0f) ? m + __log2f(lt) : -INFINITY;
  }
}

}  // namespace

int rowstat_bf16_rows_per_unit() { return kBM; }

hipError_t launch_rowstat_bf16(const AttnArgs& a_in, hipStream_t s) {
  AttnArgs a = a_in;
  a.stats_only = 1;
  const int n = attn_total_units(a);
  if (n == 0) return hipSuccess;
  a.xcd_chunk = max(1, a.n_q_units / a.Hkv);
  const dim3 grid(xcd_grid(n, a.xcd_chunk));
  if (a.D == 128)
    hipLaunchKernelGGL((rowstat_bf16_kernel<128>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((rowstat_bf16_kernel<64>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace spava
