// Block scoring and top-lp selection.
//
// Scoring (Figure 5 caption of the Spava page: the query block's logits
// against block h rank that block's keys; "What carries the argument" in the APB-V review: keys ranked by
// query-to-context attention scores).  For block h and KV head g the score of
// key j is the sum over the query block's rows r = (token i, head a in g) of
// softmax_j(q_r . k_j * scale) over the block's L keys.  It takes two passes
// over the block: the row log-sum-exp, then the column sums.  This file holds
// the float32 path (vector ALUs) and the top-lp selection; bf16 inputs use the
// MFMA kernels of score_bf16.hip.  Probabilities are float32, column sums
// accumulate in float64 in a fixed order, so the result is deterministic and
// its relative error stays far below 1e-6.
//
// With AttnArgs::score_ctx set the rows are block h's own tokens instead (the
// context-driven selector of the APB-V review's Referee Report, major comment
// 1), each attending causally over the block's keys: key j counts for token t
// iff j <= t.
//
// Selection (ArgTop_lp in the APB-V review's axiom ledger): an exact radix
// select on the order-preserving integer image of the float32 scores finds
// the lp-th largest value; ties at that value go to the lower indices; the
// kept indices are written in ascending order by a block-wide prefix sum.
#include "spava_common.h"

namespace spava {
namespace {

// float32 inputs: row statistics and column sums on the vector ALUs.
template <int D>
__global__ __launch_bounds__(256) void rowstat_f32_kernel(AttnArgs a) {
  const int R = score_rows(a, 0).R;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)a.V * a.Hkv * R) return;
  const int r = (int)(gid % R);
  const int hg = (int)(gid / R);
  const int h = hg / a.Hkv, g = hg % a.Hkv;
  const ScoreRows sr = score_rows(a, h);
  const int tok = sr.tok0 + r % sr.ntok;
  const int head = g * a.G + r / sr.ntok;
  const int nkeys = a.score_ctx ? r % sr.ntok + 1 : a.L;   // keys [0, nkeys) are visible
  const float* q = (const float*)a.q + (long)tok * a.q_st + (long)head * a.q_sh;
  float qv[D];
#pragma unroll
  for (int c = 0; c < D; ++c) qv[c] = q[c];
  const long kstr = a.kv_st;
  const float* kb = (const float*)a.k + (long)(a.la + h * a.L) * kstr + (long)g * a.kv_sh;
  float m = -INFINITY, l = 0.0f;
  for (int j = 0; j < nkeys; ++j) {
    const float* kr = kb + (long)j * kstr;
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < D; ++c) s = fmaf(qv[c], kr[c], s);
    const float x = s * a.scale_log2;
    const float mn = fmaxf(m, x);
    l = l * __builtin_amdgcn_exp2f(m - mn) + __builtin_amdgcn_exp2f(x - mn);
    m = mn;
  }
  a.stats[gid] = m + __log2f(l);
}

template <int D>
__global__ __launch_bounds__(256) void colsum_f32_kernel(AttnArgs a, float* __restrict__ scores) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)a.V * a.Hkv * a.L) return;
  const int j = (int)(gid % a.L);
  const int hg = (int)(gid / a.L);
  const int h = hg / a.Hkv, g = hg % a.Hkv;
  const ScoreRows sr = score_rows(a, h);
  const int R = sr.R;
  const float* kr = (const float*)a.k + (long)(a.la + h * a.L + j) * a.kv_st + (long)g * a.kv_sh;
  float kv[D];
#pragma unroll
  for (int c = 0; c < D; ++c) kv[c] = kr[c];
  const float* lse2 = a.stats + (long)hg * R;
  // Query rows after the attention's first phase: the query partial over
  // block h holds each row's natural-log LSE over the block's keys.
  const bool from_part = a.score_from_partials && !a.score_ctx;
  const float* lse_nat = a.lse_part + (long)(h + 1) * a.Hq * a.nq;
  double acc = 0.0;
  for (int r = 0; r < R; ++r) {
    if (a.score_ctx && r % sr.ntok < j) continue;   // token r % L does not see key j
    const int tok = sr.tok0 + r % sr.ntok;
    const int head = g * a.G + r / sr.ntok;
    const float* q = (const float*)a.q + (long)tok * a.q_st + (long)head * a.q_sh;
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < D; ++c) s = fmaf(q[c], kv[c], s);
    const float l2 = from_part ? lse_nat[(long)head * a.nq + r % a.nq] * 1.44269504088896340736f : lse2[r];
    acc += (double)__builtin_amdgcn_exp2f(s * a.scale_log2 - l2);
  }
  scores[gid] = (float)acc;
}

__global__ void fill_zero_kernel(float* p, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// ---------------------------------------------------------------------------
// Exact top-lp selection, one workgroup per (block, KV head) list.
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Each thread owns the contiguous keys [j0, j1) of the list, so the kept
// indices come out in index order.  With NPT > 0 (lists of at most
// NPT * kTopkThreads keys) the thread reads its keys from memory once and
// every pass below works on registers; NPT = 0 reads them again per pass.
//
// Radix select of the lp-th largest order key.  All keys lie between the
// list's smallest and largest key, so they share those two keys' common
// leading bits: the passes start below them, 8 bits at a time.  After each
// pass's histogram every wave reads all 256 bins and finds the digit itself,
// so a pass costs one barrier.  The emit takes one scan of two counts per
// thread (keys above the threshold, keys equal to it): the equal keys kept
// are the take_eq lowest-indexed ones, so a thread's first output position
// is (keys above, before it) + min(equal keys before it, take_eq).
template <int NPT>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores,
                                                            int32_t* __restrict__ idx, int L, int lp) {
  constexpr int kWaves = kTopkThreads / 64;
  constexpr int kPasses = 4;                 // 32 bits, 8 per pass
  __shared__ int sHist[kPasses * 256];
  __shared__ uint32_t sLo[kWaves], sHi[kWaves];
  __shared__ int sGt[kWaves], sEq[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const float* sc = scores + (long)blockIdx.x * L;
  int32_t* out = idx + (long)blockIdx.x * lp;

  const int chunk = (L + kTopkThreads - 1) / kTopkThreads;
  const int j0 = min(L, tid * chunk), j1 = min(L, j0 + chunk);
  const int n = j1 - j0;
  constexpr int NR = NPT > 0 ? NPT : 1;
  uint32_t cache[NR];
  if (NPT > 0) {
#pragma unroll
    for (int e = 0; e < NR; ++e) {
      const uint32_t u = order_key(sc[min(j0 + e, L - 1)]);   // in the list even past its end
      cache[e] = (e < n) ? u : 0u;
    }
  }
  auto key = [&](int e) -> uint32_t { return NPT > 0 ? cache[e] : order_key(sc[j0 + e]); };
  const int n_loop = NPT > 0 ? NPT : n;

  for (int i = tid; i < kPasses * 256; i += kTopkThreads) sHist[i] = 0;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int e = 0; e < n_loop; ++e) {
    if (e >= n) break;
    const uint32_t u = key(e);
    lo = min(lo, u);
    hi = max(hi, u);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
  }
  if (lane == 0) {
    sLo[wave] = lo;
    sHi[wave] = hi;
  }
  __syncthreads();
  lo = sLo[0];
  hi = sHi[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    lo = min(lo, sLo[w]);
    hi = max(hi, sHi[w]);
  }
  // Bits at and above 'top' are decided: prefix holds them, pmask marks them.
  int top = (lo == hi) ? 0 : 32 - __clz(lo ^ hi);
  uint32_t pmask = top >= 32 ? 0u : ~((1u << top) - 1u);
  uint32_t prefix = lo & pmask;
  int need = lp;   // rank still to find among the keys that match prefix
  for (int pass = 0; top > 0; ++pass) {
    const int w = min(8, top);
    const int shift = top - w;
    const uint32_t dm = (1u << w) - 1u;
    int* h = sHist + pass * 256;
#pragma unroll
    for (int e = 0; e < n_loop; ++e) {
      if (e >= n) break;
      const uint32_t u = key(e);
      if ((u & pmask) == prefix) atomicAdd(&h[(u >> shift) & dm], 1);
    }
    __syncthreads();
    // Lane l holds bins 255-4l .. 252-4l (lane 0 the highest digits).
    int c[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = h[255 - 4 * lane - i];
      sum += c[i];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int above = incl - sum;   // keys in higher digits than this lane's bins
    const bool mine = above < need && need <= incl;
    int dsel = 0, nsel = 0;
    if (mine) {
      int a = above;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (a < need && need <= a + c[i]) {
          dsel = 255 - 4 * lane - i;
          nsel = need - a;
        }
        a += c[i];
      }
    }
    const unsigned long long bal = __ballot(mine);
    const int src = bal ? __ffsll((long long)bal) - 1 : 0;
    dsel = __shfl(dsel, src);
    nsel = __shfl(nsel, src);
    prefix |= ((uint32_t)dsel & dm) << shift;
    pmask |= dm << shift;
    need = nsel;
    top = shift;
  }
  const uint32_t thr = prefix;  // order key of the lp-th largest score
  const int take_eq = need;     // keys equal to thr that are kept (lowest indices)

  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < n_loop; ++e) {
    if (e >= n) break;
    const uint32_t u = key(e);
    n_gt += (u > thr);
    n_eq += (u == thr);
  }
  int ig = n_gt, ie = n_eq;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int yg = __shfl_up(ig, o);
    const int ye = __shfl_up(ie, o);
    if (lane >= o) {
      ig += yg;
      ie += ye;
    }
  }
  if (lane == 63) {
    sGt[wave] = ig;
    sEq[wave] = ie;
  }
  __syncthreads();
  int og = 0, oe = 0;
  for (int w = 0; w < wave; ++w) {
    og += sGt[w];
    oe += sEq[w];
  }
  const int eq_before = oe + ie - n_eq;
  int pos = og + ig - n_gt + min(eq_before, take_eq);
  int q = eq_before;
#pragma unroll
  for (int e = 0; e < n_loop; ++e) {
    if (e >= n) break;
    const uint32_t u = key(e);
    bool keep = false;
    if (u > thr) keep = true;
    else if (u == thr) { keep = q < take_eq; ++q; }
    if (keep && pos < lp) out[pos++] = j0 + e;
  }
}

// ---------------------------------------------------------------------------
// Overlap of two selections ("What would settle it" in the APB-V review: how
// many of the keys kept by the query-driven rule the context-driven rule also
// keeps).  One workgroup per list pair; every entry of list a is looked up in
// list b by binary search.  Both lists must be strictly ascending (as the
// top-lp selection writes them); a pair where either is not gets -1.
// ---------------------------------------------------------------------------
constexpr int kOverlapThreads = 256;

__global__ __launch_bounds__(kOverlapThreads) void overlap_kernel(const int32_t* __restrict__ idx_a,
                                                                  const int32_t* __restrict__ idx_b,
                                                                  int32_t* __restrict__ counts, int lp) {
  __shared__ int sCount[kOverlapThreads / 64];
  __shared__ int sBad[kOverlapThreads / 64];
  const int tid = threadIdx.x;
  const int32_t* A = idx_a + (long)blockIdx.x * lp;
  const int32_t* B = idx_b + (long)blockIdx.x * lp;
  int n = 0, bad = 0;
  for (int i = tid; i < lp; i += kOverlapThreads) {
    if (i + 1 < lp) bad |= (A[i] >= A[i + 1]) | (B[i] >= B[i + 1]);
    const int x = A[i];
    int lo = 0, hi = lp;               // first position in B whose value is >= x
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (B[mid] < x) lo = mid + 1;
      else hi = mid;
    }
    n += (lo < lp && B[lo] == x);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    n += __shfl_xor(n, o);
    bad |= __shfl_xor(bad, o);
  }
  if ((tid & 63) == 0) {
    sCount[tid >> 6] = n;
    sBad[tid >> 6] = bad;
  }
  __syncthreads();
  if (tid == 0) {
    int tot = 0, any_bad = 0;
    for (int w = 0; w < kOverlapThreads / 64; ++w) {
      tot += sCount[w];
      any_bad |= sBad[w];
    }
    counts[blockIdx.x] = any_bad ? -1 : tot;
  }
}

}  // namespace

hipError_t launch_overlap(const int32_t* idx_a, const int32_t* idx_b, int32_t* counts, int n_lists, int lp,
                          hipStream_t s) {
  if (n_lists == 0) return hipSuccess;
  hipLaunchKernelGGL(overlap_kernel, dim3(n_lists), dim3(kOverlapThreads), 0, s, idx_a, idx_b, counts, lp);
  return hipGetLastError();
}

hipError_t launch_rowstat_f32(const AttnArgs& a, hipStream_t s) {
  const long nr = (long)a.V * a.Hkv * score_rows(a, 0).R;
  if (nr == 0) return hipSuccess;
  const dim3 grid((unsigned)((nr + 255) / 256));
  if (a.D == 128)
    hipLaunchKernelGGL((rowstat_f32_kernel<128>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((rowstat_f32_kernel<64>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// Column sums; a.stats must already hold the row statistics.  With no
// scoring rows (an empty query block) every score is 0 (a sum over no rows).
hipError_t launch_colsum_f32(const AttnArgs& a, float* scores, hipStream_t s) {
  const long n = (long)a.V * a.Hkv * a.L;
  if (n == 0) return hipSuccess;
  if (score_rows(a, 0).R == 0) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, scores, n);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((n + 255) / 256));
  if (a.D == 128)
    hipLaunchKernelGGL((colsum_f32_kernel<128>), grid, dim3(256), 0, s, a, scores);
  else
    hipLaunchKernelGGL((colsum_f32_kernel<64>), grid, dim3(256), 0, s, a, scores);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int32_t* idx, int n_lists, int L, int lp, hipStream_t s) {
  if (n_lists == 0 || lp == 0) return hipSuccess;
  const int chunk = (L + kTopkThreads - 1) / kTopkThreads;
  if (chunk <= 4)
    hipLaunchKernelGGL(topk_kernel<4>, dim3(n_lists), dim3(kTopkThreads), 0, s, scores, idx, L, lp);
  else if (chunk <= 8)
    hipLaunchKernelGGL(topk_kernel<8>, dim3(n_lists), dim3(kTopkThreads), 0, s, scores, idx, L, lp);
  else if (chunk <= 16)
    hipLaunchKernelGGL(topk_kernel<16>, dim3(n_lists), dim3(kTopkThreads), 0, s, scores, idx, L, lp);
  else
    hipLaunchKernelGGL(topk_kernel<0>, dim3(n_lists), dim3(kTopkThreads), 0, s, scores, idx, L, lp);
  return hipGetLastError();
}

}  // namespace spava
