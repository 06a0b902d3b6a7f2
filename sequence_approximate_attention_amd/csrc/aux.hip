// Data-movement kernels: passing-block gather and LSE merge.
#include "spava_common.h"

namespace spava {
namespace {

// ---------------------------------------------------------------------------
// Passing blocks (Figure 2 caption of the Spava page: each context block is
// compressed to its selected KVs, then passed on).
//   kp[g][h][t] = k[la + h*L + idx[h][g][t]][g],  same for v.
// One thread moves one 16-byte chunk; consecutive threads cover one row, so
// both the gathered reads and the writes are coalesced per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t* __restrict__ k,
                                                     const uint8_t* __restrict__ v,
                                                     const int32_t* __restrict__ idx,
                                                     uint8_t* __restrict__ kp,
                                                     uint8_t* __restrict__ vp, int la, int V,
                                                     int L, int Hkv, int lp, int row_bytes,
                                                     long kv_st_bytes, long kv_sh_bytes, long total_chunks) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total_chunks) return;
  const int cpr = row_bytes / 16;
  const long half = total_chunks / 2;
  const int which = gid >= half;          // 0: K, 1: V
  const long cidx = which ? gid - half : gid;
  const int c = (int)(cidx % cpr);
  const long ri = cidx / cpr;             // (g, h, t) row of kp/vp
  const int t = (int)(ri % lp);
  const int h = (int)((ri / lp) % V);
  const int g = (int)(ri / ((long)lp * V));
  int j = idx[((long)h * Hkv + g) * lp + t];
  j = min(max(j, 0), L - 1);
  const long tok = (long)la + (long)h * L + j;
  const uint8_t* src = (which ? v : k) + tok * kv_st_bytes + g * kv_sh_bytes + c * 16;
  uint8_t* dst = (which ? vp : kp) + ri * row_bytes + c * 16;
  *(uint4*)dst = *(const uint4*)src;
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of partial attention results (axiom on Eq. 5 / Appendix A
// in the APB-V review: merging through the FlashAttention lse is exact).
// One thread per (row, head, 4 channels); it walks the partials in order and
// merges them online: the running maximum m, the weight sum and the weighted
// O are rescaled when a partial raises m, so each weight is exp(lse - m) with
// m the maximum so far.  The sums run in partial order, so the result is
// deterministic.
//
// A ring of PF slots keeps PF partials' loads in flight: each slot is
// refilled with partial p + PF right after partial p is merged.  The partials
// of one (row, head) lie n_rows*n_heads*d*4 bytes apart (7 MiB at the 256K
// frame shape), so every partial in flight is another far-apart region per
// wave.  A shallow ring (PF = 2) keeps the chip's reads in few DRAM regions
// at a time, and reads faster than issuing a dozen partials at once (67 %
// against 59 % of HBM bandwidth at 33 partials).  Grids of fewer than two
// workgroups per CU take a deeper ring (PF = 8) so that enough bytes are in
// flight.
// ---------------------------------------------------------------------------
template <int PF>
__global__ __launch_bounds__(256) void merge_kernel(int P, int R, int H, int D,
                                                    const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part,
                                                    void* __restrict__ o, long o_row_stride,
                                                    float* __restrict__ lse, long lse_head_stride,
                                                    int out_bf16) {
  const int cq = D / 4;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long total = (long)R * H * cq;
  if (gid >= total) return;
  const int c4 = (int)(gid % cq);
  const long ra = gid / cq;               // r * H + a
  const int a = (int)(ra % H);
  const int r = (int)(ra / H);
  const float* lp_ra = lse_part + (long)a * R + r;   // + p * H * R
  const float* op_ra = o_part + ra * D + c4 * 4;     // + p * R * H * D
  const long lp_step = (long)H * R, op_step = (long)R * H * D;
  float lb[PF];
  float4 xb[PF];
#pragma unroll
  for (int q = 0; q < PF; ++q) {
    if (q < P) {
      lb[q] = lp_ra[q * lp_step];
      xb[q] = *(const float4*)(op_ra + q * op_step);
    }
  }
  float m = -INFINITY, wsum = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = 0; p0 < P; p0 += PF) {
#pragma unroll
    for (int sl = 0; sl < PF; ++sl) {
      const int p = p0 + sl;
      if (p >= P) break;
      const float l = lb[sl];
      const float4 x = xb[sl];
      // A partial with lse = -inf has weight 0 and its O is not read into
      // the sums; while m is -inf (no finite partial yet) the sums are 0.
      const bool up = l > m;
      const float m_new = up ? l : m;
      const float sc = up ? expf(m - l) : 1.0f;   // exp(-inf) = 0 for the first finite partial
      const float w = (l == -INFINITY) ? 0.0f : expf(l - m_new);
      acc.x = acc.x * sc + w * x.x;
      acc.y = acc.y * sc + w * x.y;
      acc.z = acc.z * sc + w * x.z;
      acc.w = acc.w * sc + w * x.w;
      wsum = wsum * sc + w;
      m = m_new;
      const int pn = p + PF;
      if (pn < P) {                       // refill the slot just merged
        lb[sl] = lp_ra[pn * lp_step];
        xb[sl] = *(const float4*)(op_ra + pn * op_step);
      }
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  acc.x *= inv;
  acc.y *= inv;
  acc.z *= inv;
  acc.w *= inv;
  const long off = (long)r * o_row_stride + (long)a * D + c4 * 4;
  if (out_bf16) {
    union { __bf16 h[4]; uint2 u; } pk;
    pk.h[0] = (__bf16)acc.x;
    pk.h[1] = (__bf16)acc.y;
    pk.h[2] = (__bf16)acc.z;
    pk.h[3] = (__bf16)acc.w;
    *(uint2*)((uint16_t*)o + off) = pk.u;
  } else {
    *(float4*)((float*)o + off) = acc;
  }
  if (c4 == 0) lse[(long)a * lse_head_stride + r] = (wsum > 0.0f) ? m + logf(wsum) : -INFINITY;
}

// Workgroups below which the merge takes the deeper load ring (two per CU).
constexpr long kMergeDeepBelow = 512;

}  // namespace

hipError_t launch_gather(const void* k, const void* v, const int32_t* idx, void* kp, void* vp,
                         int la, int V, int L, int Hkv, int lp, int row_bytes, long kv_st_bytes,
                         long kv_sh_bytes, hipStream_t s) {
  const long total = 2L * Hkv * V * lp * (row_bytes / 16);
  if (total == 0) return hipSuccess;
  const long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint8_t*)k,
                     (const uint8_t*)v, idx, (uint8_t*)kp, (uint8_t*)vp, la, V, L, Hkv, lp,
                     row_bytes, kv_st_bytes, kv_sh_bytes, total);
  return hipGetLastError();
}

hipError_t launch_merge(int P, int R, int H, int D, const float* o_part, const float* lse_part,
                        void* o, long o_row_stride, float* lse, long lse_head_stride,
                        int out_bf16, hipStream_t s) {
  const long total = (long)R * H * (D / 4);
  if (total == 0) return hipSuccess;
  const long blocks = (total + 255) / 256;
  if (blocks < kMergeDeepBelow)
    hipLaunchKernelGGL(merge_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, s, P, R, H, D, o_part,
                       lse_part, o, o_row_stride, lse, lse_head_stride, out_bf16);
  else
    hipLaunchKernelGGL(merge_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, P, R, H, D, o_part,
                       lse_part, o, o_row_stride, lse, lse_head_stride, out_bf16);
  return hipGetLastError();
}

}  // namespace spava
