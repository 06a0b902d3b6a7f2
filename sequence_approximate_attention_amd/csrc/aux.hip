// Data-movement kernels: passing-block gather, key-contiguous V copy, LSE merge.
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
// Key-contiguous copy of V for the bf16 attention kernel (V^T per KV head).
// Tile = 64 key positions x D channels, transposed through LDS.  Padding key
// positions are written as zeros (their probabilities are masked to 0, and
// 0 * 0 keeps the PV product finite).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void vtranspose_kernel(AttnArgs a, uint16_t* __restrict__ vt,
                                                         uint16_t* __restrict__ vpt, int tile0) {
  constexpr int TS = kKeyTile + 2;  // LDS row stride (elements) of the [D][keys] tile
  __shared__ uint16_t sT[D * TS];
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int main_tiles = a.vl.main_len / kKeyTile;
  const int tt = tile0 + blockIdx.x;
  const bool pass = tt >= main_tiles;
  const int p0 = (pass ? tt - main_tiles : tt) * kKeyTile;

  // Which source rows feed this tile.
  long src_row0 = 0;   // element offset of key 0 of the run in v / vp
  long src_stride = 0; // elements between keys
  int n_valid = 0;     // keys of the tile that exist
  const uint16_t* src = nullptr;
  if (pass) {
    src = (const uint16_t*)a.vp;
    const int total = a.V * a.lp;
    n_valid = max(0, min(kKeyTile, total - p0));
    src_row0 = ((long)g * total + p0) * D;
    src_stride = D;
  } else {
    src = (const uint16_t*)a.v;
    int tok0, len, off;
    if (p0 < a.vl.off_block0) {
      tok0 = 0; len = a.la; off = p0;
    } else if (p0 < a.vl.off_query) {
      const int h = (p0 - a.vl.off_block0) / a.vl.pad_block;
      off = (p0 - a.vl.off_block0) % a.vl.pad_block;
      tok0 = a.la + h * a.L; len = a.L;
    } else {
      off = p0 - a.vl.off_query;
      tok0 = a.la + a.V * a.L; len = a.nq;
    }
    n_valid = max(0, min(kKeyTile, len - off));
    src_stride = a.kv_st;
    src_row0 = (long)(tok0 + off) * src_stride + (long)g * a.kv_sh;
  }

  constexpr int CPR = D / 8;
  for (int ch = tid; ch < kKeyTile * CPR; ch += 256) {
    const int key = ch / CPR;
    const int c = ch % CPR;
    union { uint4 u; uint16_t h[8]; } x;
    if (key < n_valid) {
      x.u = *(const uint4*)(src + src_row0 + (long)key * src_stride + c * 8);
    } else {
      x.u = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sT[(c * 8 + e) * TS + key] = x.h[e];
  }
  __syncthreads();
  const int rowlen = pass ? a.vl.pass_len : a.vl.main_len;
  uint16_t* dst = (pass ? vpt : vt) + (long)g * D * rowlen + p0;
  for (int ch = tid; ch < D * (kKeyTile / 8); ch += 256) {
    const int d = ch / (kKeyTile / 8);
    const int kc = ch % (kKeyTile / 8);
    union { uint4 u; uint32_t w[4]; } y;
    const uint16_t* s = sT + d * TS + kc * 8;
#pragma unroll
    for (int e = 0; e < 4; ++e) y.w[e] = (uint32_t)s[2 * e] | ((uint32_t)s[2 * e + 1] << 16);
    *(uint4*)(dst + (long)d * rowlen + kc * 8) = y.u;
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of partial attention results (axiom on Eq. 5 / Appendix A
// in the APB-V review: merging through the FlashAttention lse is exact).
// One thread per (row, head, 4 channels).
// ---------------------------------------------------------------------------
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
  const int a = (int)((gid / cq) % H);
  const int r = (int)(gid / ((long)cq * H));
  const float* lp_ra = lse_part + (long)a * R + r;                  // + p * H * R
  const float* op_ra = o_part + ((long)r * H + a) * D + c4 * 4;      // + p * R * H * D
  const long lp_step = (long)H * R, op_step = (long)R * H * D;
  float m = -INFINITY;
#pragma unroll 8
  for (int p = 0; p < P; ++p) m = fmaxf(m, lp_ra[p * lp_step]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.0f;
  if (m != -INFINITY) {
    // The partials are read kMergeBatch at a time, all loads first, so each
    // wave keeps that many reads in flight; the sums still run in p order.
    constexpr int kMergeBatch = 8;
    int p = 0;
    for (; p + kMergeBatch <= P; p += kMergeBatch) {
      float l[kMergeBatch];
      float4 x[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        l[u] = lp_ra[(p + u) * lp_step];
        x[u] = *(const float4*)(op_ra + (p + u) * op_step);
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const float w = expf(l[u] - m);
        acc.x += w * x[u].x;
        acc.y += w * x[u].y;
        acc.z += w * x[u].z;
        acc.w += w * x[u].w;
        wsum += w;
      }
    }
    for (; p < P; ++p) {
      const float w = expf(lp_ra[p * lp_step] - m);
      const float4 x = *(const float4*)(op_ra + p * op_step);
      acc.x += w * x.x;
      acc.y += w * x.y;
      acc.z += w * x.z;
      acc.w += w * x.w;
      wsum += w;
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

hipError_t launch_vtranspose(const AttnArgs& a, uint16_t* vt, uint16_t* vpt, int phase, hipStream_t s) {
  const int main_tiles = a.vl.main_len / kKeyTile;
  const int pass_tiles = a.vl.pass_len / kKeyTile;
  const int tile0 = phase == kPhasePassing ? main_tiles : 0;
  const int tiles = (phase == kPhaseLocal ? 0 : pass_tiles) + (phase == kPhasePassing ? 0 : main_tiles);
  if (tiles == 0) return hipSuccess;
  dim3 grid(tiles, a.Hkv);
  if (a.D == 128)
    hipLaunchKernelGGL((vtranspose_kernel<128>), grid, dim3(256), 0, s, a, vt, vpt, tile0);
  else
    hipLaunchKernelGGL((vtranspose_kernel<64>), grid, dim3(256), 0, s, a, vt, vpt, tile0);
  return hipGetLastError();
}

hipError_t launch_merge(int P, int R, int H, int D, const float* o_part, const float* lse_part,
                        void* o, long o_row_stride, float* lse, long lse_head_stride,
                        int out_bf16, hipStream_t s) {
  const long total = (long)R * H * (D / 4);
  if (total == 0) return hipSuccess;
  const long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, P, R, H, D, o_part,
                     lse_part, o, o_row_stride, lse, lse_head_stride, out_bf16);
  return hipGetLastError();
}

}  // namespace spava
