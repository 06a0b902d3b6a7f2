// Approximate-attention forward for float32 inputs (vector ALUs).
//
// Same units and key segments as the bf16 MFMA kernel; one thread owns one
// query row and walks its keys with an online softmax in float32.  This path
// exists so that float32 inputs are computed in float32 end to end; it is
// sized for small workloads, not for throughput.
#include "spava_common.h"

namespace spava {
namespace {

constexpr int kRows = 128;

template <int D>
__global__ __launch_bounds__(kRows) void attn_f32_kernel(AttnArgs a) {
  const Unit u = unit_decode(a, a.unit_lo + blockIdx.x);
  Seg segs[3];
  const int nseg = unit_segments(a, u, segs);
  const int r = u.tile * kRows + threadIdx.x;
  const RowId row = unit_row(a, u, r);
  if (!row.valid) return;
  const float* qp = (const float*)a.q + (long)row.tok * a.q_st + (long)row.head * a.q_sh;
  float qv[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = qp[c];
    acc[c] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int s = 0; s < nseg; ++s) {
    const Seg& sg = segs[s];
    const float* kb = (const float*)(sg.kind ? a.kp : a.k) + sg.k_off;
    const float* vb = (const float*)(sg.kind ? a.vp : a.v) + sg.v_off;
    int n = sg.len;
    if (sg.causal) n = min(n, row.tok - sg.tok0 + 1);
    for (int j = 0; j < n; ++j) {
      const float* kr = kb + (long)j * sg.k_stride;
      float dot = 0.0f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(qv[c], kr[c], dot);
      const float x = dot * a.scale_log2;
      const float mn = fmaxf(m, x);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      const float p = __builtin_amdgcn_exp2f(x - mn);
      l = l * alpha + p;
      const float* vr = vb + (long)j * sg.v_stride;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(p, vr[c], acc[c] * alpha);
      m = mn;
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const float lse = l > 0.0f ? (m + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
  if (u.kind == kAnchor || u.kind == kContext) {
    float* op = (float*)a.o + ((long)row.tok * a.Hq + row.head) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) op[c] = acc[c] * inv;
    a.lse[(long)row.head * a.N + row.tok] = lse;
  } else {
    const int p = (u.kind == kQueryHead) ? 0 : u.host + 1;
    const int i = row.tok - (a.la + a.V * a.L);
    float* op = a.o_part + (((long)p * a.nq + i) * a.Hq + row.head) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) op[c] = acc[c] * inv;
    a.lse_part[((long)p * a.Hq + row.head) * a.nq + i] = lse;
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  const int n = a.unit_hi - a.unit_lo;
  if (n <= 0) return hipSuccess;
  if (a.D == 128)
    hipLaunchKernelGGL((attn_f32_kernel<128>), dim3(n), dim3(kRows), 0, s, a);
  else
    hipLaunchKernelGGL((attn_f32_kernel<64>), dim3(n), dim3(kRows), 0, s, a);
  return hipGetLastError();
}

}  // namespace spava
