// Fused approximate-attention forward for bf16 inputs on gfx950 (CDNA4).
//
// One workgroup = 4 waves = one unit of 128 query rows (32 per wave).  The
// unit's key segments (anchor / passing blocks / own block / query block,
// see unit_segments) are walked in 64-key tiles staged through LDS:
//   K tile   [64 keys][D]   row-major, read as the MFMA A operand
//   V^T tile [D][64 keys]   key-contiguous, read as the MFMA A operand
// Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so that every
// lane owns one query column: the online-softmax row statistics then live in
// one lane pair (l, l^32) and the rescale of O^T is lane-uniform.  P^T leaves
// the accumulator registers directly as the B operand of O^T += V^T P^T.
// A-operand rows of the K tile are read in a permuted order (bits 2 and 3 of
// the row swapped) so that the accumulator layout of S^T equals the B-operand
// layout P^T needs, with keys in natural order.
//
// STATS = true: rows only accumulate the running max and sum (no PV) and
// write the log2-domain row log-sum-exp used by the block scoring
// (Figure 5 caption of the Spava page: Q_qr K^(h)T estimates KV importance).
#include "spava_common.h"

namespace spava {
namespace {

constexpr int kBM = 128;   // rows per workgroup
constexpr int kBN = kKeyTile;
constexpr int kThreads = 256;

__device__ __forceinline__ int perm_row(int m) {  // swap bits 2 and 3
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ float wave_max_xor32(float x) {
  return fmaxf(x, __shfl_xor(x, 32));
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

template <int D>
struct TileRegs {
  uint4 k[D / 32];
  uint4 v[D / 32];
};

template <int D, bool STATS>
__device__ __forceinline__ void load_tile(const AttnArgs& a, const Seg& sg, int t, int tid,
                                          TileRegs<D>& r) {
  constexpr int CPR = D / 8;           // 16-byte chunks per K row
  constexpr int RPP = kThreads / CPR;  // K rows per pass
  const uint16_t* kbase = (const uint16_t*)(sg.kind ? a.kp : a.k) + sg.k_off;
  const int kb0 = t * kBN;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    int row = tid / CPR + i * RPP;
    int j = min(kb0 + row, sg.len - 1);
    r.k[i] = *(const uint4*)(kbase + (long)j * sg.k_stride + (tid % CPR) * 8);
  }
  if (!STATS) {
    const int rowlen = sg.vt_pass ? a.vl.pass_len : a.vl.main_len;
    const uint16_t* vbase = (sg.vt_pass ? a.vpt : a.vt) + sg.vt_off + kb0;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      int drow = tid / 8 + i * 32;
      r.v[i] = *(const uint4*)(vbase + (long)drow * rowlen + (tid % 8) * 8);
    }
  }
}

template <int D, bool STATS>
__device__ __forceinline__ void store_tile(uint16_t* sK, uint16_t* sV, int tid, const TileRegs<D>& r) {
  constexpr int CPR = D / 8;
  constexpr int RPP = kThreads / CPR;
  constexpr int KS = D + 8;
  constexpr int VS = kBN + 8;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    int row = tid / CPR + i * RPP;
    *(uint4*)(sK + row * KS + (tid % CPR) * 8) = r.k[i];
  }
  if (!STATS) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      int drow = tid / 8 + i * 32;
      *(uint4*)(sV + drow * VS + (tid % 8) * 8) = r.v[i];
    }
  }
}

template <int D, bool STATS>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KS = D + 8;
  constexpr int VS = kBN + 8;
  constexpr int NC = D / 16;  // 16-wide d chunks (MFMA K steps of S)
  constexpr int NDB = D / 32; // 32-row d blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[STATS ? 8 : D * VS];
  __shared__ int sTok[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 5;
  const int col = lane & 31;

  const Unit u = unit_decode(a, blockIdx.x);
  Seg segs[3];
  const int nseg = unit_segments(a, u, segs);

  const int r = u.tile * kBM + wave * kRowsPerWave + col;
  const RowId row = unit_row(a, u, r);

  // Q^T fragments (B operand): lane holds its query's d = 16c + 8*hi .. +7.
  bf16x8 qf[NC];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((long)row.tok * a.Hq + row.head) * D + 8 * hi;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (row.valid) {
        qf[c] = *(const bf16x8*)(qp + 16 * c);
      } else {
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

  int ntile[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    ntile[s] = 0;
    if (s < nseg) {
      int n = segs[s].len;
      if (segs[s].causal) n = min(n, gmax - segs[s].tok0 + 1);
      ntile[s] = n > 0 ? ceil_div(n, kBN) : 0;
    }
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const float sl2 = a.scale_log2;

  int cs = 0, ct = 0;
  while (cs < nseg && ntile[cs] == 0) ++cs;
  TileRegs<D> regs;
  if (cs < nseg) load_tile<D, STATS>(a, segs[cs], 0, tid, regs);

  while (cs < nseg) {
    __syncthreads();
    store_tile<D, STATS>(sK, sV, tid, regs);
    __syncthreads();
    // Prefetch the next tile while this one is consumed.
    int ns = cs, nt = ct + 1;
    if (nt >= ntile[ns]) {
      nt = 0;
      ++ns;
      while (ns < nseg && ntile[ns] == 0) ++ns;
    }
    if (ns < nseg) load_tile<D, STATS>(a, segs[ns], nt, tid, regs);

    const Seg& sg = segs[cs];
    const int kb0 = ct * kBN;
    const bool skip = sg.causal && (sg.tok0 + kb0 > wmax);
    if (!skip) {
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.0f;
        const uint16_t* kr = sK + (32 * kb + perm_row(col)) * KS + 8 * hi;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          bf16x8 af = *(const bf16x8*)(kr + 16 * c);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[c], sacc[kb], 0, 0, 0);
        }
      }
      const bool need_mask = (kb0 + kBN > sg.len) || (sg.causal && sg.tok0 + kb0 + kBN - 1 > wmin);
      if (need_mask) {
        // Tile-local key j is visible iff j < lim.
        int lim = sg.len - kb0;
        if (sg.causal) lim = min(lim, row.tok - sg.tok0 - kb0 + 1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            int j = 32 * kb + (i & 7) + 8 * hi + 16 * (i >> 3);
            if (j >= lim) sacc[kb][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = wave_max_xor32(mx);
      const float m_new = fmaxf(m_run, mx * sl2);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = __builtin_amdgcn_exp2f(sacc[kb][i] * sl2 - m_use);
          sacc[kb][i] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (!STATS) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const int kb = kc >> 1;
          const int base = 8 * (kc & 1);
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sacc[kb][base + e];
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8 vf = *(const bf16x8*)(sV + (32 * db + col) * VS + 16 * kc + 8 * hi);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, oacc[db], 0, 0, 0);
          }
        }
      }
    }
    cs = ns;
    ct = nt;
  }

  // Epilogue.
  const float lt = l_run + __shfl_xor(l_run, 32);
  const float lse2 = (lt > 0.0f) ? m_run + __log2f(lt) : -INFINITY;
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
        for (int e = 0; e < 4; ++e) pk.h[e] = (__bf16)(oacc[db][4 * g4 + e] * inv);
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
        w.x = oacc[db][4 * g4 + 0] * inv;
        w.y = oacc[db][4 * g4 + 1] * inv;
        w.z = oacc[db][4 * g4 + 2] * inv;
        w.w = oacc[db][4 * g4 + 3] * inv;
        *(float4*)(op + d0) = w;
      }
    if (hi == 0) a.lse_part[((long)p * a.Hq + row.head) * a.nq + i] = lse_nat;
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  const int n = attn_total_units(a);
  if (n == 0) return hipSuccess;
  if (a.D == 128) {
    if (a.stats_only)
      hipLaunchKernelGGL((attn_bf16_kernel<128, true>), dim3(n), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<128, false>), dim3(n), dim3(kThreads), 0, s, a);
  } else {
    if (a.stats_only)
      hipLaunchKernelGGL((attn_bf16_kernel<64, true>), dim3(n), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((attn_bf16_kernel<64, false>), dim3(n), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace spava
