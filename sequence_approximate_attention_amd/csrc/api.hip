// C ABI of libspava: argument checks and launch sequencing (see include/spava.h).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "spava_common.h"

namespace spava {
namespace {

constexpr int kRowsPerUnitF32 = 128;  // query rows per workgroup of the float32 kernel

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Scratch memory of spava_score_topk_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address: the device address of each GPU's copy comes
// from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = SPAVA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, or NULL (with the
// error recorded) if it cannot be had.
void* scratch_on_current_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(SPAVA_ELAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(SPAVA_EUNSUPPORTED, "device %d is beyond the %d devices the scratch table covers", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(SPAVA_ELAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

int check_plan(const spava_plan* p) {
  if (!p) return fail(SPAVA_EINVAL, "plan is NULL");
  if (p->dtype != SPAVA_BF16 && p->dtype != SPAVA_F32)
    return fail(SPAVA_EUNSUPPORTED, "dtype %d is not SPAVA_BF16 or SPAVA_F32", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(SPAVA_EUNSUPPORTED, "head_dim %d is not 64 or 128", p->head_dim);
  if (p->n_anchor < 0 || p->n_hosts < 1 || p->host_len < 1 || p->n_query < 0)
    return fail(SPAVA_EINVAL, "need n_anchor>=0, n_hosts>=1, host_len>=1, n_query>=0");
  if (p->n_q_heads < 1 || p->n_kv_heads < 1 || p->n_q_heads % p->n_kv_heads != 0)
    return fail(SPAVA_EINVAL, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                p->n_q_heads, p->n_kv_heads);
  if (p->lp < 0 || p->lp > p->host_len)
    return fail(SPAVA_EINVAL, "lp (%d) must lie in [0, host_len=%d]", p->lp, p->host_len);
  if (!(p->scale >= 0.0f) || isinf(p->scale))
    return fail(SPAVA_EINVAL, "scale must be finite and >= 0 (0 = 1/sqrt(d))");
  const double N = (double)p->n_anchor + (double)p->n_hosts * p->host_len + p->n_query;
  const double H = p->n_q_heads > p->n_kv_heads ? p->n_q_heads : p->n_kv_heads;
  if (N * H * p->head_dim >= 2147483648.0)
    return fail(SPAVA_EINVAL, "N*heads*head_dim must stay below 2^31");
  // Strides: multiples of 16 bytes, extents below 2^31 elements, and every
  // run of keys (a block, the anchor, the query block) below 2^31 bytes.
  const int esz = p->dtype == SPAVA_F32 ? 4 : 2;
  const int64_t st[4] = {p->q_stride_tok, p->q_stride_head, p->kv_stride_tok, p->kv_stride_head};
  for (int i = 0; i < 4; ++i)
    if (st[i] < 0 || st[i] % (16 / esz) != 0)
      return fail(SPAVA_EINVAL, "strides must be >= 0 and multiples of %d elements", 16 / esz);
  const double q_st = p->q_stride_tok ? (double)p->q_stride_tok : (double)p->n_q_heads * p->head_dim;
  const double q_sh = p->q_stride_head ? (double)p->q_stride_head : (double)p->head_dim;
  const double kv_st = p->kv_stride_tok ? (double)p->kv_stride_tok : (double)p->n_kv_heads * p->head_dim;
  const double kv_sh = p->kv_stride_head ? (double)p->kv_stride_head : (double)p->head_dim;
  // A token's d channels end before the next token starts (copies of a run
  // end at its last row's d channels), and a token stride stays below 2^24
  // bytes (tile-row offsets are 24-bit products).
  if (q_st < p->head_dim || kv_st < p->head_dim)
    return fail(SPAVA_EINVAL, "token strides must be at least head_dim (%d) elements", p->head_dim);
  if (q_st * esz >= 16777216.0 || kv_st * esz >= 16777216.0)
    return fail(SPAVA_EINVAL, "token strides must stay below 2^24 bytes");
  if ((N - 1) * q_st + (p->n_q_heads - 1) * q_sh + p->head_dim >= 2147483648.0 ||
      (N - 1) * kv_st + (p->n_kv_heads - 1) * kv_sh + p->head_dim >= 2147483648.0)
    return fail(SPAVA_EINVAL, "q or k/v extends over 2^31 elements under its strides");
  double run = p->host_len;
  if (p->n_anchor > run) run = p->n_anchor;
  if (p->n_query > run) run = p->n_query;
  if (run * kv_st * esz >= 2147483648.0 || run * q_st * esz >= 2147483648.0)
    return fail(SPAVA_EINVAL, "a run of keys spans 2^31 bytes or more under the token strides");
  if ((double)p->n_hosts * p->lp * p->n_kv_heads * p->head_dim >= 2147483648.0)
    return fail(SPAVA_EINVAL, "passing blocks too large");
  return SPAVA_OK;
}

// Launch arguments of a plan; units are sized for the attention kernel of the
// plan's dtype.
AttnArgs make_args(const spava_plan* p) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.Hq = p->n_q_heads;
  a.Hkv = p->n_kv_heads;
  a.G = a.Hq / a.Hkv;
  a.D = p->head_dim;
  a.la = p->n_anchor;
  a.V = p->n_hosts;
  a.L = p->host_len;
  a.nq = p->n_query;
  a.lp = p->lp;
  a.N = a.la + a.V * a.L + a.nq;
  a.q_st = p->q_stride_tok ? p->q_stride_tok : (long)a.Hq * a.D;
  a.q_sh = p->q_stride_head ? p->q_stride_head : a.D;
  a.kv_st = p->kv_stride_tok ? p->kv_stride_tok : (long)a.Hkv * a.D;
  a.kv_sh = p->kv_stride_head ? p->kv_stride_head : a.D;
  a.scale = p->scale > 0.0f ? p->scale : 1.0f / sqrtf((float)a.D);
  a.scale_log2 = a.scale * 1.44269504088896340736f;
  a.f32 = p->dtype == SPAVA_F32;
  const int bm = a.f32 ? kRowsPerUnitF32 : attn_bf16_rows_per_unit();
  a.rows_per_unit = bm;
  a.n_ctx_units_per_host = ceil_div(a.L, bm) * a.Hq;
  a.n_q_units = ceil_div(a.nq * a.G, bm) * a.Hkv;
  a.n_anchor_units = ceil_div(a.la, bm) * a.Hq;
  // Query-block partials (ceil(L/64) tiles each) go after the hosts whose
  // shortest context unit (first row tile) walks at least as many tiles.
  const int t_qblk = ceil_div(a.L, kKeyTile);
  a.n_ctx_first = 0;
  for (int h = 0; h < a.V; ++h) {
    const int t_min = ceil_div(a.la, kKeyTile) + (h > 0 ? ceil_div(h * a.lp, kKeyTile) : 0) +
                      ceil_div(a.L < bm ? a.L : bm, kKeyTile);
    if (t_min >= t_qblk) ++a.n_ctx_first;
  }
  attn_phase_units(a, kPhaseAll, &a.unit_lo, &a.unit_hi);
  return a;
}

// Scoring workspace: float32 inputs keep one log2-domain LSE per (block, KV
// head, scoring row); bf16 inputs keep a (max, sum) pair per key chunk.  The
// query selector's rows are the query block's tokens, the context selector's
// the block's own tokens (each times the G heads of a group).
size_t stats_bytes(const spava_plan* p, bool ctx) {
  size_t bytes;
  if (p->dtype == SPAVA_F32) {
    const size_t ntok = ctx ? (size_t)p->host_len : (size_t)p->n_query;
    bytes = (size_t)p->n_hosts * p->n_kv_heads * ntok * (p->n_q_heads / p->n_kv_heads) * sizeof(float);
  } else {
    AttnArgs a = make_args(p);
    a.score_ctx = ctx ? 1 : 0;
    bytes = score_bf16_ws_bytes(a);
  }
  return (bytes + 255) / 256 * 256;
}

// Room for the scores when the caller passes none: float32 [V][Hkv][L] after
// the statistics.
size_t scores_bytes(const spava_plan* p) {
  return ((size_t)p->n_hosts * p->n_kv_heads * p->host_len * sizeof(float) + 255) / 256 * 256;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SPAVA_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = 0;
  return SPAVA_OK;
}

// Argument checks and launches of the attention, all units or one phase.
int attn_fwd(const char* name, int phase, const spava_plan* plan, const void* q, const void* k, const void* v,
             const void* kp, const void* vp, void* o, float* lse, float* o_part, float* lse_part, void* stream) {
  int rc = check_plan(plan);
  if (rc) return rc;
  const bool need_pass = phase != kPhaseLocal && plan->lp > 0 && plan->n_hosts > 1;
  const bool need_part = phase != kPhasePassing && plan->n_query > 0;
  if (!q || !k || !v || !o || !lse || (need_pass && (!kp || !vp)) || (need_part && (!o_part || !lse_part)))
    return fail(SPAVA_EINVAL, "%s: NULL pointer", name);
  const void* ptrs[] = {q, k, v, kp, vp, o, lse, o_part, lse_part};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SPAVA_EINVAL, "%s: pointers must be 16-byte aligned", name);
  hipStream_t s = (hipStream_t)stream;
  AttnArgs a = make_args(plan);
  if (phase != kPhaseAll) a.n_ctx_first = a.V;   // phases split the order after host 1
  attn_phase_units(a, phase, &a.unit_lo, &a.unit_hi);
  a.q = q;
  a.k = k;
  a.v = v;
  a.kp = kp;
  a.vp = vp;
  a.o = o;
  a.lse = lse;
  a.o_part = o_part;
  a.lse_part = lse_part;
  hipError_t e;
  if (a.f32) {
    e = launch_attn_f32(a, s);
    return launched(e, "attention (float32)");
  }
  e = launch_attn_bf16(a, s);
  return launched(e, "attention (bf16)");
}

// Block scores and top-lp selection with the query rows (ctx = false) or the
// block's own tokens (ctx = true) as the scoring rows.
int score_topk(const char* name, bool ctx, const spava_plan* plan, const void* q, const void* k,
               float* scores, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_plan(plan);
  if (rc) return rc;
  if (!q || !k || !ws || (plan->lp > 0 && !idx))
    return fail(SPAVA_EINVAL, "%s: q, k, ws (and idx when lp > 0) must be non-NULL", name);
  if (!aligned16(q) || !aligned16(k) || (scores && !aligned16(scores)) || !aligned16(ws) ||
      (idx && !aligned16(idx)))
    return fail(SPAVA_EINVAL, "%s: pointers must be 16-byte aligned", name);
  const size_t need = stats_bytes(plan, ctx) + (scores ? 0 : scores_bytes(plan));
  if (ws_bytes < need) return fail(SPAVA_EWORKSPACE, "%s: workspace %zu < %zu bytes", name, ws_bytes, need);
  if (!scores) scores = (float*)((char*)ws + stats_bytes(plan, ctx));
  if (ctx && (double)plan->host_len * (plan->n_q_heads / plan->n_kv_heads) >= 2147483648.0)
    return fail(SPAVA_EINVAL, "%s: host_len * (n_q_heads / n_kv_heads) must stay below 2^31", name);
  hipStream_t s = (hipStream_t)stream;
  AttnArgs a = make_args(plan);
  a.q = q;
  a.k = k;
  a.score_ctx = ctx ? 1 : 0;
  hipError_t e = hipSuccess;
  if (a.f32) {
    a.stats = (float*)ws;
    if (score_rows(a, 0).R > 0) {
      e = launch_rowstat_f32(a, s);
      if (e != hipSuccess) return launched(e, "row statistics");
    }
    e = launch_colsum_f32(a, scores, s);
  } else {
    e = launch_score_bf16(a, ws, scores, s);
  }
  if (e != hipSuccess) return launched(e, "block scores");
  e = launch_topk(scores, idx, a.V * a.Hkv, a.L, a.lp, s);
  return launched(e, "top-lp selection");
}



}  // namespace
}  // namespace spava

using namespace spava;

extern "C" {

int spava_version(void) { return SPAVA_VERSION; }

const char* spava_last_error(void) { return g_err; }

int spava_plan_check(const spava_plan* plan) {
  int rc = check_plan(plan);
  if (rc == SPAVA_OK) g_err[0] = 0;
  return rc;
}

size_t spava_score_topk_ws_bytes(const spava_plan* plan) {
  if (check_plan(plan) != SPAVA_OK) return 0;
  return stats_bytes(plan, false) + scores_bytes(plan);
}

int spava_score_topk(const spava_plan* plan, const void* q, const void* k, float* scores,
                     int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  return score_topk("spava_score_topk", false, plan, q, k, scores, idx, ws, ws_bytes, stream);
}

int spava_score_topk_noalloc(const spava_plan* plan, const void* q, const void* k, float* scores,
                             int32_t* idx, void* stream) {
  const char* name = "spava_score_topk_noalloc";
  int rc = check_plan(plan);
  if (rc) return rc;
  // The same checks as spava_score_topk, then the size, all before the
  // device is touched.
  if (!q || !k || (plan->lp > 0 && !idx))
    return fail(SPAVA_EINVAL, "%s: q, k (and idx when lp > 0) must be non-NULL", name);
  if (!aligned16(q) || !aligned16(k) || (scores && !aligned16(scores)) || (idx && !aligned16(idx)))
    return fail(SPAVA_EINVAL, "%s: pointers must be 16-byte aligned", name);
  const size_t need = stats_bytes(plan, false) + (scores ? 0 : scores_bytes(plan));
  if (need > kScratchBytes)
    return fail(SPAVA_EWORKSPACE, "%s: this plan needs %zu bytes of scratch; the static scratch holds %zu "
                "(pass scores, or use spava_score_topk with a workspace)", name, need, kScratchBytes);
  void* ws = scratch_on_current_device();
  if (!ws) return SPAVA_ELAUNCH;
  return score_topk(name, false, plan, q, k, scores, idx, ws, kScratchBytes, stream);
}

size_t spava_score_topk_context_ws_bytes(const spava_plan* plan) {
  if (check_plan(plan) != SPAVA_OK) return 0;
  return stats_bytes(plan, true) + scores_bytes(plan);
}

int spava_score_topk_context(const spava_plan* plan, const void* q, const void* k, float* scores,
                             int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  return score_topk("spava_score_topk_context", true, plan, q, k, scores, idx, ws, ws_bytes, stream);
}

int spava_kv_overlap(int32_t n_lists, int32_t lp, const int32_t* idx_a, const int32_t* idx_b,
                     int32_t* counts, void* stream) {
  if (n_lists < 0 || lp < 0) return fail(SPAVA_EINVAL, "spava_kv_overlap: need n_lists >= 0 and lp >= 0");
  if (n_lists == 0) {
    g_err[0] = 0;
    return SPAVA_OK;
  }
  if (!counts || (lp > 0 && (!idx_a || !idx_b)))
    return fail(SPAVA_EINVAL, "spava_kv_overlap: NULL pointer");
  if (((uintptr_t)counts | (uintptr_t)idx_a | (uintptr_t)idx_b) & 3u)
    return fail(SPAVA_EINVAL, "spava_kv_overlap: pointers must be 4-byte aligned");
  if ((double)n_lists * lp >= 2147483648.0)
    return fail(SPAVA_EINVAL, "spava_kv_overlap: n_lists * lp must stay below 2^31");
  return launched(launch_overlap(idx_a, idx_b, counts, n_lists, lp, (hipStream_t)stream), "overlap");
}

int spava_gather_passing(const spava_plan* plan, const void* k, const void* v, const int32_t* idx,
                         void* kp, void* vp, void* stream) {
  int rc = check_plan(plan);
  if (rc) return rc;
  if (plan->lp == 0) {
    g_err[0] = 0;
    return SPAVA_OK;
  }
  if (!k || !v || !idx || !kp || !vp)
    return fail(SPAVA_EINVAL, "spava_gather_passing: NULL pointer");
  if (!aligned16(k) || !aligned16(v) || !aligned16(kp) || !aligned16(vp))
    return fail(SPAVA_EINVAL, "spava_gather_passing: pointers must be 16-byte aligned");
  const int esz = plan->dtype == SPAVA_F32 ? 4 : 2;
  const AttnArgs a = make_args(plan);
  hipError_t e = launch_gather(k, v, idx, kp, vp, plan->n_anchor, plan->n_hosts, plan->host_len,
                               plan->n_kv_heads, plan->lp, plan->head_dim * esz, a.kv_st * esz, a.kv_sh * esz,
                               (hipStream_t)stream);
  return launched(e, "gather");
}

int spava_attn_fwd(const spava_plan* plan, const void* q, const void* k, const void* v,
                   const void* kp, const void* vp, void* o, float* lse, float* o_part,
                   float* lse_part, void* stream) {
  return attn_fwd("spava_attn_fwd", kPhaseAll, plan, q, k, v, kp, vp, o, lse, o_part, lse_part, stream);
}

int spava_attn_fwd_phase(const spava_plan* plan, int32_t phase, const void* q, const void* k, const void* v,
                         const void* kp, const void* vp, void* o, float* lse, float* o_part,
                         float* lse_part, void* stream) {
  if (phase != SPAVA_PHASE_ALL && phase != SPAVA_PHASE_LOCAL && phase != SPAVA_PHASE_PASSING)
    return fail(SPAVA_EINVAL, "spava_attn_fwd_phase: phase %d is not SPAVA_PHASE_ALL, _LOCAL or _PASSING", phase);
  return attn_fwd("spava_attn_fwd_phase", phase, plan, q, k, v, kp, vp, o, lse, o_part, lse_part, stream);
}

int spava_score_topk_from_partials(const spava_plan* plan, const void* q, const void* k, const float* lse_part,
                                   float* scores, int32_t* idx, void* stream) {
  int rc = check_plan(plan);
  if (rc) return rc;
  const char* name = "spava_score_topk_from_partials";
  if (!q || !k || !scores || (plan->lp > 0 && !idx) || (plan->n_query > 0 && !lse_part))
    return fail(SPAVA_EINVAL, "%s: q, k, scores (idx when lp > 0, lse_part when n_query > 0) must be non-NULL",
                name);
  if (!aligned16(q) || !aligned16(k) || !aligned16(scores) || (idx && !aligned16(idx)) ||
      (lse_part && !aligned16(lse_part)))
    return fail(SPAVA_EINVAL, "%s: pointers must be 16-byte aligned", name);
  hipStream_t s = (hipStream_t)stream;
  AttnArgs a = make_args(plan);
  a.q = q;
  a.k = k;
  a.lse_part = (float*)lse_part;
  a.score_from_partials = 1;
  hipError_t e = a.f32 ? launch_colsum_f32(a, scores, s) : launch_score_bf16(a, nullptr, scores, s);
  if (e != hipSuccess) return launched(e, "block scores");
  e = launch_topk(scores, idx, a.V * a.Hkv, a.L, a.lp, s);
  return launched(e, "top-lp selection");
}

int spava_lse_merge(int32_t n_parts, int32_t n_rows, int32_t n_heads, int32_t head_dim,
                    const float* o_part, const float* lse_part, void* o, int64_t o_row_stride,
                    float* lse, int64_t lse_head_stride, int32_t out_dtype, void* stream) {
  if (n_parts < 1 || n_rows < 0 || n_heads < 1 || head_dim < 4 || head_dim % 4 != 0)
    return fail(SPAVA_EINVAL, "spava_lse_merge: need n_parts>=1, n_rows>=0, n_heads>=1, head_dim%%4==0");
  if (out_dtype != SPAVA_BF16 && out_dtype != SPAVA_F32)
    return fail(SPAVA_EUNSUPPORTED, "spava_lse_merge: out_dtype %d", out_dtype);
  if (n_rows == 0) {
    g_err[0] = 0;
    return SPAVA_OK;
  }
  if (!o_part || !lse_part || !o || !lse) return fail(SPAVA_EINVAL, "spava_lse_merge: NULL pointer");
  if (!aligned16(o_part) || ((uintptr_t)o & (out_dtype == SPAVA_F32 ? 15u : 7u)) ||
      (o_row_stride % 4) != 0 || ((uintptr_t)lse & 3u))
    return fail(SPAVA_EINVAL, "spava_lse_merge: misaligned pointer or row stride");
  if (o_row_stride < (int64_t)n_heads * head_dim || lse_head_stride < n_rows)
    return fail(SPAVA_EINVAL, "spava_lse_merge: strides too small");
  hipError_t e = launch_merge(n_parts, n_rows, n_heads, head_dim, o_part, lse_part, o, o_row_stride,
                              lse, lse_head_stride, out_dtype == SPAVA_BF16, (hipStream_t)stream);
  return launched(e, "merge");
}

}  // extern "C"
