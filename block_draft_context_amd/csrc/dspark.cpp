// C ABI of the draft-block library: argument checks, workspace planning and
// the launch sequence of each entry point (include/dspark.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/dspark.h"
#include "kernels.h"

namespace dspark {

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
static thread_local std::string g_err;

static dspark_status fail(dspark_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define DSPARK_HIP(expr)                                                             \
  do {                                                                               \
    hipError_t e_ = (expr);                                                          \
    if (e_ != hipSuccess)                                                            \
      return fail(DSPARK_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));       \
  } while (0)

// ---------------------------------------------------------------------------
// tracing (per-kernel HIP events)
// ---------------------------------------------------------------------------
static const char* kNames[K_COUNT] = {
    "gemm_ctx_fuse",      "setup",      "gemm_ctx_kv", "attn_split_k",
    "attn_combine_oproj", "block_gemm", "block_rows",  "markov"};

const char* kernel_name(int kind) { return (kind >= 0 && kind < K_COUNT) ? kNames[kind] : ""; }

struct Trace {
  bool on = false;
  uint64_t mask = 0;
  int cap = 0;
  int used = 0;
  bool open = false;
  std::vector<hipEvent_t> ev;
  std::vector<int> kind;
};
static Trace g_trace;

void trace_pre(int kind, hipStream_t s) {
  Trace& t = g_trace;
  if (!t.on || !((t.mask >> kind) & 1ull) || t.used >= t.cap) return;
  (void)hipEventRecord(t.ev[2 * t.used], s);
  t.open = true;
}

void trace_post(int kind, hipStream_t s) {
  Trace& t = g_trace;
  if (!t.on || !t.open) return;
  (void)hipEventRecord(t.ev[2 * t.used + 1], s);
  t.kind[t.used] = kind;
  t.used += 1;
  t.open = false;
}

// ---------------------------------------------------------------------------
// planning
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }


struct Plan {
  int64_t T = 0, Tpad = 0;
  int hd = 0, M = 0, chunk = 0, total_chunks = 0, kv_layers = 0;
  int nkv = 0, kvd = 0;   // K/V heads and K/V columns (kvd = nkv * hd)
  CtxSplit ctx;   // K splits of the Eq 2 projection
  size_t esz = 4;
  // workspace offsets (bytes)
  // ppart: the Eq 2 split-K partials, or with ctx.fused its Y rows; ysum: the
  // fused epilogue's row sums
  size_t wkvt = 0, ppart = 0, ysum = 0, ptail = 0, hctx = 0, rinv = 0, kv = 0, prefix = 0, po = 0, pml = 0,
         rowmap = 0;
  size_t D = 0, D2 = 0, Q = 0, Kd = 0, Vd = 0, E = 0, GU = 0, O = 0;
  size_t total = 0;
};

static dspark_status check_dims(const dspark_dims* dm, int op) {
  if (!dm) return fail(DSPARK_EINVAL, "dims is NULL");
  if (dm->dtype != DSPARK_F32 && dm->dtype != DSPARK_BF16)
    return fail(DSPARK_EUNSUPPORTED, "dtype %d not supported (0 = f32, 1 = bf16)", dm->dtype);
  if (dm->d <= 0 || dm->n_heads <= 0 || dm->gamma < 1 || dm->m < 1 || dm->H <= 0 || dm->ff <= 0)
    return fail(DSPARK_EINVAL, "sizes must be positive (m=%d H=%d d=%d n_heads=%d gamma=%d ff=%d)",
                dm->m, dm->H, dm->d, dm->n_heads, dm->gamma, dm->ff);
  if (dm->d % dm->n_heads != 0)
    return fail(DSPARK_EINVAL, "dDraft %d not divisible by nHeads %d", dm->d, dm->n_heads);
  const int hd = dm->d / dm->n_heads;
  if (hd != 32 && hd != 64 && hd != 128)
    return fail(DSPARK_EUNSUPPORTED, "head_dim %d not in {32, 64, 128}", hd);
  if (dm->gamma > kMaxGamma) return fail(DSPARK_EUNSUPPORTED, "gamma %d > %d", dm->gamma, kMaxGamma);
  if (dm->m > kMaxSegs) return fail(DSPARK_EUNSUPPORTED, "m %d > %d taps", dm->m, kMaxSegs);
  if (dm->d % 128 != 0 || dm->d > 2048)
    return fail(DSPARK_EUNSUPPORTED, "d %d must be a multiple of 128 and <= 2048", dm->d);
  if (dm->H % 64 != 0) return fail(DSPARK_EUNSUPPORTED, "H %d must be a multiple of 64", dm->H);
  if (dm->ff % 128 != 0) return fail(DSPARK_EUNSUPPORTED, "ff %d must be a multiple of 128", dm->ff);
  if (dm->ff > 16256) return fail(DSPARK_EUNSUPPORTED, "ff %d above the supported 16256", dm->ff);
  if (!(dm->eps >= 0.f) || !std::isfinite(dm->eps)) return fail(DSPARK_EINVAL, "eps must be finite and >= 0");
  const int nkv = dm->n_kv_heads == 0 ? dm->n_heads : dm->n_kv_heads;
  if (nkv < 1 || dm->n_heads % nkv != 0)
    return fail(DSPARK_EINVAL, "n_kv_heads %d must divide n_heads %d", dm->n_kv_heads, dm->n_heads);
  if ((nkv * hd) % 128 != 0)
    return fail(DSPARK_EUNSUPPORTED, "n_kv_heads * head_dim = %d must be a multiple of 128", nkv * hd);
  if (dm->variant & ~(DSPARK_QK_NORM | DSPARK_PLAIN_CTX_KV | DSPARK_GELU_FFN))
    return fail(DSPARK_EINVAL, "unknown variant bits 0x%x", dm->variant);
  if (!(dm->rope_theta >= 0.f) || !std::isfinite(dm->rope_theta) || (dm->rope_theta > 0.f && dm->rope_theta <= 1.f))
    return fail(DSPARK_EINVAL, "rope_theta must be 0 (no rotary positions) or finite and > 1");
  if ((op == DSPARK_OP_BLOCK_FORWARD || op == DSPARK_OP_CTX_APPEND || op == DSPARK_OP_BLOCK_PROPOSE) &&
      (dm->n_layers < 1 || dm->n_layers > 16))
    return fail(dm->n_layers < 1 ? DSPARK_EINVAL : DSPARK_EUNSUPPORTED, "n_layers %d not in [1, 16]",
                dm->n_layers);
  return DSPARK_OK;
}

static dspark_status check_cu(int32_t A, const int32_t* cu_host, int gamma, int64_t* T) {
  if (A < 1) return fail(DSPARK_EINVAL, "A = %d < 1", A);
  if ((int64_t)A * gamma > 1024) return fail(DSPARK_EUNSUPPORTED, "A * gamma = %lld > 1024", (long long)A * gamma);
  if (!cu_host) return fail(DSPARK_EINVAL, "cu_host is NULL");
  if (cu_host[0] != 0) return fail(DSPARK_EINVAL, "cu[0] = %d, expected 0", cu_host[0]);
  for (int b = 0; b < A; ++b)
    if (cu_host[b + 1] < cu_host[b]) return fail(DSPARK_EINVAL, "cu is decreasing at %d", b);
  *T = cu_host[A];
  if (*T > (1ll << 30)) return fail(DSPARK_EUNSUPPORTED, "T = %lld too large", (long long)*T);
  return DSPARK_OK;
}

static dspark_status make_plan(int op, const dspark_dims* dm, int32_t A, const int32_t* cu_host, Plan* p) {
  dspark_status st = check_dims(dm, op);
  if (st != DSPARK_OK) return st;
  int64_t T = 0;
  st = check_cu(A, cu_host, dm->gamma, &T);
  if (st != DSPARK_OK) return st;
  const bool bf = dm->dtype == DSPARK_BF16;
  p->esz = bf ? 2 : 4;
  p->T = T;
  p->Tpad = ((T + 63) / 64) * 64;
  p->hd = dm->d / dm->n_heads;
  p->nkv = dm->n_kv_heads == 0 ? dm->n_heads : dm->n_kv_heads;
  p->kvd = p->nkv * p->hd;
  p->M = A * dm->gamma;
  // The context projections address H_ctx (the A operand of the K/V
  // product) and W_c with 32-bit byte offsets (the taps are checked with
  // their leading dimension in check_taps).
  // The ops' parts: Eq 2 (the fuse product), the context K/V product (over
  // H_ctx rows), and the block side (attention over context K/V in the
  // workspace or in a draft cache).
  const bool runs_eq2 = op == DSPARK_OP_CTX_FUSE || op == DSPARK_OP_BLOCK_FORWARD || op == DSPARK_OP_CTX_APPEND;
  const bool runs_kv = op == DSPARK_OP_BLOCK_LAYER || op == DSPARK_OP_BLOCK_FORWARD || op == DSPARK_OP_CTX_APPEND;
  const bool runs_block = op == DSPARK_OP_BLOCK_LAYER || op == DSPARK_OP_BLOCK_FORWARD ||
                          op == DSPARK_OP_BLOCK_PROPOSE;
  const int64_t kMaxBytes = (int64_t)1 << 32;
  if (op != DSPARK_OP_BLOCK_PROPOSE && T * dm->d * p->esz >= kMaxBytes)
    return fail(DSPARK_EUNSUPPORTED, "H_ctx spans %lld bytes (T * d); at most 4 GiB is supported",
                (long long)(T * dm->d * p->esz));
  if (runs_eq2 && (int64_t)dm->d * dm->m * dm->H * p->esz >= kMaxBytes)
    return fail(DSPARK_EUNSUPPORTED, "W_c spans %lld bytes (d * m * H); at most 4 GiB is supported",
                (long long)((int64_t)dm->d * dm->m * dm->H * p->esz));
  const int d = dm->d, mH = dm->m * dm->H, ff = dm->ff, M = p->M;
  p->ctx = ctx_gemm_split(dm->dtype, T, d, mH);
  p->chunk = attention_chunk(cu_host, A, dm->n_heads);
  p->total_chunks = (int)attention_tiles(cu_host, A, p->chunk);
  p->kv_layers = op == DSPARK_OP_BLOCK_LAYER ? 1 : dm->n_layers;

  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  const bool fused = runs_eq2 && p->ctx.fused;
  if (fused) {
    p->ppart = take((size_t)T * d * 2);
    p->ysum = take((size_t)T * (d / kCtxSumCols) * 2 * 4);
    if (p->ctx.tail_row < T) p->ptail = take((size_t)p->ctx.tail_splits * (T - p->ctx.tail_row) * d * 4);
  } else if (runs_eq2) {
    p->ppart = take((size_t)p->ctx.splits * T * d * 4);
  }
  if (runs_kv) {
    if (bf) p->wkvt = take((size_t)2 * p->kv_layers * p->kvd * d * 2);
    // the K/V product reads H_ctx, or with the fused Eq 2 path the Y rows
    if (op != DSPARK_OP_BLOCK_LAYER && !fused) p->hctx = take((size_t)T * d * p->esz);
    p->rinv = take((size_t)T * 4);
    if (op == DSPARK_OP_CTX_APPEND) p->rowmap = take((size_t)T * 4);
    else p->kv = take((size_t)p->kv_layers * 2 * p->Tpad * p->kvd * p->esz);
  }
  if (runs_block) {
    p->prefix = take((size_t)(A + 1) * 4);
    p->po = take((size_t)p->total_chunks * dm->n_heads * dm->gamma * p->hd * 4);
    p->pml = take((size_t)p->total_chunks * dm->n_heads * dm->gamma * 2 * 4);
    const size_t row = (size_t)M * d * 4;
    p->D = take(row);
    p->D2 = take(row);
    p->Q = take(row);
    p->Kd = take(row);
    p->Vd = take(row);
    p->E = take(row);   // D + Attn Wo^T of the current layer
    p->O = take(row);   // Attn: the heads' attention outputs
    p->GU = take((size_t)M * 2 * ff * 4);
  }
  p->total = off == 0 ? 256 : off;
  return DSPARK_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define NEED_PTR(p)                                                                  \
  do {                                                                               \
    if (!(p)) return fail(DSPARK_EINVAL, "%s is NULL", #p);                          \
    if (!aligned16(p)) return fail(DSPARK_EINVAL, "%s is not 16-byte aligned", #p);  \
  } while (0)
#define OPT_PTR(p)                                                                   \
  do {                                                                               \
    if ((p) && !aligned16(p)) return fail(DSPARK_EINVAL, "%s is not 16-byte aligned", #p); \
  } while (0)

static dspark_status check_layer(const dspark_layer_weights* lw, int i, const dspark_dims* dm) {
  if (!lw) return fail(DSPARK_EINVAL, "layer weights %d is NULL", i);
  if (dm->variant & DSPARK_QK_NORM) {
    if (!lw->q_norm || !lw->k_norm) return fail(DSPARK_EINVAL, "layer %d: q_norm / k_norm is NULL", i);
    if (!aligned16(lw->q_norm) || !aligned16(lw->k_norm))
      return fail(DSPARK_EINVAL, "layer %d: q_norm / k_norm is not 16-byte aligned", i);
  }
  const void* ptrs[9] = {lw->attn_norm, lw->wq, lw->wk, lw->wv, lw->wo,
                         lw->ff_norm,   lw->w_gate, lw->w_up, lw->w_down};
  static const char* names[9] = {"attn_norm", "wq", "wk", "wv", "wo", "ff_norm", "w_gate", "w_up", "w_down"};
  for (int k = 0; k < 9; ++k) {
    if (!ptrs[k]) return fail(DSPARK_EINVAL, "layer %d: %s is NULL", i, names[k]);
    if (!aligned16(ptrs[k])) return fail(DSPARK_EINVAL, "layer %d: %s is not 16-byte aligned", i, names[k]);
  }
  return DSPARK_OK;
}

static dspark_status check_taps(const dspark_dims* dm, const void* const* taps, int64_t ld_tap, int64_t T) {
  if (!taps) return fail(DSPARK_EINVAL, "taps is NULL");
  if (ld_tap < dm->H) return fail(DSPARK_EINVAL, "ld_tap %lld < H %d", (long long)ld_tap, dm->H);
  const int esz = dm->dtype == DSPARK_BF16 ? 2 : 4;
  if ((ld_tap * esz) % 16 != 0) return fail(DSPARK_EINVAL, "ld_tap * element size must be a multiple of 16 bytes");
  // the projection kernels address a tap with 32-bit byte offsets
  if (T * ld_tap * esz >= (int64_t)1 << 32)
    return fail(DSPARK_EUNSUPPORTED, "a tap spans %lld bytes (T * ld_tap); at most 4 GiB is supported",
                (long long)(T * ld_tap * esz));
  for (int j = 0; j < dm->m; ++j) {
    if (T > 0 && !taps[j]) return fail(DSPARK_EINVAL, "taps[%d] is NULL", j);
    if (!aligned16(taps[j])) return fail(DSPARK_EINVAL, "taps[%d] is not 16-byte aligned", j);
  }
  return DSPARK_OK;
}

template <typename T>
static T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

// ---------------------------------------------------------------------------
// launch sequences
// ---------------------------------------------------------------------------
// Eq 2 projection: split-K fp32 partials of X . W_c^T into the workspace, or
// in one split Y = P * ctx_norm and its row sums (the RMSNorm row pass, or
// the row scales, run in the set-up launch).
static dspark_status run_ctx_gemm(const dspark_dims* dm, const Plan& p, const void* const* taps,
                                  int64_t ld_tap, const void* w_c, const float* ctx_norm, void* ws,
                                  hipStream_t s) {
  if (p.T == 0) return DSPARK_OK;
  const int d = dm->d, mH = dm->m * dm->H;
  ASegs a{};
  for (int j = 0; j < dm->m; ++j) a.seg[j] = taps[j];
  a.ld = ld_tap;
  a.seg_k = dm->H;
  a.nseg = dm->m;
  BMats b{};
  b.mat[0] = w_c;
  b.gain[0] = nullptr;
  b.n_per = d;
  b.nmat = 1;
  // W_c [d, m*H] is already the K-contiguous B operand
  CtxOut o;
  if (p.ctx.fused) {
    o.y = at<char>(ws, p.ppart);
    o.sums = at<float>(ws, p.ysum);
    o.g = ctx_norm;
    if (p.ctx.tail_row < p.T) o.tail_part = at<float>(ws, p.ptail);
  } else {
    o.part = at<float>(ws, p.ppart);
  }
  DSPARK_HIP(launch_gemm_ctx(dm->dtype, a, b, w_c, o, (int)p.T, d, mH, p.ctx, s));
  return DSPARK_OK;
}

// The K/V GEMM's B operand: W_K, W_V ([kvd, d] each) of `nl` layers with the
// attn_norm gains (none when the context rows enter W_K / W_V unnormalised).
static BMats kv_mats(const dspark_dims* dm, const dspark_layer_weights* layers, int nl, int kvd) {
  const bool plain = (dm->variant & DSPARK_PLAIN_CTX_KV) != 0;
  BMats b{};
  for (int i = 0; i < nl; ++i) {
    b.mat[2 * i] = layers[i].wk;
    b.mat[2 * i + 1] = layers[i].wv;
    b.gain[2 * i] = plain ? nullptr : layers[i].attn_norm;
    b.gain[2 * i + 1] = plain ? nullptr : layers[i].attn_norm;
  }
  b.n_per = kvd;
  b.nmat = 2 * nl;
  return b;
}

// k_norm and rotary positions on the context keys the K/V product just
// wrote (the variant's contextNormRope); nothing for the plain method.
static dspark_status run_k_post(const dspark_dims* dm, const Plan& p, const dspark_layer_weights* layers,
                                int nl, const KVDesc& kv, const int32_t* cu_dev, int A, hipStream_t s) {
  const bool qkn = (dm->variant & DSPARK_QK_NORM) != 0;
  if ((!qkn && dm->rope_theta <= 0.f) || p.T == 0) return DSPARK_OK;
  KPostArgs a;
  a.base = kv.base;
  a.Tpad = kv.Tpad;
  a.T = p.T;
  a.n_kv = p.nkv;
  a.hd = p.hd;
  a.n_layers = nl;
  for (int i = 0; i < nl; ++i) a.k_norm[i] = qkn ? layers[i].k_norm : nullptr;
  a.eps = dm->eps;
  a.rope = dm->rope_theta > 0.f;
  a.log2_theta = dm->rope_theta > 0.f ? std::log2((double)dm->rope_theta) : 0.0;
  a.cu = cu_dev;
  a.A = A;
  a.dst_row = kv.dst_row;
  a.cap = kv.seq_stride;
  DSPARK_HIP(launch_k_post(dm->dtype, a, s));
  return DSPARK_OK;
}

// Context K/V of `nl` layers from H_ctx (rinv, and for bf16 the stacked
// weights, already written by the set-up pass).
static dspark_status run_ctx_kv(const dspark_dims* dm, const Plan& p, const void* h_ctx, const float* rinv,
                                const dspark_layer_weights* layers, int nl, const KVDesc& kv, void* ws,
                                hipStream_t s) {
  if (p.T == 0) return DSPARK_OK;
  const int d = dm->d;
  const BMats b = kv_mats(dm, layers, nl, p.kvd);
  void* wkvt = dm->dtype == DSPARK_BF16 ? at<char>(ws, p.wkvt) : nullptr;
  DSPARK_HIP(launch_gemm_kv(dm->dtype, h_ctx, b, wkvt, rinv, kv, d, p.kvd, nl, s));
  return DSPARK_OK;
}

// The context K/V of a forward or a layer: packed rows in the workspace.
static KVDesc ws_kv(const dspark_dims* dm, const Plan& p, void* ws) {
  KVDesc kv{};
  kv.base = at<char>(ws, p.kv);
  kv.Tpad = p.Tpad;
  kv.T = (int)p.T;
  kv.hd = p.hd;
  kv.n_heads = p.nkv;
  return kv;
}

// A draft cache of A sequences with `cap` rows each; T = cached rows in
// total (the attention side) or the new rows of an append (the K/V side).
static KVDesc cache_kv(const dspark_dims* dm, const Plan& p, int A, int cap, void* cache,
                       const int32_t* dst_row) {
  KVDesc kv{};
  kv.base = cache;
  kv.Tpad = (int64_t)A * cap;
  kv.T = (int)p.T;
  kv.hd = p.hd;
  kv.n_heads = p.nkv;
  kv.seq_stride = cap;
  kv.dst_row = dst_row;
  return kv;
}

// Set-up roles shared by the block ops: tile plan and, for bf16, the stacked
// K/V weights.
static void setup_block_roles(const dspark_dims* dm, const Plan& p, int A, const int32_t* cu_dev,
                              void* ws, SetupArgs* sa) {
  sa->cu = cu_dev;
  sa->A = A;
  sa->chunk = p.chunk;
  sa->prefix = at<int32_t>(ws, p.prefix);

}

// The K/V product's stacked, gain-folded weights (bf16 only).
static void setup_prep_role(const dspark_dims* dm, const Plan& p, const dspark_layer_weights* layers, int nl,
                            void* ws, SetupArgs* sa) {
  if (dm->dtype == DSPARK_BF16 && p.T > 0) {
    sa->b = kv_mats(dm, layers, nl, p.kvd);
    sa->Bt = at<char>(ws, p.wkvt);
  }
}

// One draft layer on the block rows D (float32 [M][d]); writes D_next.
static dspark_status run_layer(const dspark_dims* dm, const Plan& p, int A, const int32_t* cu_dev,
                               const dspark_layer_weights& lw, int kv_layer, const KVDesc& kv,
                               const float* D, float* D_next, void* ws, hipStream_t s) {
  const int d = dm->d, ff = dm->ff, M = p.M, G = dm->gamma;
  const int dt = dm->dtype;
  float* Q = at<float>(ws, p.Q);
  float* Kd = at<float>(ws, p.Kd);
  float* Vd = at<float>(ws, p.Vd);
  float* E = at<float>(ws, p.E);
  float* GU = at<float>(ws, p.GU);

  // Q (pre-scaled for the base-2 softmax), K_d, V_d from RMSNorm(D; attn_norm).
  // The weights go in as kvd-row pieces: W_Q as d / kvd of them, then W_K, W_V.
  const float qscale = (float)(1.0 / std::sqrt((double)p.hd) * 1.4426950408889634);
  const bool qkn = (dm->variant & DSPARK_QK_NORM) != 0, rope = dm->rope_theta > 0.f;
  const size_t esz = dt == DSPARK_BF16 ? 2 : 4;
  const int kvd = p.kvd, npq = d / kvd;
  RowGemmArgs r{};
  r.X = D; r.ldx = d; r.M = M; r.K = d; r.N = d + 2 * kvd;
  r.g = lw.attn_norm; r.eps = dm->eps;
  for (int i = 0; i < npq; ++i) r.b.mat[i] = static_cast<const char*>(lw.wq) + (size_t)i * kvd * d * esz;
  r.b.mat[npq] = lw.wk; r.b.mat[npq + 1] = lw.wv;
  r.b.n_per = kvd; r.b.nmat = npq + 2;
  r.q = Q; r.kd = Kd; r.vd = Vd; r.d = d; r.kvd = kvd;
  r.qscale = (qkn || rope) ? 1.f : qscale;   // with head norms / rotary positions the post pass scales
  DSPARK_HIP(launch_rowgemm(dt, RP_RMSNORM, RE_QKV, r, s));
  if (qkn || rope) {   // the variant's noiseNormRope on the block rows
    QkPostArgs qa;
    qa.Q = Q; qa.Kd = Kd; qa.M = M; qa.gamma = G; qa.n_heads = dm->n_heads; qa.n_kv = p.nkv; qa.hd = p.hd;
    qa.q_norm = qkn ? lw.q_norm : nullptr;
    qa.k_norm = qkn ? lw.k_norm : nullptr;
    qa.eps = dm->eps;
    qa.rope = rope;
    qa.log2_theta = rope ? std::log2((double)dm->rope_theta) : 0.0;
    qa.cu = cu_dev;
    qa.qscale = qscale;
    DSPARK_HIP(launch_qk_post(qa, s));
  }
  // attention over [context ++ block]: split-K partials, then the combine
  // with the output projection, E = D + Attn Wo^T
  AttnArgs aa{};
  aa.Q = Q; aa.Kd = Kd; aa.Vd = Vd;
  aa.kv = kv;
  aa.n_heads = dm->n_heads;
  aa.layer = kv_layer;
  aa.cu = cu_dev;
  aa.prefix = at<int32_t>(ws, p.prefix);
  aa.A = A; aa.gamma = G; aa.chunk = p.chunk; aa.total_tiles = p.total_chunks;
  aa.part_o = at<float>(ws, p.po);
  aa.part_ml = at<float>(ws, p.pml);
  // the combine writes Attn; E = D + Attn Wo^T is a row GEMM (the heads'
  // shares summed in a fixed order: the block rows repeat bitwise)
  float* O = at<float>(ws, p.O);
  aa.attn = O;
  DSPARK_HIP(launch_attention(dt, aa, s));
  r = RowGemmArgs{};
  r.X = O; r.ldx = d; r.M = M; r.K = d; r.N = d;
  r.b.mat[0] = lw.wo; r.b.n_per = d; r.b.nmat = 1;
  r.res = D; r.out = E; r.ldo = d;
  DSPARK_HIP(launch_rowgemm(dt, RP_NONE, RE_RESID, r, s));
  // H = SiLU(Z Wgate^T) * (Z Wup^T), Z = RMSNorm(E; ff_norm)
  r = RowGemmArgs{};
  r.X = E; r.ldx = d; r.M = M; r.K = d; r.N = 2 * ff;
  r.g = lw.ff_norm; r.eps = dm->eps;
  r.b.mat[0] = lw.w_gate; r.b.mat[1] = lw.w_up; r.b.n_per = ff; r.b.nmat = 2;
  r.out = GU; r.ldo = ff;
  r.act = (dm->variant & DSPARK_GELU_FFN) ? 1 : 0;
  DSPARK_HIP(launch_rowgemm(dt, RP_RMSNORM, RE_SWIGLU, r, s));
  // D' = E + H Wdown^T
  r = RowGemmArgs{};
  r.X = GU; r.ldx = ff; r.M = M; r.K = ff; r.N = d;
  r.b.mat[0] = lw.w_down; r.b.n_per = d; r.b.nmat = 1;
  r.res = E; r.out = D_next; r.ldo = d;
  DSPARK_HIP(launch_rowgemm(dt, RP_NONE, RE_RESID, r, s));
  return DSPARK_OK;
}

}  // namespace dspark

using namespace dspark;

extern "C" {

// The set-up pass's Eq 2 row work. Split-K: sum the splits, H_ctx =
// RMSNorm(.; ctx_norm) into `h`, and rinv from the stored rows. Fused: rinv
// from the epilogue's row sums, and H_ctx into `h` only if `h` is given.
static void setup_eq2_role(const dspark_dims* dm, const Plan& p, const float* ctx_norm, void* h, float* rinv,
                           void* ws, SetupArgs* sa) {
  sa->T = p.T;
  sa->rinv = rinv;
  sa->rinv_one = (dm->variant & DSPARK_PLAIN_CTX_KV) != 0;
  sa->h = h;
  if (p.ctx.fused) {
    sa->rsum = at<float>(ws, p.ysum);
    sa->nts = dm->d / kCtxSumCols;
    sa->y = at<char>(ws, p.ppart);
    if (p.ctx.tail_row < p.T) {
      sa->tail_part = at<float>(ws, p.ptail);
      sa->tail_splits = p.ctx.tail_splits;
      sa->tail_from = p.ctx.tail_row;
      sa->g = ctx_norm;
    }
  } else {
    sa->part = at<float>(ws, p.ppart);
    sa->splits = p.ctx.splits;
    sa->g = ctx_norm;
  }
}

// The K/V product's A operand after Eq 2: H_ctx, or the fused path's Y rows.
static const void* kv_rows(const Plan& p, const void* h_ctx, void* ws) {
  return p.ctx.fused ? static_cast<const void*>(at<char>(ws, p.ppart)) : h_ctx;
}

size_t dspark_workspace_size(int32_t op, const dspark_dims* dims, int32_t A, const int32_t* cu_host) {
  if (op < DSPARK_OP_CTX_FUSE || op > DSPARK_OP_BLOCK_PROPOSE) {
    fail(DSPARK_EINVAL, "unknown op %d", op);
    return 0;
  }
  Plan p;
  if (make_plan(op, dims, A, cu_host, &p) != DSPARK_OK) return 0;
  return p.total;
}

dspark_status dspark_ctx_fuse(const dspark_dims* dims, int32_t A, const int32_t* cu_host,
                              const int32_t* cu_dev, const void* const* taps, int64_t ld_tap,
                              const void* w_c, const float* ctx_norm, void* h_ctx, void* ws,
                              size_t ws_bytes, void* stream) {
  Plan p;
  dspark_status st = make_plan(DSPARK_OP_CTX_FUSE, dims, A, cu_host, &p);
  if (st != DSPARK_OK) return st;
  NEED_PTR(cu_dev);
  st = check_taps(dims, taps, ld_tap, p.T);
  if (st != DSPARK_OK) return st;
  NEED_PTR(w_c);
  NEED_PTR(ctx_norm);
  if (p.T > 0) NEED_PTR(h_ctx);
  NEED_PTR(ws);
  if (ws_bytes < p.total)
    return fail(DSPARK_EWORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, p.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.T == 0) return DSPARK_OK;
  st = run_ctx_gemm(dims, p, taps, ld_tap, w_c, ctx_norm, ws, s);
  if (st != DSPARK_OK) return st;
  SetupArgs sa{};
  sa.d = dims->d;
  sa.eps = dims->eps;
  setup_eq2_role(dims, p, ctx_norm, h_ctx, nullptr, ws, &sa);
  DSPARK_HIP(launch_setup(dims->dtype, sa, s));
  return DSPARK_OK;
}

static dspark_status block_layer_impl(const dspark_dims* dims, int32_t A, const int32_t* cu_host,
                                      const int32_t* cu_dev, const void* h_ctx, const float* d_in,
                                      float* d_out, const dspark_layer_weights* lw, void* ws,
                                      size_t ws_bytes, void* stream, const Plan& p) {
  dspark_status st;
  NEED_PTR(cu_dev);
  if (p.T > 0) NEED_PTR(h_ctx);
  NEED_PTR(d_in);
  NEED_PTR(d_out);
  st = check_layer(lw, 0, dims);
  if (st != DSPARK_OK) return st;
  NEED_PTR(ws);
  if (ws_bytes < p.total)
    return fail(DSPARK_EWORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, p.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* rinv = at<float>(ws, p.rinv);
  SetupArgs sa{};
  sa.d = dims->d;
  sa.eps = dims->eps;
  setup_block_roles(dims, p, A, cu_dev, ws, &sa);
  setup_prep_role(dims, p, lw, 1, ws, &sa);
  if (p.T > 0) {
    sa.T = p.T;
    sa.h_in = h_ctx;
    sa.rinv = rinv;
    sa.rinv_one = (dims->variant & DSPARK_PLAIN_CTX_KV) != 0;
  }
  DSPARK_HIP(launch_setup(dims->dtype, sa, s));
  const KVDesc kv = ws_kv(dims, p, ws);
  st = run_ctx_kv(dims, p, h_ctx, rinv, lw, 1, kv, ws, s);
  if (st != DSPARK_OK) return st;
  st = run_k_post(dims, p, lw, 1, kv, cu_dev, A, s);
  if (st != DSPARK_OK) return st;
  return run_layer(dims, p, A, cu_dev, *lw, 0, kv, d_in, d_out, ws, s);
}

dspark_status dspark_block_layer(const dspark_dims* dims, int32_t A, const int32_t* cu_host,
                                 const int32_t* cu_dev, const void* h_ctx, const float* d_in,
                                 float* d_out, const dspark_layer_weights* lw, void* ws,
                                 size_t ws_bytes, void* stream) {
  Plan p;
  dspark_status st = make_plan(DSPARK_OP_BLOCK_LAYER, dims, A, cu_host, &p);
  if (st != DSPARK_OK) return st;
  return block_layer_impl(dims, A, cu_host, cu_dev, h_ctx, d_in, d_out, lw, ws, ws_bytes, stream, p);
}

dspark_status dspark_block_layer_noalloc(const dspark_dims* dims, int32_t A, const int32_t* cu_host,
                                         const int32_t* cu_dev, const void* h_ctx, const float* d_in,
                                         float* d_out, const dspark_layer_weights* lw, void* stream) {
  Plan p;
  dspark_status st = make_plan(DSPARK_OP_BLOCK_LAYER, dims, A, cu_host, &p);
  if (st != DSPARK_OK) return st;
  if (p.total > kNoAllocScratchBytes)
    return fail(DSPARK_EUNSUPPORTED,
                "this layer needs %zu bytes of scratch; dspark_block_layer_noalloc holds at most %zu "
                "(use dspark_block_layer with a workspace)",
                p.total, kNoAllocScratchBytes);
  void* ws = nullptr;
  DSPARK_HIP(noalloc_scratch(&ws));
  return block_layer_impl(dims, A, cu_host, cu_dev, h_ctx, d_in, d_out, lw, ws, kNoAllocScratchBytes,
                          stream, p);
}

// The forward's launch sequence; key_mask (nullable) marks the context rows
// that are keys (a padded batch); `pre` runs first on the stream (nullable).
static dspark_status forward_impl(const dspark_dims* dims, int32_t A, const int32_t* cu_dev,
                                  const void* const* taps, int64_t ld_tap, const void* w_c,
                                  const float* ctx_norm, const float* block_in, const float* block_pos,
                                  const dspark_layer_weights* layers, const float* out_norm, void* h_ctx_out,
                                  float* block_out, void* ws, size_t ws_bytes, void* stream, const Plan& p,
                                  const uint8_t* key_mask, int32_t* fill_cu, int32_t fill_L) {
  dspark_status st;
  if (!fill_cu) NEED_PTR(cu_dev);
  st = check_taps(dims, taps, ld_tap, p.T);
  if (st != DSPARK_OK) return st;
  NEED_PTR(w_c);
  NEED_PTR(ctx_norm);
  NEED_PTR(block_in);
  NEED_PTR(block_pos);
  if (!layers) return fail(DSPARK_EINVAL, "layers is NULL");
  for (int i = 0; i < dims->n_layers; ++i) {
    st = check_layer(&layers[i], i, dims);
    if (st != DSPARK_OK) return st;
  }
  OPT_PTR(out_norm);
  OPT_PTR(h_ctx_out);
  NEED_PTR(block_out);
  NEED_PTR(ws);
  if (ws_bytes < p.total)
    return fail(DSPARK_EWORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, p.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fill_cu) {   // the offsets b * L of a padded batch, written in the workspace
    DSPARK_HIP(launch_fill_offsets(fill_cu, A, fill_L, s));
    cu_dev = fill_cu;
  }
  // H_ctx: the caller's buffer, else (split-K Eq 2) the workspace's; the
  // fused Eq 2 path writes it only for the caller
  void* h_ctx = h_ctx_out ? h_ctx_out : (p.ctx.fused ? nullptr : at<char>(ws, p.hctx));
  float* rinv = at<float>(ws, p.rinv);
  float* Da = at<float>(ws, p.D);
  float* Db = at<float>(ws, p.D2);
  st = run_ctx_gemm(dims, p, taps, ld_tap, w_c, ctx_norm, ws, s);
  if (st != DSPARK_OK) return st;
  // Eq 2's row norm, K/V weight prep, tile plan and D0 = block_in + block_pos
  SetupArgs sa{};
  sa.d = dims->d;
  sa.eps = dims->eps;
  setup_block_roles(dims, p, A, cu_dev, ws, &sa);
  setup_prep_role(dims, p, layers, dims->n_layers, ws, &sa);
  sa.block_in = block_in;
  sa.block_pos = block_pos;
  sa.gamma = dims->gamma;
  sa.D0 = Da;
  if (p.T > 0) setup_eq2_role(dims, p, ctx_norm, h_ctx, rinv, ws, &sa);
  DSPARK_HIP(launch_setup(dims->dtype, sa, s));
  KVDesc kv = ws_kv(dims, p, ws);
  kv.key_mask = key_mask;
  st = run_ctx_kv(dims, p, kv_rows(p, h_ctx, ws), rinv, layers, dims->n_layers, kv, ws, s);
  if (st != DSPARK_OK) return st;
  st = run_k_post(dims, p, layers, dims->n_layers, kv, cu_dev, A, s);
  if (st != DSPARK_OK) return st;
  const int N = dims->n_layers;
  for (int i = 0; i < N; ++i) {
    float* Dn = (i == N - 1 && !out_norm) ? block_out : Db;
    st = run_layer(dims, p, A, cu_dev, layers[i], i, kv, Da, Dn, ws, s);
    if (st != DSPARK_OK) return st;
    std::swap(Da, Db);
  }
  if (out_norm)   // out = RMSNorm(D^N; out_norm)
    DSPARK_HIP(launch_block_rows(Da, nullptr, A, dims->gamma, dims->d, out_norm, dims->eps, nullptr,
                                 block_out, s));
  return DSPARK_OK;
}

dspark_status dspark_block_forward(const dspark_dims* dims, int32_t A, const int32_t* cu_host,
                                   const int32_t* cu_dev, const void* const* taps, int64_t ld_tap,
                                   const void* w_c, const float* ctx_norm, const float* block_in,
                                   const float* block_pos, const dspark_layer_weights* layers,
                                   const float* out_norm, void* h_ctx_out, float* block_out,
                                   void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  dspark_status st = make_plan(DSPARK_OP_BLOCK_FORWARD, dims, A, cu_host, &p);
  if (st != DSPARK_OK) return st;
  return forward_impl(dims, A, cu_dev, taps, ld_tap, w_c, ctx_norm, block_in, block_pos, layers, out_norm,
                      h_ctx_out, block_out, ws, ws_bytes, stream, p, nullptr, nullptr, 0);
}

// A padded batch: A sequences of L_ctx rows each (offsets b * L_ctx), with
// the key-padding mask; the plan of the equal-length packed batch plus the
// device copy of its offsets.
static dspark_status padded_plan(const dspark_dims* dims, int32_t A, int32_t L_ctx, Plan* p, size_t* cu_off) {
  if (A < 1) return fail(DSPARK_EINVAL, "A = %d < 1", A);
  if (L_ctx < 0 || (int64_t)A * L_ctx > (1ll << 30))
    return fail(L_ctx < 0 ? DSPARK_EINVAL : DSPARK_EUNSUPPORTED, "L_ctx = %d not supported", L_ctx);
  std::vector<int32_t> cu(A + 1);
  for (int b = 0; b <= A; ++b) cu[b] = b * L_ctx;
  dspark_status st = make_plan(DSPARK_OP_BLOCK_FORWARD, dims, A, cu.data(), p);
  if (st != DSPARK_OK) return st;
  *cu_off = p->total;
  p->total += align256((size_t)(A + 1) * 4);
  return DSPARK_OK;
}

size_t dspark_padded_workspace_size(const dspark_dims* dims, int32_t A, int32_t L_ctx) {
  Plan p;
  size_t cu_off = 0;
  if (padded_plan(dims, A, L_ctx, &p, &cu_off) != DSPARK_OK) return 0;
  return p.total;
}

dspark_status dspark_block_forward_padded(const dspark_dims* dims, int32_t A, int32_t L_ctx,
                                          const void* const* taps, int64_t ld_tap, const void* w_c,
                                          const float* ctx_norm, const uint8_t* ctx_mask,
                                          const float* block_in, const float* block_pos,
                                          const dspark_layer_weights* layers, const float* out_norm,
                                          void* h_ctx_out, float* block_out, void* ws, size_t ws_bytes,
                                          void* stream) {
  Plan p;
  size_t cu_off = 0;
  dspark_status st = padded_plan(dims, A, L_ctx, &p, &cu_off);
  if (st != DSPARK_OK) return st;
  if (p.T > 0 && !ctx_mask) return fail(DSPARK_EINVAL, "ctx_mask is NULL");
  if (!ws) return fail(DSPARK_EINVAL, "ws is NULL");
  return forward_impl(dims, A, nullptr, taps, ld_tap, w_c, ctx_norm, block_in, block_pos, layers, out_norm,
                      h_ctx_out, block_out, ws, ws_bytes, stream, p, ctx_mask, at<int32_t>(ws, cu_off), L_ctx);
}

dspark_status dspark_block_build(const dspark_dims* dims, int32_t A, const float* anchor_emb,
                                 const void* tok_proj, const float* mask_emb, float* block_in, void* stream) {
  dspark_status st = check_dims(dims, DSPARK_OP_BLOCK_LAYER);
  if (st != DSPARK_OK) return st;
  if (A < 1 || (int64_t)A * dims->gamma > 1024)
    return fail(A < 1 ? DSPARK_EINVAL : DSPARK_EUNSUPPORTED, "A = %d (A * gamma must be in [1, 1024])", A);
  if (dims->H > 16256) return fail(DSPARK_EUNSUPPORTED, "H %d above the supported 16256", dims->H);
  NEED_PTR(anchor_emb);
  NEED_PTR(tok_proj);
  if (dims->gamma > 1) NEED_PTR(mask_emb);
  NEED_PTR(block_in);
  DSPARK_HIP(launch_block_build(dims->dtype, anchor_emb, A, dims->H, tok_proj, mask_emb, dims->gamma, dims->d,
                                block_in, static_cast<hipStream_t>(stream)));
  return DSPARK_OK;
}

// ---------------------------------------------------------------------------
// incremental context: a draft cache, appends, and the block side over it
// ---------------------------------------------------------------------------
static dspark_status check_cache(const dspark_dims* dims, int32_t A, int32_t cap, size_t* bytes) {
  dspark_status st = check_dims(dims, DSPARK_OP_BLOCK_PROPOSE);
  if (st != DSPARK_OK) return st;
  if (A < 1) return fail(DSPARK_EINVAL, "A = %d < 1", A);
  if (cap < 64 || cap % 64 != 0) return fail(DSPARK_EINVAL, "cap %d must be a positive multiple of 64", cap);
  if ((int64_t)A * cap > (int64_t)INT32_MAX)
    return fail(DSPARK_EUNSUPPORTED, "A * cap = %lld rows; at most 2^31 - 1 are supported",
                (long long)A * cap);
  const size_t esz = dims->dtype == DSPARK_BF16 ? 2 : 4;
  const int nkv = dims->n_kv_heads == 0 ? dims->n_heads : dims->n_kv_heads;
  *bytes = (size_t)dims->n_layers * 2 * (size_t)A * cap * nkv * (dims->d / dims->n_heads) * esz;
  return DSPARK_OK;
}

size_t dspark_cache_bytes(const dspark_dims* dims, int32_t A, int32_t cap) {
  size_t bytes = 0;
  if (check_cache(dims, A, cap, &bytes) != DSPARK_OK) return 0;
  return bytes;
}

dspark_status dspark_cache_reset(const dspark_dims* dims, int32_t A, int32_t cap, void* cache,
                                 void* stream) {
  size_t bytes = 0;
  dspark_status st = check_cache(dims, A, cap, &bytes);
  if (st != DSPARK_OK) return st;
  NEED_PTR(cache);
  SetupArgs sa{};
  sa.d = dims->d;
  sa.zero = static_cast<float*>(cache);
  sa.zero_n = (int64_t)(bytes / 4);
  DSPARK_HIP(launch_setup(dims->dtype, sa, static_cast<hipStream_t>(stream)));
  return DSPARK_OK;
}

dspark_status dspark_ctx_append(const dspark_dims* dims, int32_t A, int32_t cap, const int32_t* ncu_host,
                                const int32_t* ncu_dev, const int32_t* pos_host, const int32_t* pos_dev,
                                const void* const* taps, int64_t ld_tap, const void* w_c,
                                const float* ctx_norm, const dspark_layer_weights* layers, void* cache,
                                void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  dspark_status st = make_plan(DSPARK_OP_CTX_APPEND, dims, A, ncu_host, &p);
  if (st != DSPARK_OK) return st;
  size_t bytes = 0;
  st = check_cache(dims, A, cap, &bytes);
  if (st != DSPARK_OK) return st;
  if (!pos_host) return fail(DSPARK_EINVAL, "pos_host is NULL");
  for (int b = 0; b < A; ++b) {
    const int64_t n = ncu_host[b + 1] - ncu_host[b];
    if (pos_host[b] < 0 || (int64_t)pos_host[b] + n > cap)
      return fail(DSPARK_EINVAL, "sequence %d: %lld rows at position %d do not fit a cache of %d rows", b,
                  (long long)n, pos_host[b], cap);
  }
  NEED_PTR(ncu_dev);
  NEED_PTR(pos_dev);
  st = check_taps(dims, taps, ld_tap, p.T);
  if (st != DSPARK_OK) return st;
  NEED_PTR(w_c);
  NEED_PTR(ctx_norm);
  if (!layers) return fail(DSPARK_EINVAL, "layers is NULL");
  for (int i = 0; i < dims->n_layers; ++i) {
    st = check_layer(&layers[i], i, dims);
    if (st != DSPARK_OK) return st;
  }
  NEED_PTR(cache);
  NEED_PTR(ws);
  if (ws_bytes < p.total)
    return fail(DSPARK_EWORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, p.total);
  if (p.T == 0) return DSPARK_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_ctx_gemm(dims, p, taps, ld_tap, w_c, ctx_norm, ws, s);
  if (st != DSPARK_OK) return st;
  // Eq 2's row norm of the new rows, the stacked K/V weights, the row map
  SetupArgs sa{};
  sa.d = dims->d;
  sa.eps = dims->eps;
  sa.A = A;
  setup_prep_role(dims, p, layers, dims->n_layers, ws, &sa);
  void* h_new = p.ctx.fused ? nullptr : at<char>(ws, p.hctx);
  setup_eq2_role(dims, p, ctx_norm, h_new, at<float>(ws, p.rinv), ws, &sa);
  sa.ncu = ncu_dev;
  sa.pos = pos_dev;
  sa.cap = cap;
  sa.map_T = p.T;
  sa.dst_row = at<int32_t>(ws, p.rowmap);
  DSPARK_HIP(launch_setup(dims->dtype, sa, s));
  const KVDesc kv = cache_kv(dims, p, A, cap, cache, at<int32_t>(ws, p.rowmap));
  st = run_ctx_kv(dims, p, kv_rows(p, h_new, ws), at<float>(ws, p.rinv), layers, dims->n_layers, kv, ws, s);
  if (st != DSPARK_OK) return st;
  return run_k_post(dims, p, layers, dims->n_layers, kv, ncu_dev, A, s);
}

dspark_status dspark_block_propose(const dspark_dims* dims, int32_t A, int32_t cap, const int32_t* cu_host,
                                   const int32_t* cu_dev, const void* cache, const float* block_in,
                                   const float* block_pos, const dspark_layer_weights* layers,
                                   const float* out_norm, float* block_out, void* ws, size_t ws_bytes,
                                   void* stream) {
  Plan p;
  dspark_status st = make_plan(DSPARK_OP_BLOCK_PROPOSE, dims, A, cu_host, &p);
  if (st != DSPARK_OK) return st;
  size_t bytes = 0;
  st = check_cache(dims, A, cap, &bytes);
  if (st != DSPARK_OK) return st;
  for (int b = 0; b < A; ++b)
    if (cu_host[b + 1] - cu_host[b] > cap)
      return fail(DSPARK_EINVAL, "sequence %d has %d cached rows, more than the cache's %d", b,
                  cu_host[b + 1] - cu_host[b], cap);
  NEED_PTR(cu_dev);
  NEED_PTR(cache);
  NEED_PTR(block_in);
  NEED_PTR(block_pos);
  if (!layers) return fail(DSPARK_EINVAL, "layers is NULL");
  for (int i = 0; i < dims->n_layers; ++i) {
    st = check_layer(&layers[i], i, dims);
    if (st != DSPARK_OK) return st;
  }
  OPT_PTR(out_norm);
  NEED_PTR(block_out);
  NEED_PTR(ws);
  if (ws_bytes < p.total)
    return fail(DSPARK_EWORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, p.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* Da = at<float>(ws, p.D);
  float* Db = at<float>(ws, p.D2);
  // tile plan, cleared accumulators, D0 = block_in + block_pos
  SetupArgs sa{};
  sa.d = dims->d;
  sa.eps = dims->eps;
  setup_block_roles(dims, p, A, cu_dev, ws, &sa);
  sa.block_in = block_in;
  sa.block_pos = block_pos;
  sa.gamma = dims->gamma;
  sa.D0 = Da;
  DSPARK_HIP(launch_setup(dims->dtype, sa, s));
  const KVDesc kv = cache_kv(dims, p, A, cap, const_cast<void*>(cache), nullptr);
  const int N = dims->n_layers;
  for (int i = 0; i < N; ++i) {
    float* Dn = (i == N - 1 && !out_norm) ? block_out : Db;
    st = run_layer(dims, p, A, cu_dev, layers[i], i, kv, Da, Dn, ws, s);
    if (st != DSPARK_OK) return st;
    std::swap(Da, Db);
  }
  if (out_norm)
    DSPARK_HIP(launch_block_rows(Da, nullptr, A, dims->gamma, dims->d, out_norm, dims->eps, nullptr,
                                 block_out, s));
  return DSPARK_OK;
}

// ---------------------------------------------------------------------------
// Markov head, confidence head, greedy draft loop
// ---------------------------------------------------------------------------
struct MarkovPlan {
  size_t E1 = 0, pv = 0, pi = 0, total = 0;
};

static dspark_status markov_plan(const dspark_dims* dims, int32_t A, int32_t vocab, int32_t rank,
                                 MarkovPlan* mp) {
  if (!dims) return fail(DSPARK_EINVAL, "dims is NULL");
  if (dims->dtype != DSPARK_F32 && dims->dtype != DSPARK_BF16)
    return fail(DSPARK_EUNSUPPORTED, "dtype %d not supported (0 = f32, 1 = bf16)", dims->dtype);
  if (dims->d <= 0 || dims->d % 4 != 0) return fail(DSPARK_EINVAL, "d %d must be a positive multiple of 4", dims->d);
  if (dims->gamma < 1 || dims->gamma > kMaxGamma)
    return fail(DSPARK_EUNSUPPORTED, "gamma %d not in [1, %d]", dims->gamma, kMaxGamma);
  if (A < 1 || (int64_t)A * dims->gamma > 1024)
    return fail(A < 1 ? DSPARK_EINVAL : DSPARK_EUNSUPPORTED, "A = %d (A * gamma must be in [1, 1024])", A);
  if (vocab < 8 || vocab % 8 != 0) return fail(DSPARK_EUNSUPPORTED, "vocab %d must be a multiple of 8", vocab);
  if ((int64_t)dims->gamma * vocab >= ((int64_t)1 << 31))
    return fail(DSPARK_EUNSUPPORTED, "gamma * vocab = %lld too large", (long long)dims->gamma * vocab);
  if (rank < 64 || rank % 64 != 0 || rank > 16256)
    return fail(DSPARK_EUNSUPPORTED, "rank %d must be a multiple of 64 in [64, 16256]", rank);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  const MarkovGrid mg = markov_grid(dims->dtype, vocab, rank, A);
  const int P = mg.P;
  if (mg.mfma) {
    // two positions' (value, index) partials; the kernels read w1 rows directly
    mp->pv = take((size_t)2 * A * P * 8);
  } else {
    mp->E1 = take((size_t)A * rank * 4);
    mp->pv = take((size_t)A * P * 4);
    mp->pi = take((size_t)A * P * 4);
  }
  mp->total = off;
  return DSPARK_OK;
}

size_t dspark_markov_workspace_size(const dspark_dims* dims, int32_t A, int32_t vocab, int32_t rank) {
  MarkovPlan mp;
  if (markov_plan(dims, A, vocab, rank, &mp) != DSPARK_OK) return 0;
  return mp.total;
}

dspark_status dspark_markov_draft(const dspark_dims* dims, int32_t A, int32_t vocab, int32_t rank,
                                  const float* block, const float* base_logits, const int32_t* anchor,
                                  const void* w1, const void* w2, const float* conf_w, const float* conf_b,
                                  int32_t* tokens, float* conf, float* draft_logits, void* ws,
                                  size_t ws_bytes, void* stream) {
  MarkovPlan mp;
  dspark_status st = markov_plan(dims, A, vocab, rank, &mp);
  if (st != DSPARK_OK) return st;
  NEED_PTR(block);
  NEED_PTR(base_logits);
  NEED_PTR(anchor);
  NEED_PTR(w1);
  NEED_PTR(w2);
  NEED_PTR(conf_w);
  if (!conf_b) return fail(DSPARK_EINVAL, "conf_b is NULL");
  NEED_PTR(tokens);
  NEED_PTR(conf);
  NEED_PTR(draft_logits);
  NEED_PTR(ws);
  if (ws_bytes < mp.total)
    return fail(DSPARK_EWORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, mp.total);
  MarkovArgs a;
  a.A = A;
  a.gamma = dims->gamma;
  a.d = dims->d;
  a.vocab = vocab;
  a.rank = rank;
  a.block = block;
  a.base_logits = base_logits;
  a.anchor = anchor;
  a.w1 = w1;
  a.w2 = w2;
  a.conf_w = conf_w;
  a.conf_b = conf_b;
  a.tokens = tokens;
  a.conf = conf;
  a.logits = draft_logits;
  a.E1 = at<float>(ws, mp.E1);
  a.part_v = at<float>(ws, mp.pv);
  a.part_i = at<int32_t>(ws, mp.pi);
  DSPARK_HIP(launch_markov(dims->dtype, a, static_cast<hipStream_t>(stream)));
  return DSPARK_OK;
}

int32_t dspark_plan_info(int32_t op, const dspark_dims* dims, int32_t A, const int32_t* cu_host,
                         int64_t* out, int32_t n) {
  if (op < DSPARK_OP_CTX_FUSE || op > DSPARK_OP_BLOCK_PROPOSE) {
    fail(DSPARK_EINVAL, "unknown op %d", op);
    return 0;
  }
  if (!out || n < 1) {
    fail(DSPARK_EINVAL, "out is NULL or n < 1");
    return 0;
  }
  Plan p;
  if (make_plan(op, dims, A, cu_host, &p) != DSPARK_OK) return 0;
  const bool eq2 = op == DSPARK_OP_CTX_FUSE || op == DSPARK_OP_BLOCK_FORWARD || op == DSPARK_OP_CTX_APPEND;
  const int64_t v[DSPARK_PLAN_COUNT] = {p.ctx.splits, p.ctx.k_per_split, p.chunk, p.total_chunks,
                                        p.chunk != 64 ? 1 : 0, (int64_t)p.total, eq2 && p.ctx.fused ? 1 : 0,
                                        eq2 && p.ctx.fused ? p.T - p.ctx.tail_row : 0};
  const int k = std::min<int32_t>(n, DSPARK_PLAN_COUNT);
  for (int i = 0; i < k; ++i) out[i] = v[i];
  return k;
}

const char* dspark_last_error(void) { return g_err.c_str(); }

const char* dspark_version(void) { return "dspark-mi355x 0.1.0 (gfx950)"; }

int32_t dspark_kernel_kinds(void) { return K_COUNT; }

const char* dspark_kernel_name(int32_t kind) { return kernel_name(kind); }

dspark_status dspark_trace_begin(uint64_t mask, int32_t capacity) {
  Trace& t = g_trace;
  if (capacity < 1) return fail(DSPARK_EINVAL, "capacity must be >= 1");
  if ((int)t.ev.size() < 2 * capacity) {
    const size_t old = t.ev.size();
    t.ev.resize(2 * capacity);
    for (size_t i = old; i < t.ev.size(); ++i) DSPARK_HIP(hipEventCreate(&t.ev[i]));
  }
  t.kind.assign(capacity, -1);
  t.mask = mask;
  t.cap = capacity;
  t.used = 0;
  t.open = false;
  t.on = true;
  return DSPARK_OK;
}

dspark_status dspark_trace_end(double* total_ms, int64_t* launches, int32_t n_kinds) {
  Trace& t = g_trace;
  t.on = false;
  if (!total_ms || !launches) return fail(DSPARK_EINVAL, "output arrays are NULL");
  for (int k = 0; k < n_kinds; ++k) {
    total_ms[k] = 0.0;
    launches[k] = 0;
  }
  for (int i = 0; i < t.used; ++i) {
    DSPARK_HIP(hipEventSynchronize(t.ev[2 * i + 1]));
    float ms = 0.f;
    DSPARK_HIP(hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]));
    const int k = t.kind[i];
    if (k >= 0 && k < n_kinds) {
      total_ms[k] += ms;
      launches[k] += 1;
    }
  }
  t.used = 0;
  return DSPARK_OK;
}

}  // extern "C"
