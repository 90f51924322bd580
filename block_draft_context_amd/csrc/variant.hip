// Per-head norms and rotary positions of the layer variant that the page
// "src/dspark-runtime.js" runs: its noiseNormRope kernel applies q_norm /
// k_norm and rotary positions to the block's queries and keys, and its
// contextNormRope kernel k_norm and rotary positions to the context keys
// before they are stored. module-dflash.ts has neither.
//
//   head norm   x_h <- x_h * (mean_c x_h[c]^2 + eps)^(-1/2) * g       (g: [hd])
//   RoPE        (x[c], x[c + hd/2]) <- (x[c] cos a - x[c + hd/2] sin a,
//                                       x[c + hd/2] cos a + x[c] sin a),
//               a = pos * theta^(-2c/hd), c < hd/2
// A context row's position is its index in its sequence; block row j of
// sequence b sits at L_b + j, right after the sequence's context. The angle
// is formed and reduced to [-pi, pi] in double precision before the float
// sine and cosine, so long positions keep float accuracy.
#include "common.h"
#include "kernels.h"
#include "kv_layout.h"

namespace dspark {

DSPARK_DEV void rope_sincos(int64_t pos, int c, int hd, double log2_theta, float& sn, float& cs) {
  const double inv = exp2(-2.0 * (double)c / (double)hd * log2_theta);
  double ang = (double)pos * inv;
  ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
  sincosf((float)ang, &sn, &cs);
}

// Block rows: grid (M, n_heads + n_kv), one wave per (row, head); lane c < hd/2
// holds the pair (c, c + hd/2). Queries are scaled by qscale last.
__global__ __launch_bounds__(64) void qk_post_kernel(float* __restrict__ Q, float* __restrict__ Kd, int gamma,
                                                     int n_heads, int n_kv, int hd, const float* __restrict__ q_norm,
                                                     const float* __restrict__ k_norm, float eps, int rope,
                                                     double log2_theta, const int32_t* __restrict__ cu,
                                                     float qscale) {
  const int m = blockIdx.x, hh = blockIdx.y, lane = threadIdx.x;
  const bool isq = hh < n_heads;
  const int head = isq ? hh : hh - n_heads;
  float* x = isq ? Q + (int64_t)m * n_heads * hd + head * hd : Kd + (int64_t)m * n_kv * hd + head * hd;
  const float* g = isq ? q_norm : k_norm;
  const int half = hd / 2;
  const bool on = lane < half;
  float x1 = on ? x[lane] : 0.f, x2 = on ? x[lane + half] : 0.f;
  if (g) {
    const float ss = wave_sum(x1 * x1 + x2 * x2);
    const float r = rsqrtf(ss / (float)hd + eps);
    if (on) {
      x1 *= r * g[lane];
      x2 *= r * g[lane + half];
    }
  }
  if (rope && on) {
    const int b = m / gamma, j = m % gamma;
    const int64_t pos = (int64_t)(cu[b + 1] - cu[b]) + j;
    float sn, cs;
    rope_sincos(pos, lane, hd, log2_theta, sn, cs);
    const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
    x1 = y1;
    x2 = y2;
  }
  if (isq) {
    x1 *= qscale;
    x2 *= qscale;
  }
  if (on) {
    x[lane] = x1;
    x[lane + half] = x2;
  }
}

hipError_t launch_qk_post(const QkPostArgs& a, hipStream_t s) {
  trace_pre(K_ROWGEMM, s);
  qk_post_kernel<<<dim3(a.M, a.n_heads + a.n_kv), 64, 0, s>>>(a.Q, a.Kd, a.gamma, a.n_heads, a.n_kv, a.hd,
                                                             a.q_norm, a.k_norm, a.eps, a.rope, a.log2_theta,
                                                             a.cu, a.qscale);
  trace_post(K_ROWGEMM, s);
  return hipGetLastError();
}

// Context keys in place, in the attention layout: grid (ceil(T / 64), n_kv,
// n_layers), lane = one of the T rows the K/V product wrote (slab row
// dst_row[r] in a cache, else r). The lane reads the row's hd values (hd / E
// vectors, each a 1 KiB run across the wave), normalises, rotates and
// stores them.
template <typename S, int HD>
__global__ __launch_bounds__(64) void k_post_kernel(KPostArgs a) {
  using L = KVLayout<S>;
  constexpr int E = L::E, NV = HD / E;
  const int64_t r = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (r >= a.T) return;
  const int kvh = blockIdx.y, layer = blockIdx.z;
  int64_t t, pos;
  if (a.dst_row) {
    t = a.dst_row[r];
    pos = t % a.cap;
  } else {
    t = r;
    int lo = 0, hi = a.A - 1;   // the sequence owning row r: the last b with cu[b] <= r
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu[mid] <= r) lo = mid; else hi = mid - 1;
    }
    pos = r - a.cu[lo];
  }
  S* K = static_cast<S*>(a.base) + L::head_base(layer, 0, kvh, a.n_kv, a.Tpad, HD);
  float x[HD];
  u32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = ld16(K + L::k_off(t, i * E, HD));
#pragma unroll
  for (int i = 0; i < NV; ++i) Vec16<S>::unpack(v[i], x + i * E);
  const float* g = a.k_norm[layer];
  if (g) {
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < HD; ++c) ss += x[c] * x[c];
    const float rs = rsqrtf(ss / (float)HD + a.eps);
#pragma unroll
    for (int c = 0; c < HD; ++c) x[c] *= rs * g[c];
  }
  if (a.rope) {
#pragma unroll
    for (int c = 0; c < HD / 2; ++c) {
      float sn, cs;
      rope_sincos(pos, c, HD, a.log2_theta, sn, cs);
      const float x1 = x[c], x2 = x[c + HD / 2];
      x[c] = x1 * cs - x2 * sn;
      x[c + HD / 2] = x2 * cs + x1 * sn;
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    u32x4 o;
    if constexpr (sizeof(S) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = pack_bf16x2(x[i * E + 2 * w], x[i * E + 2 * w + 1]);
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = __float_as_uint(x[i * E + w]);
    }
    st16(K + L::k_off(t, i * E, HD), o);
  }
}

hipError_t launch_k_post(int dtype, const KPostArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  dim3 grid((unsigned)((a.T + 63) / 64), a.n_kv, a.n_layers);
  trace_pre(K_GEMM_KV, s);
#define DSPARK_KP(SS, H)                                                       \
  if (a.hd == H) k_post_kernel<SS, H><<<grid, 64, 0, s>>>(a);
  if (dtype == 1) {
    DSPARK_KP(bf16, 32) DSPARK_KP(bf16, 64) DSPARK_KP(bf16, 128)
  } else {
    DSPARK_KP(float, 32) DSPARK_KP(float, 64) DSPARK_KP(float, 128)
  }
#undef DSPARK_KP
  trace_post(K_GEMM_KV, s);
  return hipGetLastError();
}

}  // namespace dspark
