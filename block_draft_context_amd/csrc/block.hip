// Block-side work of Eq 3 (#layer of module-dflash.ts) on the A*gamma block
// rows, kept in float32 between kernels:
//   U = RMSNorm(D; attn_norm);  Q, K_d, V_d = U Wq, U Wk, U Wv
//   E = D + Attn Wo;  Z = RMSNorm(E; ff_norm)
//   D' = E + (SiLU(Z Wgate) * (Z Wup)) Wdown
// With at most a few dozen rows these products are weight-streaming bound, so
// each one is a split-K "skinny" GEMM: every workgroup streams a 128-column x
// KS-row slab of the [in, out] weight once (16-byte loads along the output
// columns), multiplies it with the matching slab of the rows held in LDS, and
// writes a float32 partial; small row kernels then reduce the partials and
// apply the residual, the norms and the SiLU gate.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace dspark {

constexpr int SK_TN = 16;            // threads along columns (8 columns each)
constexpr int SK_TK = 16;            // thread rows along K
constexpr int SK_COLS = 8 * SK_TN;   // 128 columns per workgroup
constexpr int SK_MT = 8;             // block rows per pass

// K rows per thread (RPT) and K slabs (splits) so that (N/128) * splits
// covers the GPU a few times over; the last slab may be partial.
SkinnyPlan skinny_plan(int M, int N, int K) {
  (void)M;
  const int nb = N / SK_COLS;
  const int want = (1024 + nb - 1) / nb;
  int rpt = 1;
  while (rpt < 16 && (int64_t)SK_TK * rpt * want < K) rpt *= 2;
  SkinnyPlan p;
  p.rpt = rpt;
  p.splits = (K + SK_TK * rpt - 1) / (SK_TK * rpt);
  return p;
}

template <typename S, int RPT>
__global__ __launch_bounds__(256) void skinny_kernel(const float* __restrict__ X, int M, int K,
                                                     BMats b, int N, float* __restrict__ part) {
  constexpr int KS = SK_TK * RPT;
  __shared__ __attribute__((aligned(16))) float xs[KS][SK_MT];
  __shared__ float red[SK_TK][SK_MT][SK_COLS + 4];
  const int tid = threadIdx.x;
  const int tn = tid % SK_TN, tk = tid / SK_TN;
  const int n0 = blockIdx.x * SK_COLS;
  const int z = blockIdx.y;
  const int kbase = z * KS;
  const int mi = n0 / b.n_per;
  const int c0 = n0 % b.n_per + tn * 8;
  const S* __restrict__ W = static_cast<const S*>(b.mat[mi]);

  // this thread's weights: rows kbase + tk + SK_TK * r (< K), 8 columns
  float w[RPT][8];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int k = kbase + tk + SK_TK * r;
    if (k < K) {
      const S* p = W + (int64_t)k * b.n_per + c0;
      Vec16<S>::unpack(ld16(p), w[r]);
      if constexpr (sizeof(S) == 4) Vec16<S>::unpack(ld16(p + 4), w[r] + 4);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) w[r][c] = 0.f;
    }
  }

  for (int m0 = 0; m0 < M; m0 += SK_MT) {
    __syncthreads();
    for (int i = tid; i < KS * SK_MT; i += 256) {
      const int kk = i / SK_MT, mm = i % SK_MT;
      xs[kk][mm] = (m0 + mm < M && kbase + kk < K) ? X[(int64_t)(m0 + mm) * K + kbase + kk] : 0.f;
    }
    __syncthreads();
    float acc[SK_MT][8];
#pragma unroll
    for (int mm = 0; mm < SK_MT; ++mm)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[mm][c] = 0.f;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int kk = tk + SK_TK * r;
      const f32x4 xa = *reinterpret_cast<const f32x4*>(&xs[kk][0]);
      const f32x4 xb = *reinterpret_cast<const f32x4*>(&xs[kk][4]);
      const float xv[8] = {xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};
#pragma unroll
      for (int mm = 0; mm < SK_MT; ++mm)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[mm][c] = fmaf(xv[mm], w[r][c], acc[mm][c]);
    }
#pragma unroll
    for (int mm = 0; mm < SK_MT; ++mm)
#pragma unroll
      for (int c = 0; c < 8; ++c) red[tk][mm][tn * 8 + c] = acc[mm][c];
    __syncthreads();
    for (int i = tid; i < SK_MT * SK_COLS; i += 256) {
      const int mm = i / SK_COLS, cc = i % SK_COLS;
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < SK_TK; ++q) v += red[q][mm][cc];
      if (m0 + mm < M) part[((int64_t)z * M + m0 + mm) * N + n0 + cc] = v;
    }
  }
}

hipError_t launch_skinny(int dtype, const float* X, int M, int K, const BMats& b, int N, int splits,
                         float* part, hipStream_t s) {
  const SkinnyPlan plan = skinny_plan(M, N, K);
  if (plan.splits != splits) return hipErrorInvalidValue;
  const int rpt = plan.rpt;
  dim3 grid(N / SK_COLS, splits);
  trace_pre(K_SKINNY, s);
  bool ok = true;
#define DSPARK_SK(R)                                                                     \
  case R:                                                                                \
    if (dtype == 1)                                                                      \
      skinny_kernel<bf16, R><<<grid, 256, 0, s>>>(X, M, K, b, N, part);                  \
    else                                                                                 \
      skinny_kernel<float, R><<<grid, 256, 0, s>>>(X, M, K, b, N, part);                 \
    break;
  switch (rpt) {
    DSPARK_SK(1) DSPARK_SK(2) DSPARK_SK(4) DSPARK_SK(8) DSPARK_SK(16)
    default: ok = false;
  }
#undef DSPARK_SK
  trace_post(K_SKINNY, s);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// reductions of the split-K partials
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void finish_qkv_kernel(const float* __restrict__ part, int splits,
                                                         int M, int d, float qscale,
                                                         float* __restrict__ Q, float* __restrict__ Kd,
                                                         float* __restrict__ Vd) {
  const int64_t n3 = 3 * (int64_t)d;
  const int64_t total = (int64_t)M * n3;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    float v = 0.f;
    for (int z = 0; z < splits; ++z) v += part[(int64_t)z * total + i];
    const int64_t r = i / n3, c = i % n3;
    if (c < d) Q[r * d + c] = v * qscale;
    else if (c < 2 * d) Kd[r * d + c - d] = v;
    else Vd[r * d + c - 2 * d] = v;
  }
}

hipError_t launch_finish_qkv(const float* part, int splits, int M, int d, float qscale, float* Q,
                             float* Kd, float* Vd, hipStream_t s) {
  const int64_t total = (int64_t)M * 3 * d;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 1024);
  trace_pre(K_FINISH_QKV, s);
  finish_qkv_kernel<<<blocks, 256, 0, s>>>(part, splits, M, d, qscale, Q, Kd, Vd);
  trace_post(K_FINISH_QKV, s);
  return hipGetLastError();
}

// one workgroup per row: full = res + sum_z part; normed = RMSNorm(full; g)
__global__ __launch_bounds__(256) void finish_res_kernel(const float* __restrict__ part, int splits,
                                                         int M, int d, const float* __restrict__ res,
                                                         const float* __restrict__ g, float eps,
                                                         float* __restrict__ full,
                                                         float* __restrict__ normed) {
  __shared__ float wsum[4];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  float ss = 0.f;
  for (int c = tid; c < d; c += 256) {
    float v = res[(int64_t)r * d + c];
    for (int z = 0; z < splits; ++z) v += part[((int64_t)z * M + r) * d + c];
    full[(int64_t)r * d + c] = v;
    ss += v * v;
  }
  if (!normed) return;
  ss = wave_sum(ss);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float tot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  const float sc = rsqrtf(tot / (float)d + eps);
  for (int c = tid; c < d; c += 256) normed[(int64_t)r * d + c] = full[(int64_t)r * d + c] * sc * g[c];
}

hipError_t launch_finish_res(const float* part, int splits, int M, int d, const float* res,
                             const float* g, float eps, float* full, float* normed, hipStream_t s) {
  trace_pre(K_FINISH_RES, s);
  finish_res_kernel<<<M, 256, 0, s>>>(part, splits, M, d, res, g, eps, full, normed);
  trace_post(K_FINISH_RES, s);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void finish_swiglu_kernel(const float* __restrict__ part, int splits,
                                                            int M, int ff, float* __restrict__ hid) {
  const int64_t n2 = 2 * (int64_t)ff;
  const int64_t total = (int64_t)M * ff;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / ff, c = i % ff;
    float gt = 0.f, up = 0.f;
    for (int z = 0; z < splits; ++z) {
      const float* p = part + ((int64_t)z * M + r) * n2;
      gt += p[c];
      up += p[ff + c];
    }
    hid[i] = gt / (1.f + __expf(-gt)) * up;
  }
}

hipError_t launch_finish_swiglu(const float* part, int splits, int M, int ff, float* hid,
                                hipStream_t s) {
  const int64_t total = (int64_t)M * ff;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 1024);
  trace_pre(K_FINISH_SWIGLU, s);
  finish_swiglu_kernel<<<blocks, 256, 0, s>>>(part, splits, M, ff, hid);
  trace_post(K_FINISH_SWIGLU, s);
  return hipGetLastError();
}

// D0[b, j] = block_in[b, j] + block_pos[j] (block_pos and D0 nullable);
// U0 = RMSNorm(D0; g). One row per workgroup.
__global__ __launch_bounds__(256) void block_init_kernel(const float* __restrict__ bin,
                                                         const float* __restrict__ bpos, int gamma,
                                                         int d, const float* __restrict__ g, float eps,
                                                         float* __restrict__ D0, float* __restrict__ U0) {
  __shared__ float wsum[4];
  const int r = blockIdx.x;
  const int j = r % gamma;
  const int tid = threadIdx.x;
  float ss = 0.f;
  for (int c = tid; c < d; c += 256) {
    float v = bin[(int64_t)r * d + c];
    if (bpos) v += bpos[(int64_t)j * d + c];
    if (D0) D0[(int64_t)r * d + c] = v;
    ss += v * v;
  }
  if (!U0) return;
  ss = wave_sum(ss);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float sc = rsqrtf((wsum[0] + wsum[1] + wsum[2] + wsum[3]) / (float)d + eps);
  for (int c = tid; c < d; c += 256) {
    float v = bin[(int64_t)r * d + c];
    if (bpos) v += bpos[(int64_t)j * d + c];
    U0[(int64_t)r * d + c] = v * sc * g[c];
  }
}

hipError_t launch_block_init(const float* block_in, const float* block_pos, int A, int gamma, int d,
                             const float* g, float eps, float* D0, float* U0, hipStream_t s) {
  trace_pre(K_BLOCK_INIT, s);
  block_init_kernel<<<A * gamma, 256, 0, s>>>(block_in, block_pos, gamma, d, g, eps, D0, U0);
  trace_post(K_BLOCK_INIT, s);
  return hipGetLastError();
}

}  // namespace dspark
