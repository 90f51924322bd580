// Block-side work of Eq 3 (#layer of module-dflash.ts) on the A*gamma block
// rows, kept in float32 between kernels:
//   U = RMSNorm(D; attn_norm);  Q, K_d, V_d = U Wq, U Wk, U Wv
//   E = D + Attn Wo;  Z = RMSNorm(E; ff_norm)
//   D' = E + (SiLU(Z Wgate) * (Z Wup)) Wdown
// With at most a few dozen rows these products are weight-streaming bound, so
// each one is a split-K "skinny" GEMM: every workgroup streams a 128-column x
// KS-row slab of the [in, out] weight once (16-byte loads along the output
// columns), multiplies it with the matching slab of the rows held in LDS and
// writes a float32 partial. The last workgroup to finish a column slab (an
// atomic ticket; nobody waits) sums the slab's partials in a fixed order and
// applies the epilogue: the Q/K_d/V_d split, the residual, or SiLU(gate)*up;
// the last slab to finish then applies the row RMSNorm that the next
// projection needs.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace dspark {

constexpr int SK_TN = 16;            // threads along columns (8 columns each)
constexpr int SK_TK = 16;            // thread rows along K
constexpr int SK_COLS = 8 * SK_TN;   // 128 columns per workgroup
constexpr int SK_MT = 8;             // block rows per pass

// K rows per thread (RPT) and K slabs (splits): about 256 workgroups over
// the (N/128) column slabs, at least 2 rows per thread, and few enough slabs
// that the last-arriving workgroup's reduction (M rows x 128 columns x splits
// partials) stays short. The last slab may be partial.
SkinnyPlan skinny_plan(int M, int N, int K) {
  const int nb = N / SK_COLS;
  int want = (256 + nb - 1) / nb;
  const int cap = std::max(2, 512 / std::max(M, 1));
  if (want > cap) want = cap;
  int rpt = 2;
  while (rpt < 16 && (int64_t)SK_TK * rpt * want < K) rpt *= 2;
  SkinnyPlan p;
  p.rpt = rpt;
  p.splits = (K + SK_TK * rpt - 1) / (SK_TK * rpt);
  return p;
}

template <typename S, int RPT>
__global__ __launch_bounds__(256) void skinny_kernel(const float* __restrict__ X, int M, int K,
                                                     BMats b, int N, float* __restrict__ part,
                                                     SkinnyEpi epi) {
  constexpr int KS = SK_TK * RPT;
  __shared__ __attribute__((aligned(16))) float xs[KS][SK_MT];
  __shared__ float red[SK_TK][SK_MT][SK_COLS + 4];
  __shared__ unsigned s_ticket;
  const int tid = threadIdx.x;
  const int tn = tid % SK_TN, tk = tid / SK_TN;
  const int nb = blockIdx.x;
  const int z = blockIdx.y;
  const int nsplit = gridDim.y;
  const int kbase = z * KS;
  // this thread's 8 output columns: matrix `mi`, columns c0 .. c0+7 of it
  int mi, c0;
  if (epi.mode == SK_SWIGLU) {          // gate columns, then the matching up columns
    mi = tn >> 3;
    c0 = nb * 64 + (tn & 7) * 8;
  } else {
    const int gc = nb * SK_COLS + tn * 8;
    mi = gc / b.n_per;
    c0 = gc % b.n_per;
  }
  const S* __restrict__ W = static_cast<const S*>(b.mat[mi]);

  // weights of rows kbase + tk + SK_TK * r (< K), all loads issued up front
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
      if (m0 + mm < M) part[((int64_t)z * M + m0 + mm) * N + nb * SK_COLS + cc] = v;
    }
  }

  // ---- the last workgroup of this column slab reduces the K slabs in a fixed
  // order and applies the epilogue (no waiting: the others simply exit).
  __threadfence();
  __syncthreads();
  if (tid == 0) s_ticket = atomicAdd(&epi.counters[nb], 1u);
  __syncthreads();
  if (s_ticket != (unsigned)(nsplit - 1)) return;
  __threadfence();
  if (tid == 0) epi.counters[nb] = 0u;

  float(*fin)[32][SK_COLS] = reinterpret_cast<float(*)[32][SK_COLS]>(&red[0][0][0]);
  const int lc = tid & (SK_COLS - 1), half = tid >> 7;
  const int zs = half == 0 ? 0 : nsplit / 2, ze = half == 0 ? nsplit / 2 : nsplit;
  const int64_t zstride = (int64_t)M * N;
  for (int m0 = 0; m0 < M; m0 += 32) {
    const int mn = min(32, M - m0);
    for (int mm = 0; mm < mn; ++mm) {
      const float* pp = part + ((int64_t)m0 + mm) * N + nb * SK_COLS + lc;
      float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
      int zz = zs;
      for (; zz + 4 <= ze; zz += 4) {
        v0 += pp[(zz + 0) * zstride];
        v1 += pp[(zz + 1) * zstride];
        v2 += pp[(zz + 2) * zstride];
        v3 += pp[(zz + 3) * zstride];
      }
      for (; zz < ze; ++zz) v0 += pp[zz * zstride];
      fin[half][mm][lc] = (v0 + v1) + (v2 + v3);
    }
    __syncthreads();
    if (epi.mode == SK_SWIGLU) {
      for (int i = tid; i < mn * 64; i += 256) {
        const int mm = i / 64, c = i % 64;
        const float g = fin[0][mm][c] + fin[1][mm][c];
        const float u = fin[0][mm][c + 64] + fin[1][mm][c + 64];
        epi.hid[(int64_t)(m0 + mm) * epi.ff + nb * 64 + c] = g / (1.f + __expf(-g)) * u;
      }
    } else {
      for (int i = tid; i < mn * SK_COLS; i += 256) {
        const int mm = i / SK_COLS, c = i % SK_COLS;
        const int m = m0 + mm;
        const float v = fin[0][mm][c] + fin[1][mm][c];
        const int gc = nb * SK_COLS + c;
        if (epi.mode == SK_QKV) {
          const int seg = gc / epi.d, col = gc % epi.d;
          const int64_t o = (int64_t)m * epi.d + col;
          if (seg == 0) epi.q[o] = v * epi.qscale;
          else if (seg == 1) epi.kd[o] = v;
          else epi.vd[o] = v;
        } else {
          const int64_t o = (int64_t)m * N + gc;
          epi.out[o] = epi.res[o] + v;
        }
      }
    }
    __syncthreads();
  }
  if (epi.mode != SK_RESID || epi.g == nullptr) return;

  // ---- the last slab to finish normalises every row: normed = RMSNorm(out; g)
  const int nslabs = gridDim.x;
  __threadfence();
  __syncthreads();
  if (tid == 0) s_ticket = atomicAdd(&epi.counters[nslabs], 1u);
  __syncthreads();
  if (s_ticket != (unsigned)(nslabs - 1)) return;
  __threadfence();
  if (tid == 0) epi.counters[nslabs] = 0u;
  const int lane = tid & 63, wave = tid >> 6;
  for (int m = wave; m < M; m += 4) {
    const float* row = epi.out + (int64_t)m * N;
    float ss = 0.f;
    for (int c = lane; c < N; c += 64) ss += row[c] * row[c];
    ss = wave_sum(ss);
    const float sc = rsqrtf(ss / (float)N + epi.eps);
    for (int c = lane; c < N; c += 64) epi.normed[(int64_t)m * N + c] = row[c] * sc * epi.g[c];
  }
}

hipError_t launch_skinny(int dtype, const float* X, int M, int K, const BMats& b, int N, int splits,
                         float* part, const SkinnyEpi& epi, hipStream_t s) {
  const SkinnyPlan plan = skinny_plan(M, N, K);
  if (plan.splits != splits) return hipErrorInvalidValue;
  const int rpt = plan.rpt;
  dim3 grid(N / SK_COLS, splits);
  trace_pre(K_SKINNY, s);
  bool ok = true;
#define DSPARK_SK(R)                                                                     \
  case R:                                                                                \
    if (dtype == 1)                                                                      \
      skinny_kernel<bf16, R><<<grid, 256, 0, s>>>(X, M, K, b, N, part, epi);             \
    else                                                                                 \
      skinny_kernel<float, R><<<grid, 256, 0, s>>>(X, M, K, b, N, part, epi);            \
    break;
  switch (rpt) {
    DSPARK_SK(2) DSPARK_SK(4) DSPARK_SK(8) DSPARK_SK(16)
    default: ok = false;
  }
#undef DSPARK_SK
  trace_post(K_SKINNY, s);
  if (!ok) return hipErrorInvalidValue;
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
