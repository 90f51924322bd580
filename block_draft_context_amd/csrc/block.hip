// Block-side work of Eq 3 (#layer of module-dflash.ts) on the A*gamma block
// rows, kept in float32 between kernels:
//   Q, K_d, V_d = RMSNorm(D; attn_norm) . {Wq, Wk, Wv}
//   E  = D + Attn . Wo
//   GU = RMSNorm(E; ff_norm) . [Wgate | Wup]
//   D' = E + (SiLU(G) * U) . Wdown
// With at most a few dozen rows these products stream their weights once and
// are bound by memory latency, so each is one "row GEMM" launch with no
// cross-workgroup communication and as many workgroups as the weights allow:
// a workgroup owns 8 output columns (one 16-byte bf16 vector per weight row)
// and the full K, and its 256 threads split K, each with its few weight
// vectors requested before anything else. The row norm / SwiGLU that feeds a
// product is applied while its input rows are staged in LDS (prologue); the
// residual and the Q/K_d/V_d split are applied on the way out (epilogue).
// Workgroup i runs on XCD i % 8, so column groups are dealt to the XCDs in
// contiguous runs: the workgroups that share a 128-byte weight line then
// share one L2.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace dspark {

constexpr int RG_COLS = 8;          // columns per workgroup
constexpr int RG_THREADS = 256;
constexpr int RG_WAVES = RG_THREADS / 64;
constexpr int RG_MC = 8;            // block rows per pass
constexpr int RG_XS = 16384;        // floats of staged rows (64 KiB)
constexpr int RG_RB = 8;            // weight rows per thread held at once
constexpr int RG_RED = 64 * 65;     // floats of one wave's reduction block
constexpr int RG_LDS = RG_XS > RG_WAVES * RG_RED ? RG_XS : RG_WAVES * RG_RED;

int rowgemm_rows_per_pass(int K) { return std::max(1, std::min(RG_MC, RG_XS / K)); }

template <typename S, int PRO, int EPI>
__global__ __launch_bounds__(RG_THREADS) void rowgemm_kernel(RowGemmArgs a) {
  __shared__ __attribute__((aligned(16))) float xs[RG_LDS];   // staged rows, then reductions
  __shared__ float part_ss[RG_WAVES][RG_MC];
  __shared__ float wred[RG_WAVES][RG_MC * RG_COLS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, M = a.M;
  const int G = gridDim.x;
  const int cg = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  const int n0 = cg * RG_COLS;
  const int mi = n0 / a.b.n_per, c0 = n0 % a.b.n_per;
  const S* __restrict__ W = static_cast<const S*>(a.b.mat[mi]);
  const int rpt = (K + RG_THREADS - 1) / RG_THREADS;          // weight rows per thread
  const int mc = max(1, min(RG_MC, RG_XS / K));
  constexpr int NV = sizeof(S) / 2;                            // 16-byte vectors per row

  // weight rows k = tid + 256 r, RG_RB at a time; loads are unconditional
  // (rows past K repeat row K-1 and are weighted by zero) so they issue back
  // to back, and the first batch is requested before the rows are staged
  u32x4 wv[RG_RB][NV];
  auto load_batch = [&](int r0) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RG_RB; ++r) {
      const int k = min(tid + RG_THREADS * (r0 + r), K - 1);
      const S* p = W + (int64_t)k * a.b.n_per + c0;
      wv[r][0] = ld16(p);
      if constexpr (NV == 2) wv[r][1] = ld16(p + 4);
    }
  };
  load_batch(0);

  for (int m0 = 0; m0 < M; m0 += mc) {
    const int mp = min(mc, M - m0);                             // live rows of this pass
    // residual of this thread's output (wave 0, lane o = m * 8 + c), early
    float resv = 0.f;
    if constexpr (EPI == RE_RESID) {
      if (wave == 0) {
        const int m = m0 + min(lane / RG_COLS, mp - 1);
        resv = a.res[(int64_t)m * a.ldo + n0 + lane % RG_COLS];
      }
    }
    // ---- stage the pass's rows (prologue applied) as xs[mm][k]: thread t
    // moves float4 t, t+256, ... of the [mp][K] block, all loads together
    __syncthreads();
    {
      const int K4 = K / 4;
      constexpr int NQ = 8;
      float ssr[RG_MC];
#pragma unroll
      for (int mm = 0; mm < RG_MC; ++mm) ssr[mm] = 0.f;
      const f32x4* gain4 = reinterpret_cast<const f32x4*>(a.g);
      for (int q0 = 0; q0 < mp * K4; q0 += RG_THREADS * NQ) {
        f32x4 v[NQ], u[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const int q = min(q0 + tid + RG_THREADS * i, mp * K4 - 1);
          const int mm = q / K4, c4 = q % K4;
          const f32x4* x = reinterpret_cast<const f32x4*>(a.X + (int64_t)(m0 + mm) * a.ldx);
          v[i] = x[c4];
          if constexpr (PRO == RP_SWIGLU) u[i] = x[K4 + c4];
          if constexpr (PRO == RP_RMSNORM) u[i] = gain4[c4];
        }
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const int q = q0 + tid + RG_THREADS * i;
          if (q < mp * K4) {
            const int mm = q / K4, c4 = q % K4;
            f32x4 val = v[i];
            if constexpr (PRO == RP_SWIGLU) {
#pragma unroll
              for (int e = 0; e < 4; ++e) val[e] = val[e] / (1.f + __expf(-val[e])) * u[i][e];
            }
            if constexpr (PRO == RP_RMSNORM) {
              const float sq = val[0] * val[0] + val[1] * val[1] + val[2] * val[2] + val[3] * val[3];
#pragma unroll
              for (int mq = 0; mq < RG_MC; ++mq) ssr[mq] += (mq == mm) ? sq : 0.f;
              val *= u[i];   // gain now, row scale below
            }
            *reinterpret_cast<f32x4*>(xs + mm * K + 4 * c4) = val;
          }
        }
      }
      if constexpr (PRO == RP_RMSNORM) {
#pragma unroll
        for (int mm = 0; mm < RG_MC; ++mm) {
          if (mm < mp) {
            const float t = wave_sum(ssr[mm]);
            if (lane == 0) part_ss[wave][mm] = t;
          }
        }
        __syncthreads();
        for (int q = tid; q < mp * K4; q += RG_THREADS) {
          const int mm = q / K4, c4 = q % K4;
          const float tot = (part_ss[0][mm] + part_ss[1][mm]) + (part_ss[2][mm] + part_ss[3][mm]);
          const float sc = rsqrtf(tot / (float)K + a.eps);
          *reinterpret_cast<f32x4*>(xs + mm * K + 4 * c4) *= sc;
        }
      }
    }
    __syncthreads();

    // ---- partial dot products over this thread's rows
    float acc[RG_MC][RG_COLS];
#pragma unroll
    for (int mm = 0; mm < RG_MC; ++mm)
#pragma unroll
      for (int c = 0; c < RG_COLS; ++c) acc[mm][c] = 0.f;
    for (int r0 = 0; r0 < rpt; r0 += RG_RB) {
      if (r0 > 0 || m0 > 0) load_batch(r0);
#pragma unroll
      for (int r = 0; r < RG_RB; ++r) {
        const int k = tid + RG_THREADS * (r0 + r);
        if (r0 + r < rpt) {
          float wf[RG_COLS];
          Vec16<S>::unpack(wv[r][0], wf);
          if constexpr (NV == 2) Vec16<S>::unpack(wv[r][1], wf + 4);
          const bool in = k < K;
#pragma unroll
          for (int mm = 0; mm < RG_MC; ++mm) {
            if (mm < mp) {
              const float xv = in ? xs[mm * K + k] : 0.f;
#pragma unroll
              for (int c = 0; c < RG_COLS; ++c) acc[mm][c] = fmaf(xv, wf[c], acc[mm][c]);
            }
          }
        }
      }
    }

    // ---- reduce: over the wave's 64 lanes through LDS (row stride 65 keeps
    // both the writes and the column reads conflict-free), then over the 4 waves
    __syncthreads();
    float* red = xs + wave * RG_RED;
#pragma unroll
    for (int mm = 0; mm < RG_MC; ++mm) {
      if (mm < mp) {
#pragma unroll
        for (int c = 0; c < RG_COLS; ++c) red[lane * 65 + mm * RG_COLS + c] = acc[mm][c];
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int o = lane;                                   // output o = mm * 8 + c
    const bool live = o / RG_COLS < mp;
    float sum = 0.f;
    if (live) {
#pragma unroll 16
      for (int j = 0; j < 64; ++j) sum += red[j * 65 + o];
    }
    wred[wave][o] = sum;
    __syncthreads();

    // ---- epilogue: wave 0, lane o
    if (wave == 0 && live) {
      const float v = (wred[0][o] + wred[1][o]) + (wred[2][o] + wred[3][o]);
      const int m = m0 + o / RG_COLS;
      const int n = n0 + o % RG_COLS;
      if constexpr (EPI == RE_QKV) {
        const int seg = n / a.d, col = n % a.d;
        const int64_t off = (int64_t)m * a.d + col;
        if (seg == 0) a.q[off] = v * a.qscale;
        else if (seg == 1) a.kd[off] = v;
        else a.vd[off] = v;
      } else if constexpr (EPI == RE_RESID) {
        a.out[(int64_t)m * a.ldo + n] = resv + v;
      } else {
        a.out[(int64_t)m * a.ldo + n] = v;
      }
    }
  }
}

hipError_t launch_rowgemm(int dtype, int pro, int epi, const RowGemmArgs& a, hipStream_t s) {
  if (a.N % RG_COLS != 0 || a.K % 64 != 0 || a.b.n_per % RG_COLS != 0 || a.K > RG_XS)
    return hipErrorInvalidValue;
  dim3 grid(a.N / RG_COLS);
  bool ok = false;
  trace_pre(K_ROWGEMM, s);
#define DSPARK_RG(P, E)                                                        \
  if (pro == P && epi == E) {                                                  \
    ok = true;                                                                 \
    if (dtype == 1) rowgemm_kernel<bf16, P, E><<<grid, RG_THREADS, 0, s>>>(a); \
    else rowgemm_kernel<float, P, E><<<grid, RG_THREADS, 0, s>>>(a);           \
  }
  DSPARK_RG(RP_RMSNORM, RE_QKV)
  DSPARK_RG(RP_NONE, RE_RESID)
  DSPARK_RG(RP_RMSNORM, RE_STORE)
  DSPARK_RG(RP_SWIGLU, RE_RESID)
#undef DSPARK_RG
  trace_post(K_ROWGEMM, s);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

// D0[b, j] = block_in[b, j] + block_pos[j] (block_pos and D0 nullable);
// U0 = RMSNorm(D0; g) (nullable). One row per workgroup.
__global__ __launch_bounds__(256) void block_rows_kernel(const float* __restrict__ bin,
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

hipError_t launch_block_rows(const float* block_in, const float* block_pos, int A, int gamma, int d,
                             const float* g, float eps, float* D0, float* U0, hipStream_t s) {
  trace_pre(K_BLOCK_ROWS, s);
  block_rows_kernel<<<A * gamma, 256, 0, s>>>(block_in, block_pos, gamma, d, g, eps, D0, U0);
  trace_post(K_BLOCK_ROWS, s);
  return hipGetLastError();
}

}  // namespace dspark
