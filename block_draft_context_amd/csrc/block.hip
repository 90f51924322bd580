// Block-side work of Eq 3 (#layer of module-dflash.ts) on the A*gamma block
// rows, kept in float32 between kernels:
//   Q, K_d, V_d = RMSNorm(D; attn_norm) . {Wq, Wk, Wv}
//   E  = D + Attn . Wo
//   GU = RMSNorm(E; ff_norm) . [Wgate | Wup]
//   D' = E + (SiLU(G) * U) . Wdown
// With at most a few dozen rows these products stream their weights once and
// are bound by memory latency, so each is one "row GEMM" launch with no
// cross-workgroup communication: a workgroup owns 32 output columns (a wave
// owns 8, one 16-byte bf16 vector per weight row) and the full K; its lanes
// split K, so each lane keeps 16 independent 16-byte weight loads in flight,
// and the wave reduces its lanes through LDS. The row norm / SwiGLU that feeds
// a product is applied while its input rows are staged in LDS (prologue), the
// residual and the Q/K_d/V_d split on the way out (epilogue).
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace dspark {

constexpr int RG_COLS = 8;          // columns per wave
constexpr int RG_WAVES = 4;
constexpr int RG_WG_COLS = RG_COLS * RG_WAVES;
constexpr int RG_XS = 16384;        // floats of staged rows (64 KiB)
constexpr int RG_BATCH = 16;        // weight rows per lane per batch

int rowgemm_rows_per_pass(int K) { return std::max(1, std::min(8, RG_XS / K)); }

template <typename S, int PRO, int EPI, int MC>
__global__ __launch_bounds__(256) void rowgemm_kernel(RowGemmArgs a) {
  __shared__ __attribute__((aligned(16))) float xs[RG_XS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, M = a.M;
  const int n0 = blockIdx.x * RG_WG_COLS + wave * RG_COLS;   // this wave's first column
  const int mi = n0 / a.b.n_per, c0 = n0 % a.b.n_per;
  const S* __restrict__ W = static_cast<const S*>(a.b.mat[mi]);
  const int rpl = K / 64;                                     // weight rows per lane

  // weight batches (rows k = lane + 64 r): all loads of a batch are
  // unconditional (rows past K repeat the last row and are weighted by zero)
  // so they issue back to back; the first batch is requested before the input
  // rows are staged, so the two latencies overlap
  u32x4 wv[1][RG_BATCH][sizeof(S) / 2];
  auto load_batch = [&](int buf, int r0) {
#pragma unroll
    for (int r = 0; r < RG_BATCH; ++r) {
      const int k = lane + 64 * min(r0 + r, rpl - 1);
      const S* p = W + (int64_t)k * a.b.n_per + c0;
      wv[buf][r][0] = ld16(p);
      if constexpr (sizeof(S) == 4) wv[buf][r][1] = ld16(p + 4);
    }
  };
  load_batch(0, 0);

  for (int m0 = 0; m0 < M; m0 += MC) {
    // ---- stage MC input rows (prologue applied) into LDS as xs[mm][k]: all
    // 256 threads move float4s, thread t owning column group t, t+256, ... of
    // every row, so a thread's loads are all issued together
    __shared__ float part_ss[RG_WAVES][MC];
    __syncthreads();
    {
      const int K4 = K / 4;
      constexpr int NQ = 8;                 // float4 per thread per round
      float ssr[MC];
#pragma unroll
      for (int mm = 0; mm < MC; ++mm) ssr[mm] = 0.f;
      const f32x4* gain4 = reinterpret_cast<const f32x4*>(a.g);
      for (int q0 = 0; q0 < MC * K4; q0 += 256 * NQ) {
        f32x4 v[NQ], u[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const int q = min(q0 + tid + 256 * i, MC * K4 - 1);
          const int mm = q / K4, c4 = q % K4;
          const int m = min(m0 + mm, M - 1);
          const f32x4* x = reinterpret_cast<const f32x4*>(a.X + (int64_t)m * a.ldx);
          v[i] = x[c4];
          if constexpr (PRO == RP_SWIGLU) u[i] = x[K4 + c4];
          if constexpr (PRO == RP_RMSNORM) u[i] = gain4[c4];
        }
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const int q = q0 + tid + 256 * i;
          if (q < MC * K4) {
            const int mm = q / K4, c4 = q % K4;
            f32x4 val = (m0 + mm < M) ? v[i] : f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (PRO == RP_SWIGLU) {
#pragma unroll
              for (int e = 0; e < 4; ++e) val[e] = val[e] / (1.f + __expf(-val[e])) * u[i][e];
            }
            if constexpr (PRO == RP_RMSNORM) {
              const float sq = val[0] * val[0] + val[1] * val[1] + val[2] * val[2] + val[3] * val[3];
#pragma unroll
              for (int mq = 0; mq < MC; ++mq) ssr[mq] += (mq == mm) ? sq : 0.f;
              val *= u[i];   // gain now, row scale below
            }
            *reinterpret_cast<f32x4*>(xs + mm * K + 4 * c4) = val;
          }
        }
      }
      if constexpr (PRO == RP_RMSNORM) {
#pragma unroll
        for (int mm = 0; mm < MC; ++mm) {
          const float t = wave_sum(ssr[mm]);
          if (lane == 0) part_ss[wave][mm] = t;
        }
        __syncthreads();
        for (int q = tid; q < MC * K4; q += 256) {
          const int mm = q / K4, c4 = q % K4;
          const float tot = (part_ss[0][mm] + part_ss[1][mm]) + (part_ss[2][mm] + part_ss[3][mm]);
          const float sc = rsqrtf(tot / (float)K + a.eps);
          *reinterpret_cast<f32x4*>(xs + mm * K + 4 * c4) *= sc;
        }
      }
    }
    __syncthreads();

    // ---- partial dot products over this lane's rows k = lane + 64 r
    float acc[MC][RG_COLS];
#pragma unroll
    for (int mm = 0; mm < MC; ++mm)
#pragma unroll
      for (int c = 0; c < RG_COLS; ++c) acc[mm][c] = 0.f;
    const int nbatch = (rpl + RG_BATCH - 1) / RG_BATCH;
    auto mac = [&](const u32x4 (&w)[RG_BATCH][sizeof(S) / 2], int r0) {
#pragma unroll
      for (int r = 0; r < RG_BATCH; ++r) {
        float wf[RG_COLS];
        Vec16<S>::unpack(w[r][0], wf);
        if constexpr (sizeof(S) == 4) Vec16<S>::unpack(w[r][1], wf + 4);
        const bool in = r0 + r < rpl;
        const int k = lane + 64 * min(r0 + r, rpl - 1);
#pragma unroll
        for (int mm = 0; mm < MC; ++mm) {
          const float xv = in ? xs[mm * K + k] : 0.f;
#pragma unroll
          for (int c = 0; c < RG_COLS; ++c) acc[mm][c] = fmaf(xv, wf[c], acc[mm][c]);
        }
      }
    };
    for (int bi = 0; bi < nbatch; ++bi) {
      if (bi > 0 || m0 > 0) load_batch(0, bi * RG_BATCH);
      mac(wv[0], bi * RG_BATCH);
    }

    // ---- reduce over the 64 lanes through LDS (xs is free now), 32 sums at a time
    constexpr int NH = (MC * RG_COLS + 31) / 32;
    float resv[NH];   // residual rows, requested before the reduction
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      resv[h] = 0.f;
      if constexpr (EPI == RE_RESID) {
        const int idx = h * 32 + (lane & 31);
        const int m = min(m0 + idx / RG_COLS, M - 1);
        resv[h] = a.res[(int64_t)m * a.ldo + n0 + idx % RG_COLS];
      }
    }
    __syncthreads();
    float* red = xs + wave * (32 * 65);
    float outv[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
      for (int v = 0; v < 32; ++v) {
        const int idx = h * 32 + v;
        if (idx < MC * RG_COLS) red[v * 65 + lane] = acc[idx / RG_COLS][idx % RG_COLS];
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float sum = 0.f;
      if (lane < 32) {
#pragma unroll 8
        for (int j = 0; j < 64; ++j) sum += red[lane * 65 + j];
      }
      outv[h] = sum;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- epilogue: lane < 32 owns output idx = h*32 + lane
    if (lane < 32) {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int idx = h * 32 + lane;
        if (idx >= MC * RG_COLS) continue;
        const int m = m0 + idx / RG_COLS;
        if (m >= M) continue;
        const int n = n0 + idx % RG_COLS;
        const float v = outv[h];
        if constexpr (EPI == RE_QKV) {
          const int seg = n / a.d, col = n % a.d;
          const int64_t o = (int64_t)m * a.d + col;
          if (seg == 0) a.q[o] = v * a.qscale;
          else if (seg == 1) a.kd[o] = v;
          else a.vd[o] = v;
        } else if constexpr (EPI == RE_RESID) {
          a.out[(int64_t)m * a.ldo + n] = resv[h] + v;
        } else {
          a.out[(int64_t)m * a.ldo + n] = v;
        }
      }
    }
  }
}

template <typename S, int PRO, int EPI>
static void rowgemm_mc(const RowGemmArgs& a, dim3 grid, hipStream_t s) {
  switch (rowgemm_rows_per_pass(a.K)) {
    case 8: rowgemm_kernel<S, PRO, EPI, 8><<<grid, 256, 0, s>>>(a); break;
    case 4: rowgemm_kernel<S, PRO, EPI, 4><<<grid, 256, 0, s>>>(a); break;
    case 2: rowgemm_kernel<S, PRO, EPI, 2><<<grid, 256, 0, s>>>(a); break;
    default: rowgemm_kernel<S, PRO, EPI, 1><<<grid, 256, 0, s>>>(a); break;
  }
}

hipError_t launch_rowgemm(int dtype, int pro, int epi, const RowGemmArgs& a, hipStream_t s) {
  if (a.N % RG_WG_COLS != 0 || a.K % 64 != 0 || a.b.n_per % RG_COLS != 0 || a.K > RG_XS)
    return hipErrorInvalidValue;
  dim3 grid(a.N / RG_WG_COLS);
  bool ok = false;
  trace_pre(K_ROWGEMM, s);
#define DSPARK_RG(P, E)                                                        \
  if (pro == P && epi == E) {                                                  \
    ok = true;                                                                 \
    if (dtype == 1) rowgemm_mc<bf16, P, E>(a, grid, s);                        \
    else rowgemm_mc<float, P, E>(a, grid, s);                                  \
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
