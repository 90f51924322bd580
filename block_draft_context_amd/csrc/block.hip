// Block-side work of Eq 3 (#layer of module-dflash.ts) on the A*gamma block
// rows, kept in float32 between kernels:
//   Q, K_d, V_d = RMSNorm(D; attn_norm) . {Wq, Wk, Wv}
//   E  = D + Attn . Wo
//   H  = SiLU(Z . Wgate) * (Z . Wup),  Z = RMSNorm(E; ff_norm)
//   D' = E + H . Wdown
// With at most a few dozen rows these products stream their weights once and
// are bound by memory latency, so each is one "row GEMM" launch with no
// cross-workgroup communication and as many workgroups as the weights allow.
// Weights are [out, in] row-major, so an output column's weights are one
// contiguous run over K: a workgroup owns COLS columns (COLS / 4 per wave),
// and the 64 lanes of a wave read consecutive 16-byte chunks of a column's
// run (1 KiB per load instruction), every load issued before anything else.
// The input rows are staged in LDS once per workgroup with the RMSNorm gain
// applied; the RMSNorm row scale, which factors out of the dot products, the
// residual, the Q/K_d/V_d split and the SwiGLU (a wave owns one gate column
// and the matching up column) are applied on the outputs.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace dspark {

constexpr int RG_THREADS = 256;
constexpr int RG_WAVES = RG_THREADS / 64;
constexpr int RG_MC = 8;            // block rows per pass
constexpr int RG_XS = 16256;        // floats of staged rows (with the static arrays <= 64 KiB)
constexpr int RG_JB = 4;            // weight chunks per lane and column held at once
constexpr int RG_XC = 2;            // float4 input columns per thread per staging round

int rowgemm_rows_per_pass(int K) { return std::max(1, std::min(RG_MC, RG_XS / K)); }
// rows staged per pass for M block rows (LDS is sized to them at launch)
static int rowgemm_mc(int M, int K) { return std::max(1, std::min(std::min(RG_MC, M), RG_XS / K)); }

// Sum of v[] over the 64 lanes, scattered: V values are halved at each of the
// butterfly levels 32, 16, 8, ... (lanes whose level bit is set keep the
// upper half), then the last value is summed over the remaining levels.
// Afterwards every lane holds the full sum of value index lane / (64 / V).
// Levels 32 and 16 use the permlane swaps (a lane receives its own and its
// partner's value of a pair at once), levels 8 .. 1 the DPP row mirrors and
// quad permutations; nothing goes through LDS.
template <int S>
DSPARK_DEV float partner(float x) {
  if constexpr (S == 8) return dpp_f<kDppMirror>(x);
  else if constexpr (S == 4) return dpp_f<kDppHalfMirror>(x);
  else if constexpr (S == 2) return dpp_f<kDppXor2>(x);
  else return dpp_f<kDppXor1>(x);
}

template <int S, int N>
DSPARK_DEV void rs_level(float (&v)[64], int lane) {
  if constexpr (N > 1) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      if constexpr (S >= 16) {
        // lanes below the partner keep value i, the others value i + N/2:
        // a swap of (v[i], v[i + N/2]) hands each lane both terms of its sum
        const auto r = S == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]),
                                                                   __float_as_uint(v[i + N / 2]), false, false)
                               : __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]),
                                                                   __float_as_uint(v[i + N / 2]), false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      } else {
        const bool up = (lane & S) != 0;
        const float keep = up ? v[i + N / 2] : v[i];
        const float send = up ? v[i] : v[i + N / 2];
        v[i] = keep + partner<S>(send);
      }
    }
    rs_level<S / 2, N / 2>(v, lane);
  } else if constexpr (S >= 1) {
    // one value left: sum it over the remaining levels
    if constexpr (S >= 16) {
      float a, b;
      if constexpr (S == 32) swap32(v[0], a, b); else swap16(v[0], a, b);
      v[0] = a + b;
    } else {
      v[0] += partner<S>(v[0]);
    }
    rs_level<S / 2, 1>(v, lane);
  }
}

template <int V>
DSPARK_DEV float reduce_scatter64(float (&v)[V], int lane) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V power of two");
  float w[64];
#pragma unroll
  for (int i = 0; i < V; ++i) w[i] = v[i];
  rs_level<32, V>(w, lane);
  return w[0];
}

template <typename S, int PRO, int EPI, int COLS>
__global__ __launch_bounds__(RG_THREADS) void rowgemm_kernel(RowGemmArgs a) {
  // staged rows: element k of row mm at xs[mm*K + (k/4 % 2)*(K/2) + 4*(k/8) + k%4],
  // so lane j's two 16-byte reads of chunk j (elements 8j .. 8j+7) are
  // contiguous across lanes
  extern __shared__ __attribute__((aligned(16))) float xs[];   // [mc][K], sized at launch
  __shared__ float part_ss[RG_WAVES][RG_MC];
  constexpr int CPW = COLS / RG_WAVES;                         // columns per wave
  constexpr int V = CPW * RG_MC;                               // sums per lane
  constexpr int NV = (int)sizeof(S) / 2;                       // 16-byte loads per chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, M = a.M, K4 = K / 4, nch = K / 8;
  const int cpl = (nch + 63) / 64;                             // chunks per lane
  const int mc = max(1, min(min(RG_MC, M), RG_XS / K));
  // the wave's columns: nw .. nw+CPW-1, or for RE_SWIGLU gate column nw and
  // up column nw (one pair per wave)
  const int nw = EPI == RE_SWIGLU ? blockIdx.x * RG_WAVES + wave : blockIdx.x * COLS + wave * CPW;
  static_assert(EPI != RE_SWIGLU || CPW == 2, "SwiGLU pairs");
  const S* wcol[CPW];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    if constexpr (EPI == RE_SWIGLU) {
      wcol[cc] = static_cast<const S*>(a.b.mat[cc]) + (int64_t)nw * K;
    } else {
      const int n = nw + cc;
      wcol[cc] = static_cast<const S*>(a.b.mat[n / a.b.n_per]) + (int64_t)(n % a.b.n_per) * K;
    }
  }

  u32x4 wv[RG_JB][CPW][NV];
  auto load_batch = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < RG_JB; ++b) {
      if (j0 + b < cpl) {
        const int j = min(lane + 64 * (j0 + b), nch - 1);
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
          for (int v = 0; v < NV; ++v) wv[b][cc][v] = ld16(wcol[cc] + 8 * j + 4 * v);
      }
    }
  };
  // the first weights (the larger transfer) are requested before anything
  // else, so they stream in while the input rows' latency passes
  load_batch(0);

  // One pass of mc rows per workgroup: pass blockIdx.y (the grid has one
  // row of workgroups per pass), so many block rows run as parallel passes.
  {
    const int m0 = blockIdx.y * mc;
    const int mp = min(mc, M - m0);                             // live rows of this pass
    // this lane's output after the reduction: value index lane / (64 / V)
    const int vo = lane / (64 / V);
    const int om_l = vo % RG_MC, on = EPI == RE_SWIGLU ? nw : nw + vo / RG_MC;
    const bool live = om_l < mp && (lane % (64 / V)) == 0;
    const int om = m0 + min(om_l, mp - 1);
    float resv = 0.f;
    if constexpr (EPI == RE_RESID) resv = a.res[(int64_t)om * a.ldo + on];

    // ---- stage the pass's rows: thread t moves float4 columns t, t+256, ...
    __syncthreads();
    float ssr[RG_MC];
#pragma unroll
    for (int mm = 0; mm < RG_MC; ++mm) ssr[mm] = 0.f;
    for (int q0 = 0; q0 < K4; q0 += RG_THREADS * RG_XC) {
      f32x4 v[RG_XC][RG_MC], gv[RG_XC];
#pragma unroll
      for (int i = 0; i < RG_XC; ++i) {
        const int c4 = min(q0 + tid + RG_THREADS * i, K4 - 1);
        if constexpr (PRO == RP_RMSNORM) gv[i] = reinterpret_cast<const f32x4*>(a.g)[c4];
#pragma unroll
        for (int mm = 0; mm < RG_MC; ++mm) {
          if (mm < mp) {
            const f32x4* x = reinterpret_cast<const f32x4*>(a.X + (int64_t)(m0 + mm) * a.ldx);
            v[i][mm] = x[c4];
          }
        }
      }
#pragma unroll
      for (int i = 0; i < RG_XC; ++i) {
        const int c4 = q0 + tid + RG_THREADS * i;
        if (c4 < K4) {
          float* dst = xs + (c4 & 1) * (K / 2) + 4 * (c4 >> 1);
#pragma unroll
          for (int mm = 0; mm < RG_MC; ++mm) {
            if (mm < mp) {
              f32x4 val = v[i][mm];
              if constexpr (PRO == RP_RMSNORM) {
                ssr[mm] += val[0] * val[0] + val[1] * val[1] + val[2] * val[2] + val[3] * val[3];
                val *= gv[i];
              }
              *reinterpret_cast<f32x4*>(dst + mm * K) = val;
            }
          }
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
    }
    __syncthreads();

    // ---- dot products of this lane's chunks with every live row
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < cpl; j0 += RG_JB) {
      if (j0 > 0) load_batch(j0);   // the first batch is in registers already
#pragma unroll
      for (int b = 0; b < RG_JB; ++b) {
        if (j0 + b < cpl) {
          const int j = lane + 64 * (j0 + b);
          const bool in = j < nch;
          const int jc = min(j, nch - 1);
          float wf[CPW][8];
#pragma unroll
          for (int cc = 0; cc < CPW; ++cc) {
            Vec16<S>::unpack(wv[b][cc][0], wf[cc]);
            if constexpr (NV == 2) Vec16<S>::unpack(wv[b][cc][1], wf[cc] + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) wf[cc][e] = in ? wf[cc][e] : 0.f;
          }
#pragma unroll
          for (int mm = 0; mm < RG_MC; ++mm) {
            if (mm < mp) {
              const f32x4 xl = *reinterpret_cast<const f32x4*>(xs + mm * K + 4 * jc);
              const f32x4 xh = *reinterpret_cast<const f32x4*>(xs + mm * K + K / 2 + 4 * jc);
#pragma unroll
              for (int cc = 0; cc < CPW; ++cc) {
                float t = acc[cc * RG_MC + mm];
#pragma unroll
                for (int e = 0; e < 4; ++e) t = fmaf(xl[e], wf[cc][e], t);
#pragma unroll
                for (int e = 0; e < 4; ++e) t = fmaf(xh[e], wf[cc][4 + e], t);
                acc[cc * RG_MC + mm] = t;
              }
            }
          }
        }
      }
    }

    // ---- reduce over the wave's lanes; the wave owns whole columns, so no
    // cross-wave step is needed
    float v = reduce_scatter64<V>(acc, lane);
    if constexpr (PRO == RP_RMSNORM) {
      const float tot = (part_ss[0][om_l] + part_ss[1][om_l]) + (part_ss[2][om_l] + part_ss[3][om_l]);
      v *= rsqrtf(tot / (float)K + a.eps);
    }
    if constexpr (EPI == RE_SWIGLU) {
      // lane l < 32 holds the gate sum of row l/4, lane l + 32 the up sum
      // of the same row: one swap gives every lane both
      float g, u;
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      g = __uint_as_float(r[0]);
      u = __uint_as_float(r[1]);
      if (live && lane < 32) {
        float act;
        if (a.act == 0) {
          act = g / (1.f + expf(-g));   // SiLU (dspark-runtime.js)
        } else {                        // tanh-GELU (module-dflash.ts, geluApprox)
          const float c = 0.7978845608028654f;   // sqrt(2 / pi)
          act = 0.5f * g * (1.f + tanhf(c * (g + 0.044715f * g * g * g)));
        }
        a.out[(int64_t)om * a.ldo + on] = act * u;
      }
    } else if (live) {
      if constexpr (EPI == RE_QKV) {
        if (on < a.d) a.q[(int64_t)om * a.d + on] = v * a.qscale;
        else if (on < a.d + a.kvd) a.kd[(int64_t)om * a.kvd + (on - a.d)] = v;
        else a.vd[(int64_t)om * a.kvd + (on - a.d - a.kvd)] = v;
      } else if constexpr (EPI == RE_RESID) {
        a.out[(int64_t)om * a.ldo + on] = resv + v;
      } else {
        a.out[(int64_t)om * a.ldo + on] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Row GEMM on the matrix cores, for many block rows with bf16 weights.
// With more rows than one 8-row pass, the vector-ALU kernel above re-reads
// the input rows for every 8 output columns; here a workgroup owns CB blocks
// of 16 output columns (SwiGLU: CB gate blocks and the matching up blocks)
// for RB blocks of 16 rows and multiplies on v_mfma_f32_16x16x32_bf16. The
// float32 rows enter as two bf16 terms, hi = bf16(x) and lo = bf16(x - hi), so each product is two MFMAs
// and the input keeps about 16 bits of mantissa (relative error <= 2^-16);
// the weights are bf16 as stored and the sums are float32. The four waves
// split K and keep RF_PF chunks of 32 k in flight each; their partial sums
// meet in LDS, where the epilogues of the vector-ALU kernel run unchanged.
// 16x16x32 operand layout: lane l holds A[l % 16][8 (l / 16) .. + 8) and
// B[8 (l / 16) .. + 8)[l % 16]; the result D[4 (l / 16) + r][l % 16], r < 4.
// ---------------------------------------------------------------------------

DSPARK_DEV uint32_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, from_f32<bf16>(x)); }

// x (8 floats) -> hi, lo bf16 vectors with x ~= hi + lo
DSPARK_DEV void split_bf16(const f32x4& x0, const f32x4& x1, bf16x8& hi, bf16x8& lo) {
  float xv[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bf16 h = from_f32<bf16>(xv[e]);
    hi[e] = h;
    lo[e] = from_f32<bf16>(xv[e] - static_cast<float>(h));
  }
}

// RB 16-row blocks and CB 16-column blocks per workgroup (for SwiGLU, CB
// gate blocks and the matching CB up blocks); RF_PF k chunks in flight.
template <int PRO, int EPI, int RB, int CB>
__global__ __launch_bounds__(256) void rowgemm_mfma_kernel(RowGemmArgs a) {
  constexpr int RF_RB = RB;
  constexpr int RF_PF = RB * CB > 4 ? 2 : 4;
  constexpr int NCB = EPI == RE_SWIGLU ? 2 * CB : CB;   // 16-column blocks: gate ones first for SwiGLU
  __shared__ float red[4][RF_RB][NCB][256];
  __shared__ float ssq[4][RF_RB * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, M = a.M;
  const int nb = blockIdx.x;
  const int m_base = blockIdx.y * RF_RB * 16;
  const int c16 = lane & 15, kg = lane >> 4;
  const bf16* wrow[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    if constexpr (EPI == RE_SWIGLU) {
      const int half = cb / CB, n = (nb * CB + cb % CB) * 16 + c16;
      wrow[cb] = static_cast<const bf16*>(a.b.mat[half]) + (int64_t)n * K;
    } else {
      const int n = (nb * CB + cb) * 16 + c16;
      wrow[cb] = static_cast<const bf16*>(a.b.mat[n / a.b.n_per]) + (int64_t)(n % a.b.n_per) * K;
    }
  }
  const float* xrow[RF_RB];
#pragma unroll
  for (int rb = 0; rb < RF_RB; ++rb)
    xrow[rb] = a.X + (int64_t)min(m_base + rb * 16 + c16, M - 1) * a.ldx;   // rows past M: a valid row, unused

  const int kq = K / 4;                    // this wave's quarter of K (K % 128 == 0)
  const int nch = kq / 32;
  const int kw = wave * kq + 8 * kg;       // this lane's first k

  f32x4 acc[RF_RB][NCB];
  float ss[RF_RB];
#pragma unroll
  for (int rb = 0; rb < RF_RB; ++rb) {
    ss[rb] = 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 wb[RF_PF][NCB];
  f32x4 xb[RF_PF][RF_RB][2];
  auto load = [&](int c, int slot) __attribute__((always_inline)) {
    const int k = kw + min(c, nch - 1) * 32;   // past the last chunk: repeat it (in bounds, unused)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) wb[slot][cb] = *reinterpret_cast<const bf16x8*>(wrow[cb] + k);
#pragma unroll
    for (int rb = 0; rb < RF_RB; ++rb) {
      xb[slot][rb][0] = *reinterpret_cast<const f32x4*>(xrow[rb] + k);
      xb[slot][rb][1] = *reinterpret_cast<const f32x4*>(xrow[rb] + k + 4);
    }
  };
#pragma unroll
  for (int u = 0; u < RF_PF; ++u) load(u, u);
  for (int c0 = 0; c0 < nch; c0 += RF_PF) {
#pragma unroll
    for (int u = 0; u < RF_PF; ++u) {
      const int c = c0 + u;
      if (c < nch) {
        const int k = kw + c * 32;
        f32x4 g0 = f32x4{1.f, 1.f, 1.f, 1.f}, g1 = g0;
        if constexpr (PRO == RP_RMSNORM) {
          g0 = *reinterpret_cast<const f32x4*>(a.g + k);
          g1 = *reinterpret_cast<const f32x4*>(a.g + k + 4);
        }
#pragma unroll
        for (int rb = 0; rb < RF_RB; ++rb) {
          f32x4 x0 = xb[u][rb][0], x1 = xb[u][rb][1];
          if constexpr (PRO == RP_RMSNORM) {
#pragma unroll
            for (int e = 0; e < 4; ++e) ss[rb] += x0[e] * x0[e] + x1[e] * x1[e];
            x0 *= g0;
            x1 *= g1;
          }
          bf16x8 hi, lo;
          split_bf16(x0, x1, hi, lo);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, wb[u][cb], acc[rb][cb], 0, 0, 0);
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, wb[u][cb], acc[rb][cb], 0, 0, 0);
          }
        }
      }
      load(c + RF_PF, u);
    }
  }

  // partial sums of the four waves (K quarters) into LDS
#pragma unroll
  for (int rb = 0; rb < RF_RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      *reinterpret_cast<f32x4*>(&red[wave][rb][cb][lane * 4]) = acc[rb][cb];
  if constexpr (PRO == RP_RMSNORM) {
#pragma unroll
    for (int rb = 0; rb < RF_RB; ++rb) {
      float t = ss[rb];
      t += __shfl_xor(t, 16, kWave);
      t += __shfl_xor(t, 32, kWave);
      if (kg == 0) ssq[wave][rb * 16 + c16] = t;
    }
  }
  __syncthreads();

  // epilogue: element q = 4 * l + r of a 16x16 block is row 4 (l / 16) + r,
  // column l % 16 of the block
#pragma unroll
  for (int rb = 0; rb < RF_RB; ++rb)
#pragma unroll
  for (int cc = 0; cc < CB; ++cc) {
    const int q = tid;
    const int l = q >> 2, r = q & 3;
    const int row = 4 * (l >> 4) + r, col = l & 15;
    const int om = m_base + rb * 16 + row;
    constexpr int NV = EPI == RE_SWIGLU ? 2 : 1;
    float v[NV];
#pragma unroll
    for (int h = 0; h < NV; ++h) {
      const int cb = cc + h * CB;
      v[h] = (red[0][rb][cb][q] + red[1][rb][cb][q]) + (red[2][rb][cb][q] + red[3][rb][cb][q]);
    }
    if constexpr (PRO == RP_RMSNORM) {
      const int i = rb * 16 + row;
      const float tot = (ssq[0][i] + ssq[1][i]) + (ssq[2][i] + ssq[3][i]);
      const float rs = rsqrtf(tot / (float)K + a.eps);
#pragma unroll
      for (int h = 0; h < NV; ++h) v[h] *= rs;
    }
    if (om >= M) continue;
    const int on = (nb * CB + cc) * 16 + col;
    if constexpr (EPI == RE_SWIGLU) {
      const float g = v[0], u = v[1];
      float act;
      if (a.act == 0) {
        act = g / (1.f + expf(-g));
      } else {
        const float c = 0.7978845608028654f;
        act = 0.5f * g * (1.f + tanhf(c * (g + 0.044715f * g * g * g)));
      }
      a.out[(int64_t)om * a.ldo + on] = act * u;
    } else if constexpr (EPI == RE_QKV) {
      if (on < a.d) a.q[(int64_t)om * a.d + on] = v[0] * a.qscale;
      else if (on < a.d + a.kvd) a.kd[(int64_t)om * a.kvd + (on - a.d)] = v[0];
      else a.vd[(int64_t)om * a.kvd + (on - a.d - a.kvd)] = v[0];
    } else if constexpr (EPI == RE_RESID) {
      a.out[(int64_t)om * a.ldo + on] = a.res[(int64_t)om * a.ldo + on] + v[0];
    } else {
      a.out[(int64_t)om * a.ldo + on] = v[0];
    }
  }
}

static bool use_rowgemm_mfma(int dtype, int epi, const RowGemmArgs& a) {
  const int cols = epi == RE_SWIGLU ? a.b.n_per : a.N;
  return dtype == 1 && a.M > rowgemm_mc(a.M, a.K) && a.K % 128 == 0 && cols % 16 == 0 && a.b.n_per % 16 == 0;
}

// Workgroup shape of the matrix-core row GEMM: RB 16-row blocks by CB
// 16-column blocks (column pairs for SwiGLU). At 80 block rows (16
// sequences) alternating runs of a layer's four row GEMMs measured (RB, CB)
// = (1, 2) 14% faster than (2, 1) and (2, 2) 5% faster, with (5, 1), (3, 2),
// (1, 1) and (2, 4) no faster or slower: more workgroups with fewer rows
// each beat fewer re-reads of the block rows. Beyond 128 rows the weights'
// re-reads per 16-row block weigh more, so two row blocks.
struct MfmaShape {
  int rb, cb;
};
static MfmaShape rowgemm_mfma_shape(int epi, const RowGemmArgs& a) {
  const int cols = epi == RE_SWIGLU ? a.b.n_per : a.N;
  MfmaShape sh{a.M <= 128 ? 1 : 2, 2};
  if (cols % (16 * sh.cb) != 0 || a.b.n_per % (16 * sh.cb) != 0) sh.cb = 1;
  // One row block (at most 16 rows) that would fill fewer than one
  // workgroup per CU: 16-column workgroups, twice as many streaming the
  // weights (the rows they re-read are few). Measured at 8 rows of d = 2048:
  // a forward's row GEMMs 300 instead of 357 us; at 80 rows the same switch
  // made the output and down projections 10% slower.
  if (sh.cb == 2 && a.M <= 16 && cols / 32 < 256) sh.cb = 1;
  return sh;
}

hipError_t launch_rowgemm(int dtype, int pro, int epi, const RowGemmArgs& a, hipStream_t s) {
  if (use_rowgemm_mfma(dtype, epi, a)) {
    const MfmaShape sh = rowgemm_mfma_shape(epi, a);
    const int nblk = (epi == RE_SWIGLU ? a.b.n_per : a.N) / (16 * sh.cb);
    dim3 grid(nblk, (a.M + sh.rb * 16 - 1) / (sh.rb * 16));
    bool ok = false;
    trace_pre(K_ROWGEMM, s);
#define DSPARK_RM(P, E)                                                                   \
    if (pro == P && epi == E) {                                                           \
      ok = true;                                                                          \
      if (sh.rb == 1 && sh.cb == 1) rowgemm_mfma_kernel<P, E, 1, 1><<<grid, 256, 0, s>>>(a); \
      else if (sh.rb == 1) rowgemm_mfma_kernel<P, E, 1, 2><<<grid, 256, 0, s>>>(a);        \
      else if (sh.cb == 1) rowgemm_mfma_kernel<P, E, 2, 1><<<grid, 256, 0, s>>>(a);        \
      else rowgemm_mfma_kernel<P, E, 2, 2><<<grid, 256, 0, s>>>(a);                        \
    }
    DSPARK_RM(RP_RMSNORM, RE_QKV)
    DSPARK_RM(RP_NONE, RE_RESID)
    DSPARK_RM(RP_RMSNORM, RE_SWIGLU)
    DSPARK_RM(RP_NONE, RE_STORE)
#undef DSPARK_RM
    trace_post(K_ROWGEMM, s);
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (a.N % 8 != 0 || a.K % 64 != 0 || a.b.n_per % 8 != 0 || a.K > RG_XS) return hipErrorInvalidValue;
  const bool narrow = epi != RE_SWIGLU && a.N / 8 < 256;   // SwiGLU pairs need 2 columns per wave
  // one workgroup row per pass of rowgemm_mc rows; with N / COLS a multiple
  // of 8 the workgroups of one column set land on one XCD (id % 8), so the
  // passes re-read that set's weights from the XCD's L2
  const int passes = (a.M + rowgemm_mc(a.M, a.K) - 1) / rowgemm_mc(a.M, a.K);
  dim3 grid(a.N / (narrow ? 4 : 8), passes);
  const size_t lds = (size_t)rowgemm_mc(a.M, a.K) * a.K * sizeof(float);
  bool ok = false;
  trace_pre(K_ROWGEMM, s);
#define DSPARK_RG(P, E)                                                                      \
  if (pro == P && epi == E) {                                                                \
    ok = true;                                                                               \
    if (dtype == 1) {                                                                        \
      if (narrow) rowgemm_kernel<bf16, P, E, E == RE_SWIGLU ? 8 : 4><<<grid, RG_THREADS, lds, s>>>(a); \
      else rowgemm_kernel<bf16, P, E, 8><<<grid, RG_THREADS, lds, s>>>(a);                     \
    } else {                                                                                 \
      if (narrow) rowgemm_kernel<float, P, E, E == RE_SWIGLU ? 8 : 4><<<grid, RG_THREADS, lds, s>>>(a); \
      else rowgemm_kernel<float, P, E, 8><<<grid, RG_THREADS, lds, s>>>(a);                    \
    }                                                                                        \
  }
  DSPARK_RG(RP_RMSNORM, RE_QKV)
  DSPARK_RG(RP_NONE, RE_RESID)
  DSPARK_RG(RP_RMSNORM, RE_SWIGLU)
  DSPARK_RG(RP_NONE, RE_STORE)
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

namespace dspark {

// Rows 1 .. gamma-1 of every sequence's block: the shared mask embeddings
// (#buildBlock); row 0 (the anchor row) is written by the row GEMM.
__global__ __launch_bounds__(256) void mask_rows_kernel(const float* __restrict__ mask_emb, int gamma, int d,
                                                        float* __restrict__ block_in) {
  const int b = blockIdx.y, j = blockIdx.x + 1;
  const f32x4* src = reinterpret_cast<const f32x4*>(mask_emb + (int64_t)(j - 1) * d);
  f32x4* dst = reinterpret_cast<f32x4*>(block_in + ((int64_t)b * gamma + j) * d);
  for (int c = threadIdx.x; c < d / 4; c += 256) dst[c] = src[c];
}

hipError_t launch_block_build(int dtype, const float* anchor_emb, int A, int H, const void* tok_proj,
                              const float* mask_emb, int gamma, int d, float* block_in, hipStream_t s) {
  RowGemmArgs r{};
  r.X = anchor_emb;
  r.ldx = H;
  r.M = A;
  r.K = H;
  r.N = d;
  r.b.mat[0] = tok_proj;
  r.b.n_per = d;
  r.b.nmat = 1;
  r.out = block_in;          // row 0 of sequence b: block_in[b * gamma * d]
  r.ldo = gamma * d;
  hipError_t e = launch_rowgemm(dtype, RP_NONE, RE_STORE, r, s);
  if (e != hipSuccess || gamma == 1) return e;
  trace_pre(K_BLOCK_ROWS, s);
  mask_rows_kernel<<<dim3(gamma - 1, A), 256, 0, s>>>(mask_emb, gamma, d, block_in);
  trace_post(K_BLOCK_ROWS, s);
  return hipGetLastError();
}

}  // namespace dspark
