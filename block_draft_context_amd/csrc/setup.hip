// The forward's row passes and independent set-up work, in one launch.
//
// After the Eq 2 projection, these pieces of work need nothing but the call's
// inputs and that projection, and none needs another:
//   plan   the split-K attention's tile prefix over the ragged context lengths
//   D0     block_in + block_pos (the block rows entering the first layer)
//   prep   every layer's W_K, W_V stacked into the K/V GEMM's B operand, with
//          the layer's attn_norm gain folded into the columns
//   norm   H_ctx = RMSNorm(sum of the projection's K splits; ctx_norm) and the
//          inverse RMS of each stored row, or, when H_ctx is given, only the
//          inverse RMS ("DFlash draft layer", `#buildContext` and `#layer`);
//          after the fused one-split projection, the row scales from its
//          row sums (and H_ctx only when asked for)
//   zero   clears the per-layer accumulators that the attention output
//          projection adds its heads' shares into
// Each is a range of workgroups of one grid (256 threads, one wave per row),
// so a forward pays one kernel boundary for all of them.
#include "common.h"
#include "kernels.h"

namespace dspark {


// chunk_prefix[b] = sum_{b' < b} max(1, ceil(L_b' / chunk)) for b = 0..A. An
// empty sequence still gets one tile, which finds no keys and leaves an empty
// partial. One workgroup.
__device__ __forceinline__ void plan_role(const int32_t* __restrict__ cu, int A, int chunk,
                                          int32_t* __restrict__ prefix, int32_t* sums) {
  const int tid = threadIdx.x;
  const int per = (A + 255) / 256;
  const int b0 = tid * per, b1 = min(A, b0 + per);
  int32_t local = 0;
  for (int b = b0; b < b1; ++b) {
    const int32_t L = cu[b + 1] - cu[b];
    local += L > 0 ? (L + chunk - 1) / chunk : 1;
  }
  sums[tid] = local;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {   // inclusive scan
    const int32_t v = tid >= off ? sums[tid - off] : 0;
    __syncthreads();
    sums[tid] += v;
    __syncthreads();
  }
  int32_t run = tid > 0 ? sums[tid - 1] : 0;
  for (int b = b0; b < b1; ++b) {
    prefix[b] = run;
    const int32_t L = cu[b + 1] - cu[b];
    run += L > 0 ? (L + chunk - 1) / chunk : 1;
  }
  if (tid == 255) prefix[A] = sums[255];
}

// D0[r] = block_in[r] + block_pos[r % gamma]; one wave per row, d / 256
// float4 per lane.
__device__ __forceinline__ void d0_row(const SetupArgs& a, int r, int lane) {
  const int j = r % a.gamma;
  const f32x4* __restrict__ bin = reinterpret_cast<const f32x4*>(a.block_in + (int64_t)r * a.d);
  const f32x4* __restrict__ pos = reinterpret_cast<const f32x4*>(a.block_pos + (int64_t)j * a.d);
  f32x4* __restrict__ out = reinterpret_cast<f32x4*>(a.D0 + (int64_t)r * a.d);
  for (int c = lane; c < a.d / 4; c += 64) out[c] = bin[c] + pos[c];
}

// Bt[row][k] = W[n][k] * g[k] (row = matrix mi, output feature n); one wave
// per row, all of the row's 16-byte loads issued before any store (K <= 2048
// gives at most four per lane).
__device__ __forceinline__ void prep_row(const SetupArgs& a, int row, int lane) {
  const int K = a.d;
  const int mi = row / a.b.n_per, n = row % a.b.n_per;
  const bf16* __restrict__ W = static_cast<const bf16*>(a.b.mat[mi]) + (int64_t)n * K;
  const float* __restrict__ g = a.b.gain[mi];
  bf16* __restrict__ out = static_cast<bf16*>(a.Bt) + (int64_t)row * K;
  const int nc = K / 8;   // 16-byte chunks in the row
  u32x4 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (lane + 64 * i < nc) w[i] = ld16(W + 8 * (lane + 64 * i));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + 64 * i;
    if (c >= nc) break;
    float f[8];
    Vec16<bf16>::unpack(w[i], f);
    if (g) {
      const f32x4 g0 = reinterpret_cast<const f32x4*>(g)[2 * c];
      const f32x4 g1 = reinterpret_cast<const f32x4*>(g)[2 * c + 1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] *= g0[e];
        f[4 + e] *= g1[e];
      }
    }
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = from_f32<bf16>(f[e]);
    *reinterpret_cast<bf16x8*>(out + 8 * c) = o;
  }
}

// H_ctx row t = RMSNorm(sum_z part[z][t]; g) in the storage type, and the
// inverse RMS of the row as stored. Lane l owns the 8-column chunks l + 64 i,
// i < CPL = ceil(d / 512); the loads of SB splits are issued together, and
// a chunk leaves as one 16-byte store (bf16) or two (float32).
template <typename S, int CPL>
__device__ __forceinline__ void norm_row(const SetupArgs& a, int64_t t, int lane) {
  constexpr int SB = 8 / CPL > 0 ? 8 / CPL : 1;   // splits per batch: <= 16 float4 in flight
  const int d = a.d, nch = d / 8;
  const int64_t T = a.T;
  f32x4 acc[CPL][2];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int z0 = 0; z0 < a.splits; z0 += SB) {
    f32x4 x[SB][CPL][2];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      const int zz = min(z0 + sb, a.splits - 1);
      const f32x4* row = reinterpret_cast<const f32x4*>(a.part + ((int64_t)zz * T + t) * d);
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = min(lane + 64 * i, nch - 1);
        x[sb][i][0] = row[2 * c];
        x[sb][i][1] = row[2 * c + 1];
      }
    }
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
      if (z0 + sb < a.splits) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          acc[i][0] += x[sb][i][0];
          acc[i][1] += x[sb][i][1];
        }
      }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i)
    if (lane + 64 * i < nch)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += acc[i][h2][e] * acc[i][h2][e];
  ss = wave_sum(ss);
  const float sc = rsqrtf(ss / (float)d + a.eps);
  const f32x4* g4 = reinterpret_cast<const f32x4*>(a.g);
  float ss2 = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      float o[8];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const f32x4 gv = g4[2 * c + h2];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[4 * h2 + e] = to_f32(from_f32<S>(acc[i][h2][e] * sc * gv[e]));
          ss2 += o[4 * h2 + e] * o[4 * h2 + e];
        }
      }
      S* h = static_cast<S*>(a.h) + t * d + 8 * c;
      if constexpr (sizeof(S) == 2) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = from_f32<bf16>(o[e]);
        *reinterpret_cast<bf16x8*>(h) = v;
      } else {
        reinterpret_cast<f32x4*>(h)[0] = f32x4{o[0], o[1], o[2], o[3]};
        reinterpret_cast<f32x4*>(h)[1] = f32x4{o[4], o[5], o[6], o[7]};
      }
    }
  }
  if (a.rinv) {
    ss2 = wave_sum(ss2);
    if (lane == 0) a.rinv[t] = a.rinv_one ? 1.f : rsqrtf(ss2 / (float)d + a.eps);
  }
}

// rinv[t] = inverse RMS of a given H_ctx row; d / 64 <= 32 values per lane,
// loaded together.
template <typename S>
__device__ __forceinline__ void stats_row(const SetupArgs& a, int64_t t, int lane) {
  const int d = a.d;
  const S* __restrict__ h = static_cast<const S*>(a.h_in);
  const int nv = d / 64;
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = to_f32(h[t * d + min(i, nv - 1) * 64 + lane]);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if (i < nv) ss += x[i] * x[i];
  ss = wave_sum(ss);
  if (lane == 0) a.rinv[t] = a.rinv_one ? 1.f : rsqrtf(ss / (float)d + a.eps);
}

// After the fused Eq 2 epilogue (bf16): the row's sums of P^2 and of the
// stored Y^2 over its nts column tiles give
//   ms = mean P^2 + eps,      H_ctx = Y / sqrt(ms)
//   mean H^2 = (mean Y^2) / ms, so the layer norm of an H_ctx row scales Y by
//   1 / (sqrt(ms) * sqrt(mean H^2 + eps)) = 1 / sqrt(mean Y^2 + eps * ms)
// which is the K/V product's row scale for Y rows (1 / sqrt(ms) when the
// context rows enter W_K / W_V unnormalised).
struct RowScales {
  float inv_rms, kv;
};
__device__ __forceinline__ RowScales fused_scales(const SetupArgs& a, int64_t t) {
  const f32x2* sm = reinterpret_cast<const f32x2*>(a.rsum) + t * a.nts;
  float sp = 0.f, sy = 0.f;
  for (int i = 0; i < a.nts; ++i) {
    const f32x2 v = sm[i];
    sp += v[0];
    sy += v[1];
  }
  const float ms = sp / (float)a.d + a.eps;
  RowScales r;
  r.inv_rms = rsqrtf(ms);
  r.kv = a.rinv_one ? r.inv_rms : rsqrtf(sy / (float)a.d + a.eps * ms);
  return r;
}

// One thread per row: the row scale only.
__device__ __forceinline__ void fused_rinv(const SetupArgs& a, int64_t t) {
  a.rinv[t] = fused_scales(a, t).kv;
}

// One wave per row: the row scale and H_ctx = Y / rms(P), bf16, a 16-byte
// vector of 8 columns per lane and step.
__device__ __forceinline__ void fused_h_row(const SetupArgs& a, int64_t t, int lane) {
  const RowScales r = fused_scales(a, t);
  if (a.rinv && lane == 0) a.rinv[t] = r.kv;
  const bf16* y = static_cast<const bf16*>(a.y) + t * a.d;
  bf16* h = static_cast<bf16*>(a.h) + t * a.d;
  for (int c = lane; c < a.d / 8; c += 64) {
    float f[8];
    Vec16<bf16>::unpack(ld16(y + 8 * c), f);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = from_f32<bf16>(f[e] * r.inv_rms);
    *reinterpret_cast<bf16x8*>(h + 8 * c) = o;
  }
}

// A tail row of the fused path (t >= tail_from): P = the sum of its K
// splits, then what the fused epilogue and fused_h_row do for the other
// rows: Y = bf16(P * g) stored for the K/V product, the row scale, and H_ctx
// when asked for. Lane l owns the 8-column chunks l + 64 i, i < CPL.
template <int CPL>
__device__ __forceinline__ void fused_tail_row(const SetupArgs& a, int64_t t, int lane) {
  const int d = a.d, nch = d / 8;
  const int64_t Tt = a.T - a.tail_from, r = t - a.tail_from;
  f32x4 acc[CPL][2];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < a.tail_splits; ++z) {
    const f32x4* row = reinterpret_cast<const f32x4*>(a.tail_part + ((int64_t)z * Tt + r) * d);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = min(lane + 64 * i, nch - 1);
      acc[i][0] += row[2 * c];
      acc[i][1] += row[2 * c + 1];
    }
  }
  const f32x4* g4 = reinterpret_cast<const f32x4*>(a.g);
  bf16* y = static_cast<bf16*>(const_cast<void*>(a.y)) + t * d;
  float sp = 0.f, sy = 0.f;
  float yv[CPL][8];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      bf16x8 o;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const f32x4 gv = g4[2 * c + h2];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = acc[i][h2][e];
          const bf16 q = from_f32<bf16>(p * gv[e]);
          yv[i][4 * h2 + e] = static_cast<float>(q);
          o[4 * h2 + e] = q;
          sp += p * p;
          sy += yv[i][4 * h2 + e] * yv[i][4 * h2 + e];
        }
      }
      *reinterpret_cast<bf16x8*>(y + 8 * c) = o;
    }
  }
  sp = wave_sum(sp);
  sy = wave_sum(sy);
  const float ms = sp / (float)d + a.eps;
  const float inv_rms = rsqrtf(ms);
  if (a.rinv && lane == 0) a.rinv[t] = a.rinv_one ? inv_rms : rsqrtf(sy / (float)d + a.eps * ms);
  if (a.h) {
    bf16* h = static_cast<bf16*>(a.h) + t * d;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      if (c < nch) {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = from_f32<bf16>(yv[i][e] * inv_rms);
        *reinterpret_cast<bf16x8*>(h + 8 * c) = o;
      }
    }
  }
}

// Cache row map: new row r belongs to the sequence b with ncu[b] <= r <
// ncu[b+1] (the last b with ncu[b] <= r, which skips empty sequences) and
// lands at slab row b * cap + pos[b] + (r - ncu[b]). One thread per row.
__device__ __forceinline__ void map_rows(const SetupArgs& a, int64_t r) {
  int lo = 0, hi = a.A - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.ncu[mid] <= r) lo = mid; else hi = mid - 1;
  }
  a.dst_row[r] = (int32_t)((int64_t)lo * a.cap + a.pos[lo] + (r - a.ncu[lo]));
}

// Workgroup ranges, in dispatch order: [plan][map][zero][D0][prep][norm].
// The small roles come first so that none of them lands in the grid's tail.
struct SetupGrid {
  int plan, map, zero, d0, prep, norm, tail;
  int total() const { return plan + map + zero + d0 + prep + norm + tail; }
};
constexpr int kZeroPerBlock = 256 * 4 * 4;   // floats cleared per workgroup

static SetupGrid setup_grid(const SetupArgs& a) {
  SetupGrid g;
  g.plan = a.prefix ? 1 : 0;
  g.map = a.dst_row ? (int)((a.map_T + 255) / 256) : 0;
  g.zero = a.zero ? (int)((a.zero_n + kZeroPerBlock - 1) / kZeroPerBlock) : 0;
  g.d0 = a.D0 ? (a.A * a.gamma + 3) / 4 : 0;
  g.prep = a.Bt ? (a.b.n_per * a.b.nmat + 3) / 4 : 0;
  const int64_t rows = a.tail_part ? a.tail_from : a.T;   // rows of the norm role
  if (a.rsum) g.norm = a.h ? (int)((rows + 3) / 4) : (int)((rows + 255) / 256);
  else g.norm = (a.part || a.h_in) ? (int)((a.T + 3) / 4) : 0;
  g.tail = a.tail_part ? (int)((a.T - a.tail_from + 3) / 4) : 0;
  return g;
}

template <typename S, int CPL>
__global__ __launch_bounds__(256) void setup_kernel(SetupArgs a, SetupGrid sg) {
  __shared__ int32_t sums[256];
  int blk = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  if (blk < sg.plan) {
    plan_role(a.cu, a.A, a.chunk, a.prefix, sums);
    return;
  }
  blk -= sg.plan;
  if (blk < sg.map) {
    const int64_t r = (int64_t)blk * 256 + threadIdx.x;
    if (r < a.map_T) map_rows(a, r);
    return;
  }
  blk -= sg.map;
  if (blk < sg.zero) {
    f32x4* z = reinterpret_cast<f32x4*>(a.zero) + (int64_t)blk * (kZeroPerBlock / 4);
    const int64_t n4 = a.zero_n / 4 - (int64_t)blk * (kZeroPerBlock / 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = i * 256 + threadIdx.x;
      if (e < n4) z[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  blk -= sg.zero;
  if (blk < sg.d0) {
    const int r = blk * 4 + w;
    if (r < a.A * a.gamma) d0_row(a, r, lane);
    return;
  }
  blk -= sg.d0;
  if (blk < sg.prep) {
    if constexpr (sizeof(S) == 2) {
      const int row = blk * 4 + w;
      if (row < a.b.n_per * a.b.nmat) prep_row(a, row, lane);
    }
    return;
  }
  blk -= sg.prep;
  if (blk >= sg.norm) {   // tail rows of the fused path
    if constexpr (sizeof(S) == 2) {
      const int64_t t = a.tail_from + (int64_t)(blk - sg.norm) * 4 + w;
      if (t < a.T) fused_tail_row<CPL>(a, t, lane);
    }
    return;
  }
  const int64_t rows = a.tail_part ? a.tail_from : a.T;
  if (a.rsum && !a.h) {
    const int64_t t = (int64_t)blk * 256 + threadIdx.x;
    if (t < rows && a.rinv) fused_rinv(a, t);
    return;
  }
  const int64_t t = (int64_t)blk * 4 + w;
  if (t >= rows) return;
  if (a.rsum) {
    if constexpr (sizeof(S) == 2) fused_h_row(a, t, lane);
  } else if (a.part)
    norm_row<S, CPL>(a, t, lane);
  else
    stats_row<S>(a, t, lane);
}

// cu[b] = b * L for b = 0 .. A (the offsets of a padded batch)
__global__ __launch_bounds__(256) void fill_offsets_kernel(int32_t* __restrict__ cu, int A, int L) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b <= A) cu[b] = b * L;
}

hipError_t launch_fill_offsets(int32_t* cu, int A, int L, hipStream_t s) {
  trace_pre(K_SETUP, s);
  fill_offsets_kernel<<<(A + 1 + 255) / 256, 256, 0, s>>>(cu, A, L);
  trace_post(K_SETUP, s);
  return hipGetLastError();
}

hipError_t launch_setup(int dtype, const SetupArgs& a, hipStream_t s) {
  if (a.Bt && dtype != 1) return hipErrorInvalidValue;   // prep serves the bf16 MFMA path only
  if (a.rsum && (dtype != 1 || !a.y)) return hipErrorInvalidValue;   // the fused Eq 2 path is bf16
  if (a.tail_part && (!a.rsum || a.tail_splits < 1 || a.tail_from < 0 || a.tail_from > a.T || !a.g))
    return hipErrorInvalidValue;
  const SetupGrid sg = setup_grid(a);
  if (sg.total() == 0) return hipSuccess;
  trace_pre(K_SETUP, s);
  const int cpl = (a.d / 8 + 63) / 64;   // 8-column chunks per lane, d <= 2048
#define DSPARK_SETUP(C)                                                    \
  if (cpl == C) {                                                          \
    if (dtype == 1) setup_kernel<bf16, C><<<sg.total(), 256, 0, s>>>(a, sg); \
    else setup_kernel<float, C><<<sg.total(), 256, 0, s>>>(a, sg);           \
  }
  DSPARK_SETUP(1)
  DSPARK_SETUP(2)
  DSPARK_SETUP(3)
  DSPARK_SETUP(4)
#undef DSPARK_SETUP
  trace_post(K_SETUP, s);
  return hipGetLastError();
}

}  // namespace dspark
