// The Markov head, the confidence head and the greedy draft loop after the
// backbone (module-dflash.ts: #markov, #confidence, forwardInfer; the page
// "src/dspark-runtime.js" runs the same steps as markovEmbed -> markov ->
// addBias -> argmax for each drafted position).
//
// For every sequence b, starting from its anchor token, position k of the
// block takes
//   e1       = w1[prev]                       (the previous token's Markov embedding)
//   logits_k = base_logits[b, k] + e1 . w2^T  (w2 stored [vocab, rank])
//   token_k  = argmax logits_k                (the lowest index among equal maxima)
//   conf_k   = sigmoid([block[b, k], e1] . conf_w + conf_b)
// and prev = token_k. The positions depend on each other through the token,
// so the loop runs position by position, all sequences together:
//   the logits of a position are one weight-streaming row GEMM over the A
//   embedding rows (block.hip's row GEMM, with the base logits as its
//   residual; it writes the draft logits output directly);
//   markov_argmax_kernel reduces vocabulary chunks to (max, index) partials;
//   markov_final_kernel picks the token, computes the confidence and gathers
//   the next position's embedding rows.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace dspark {

// Larger value wins; on equal values the lower index (numpy's argmax rule).
DSPARK_DEV void arg_better(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

DSPARK_DEV void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float v2 = __shfl_xor(v, off, kWave);
    const int i2 = __shfl_xor(i, off, kWave);
    arg_better(v, i, v2, i2);
  }
}

// E1[b] = w1[clamp(tok[b])] as float32; one workgroup per sequence.
template <typename S>
__global__ __launch_bounds__(256) void markov_embed_kernel(const S* __restrict__ w1, int vocab, int rank,
                                                           const int32_t* __restrict__ tok,
                                                           float* __restrict__ E1) {
  const int b = blockIdx.x;
  const int t = min(max(tok[b], 0), vocab - 1);
  for (int i = threadIdx.x; i < rank; i += 256) E1[(int64_t)b * rank + i] = to_f32(w1[(int64_t)t * rank + i]);
}

// Partials of one position: grid (P, A); workgroup (p, b) scans vocabulary
// entries [p * chunk, min(vocab, (p+1) * chunk)) of row b of the logits
// (row stride ld) and writes its best (value, index).
__global__ __launch_bounds__(256) void markov_argmax_kernel(const float* __restrict__ logits, int64_t ld,
                                                            int vocab, int chunk, float* __restrict__ pv,
                                                            int32_t* __restrict__ pi) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int p = blockIdx.x, b = blockIdx.y, P = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* row = logits + (int64_t)b * ld;
  const int v0 = p * chunk, v1 = min(vocab, v0 + chunk);
  float best = -__builtin_inff();
  int bi = vocab;
  for (int v = v0 + tid; v < v1; v += 256) arg_better(best, bi, row[v], v);
  wave_argmax(best, bi);
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) arg_better(best, bi, sv[w], si[w]);
    pv[(int64_t)b * P + p] = best;
    pi[(int64_t)b * P + p] = bi;
  }
}

// One wave per sequence: the token of position k from the P partials, the
// confidence of position k (with the embedding rows the position used), and
// the next position's embedding rows E1[b] = w1[token].
template <typename S>
__global__ __launch_bounds__(64) void markov_final_kernel(
    const float* __restrict__ pv, const int32_t* __restrict__ pi, int P, int k, int gamma, int d, int vocab,
    int rank, const float* __restrict__ block, const float* __restrict__ conf_w, const float* __restrict__ conf_b,
    const S* __restrict__ w1, float* __restrict__ E1, int32_t* __restrict__ tokens, float* __restrict__ conf) {
  const int b = blockIdx.x, lane = threadIdx.x;
  float best = -__builtin_inff();
  int bi = vocab;
  for (int q = lane; q < P; q += 64) arg_better(best, bi, pv[(int64_t)b * P + q], pi[(int64_t)b * P + q]);
  wave_argmax(best, bi);
  const int tok = min(max(bi, 0), vocab - 1);
  const float* brow = block + ((int64_t)b * gamma + k) * d;
  float* e = E1 + (int64_t)b * rank;
  float z = 0.f;
  for (int i = lane; i < d; i += 64) z = fmaf(brow[i], conf_w[i], z);
  for (int i = lane; i < rank; i += 64) z = fmaf(e[i], conf_w[d + i], z);
  z = wave_sum(z) + conf_b[0];
  if (lane == 0) {
    tokens[(int64_t)b * gamma + k] = tok;
    conf[(int64_t)b * gamma + k] = 1.f / (1.f + expf(-z));
  }
  // every lane has read its embedding values above (z depends on them)
  for (int i = lane; i < rank; i += 64) e[i] = to_f32(w1[(int64_t)tok * rank + i]);
}

int markov_partials(int vocab) { return std::min(256, std::max(1, (vocab + 2047) / 2048)); }

hipError_t launch_markov(int dtype, const MarkovArgs& a, hipStream_t s) {
  const int P = markov_partials(a.vocab);
  const int chunk = (a.vocab + P - 1) / P;
  trace_pre(K_MARKOV, s);
  if (dtype == 1)
    markov_embed_kernel<bf16><<<a.A, 256, 0, s>>>(static_cast<const bf16*>(a.w1), a.vocab, a.rank, a.anchor, a.E1);
  else
    markov_embed_kernel<float><<<a.A, 256, 0, s>>>(static_cast<const float*>(a.w1), a.vocab, a.rank, a.anchor,
                                                   a.E1);
  trace_post(K_MARKOV, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ld = (int64_t)a.gamma * a.vocab;
  for (int k = 0; k < a.gamma; ++k) {
    // logits_k = base_logits[:, k] + E1 . w2^T, into draft_logits[:, k]
    RowGemmArgs r{};
    r.X = a.E1;
    r.ldx = a.rank;
    r.M = a.A;
    r.K = a.rank;
    r.N = a.vocab;
    r.b.mat[0] = a.w2;
    r.b.n_per = a.vocab;
    r.b.nmat = 1;
    r.res = a.base_logits + (int64_t)k * a.vocab;
    r.out = a.logits + (int64_t)k * a.vocab;
    r.ldo = (int)ld;   // gamma * vocab < 2^31 (checked on the host)
    e = launch_rowgemm(dtype, RP_NONE, RE_RESID, r, s);
    if (e != hipSuccess) return e;
    trace_pre(K_MARKOV, s);
    markov_argmax_kernel<<<dim3(P, a.A), 256, 0, s>>>(a.logits + (int64_t)k * a.vocab, ld, a.vocab, chunk,
                                                     a.part_v, a.part_i);
    if (dtype == 1)
      markov_final_kernel<bf16><<<a.A, 64, 0, s>>>(a.part_v, a.part_i, P, k, a.gamma, a.d, a.vocab, a.rank,
                                                   a.block, a.conf_w, a.conf_b,
                                                   static_cast<const bf16*>(a.w1), a.E1, a.tokens, a.conf);
    else
      markov_final_kernel<float><<<a.A, 64, 0, s>>>(a.part_v, a.part_i, P, k, a.gamma, a.d, a.vocab, a.rank,
                                                    a.block, a.conf_w, a.conf_b,
                                                    static_cast<const float*>(a.w1), a.E1, a.tokens, a.conf);
    trace_post(K_MARKOV, s);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dspark
