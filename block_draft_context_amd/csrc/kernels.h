// Internal launcher interface between the C ABI (dspark.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dspark {

constexpr int kMaxSegs = 16;     // tapped layers (A-operand segments)
constexpr int kMaxMats = 32;     // weight matrices in one batched launch (2 per layer)
constexpr int kMaxGamma = 16;

enum KernelKind : int {
  K_GEMM_CTX = 0,     // Eq 2 projection X . W_c (split-K partials)
  K_SETUP,            // Eq 2 RMSNorm row pass (or row statistics) + K/V weight prep,
                      // attention tile plan and D0, in one launch
  K_GEMM_KV,          // Eq 3 context K/V re-projection (all layers at once)
  K_ATTN,             // split-K attention partials over context chunks
  K_COMBINE,          // (m, l) combine of the partials + block keys
  K_ROWGEMM,          // block-row projections (weight streaming, fused norm/epilogue)
  K_BLOCK_ROWS,       // D0 = block_in + block_pos and row norms
  K_MARKOV,           // Markov draft loop: embedding gathers, argmax partials, token + confidence
  K_COUNT
};

// Scratch of the no-allocation entry point: a file-scope device array of
// this many bytes (noalloc.hip); noalloc_scratch gives its device address on
// the current device (taken once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

const char* kernel_name(int kind);
void trace_pre(int kind, hipStream_t s);
void trace_post(int kind, hipStream_t s);

// A operand split along K into segments of equal width (the m taps):
// A(r, k) = seg[k / seg_k][r * ld + k % seg_k].
struct ASegs {
  const void* seg[kMaxSegs];
  int64_t ld;
  int32_t seg_k;
  int32_t nseg;
};

// B operand made of several [K, n_per] matrices side by side (column n lives in
// mat[n / n_per]); an optional per-k gain g[n / n_per][k] scales row k.
struct BMats {
  const void* mat[kMaxMats];
  const float* gain[kMaxMats];
  int32_t n_per;
  int32_t nmat;
};

// Attention-side layout of the context K and V (per layer, per head):
// see kv_layout.h. Tpad is T rounded up to 64.
// Two ways of placing context rows in a slab:
//   packed (seq_stride = 0): sequence b owns rows cu[b] .. cu[b+1]-1, as the
//     packed context of one forward; the K/V product writes row r at r and
//     zeros at T .. Tpad-1;
//   cache (seq_stride = cap): sequence b owns rows b*cap .. b*cap + L_b - 1
//     of an append-only draft cache; the K/V product writes new row r at
//     dst_row[r] and nothing past its T new rows.
struct KVDesc {
  void* base;        // [n_layers][2][n_heads][Tpad][hd] in tiled order
  int64_t Tpad;      // rows per slab (A * cap for a cache)
  int32_t T;         // rows the K/V product writes (packed: context rows; cache: new rows)
  int32_t hd;
  int32_t n_heads;
  int64_t seq_stride = 0;          // attention: 0 = packed by cu, else cache rows per sequence
  const int32_t* dst_row = nullptr;  // K/V product into a cache: slab row of each new row
  const uint8_t* key_mask = nullptr; // attention: slab row t is a key only where key_mask[t] != 0
};

// ---- set-up pass ----------------------------------------------------------
// One launch of independent roles, each skipped when its output is null:
//   prefix  attention tile prefix from cu (see launch_attention)
//   D0      [A*gamma][d] = block_in + block_pos[row % gamma]
//   Bt      bf16 only: [n_per * nmat rows][d] copy of b's [out, in] matrices
//           with b.gain folded into the columns
//   h       part != null: h[t] = RMSNorm(sum_z part[z][t]; g), rinv[t] = inverse
//           RMS of the stored row (rinv nullable); part == null and h_in != null:
//           only rinv[t] of the given rows
//   zero    zero[0 .. zero_n) = 0 (zero_n a multiple of 4)
struct SetupArgs {
  int d = 0;
  float eps = 0.f;
  // plan
  const int32_t* cu = nullptr;
  int A = 0, chunk = 0;
  int32_t* prefix = nullptr;
  // D0
  const float* block_in = nullptr;
  const float* block_pos = nullptr;
  int gamma = 0;
  float* D0 = nullptr;
  // K/V weight prep
  BMats b{};
  void* Bt = nullptr;
  // row pass over the T context rows
  int64_t T = 0;
  const float* part = nullptr;
  int splits = 0;
  const float* g = nullptr;
  void* h = nullptr;
  const void* h_in = nullptr;
  float* rinv = nullptr;
  bool rinv_one = false;   // the context rows enter W_K / W_V unnormalised: rinv[t] = 1
  // or, after the fused Eq 2 epilogue: its row sums [T][nts][2] (sum P^2,
  // sum Y^2) and Y = bf16(P * ctx_norm); rinv[t] is then the K/V product's
  // row scale for Y rows, and h (if given) receives H_ctx = Y / rms(P)
  const float* rsum = nullptr;
  int nts = 0;
  const void* y = nullptr;
  // rows [tail_from, T) of the fused path come as tail_splits float32 K
  // partials [tail_splits][T - tail_from][d]: summed here into Y and the row
  // scales (tail_part null: no tail)
  const float* tail_part = nullptr;
  int tail_splits = 0;
  int64_t tail_from = 0;
  // cleared buffer
  float* zero = nullptr;
  int64_t zero_n = 0;
  // cache row map: new row r of sequence b (rows ncu[b] .. ncu[b+1]-1) goes
  // to slab row b * cap + pos[b] + (r - ncu[b]); map_T new rows
  const int32_t* ncu = nullptr;
  const int32_t* pos = nullptr;
  int32_t cap = 0;
  int64_t map_T = 0;
  int32_t* dst_row = nullptr;
};
hipError_t launch_setup(int dtype, const SetupArgs& a, hipStream_t s);
// cu[b] = b * L for b = 0 .. A
hipError_t launch_fill_offsets(int32_t* cu, int A, int L, hipStream_t s);

// ---- context side -------------------------------------------------------
// K splits of the Eq 2 projection for these sizes (sizes the partial
// buffer): split z covers columns [z * k_per_split, min(K, (z+1) * k_per_split)),
// with splits * k_per_split >= K and every split non-empty.
struct CtxSplit {
  int splits = 1;
  int k_per_split = 0;
  // one split on the big-tile kernel: its epilogue writes Y = P * ctx_norm
  // (bf16) and per-row sums instead of float32 partials
  bool fused = false;
  // fused, when its 256x256 tiles would leave the last round of the CUs at
  // most half filled: rows [tail_row, M) run instead as tail_splits K splits
  // of tail_kps columns (float32 partials), which the set-up pass sums and
  // finishes like the fused epilogue; tail_row = M when there is no tail
  int64_t tail_row = 0;
  int tail_splits = 0, tail_kps = 0;
};
CtxSplit ctx_gemm_split(int dtype, int64_t M, int N, int K);
// Where the Eq 2 product goes. Split-K: part[z][r][n] = sum_{k in split z}
// A(r,k) B(k,n) in float32. Fused: y[r][n] = bf16(P[r][n] * g[n]) and
// sums[r][n / 256] = (sum P^2, sum y^2) over that 256-column tile.
struct CtxOut {
  float* part = nullptr;
  void* y = nullptr;
  float* sums = nullptr;
  const float* g = nullptr;
  float* tail_part = nullptr;   // [tail_splits][M - tail_row][N] with a fused tail
};
hipError_t launch_gemm_ctx(int dtype, const ASegs& a, const BMats& b, const void* Bt, const CtxOut& o,
                           int M, int N, int K, const CtxSplit& sp, hipStream_t s);
constexpr int kCtxSumCols = 256;   // columns per row-sum pair of the fused Eq 2 epilogue

// K/V for all layers of `b` (2 matrices per layer: K then V) from H_ctx with
// the row scale rinv, written in the attention layout of `kv`.
// K = d input columns; kvd = K/V heads * hd output columns per K or V block.
hipError_t launch_gemm_kv(int dtype, const void* h_ctx, const BMats& b, const void* Bt,
                          const float* rinv, const KVDesc& kv, int d, int kvd, int n_layers,
                          hipStream_t s);

// ---- attention ------------------------------------------------------------
int attention_chunk(const int32_t* cu_host, int A, int n_heads);   // keys per chunk (multiple of 64)
// tiles = sum_b max(1, ceil(L_b / chunk)); the device prefix of the same sum
// comes from the set-up pass
int64_t attention_tiles(const int32_t* cu_host, int A, int chunk);

struct AttnArgs {
  const float* Q;       // [A*gamma][d], pre-scaled by hd^-1/2 * log2(e)
  const float* Kd;      // [A*gamma][kvd] block keys (kvd = kv.n_heads * hd)
  const float* Vd;      // [A*gamma][kvd] block values
  KVDesc kv;            // context K/V (attention layout; kv.n_heads = K/V heads)
  int n_heads;          // query heads (a multiple of kv.n_heads)
  int layer;
  const int32_t* cu;    // device prefix offsets [A+1]
  const int32_t* prefix;  // device tile prefix [A+1]
  int A, gamma, chunk, total_tiles;
  float* part_o;        // [tiles][n_heads][gamma][hd]
  float* part_ml;       // [tiles][n_heads][gamma][2]
  float* attn;          // out: Attn [A*gamma][d], the heads' outputs concatenated
};
// partial kernel, then the (m, l) combine into Attn
hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t s);

// ---- block side -----------------------------------------------------------
// Y = prologue(X) . W with a fused epilogue, full K per workgroup (32 columns).
enum RowPro { RP_NONE = 0, RP_RMSNORM = 1 };
// RE_SWIGLU: the columns are (gate, up) pairs: b.mat[0] = W_gate and
// b.mat[1] = W_up, both [n_per][K]; out[m][c] = SiLU(gate_c) * up_c, c < n_per.
enum RowEpi { RE_STORE = 0, RE_QKV = 1, RE_RESID = 2, RE_SWIGLU = 3 };
struct RowGemmArgs {
  const float* X = nullptr;   // [M][ldx]
  int ldx = 0;
  int M = 0, K = 0, N = 0;
  const float* g = nullptr;   // RP_RMSNORM gain [K]
  float eps = 0.f;
  BMats b{};                  // weights [out, in]: N rows of K over b.nmat matrices
  float* out = nullptr;       // RE_STORE / RE_RESID / RE_SWIGLU: out[m][n] (row stride ldo)
  int ldo = 0;
  const float* res = nullptr; // RE_RESID: out = res + X.W
  float* q = nullptr;         // RE_QKV: columns [0,d) -> q (scaled), [d,d+kvd) -> kd, [d+kvd,d+2kvd) -> vd
  float* kd = nullptr;
  float* vd = nullptr;
  int d = 0;
  int kvd = 0;                // K/V columns (grouped K/V heads: fewer than d)
  float qscale = 1.f;
  int act = 0;                // RE_SWIGLU: 0 = SiLU(gate) * up, 1 = tanh-GELU(gate) * up
};
int rowgemm_rows_per_pass(int K);
hipError_t launch_rowgemm(int dtype, int pro, int epi, const RowGemmArgs& a, hipStream_t s);
// D0 = block_in + block_pos (per sequence; block_pos, D0 nullable);
// U0 = RMSNorm(D0; g) (nullable).
hipError_t launch_block_rows(const float* block_in, const float* block_pos, int A, int gamma,
                             int d, const float* g, float eps, float* D0, float* U0,
                             hipStream_t s);

// #buildBlock's token rows: block_in[b][0] = anchor_emb[b] . tok_proj^T
// (tok_proj [d][H] storage type), block_in[b][j] = mask_emb[j-1] for j >= 1.
hipError_t launch_block_build(int dtype, const float* anchor_emb, int A, int H, const void* tok_proj,
                              const float* mask_emb, int gamma, int d, float* block_in, hipStream_t s);

// ---- layer variant: per-head norms and rotary positions -------------------
constexpr int kMaxLayers = 16;
// Block rows: Q [M][n_heads * hd], Kd [M][n_kv * hd]; q_norm / k_norm [hd]
// (nullable: no norm); rope != 0 rotates at L_b + j (cu: prefix offsets of
// the context lengths); Q is scaled by qscale last.
struct QkPostArgs {
  float* Q = nullptr;
  float* Kd = nullptr;
  int M = 0, gamma = 0, n_heads = 0, n_kv = 0, hd = 0;
  const float* q_norm = nullptr;
  const float* k_norm = nullptr;
  float eps = 0.f;
  int rope = 0;
  double log2_theta = 0.0;
  const int32_t* cu = nullptr;
  float qscale = 1.f;
};
hipError_t launch_qk_post(const QkPostArgs& a, hipStream_t s);
// Context keys in place (attention layout, every layer of the slab set):
// the T rows the K/V product wrote, slab row dst_row[r] at position
// dst_row[r] % cap (a cache), or row r of a packed context at r - cu[b].
struct KPostArgs {
  void* base = nullptr;
  int64_t Tpad = 0;
  int64_t T = 0;
  int n_kv = 0, hd = 0, n_layers = 0;
  const float* k_norm[kMaxLayers] = {};   // per layer, nullable
  float eps = 0.f;
  int rope = 0;
  double log2_theta = 0.0;
  const int32_t* cu = nullptr;
  int A = 1;
  const int32_t* dst_row = nullptr;
  int64_t cap = 0;
};
hipError_t launch_k_post(int dtype, const KPostArgs& a, hipStream_t s);

// ---- Markov head, confidence head, greedy draft loop ----------------------
struct MarkovArgs {
  int A = 0, gamma = 0, d = 0, vocab = 0, rank = 0;
  const float* block = nullptr;        // [A][gamma][d]
  const float* base_logits = nullptr;  // [A][gamma][vocab]
  const int32_t* anchor = nullptr;     // [A]
  const void* w1 = nullptr;            // [vocab][rank] storage type
  const void* w2 = nullptr;            // [vocab][rank] storage type ([out, in])
  const float* conf_w = nullptr;       // [d + rank]
  const float* conf_b = nullptr;       // [1]
  int32_t* tokens = nullptr;           // [A][gamma]
  float* conf = nullptr;               // [A][gamma]
  float* logits = nullptr;             // [A][gamma][vocab]: the draft logits
  float* E1 = nullptr;                 // workspace [A][rank] (the row-GEMM path only)
  float* part_v = nullptr;             // workspace [A][markov_grid(...).P]; the matrix-core
                                       // path: [2][A][P] (value, index) pairs
  int32_t* part_i = nullptr;
};
// Vocabulary chunks of one position: P chunks of `chunk` rows, each reduced
// to one (max, index) partial per sequence; mfma: the matrix-core logits
// kernel runs (bf16 weights, rank a multiple of 64 up to 512).
struct MarkovGrid {
  int P = 0, chunk = 0;
  bool mfma = false;
};
MarkovGrid markov_grid(int dtype, int vocab, int rank, int A);
hipError_t launch_markov(int dtype, const MarkovArgs& a, hipStream_t s);

}  // namespace dspark
