/*
 * dspark.h -- C ABI of the MI355X (gfx950) draft-block forward library.
 *
 * The library computes the DSpark / DFlash draft block with KV-injected
 * context, as stated on the page "mlx-bun 0.0.7 -> 0.0.9,
 * package/src/spec/dspark/module-dflash.ts" (header comment, Eq 2 and Eq 3;
 * methods #buildContext, #layer and #backbone of DflashDrafter):
 *
 *   Eq 2   H_ctx = RMSNorm(W_c . [H^{l1}; ...; H^{lm}]; ctx_norm)
 *   Eq 3   per draft layer i, with U = RMSNorm(D; attn_norm_i) on the block rows
 *          and Uc = RMSNorm(H_ctx; attn_norm_i) on the context rows:
 *            Q = U Wq,  K = [Uc Wk ; U Wk],  V = [Uc Wv ; U Wv]
 *            Attn = softmax(Q K^T / sqrt(hd)) V   per head, no causal mask
 *            E  = D + Attn Wo
 *            D' = E + (SiLU(Z Wgate) * (Z Wup)) Wdown,   Z = RMSNorm(E; ff_norm_i)
 *   output out = RMSNorm(D^N; out_norm)
 *
 * The gated FFN uses SiLU on the gate half as the page "src/dspark-runtime.js"
 * does (its propose() runs upGate -> silu -> down for every draft layer).
 * RMSNorm(x; g) = x * (mean_k x_k^2 + eps)^(-1/2) * g.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every matrix is row-major [out, in] and applied as y = x W^T. This is
 *   this library's own choice, not the pages': module-dflash.ts
 *   (initFromDims) keeps the parameters as [in, out] and computes x @ W, so
 *   its W is this W^T. With [out, in] an output feature's weights are one
 *   contiguous run over the input: the block-side products then read 1 KiB
 *   per wave load instead of 64 scattered lines, and W_c is directly the
 *   K-contiguous operand of the Eq 2 matrix-core product, with no per-call
 *   transpose. Norm gains are float32 [d].
 * - dims->dtype is the storage type of the long tensors: the taps, W_c, every
 *   layer matrix and H_ctx. DSPARK_BF16 means bfloat16 storage with float32
 *   accumulation; DSPARK_F32 means float32 everywhere.
 * - Block rows (block_in, d_in, d_out, block_out) and block_pos are always
 *   float32, laid out [A, gamma, d].
 * - Packing: A sequences share one context axis of T = cu[A] rows. cu holds
 *   A+1 int32 prefix offsets, cu[0] = 0, non-decreasing; sequence b owns
 *   rows cu[b] .. cu[b+1]-1 and attends only to them (the exact exclusion
 *   that the key-padding bias of #maskBias gives). L_b = 0 is allowed: the
 *   block then attends to its own gamma rows only. cu_host (host memory) and
 *   cu_dev (device memory) must hold the same values; cu_host is read during
 *   the call for validation and launch planning, cu_dev by the kernels.
 * - Every device pointer must be 16-byte aligned; host arrays (cu_host,
 *   taps, layers) are read only during the call.
 * - The caller owns all memory. Scratch lives in the caller's workspace
 *   (ws, ws_bytes); its size comes from dspark_workspace_size for the same
 *   operation, dims, A and cu. Calls that may run concurrently need distinct
 *   workspaces. The library allocates no device memory on these paths.
 * - stream is a hipStream_t (NULL = the default stream). Calls enqueue work
 *   and return without synchronising the device.
 * - Repeatability: every output is bitwise the same from call to call for
 *   the same inputs and sizes (no float atomics; every sum has a fixed
 *   order). Different sizes may take different kernels or splits and so
 *   round differently.
 * - Errors: on any non-OK status nothing has been enqueued and no output has
 *   been written; dspark_last_error() returns a message for the calling
 *   thread. A failed kernel launch returns DSPARK_EHIP (work enqueued before
 *   it in the same call may already run).
 * - Supported: head_dim = d / n_heads in {32, 64, 128}; 1 <= gamma <= 16;
 *   1 <= m <= 16; 1 <= n_layers <= 16; H a multiple of 64; d a multiple of
 *   128 up to 2048; ff a multiple of 128 up to 16256; A * gamma <= 1024;
 *   each tap spans less than 4 GiB (T * ld_tap elements), and so do H_ctx
 *   (T * d elements) and, for the calls that run Eq 2, W_c (d * m * H
 *   elements): the context projections address them with 32-bit byte
 *   offsets. Larger inputs return DSPARK_EUNSUPPORTED.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSPARK_OK = 0,
  DSPARK_EINVAL = 1,        /* bad argument: NULL, misaligned, inconsistent sizes */
  DSPARK_EUNSUPPORTED = 2,  /* valid but not built: head_dim, gamma, dtype ... */
  DSPARK_EWORKSPACE = 3,    /* ws_bytes below dspark_workspace_size */
  DSPARK_EHIP = 4           /* a HIP runtime call or kernel launch failed */
} dspark_status;

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

typedef enum {
  DSPARK_OP_CTX_FUSE = 0,
  DSPARK_OP_BLOCK_LAYER = 1,
  DSPARK_OP_BLOCK_FORWARD = 2,
  DSPARK_OP_CTX_APPEND = 3,     /* cu_host = offsets of the new rows (ncu_host) */
  DSPARK_OP_BLOCK_PROPOSE = 4   /* cu_host = offsets of the cached lengths */
} dspark_op;

/* The layer variant of the page "src/dspark-runtime.js" (its per-layer
 * q_norm / k_norm weights, noiseNormRope / contextNormRope kernels, K/V
 * heads fewer than query heads, and a context K/V projection with no
 * per-layer norm), as switches on top of module-dflash.ts's #layer:
 *   DSPARK_QK_NORM       RMSNorm over each head of the queries and keys (block
 *                        and context) with the layer's q_norm / k_norm [hd] gains
 *   DSPARK_PLAIN_CTX_KV  the context rows enter W_K / W_V as Eq 2 leaves them
 *                        (no attn_norm on the context side)
 *   DSPARK_GELU_FFN      the gated FFN's activation is tanh-GELU (module-dflash.ts
 *                        geluApprox) instead of SiLU
 * plus dims->rope_theta > 0 (rotary positions with base theta on queries and
 * keys, pairs (c, c + hd/2), angle pos * theta^(-2c/hd); context row t of a
 * sequence at position t, block row j at L_b + j) and dims->n_kv_heads (query
 * head h reads K/V head h / (n_heads / n_kv_heads)). The positions and pairing
 * are this library's reading: the page prints no formula. */
typedef enum {
  DSPARK_QK_NORM = 1,
  DSPARK_PLAIN_CTX_KV = 2,
  DSPARK_GELU_FFN = 4
} dspark_variant;

/* Problem sizes (DflashConfig and TargetDims of module-dflash.ts). */
typedef struct {
  int32_t m;         /* number of tapped target layers */
  int32_t H;         /* target hidden width */
  int32_t d;         /* draft width dDraft */
  int32_t n_heads;   /* attention (query) heads; head_dim = d / n_heads */
  int32_t gamma;     /* block size */
  int32_t n_layers;  /* draft layers (used by dspark_block_forward) */
  int32_t ff;        /* FFN width, ffMult * d */
  float eps;         /* RMSNorm epsilon (the target's rmsNormEps) */
  int32_t dtype;     /* dspark_dtype: storage type of the long tensors */
  int32_t n_kv_heads;  /* K/V heads, dividing n_heads (0 = n_heads); n_kv_heads * hd a multiple of 128 */
  int32_t variant;     /* dspark_variant bits (0 = #layer of module-dflash.ts) */
  float rope_theta;    /* rotary base (0 = no rotary positions) */
} dspark_dims;

/* One draft layer's parameters (bb.{i}.* of module-dflash.ts), device
 * pointers. Matrices in dims->dtype, gains float32. kvd = n_kv_heads * hd
 * (= d unless the K/V heads are grouped). */
typedef struct {
  const float* attn_norm;   /* [d]    shared by block and context rows */
  const void* wq;           /* [d, d]   [out, in] */
  const void* wk;           /* [kvd, d] */
  const void* wv;           /* [kvd, d] */
  const void* wo;           /* [d, d] */
  const float* ff_norm;     /* [d] */
  const void* w_gate;       /* [ff, d] */
  const void* w_up;         /* [ff, d] */
  const void* w_down;       /* [d, ff] */
  const float* q_norm;      /* [hd] with DSPARK_QK_NORM, else ignored (may be NULL) */
  const float* k_norm;      /* [hd] with DSPARK_QK_NORM, else ignored (may be NULL) */
} dspark_layer_weights;

/* Bytes of workspace that `op` needs for these sizes (0 with a message in
 * dspark_last_error() when the arguments are invalid). Pure host arithmetic. */
size_t dspark_workspace_size(int32_t op, const dspark_dims* dims, int32_t A,
                             const int32_t* cu_host);

/* Eq 2 (#buildContext): h_ctx[t, :] = RMSNorm(sum_j W_c[:, j*H:(j+1)*H] taps[j][t, :]; ctx_norm).
 *   taps     host array of m device pointers; row t of tap j starts at
 *            taps[j] + t * ld_tap elements (ld_tap >= H), T = cu_host[A] rows
 *   w_c      [d, m*H] dtype ([out, in]);  ctx_norm [d] float32
 *   h_ctx    out [T, d] dtype */
dspark_status dspark_ctx_fuse(const dspark_dims* dims, int32_t A,
                              const int32_t* cu_host, const int32_t* cu_dev,
                              const void* const* taps, int64_t ld_tap,
                              const void* w_c, const float* ctx_norm,
                              void* h_ctx, void* ws, size_t ws_bytes, void* stream);

/* Eq 3 plus the block FFN for one draft layer (#layer).
 *   h_ctx    [T, d] dtype, read-only context memory (bitwise unchanged)
 *   d_in     [A, gamma, d] float32 block rows; d_out the same shape, may alias d_in
 *   lw       host pointer to the layer's device parameters */
dspark_status dspark_block_layer(const dspark_dims* dims, int32_t A,
                                 const int32_t* cu_host, const int32_t* cu_dev,
                                 const void* h_ctx, const float* d_in, float* d_out,
                                 const dspark_layer_weights* lw,
                                 void* ws, size_t ws_bytes, void* stream);

/* dspark_block_layer for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and results, with the scratch in a
 * file-scope device array of 64 MiB inside the library instead of a
 * caller workspace. The array exists once per GPU for the life of the
 * process; its device address is resolved on the first call on each device.
 * The call allocates nothing and calls no allocating routine.
 *   - Arguments as for dspark_block_layer, without ws / ws_bytes; the
 *     stream must belong to the current device.
 *   - Sizes whose workspace (dspark_workspace_size, DSPARK_OP_BLOCK_LAYER)
 *     exceeds 64 MiB return DSPARK_EUNSUPPORTED with a message, before
 *     anything is enqueued (about 14k context rows at d = 1024 in bf16).
 *   - Every call on one GPU shares that GPU's array, so calls that overlap
 *     on one GPU (several streams, several host threads) race: serialise
 *     them. The array keeps the last call's contents; every value a call
 *     reads from it is written earlier in the same call. */
dspark_status dspark_block_layer_noalloc(const dspark_dims* dims, int32_t A,
                                         const int32_t* cu_host, const int32_t* cu_dev,
                                         const void* h_ctx, const float* d_in, float* d_out,
                                         const dspark_layer_weights* lw, void* stream);

/* The whole draft block (#backbone): Eq 2, D0 = block_in + block_pos,
 * dims->n_layers x (Eq 3 + FFN), then the output norm.
 *   block_in   [A, gamma, d] float32 token rows (anchor row, mask rows)
 *   block_pos  [gamma, d] float32 (added to every sequence's block)
 *   layers     host array of n_layers parameter sets
 *   out_norm   [d] float32, or NULL to return D^N without the output norm
 *   h_ctx_out  optional [T, d] dtype copy of H_ctx, or NULL
 *   block_out  out [A, gamma, d] float32 */
dspark_status dspark_block_forward(const dspark_dims* dims, int32_t A,
                                   const int32_t* cu_host, const int32_t* cu_dev,
                                   const void* const* taps, int64_t ld_tap,
                                   const void* w_c, const float* ctx_norm,
                                   const float* block_in, const float* block_pos,
                                   const dspark_layer_weights* layers,
                                   const float* out_norm, void* h_ctx_out,
                                   float* block_out, void* ws, size_t ws_bytes,
                                   void* stream);

/* The launch plan that `op` takes for these sizes: pure host arithmetic, for
 * tests and tools. Writes min(n, DSPARK_PLAN_COUNT) values to out, indexed by
 * dspark_plan_field, and returns that count (0 with a message in
 * dspark_last_error() when the arguments are invalid). */
typedef enum {
  DSPARK_PLAN_CTX_SPLITS = 0,     /* K splits of the Eq 2 projection */
  DSPARK_PLAN_CTX_K_PER_SPLIT,    /* columns of m*H per split (the last may cover fewer) */
  DSPARK_PLAN_ATTN_CHUNK,         /* context keys per attention tile */
  DSPARK_PLAN_ATTN_TILES,         /* attention tiles over all sequences */
  DSPARK_PLAN_ATTN_STREAMING,     /* 1: chunks of several 64-key blocks, one wave
                                     per block (long contexts); 0: one block per tile,
                                     four waves share it (short contexts) */
  DSPARK_PLAN_WORKSPACE_BYTES,    /* dspark_workspace_size for the same arguments */
  DSPARK_PLAN_CTX_FUSED_NORM,     /* 1: Eq 2 in one split whose epilogue writes
                                     H_ctx * rms(P) (bf16) and row sums, with the
                                     row norm folded into the K/V row scale */
  DSPARK_PLAN_CTX_TAIL_ROWS,      /* with it: context rows of a partly filled last
                                     round of tiles run as K splits instead */
  DSPARK_PLAN_COUNT
} dspark_plan_field;
int32_t dspark_plan_info(int32_t op, const dspark_dims* dims, int32_t A, const int32_t* cu_host,
                         int64_t* out, int32_t n);

/* ---- block construction and padded batches --------------------------------
 * #buildBlock of module-dflash.ts: the block's token rows, before block_pos
 * (dspark_block_forward adds it):
 *   block_in[b, 0] = anchor_emb[b] . tok_proj^T   (the anchor token's embedding projected)
 *   block_in[b, j] = mask_emb[j - 1]               for j = 1 .. gamma-1 (shared by all b)
 *   anchor_emb  [A, H] float32 (the target's embedding of each anchor token)
 *   tok_proj    [d, H] dims->dtype ([out, in])
 *   mask_emb    [gamma-1, d] float32 (unused when gamma = 1; may be NULL then)
 *   block_in    out [A, gamma, d] float32
 * Uses dims->H, d, gamma and dtype; H up to 16256. */
dspark_status dspark_block_build(const dspark_dims* dims, int32_t A, const float* anchor_emb,
                                 const void* tok_proj, const float* mask_emb, float* block_in,
                                 void* stream);

/* #backbone on a padded batch with #maskBias's key-padding mask: A sequences
 * of L_ctx context rows each (row t of sequence b is row b * L_ctx + t of
 * every tap), where ctx_mask[b * L_ctx + t] != 0 marks a real row and 0 a
 * padding row. Padding rows are projected like the others but are no keys:
 * the -1e9 bias that #maskBias adds to their scores makes their softmax
 * weight exactly 0 in float32, which the kernels realise by leaving them out.
 * A sequence may be all padding (its block then attends to itself only).
 * Otherwise as dspark_block_forward; h_ctx_out, when given, is [A * L_ctx, d].
 *   ctx_mask   [A, L_ctx] uint8 device memory
 *   ws_bytes   at least dspark_padded_workspace_size(dims, A, L_ctx) */
size_t dspark_padded_workspace_size(const dspark_dims* dims, int32_t A, int32_t L_ctx);
dspark_status dspark_block_forward_padded(const dspark_dims* dims, int32_t A, int32_t L_ctx,
                                          const void* const* taps, int64_t ld_tap, const void* w_c,
                                          const float* ctx_norm, const uint8_t* ctx_mask,
                                          const float* block_in, const float* block_pos,
                                          const dspark_layer_weights* layers, const float* out_norm,
                                          void* h_ctx_out, float* block_out, void* ws,
                                          size_t ws_bytes, void* stream);

/* ---- incremental context ------------------------------------------------
 * The steady-state drafting loop of the page "src/dspark-runtime.js":
 * updateContext(position, count) runs Eq 2 on `count` new context rows and,
 * for every draft layer, projects them with that layer's W_K / W_V and
 * stores them in the layer's key/value cache; propose() then runs the block
 * side of every layer over the cached keys and values. The context rows are
 * normalised with each layer's attn_norm before W_K / W_V (#layer of
 * module-dflash.ts), so a cache filled by appends holds exactly the K_c / V_c
 * that dspark_block_forward computes from the whole context, and
 * dspark_block_propose over it gives the same draft block.
 *
 * The draft cache is caller-owned device memory of dspark_cache_bytes
 * bytes for A sequences of up to `cap` context rows each (cap a multiple of
 * 64), in the layout the attention kernels stream:
 *   cache[layer][K or V][head] is a slab of A * cap rows of head_dim values;
 *   sequence b owns slab rows b * cap .. b * cap + cap - 1, and its context
 *   row t (t = 0, 1, ... in append order) is slab row b * cap + t;
 *   within a slab, row t's values sit in 64-row blocks: for K, value c of row
 *   t is element ((t / 64) * (hd / E) + c / E) * 64 * E + (t % 64) * E + c % E
 *   with E = 16 / element size; for V the block is regrouped for the
 *   probability-times-value product (KG = 128 / hd key groups of R = E / 2
 *   keys and 2 columns per 16-byte vector).
 * Rows not yet appended must hold finite values: dspark_cache_reset clears
 * the cache to zeros, and appends write only the rows they add. The caller
 * keeps each sequence's length (its number of appended rows). */

/* Bytes of a draft cache (0 with a message when the arguments are invalid):
 * n_layers * 2 * A * cap * d * element size. */
size_t dspark_cache_bytes(const dspark_dims* dims, int32_t A, int32_t cap);

/* Clear the whole cache to zeros (a fill kernel on `stream`). */
dspark_status dspark_cache_reset(const dspark_dims* dims, int32_t A, int32_t cap, void* cache,
                                 void* stream);

/* updateContext for every sequence at once: the new context rows of sequence
 * b are rows ncu[b] .. ncu[b+1]-1 of the taps (ncu: A+1 prefix offsets, as cu
 * elsewhere; a sequence may add none); they are appended at rows pos[b] ..
 * pos[b] + n_b - 1 of that sequence, where pos[b] is its current length.
 * Runs Eq 2 on the new rows only, then every layer's context K/V of them,
 * written straight into the cache. Rows outside the appended ranges are not
 * touched.
 *   ncu_host / ncu_dev, pos_host / pos_dev   the same values in host and device memory
 *   taps, ld_tap, w_c, ctx_norm               as for dspark_ctx_fuse, T = ncu[A] new rows
 *   layers                                    host array of dims->n_layers parameter sets
 *   ws, ws_bytes                              dspark_workspace_size(DSPARK_OP_CTX_APPEND, dims, A, ncu_host)
 * Errors: pos[b] + n_b > cap returns DSPARK_EINVAL (nothing is written). */
dspark_status dspark_ctx_append(const dspark_dims* dims, int32_t A, int32_t cap,
                                const int32_t* ncu_host, const int32_t* ncu_dev,
                                const int32_t* pos_host, const int32_t* pos_dev,
                                const void* const* taps, int64_t ld_tap, const void* w_c,
                                const float* ctx_norm, const dspark_layer_weights* layers,
                                void* cache, void* ws, size_t ws_bytes, void* stream);

/* propose(): the draft block over the cache. Sequence b attends to its first
 * L_b = cu[b+1] - cu[b] cached rows (cu: A+1 prefix offsets of the cached
 * lengths; L_b <= cap) and to its own gamma block rows.
 *   block_in, block_pos, layers, out_norm, block_out   as for dspark_block_forward
 *   ws, ws_bytes   dspark_workspace_size(DSPARK_OP_BLOCK_PROPOSE, dims, A, cu_host)
 * The cache is only read. */
dspark_status dspark_block_propose(const dspark_dims* dims, int32_t A, int32_t cap,
                                   const int32_t* cu_host, const int32_t* cu_dev,
                                   const void* cache, const float* block_in,
                                   const float* block_pos, const dspark_layer_weights* layers,
                                   const float* out_norm, float* block_out, void* ws,
                                   size_t ws_bytes, void* stream);

/* ---- Markov head, confidence head and the greedy draft loop --------------
 * forwardInfer of module-dflash.ts after the backbone (#markov,
 * #confidence), which the page "src/dspark-runtime.js" runs as markovEmbed
 * -> markov -> addBias -> argmax per drafted position. For every sequence b,
 * with prev = anchor[b], and for k = 0 .. gamma-1 in turn:
 *   e1           = w1[prev]                            (Markov embedding, rank values)
 *   logits[b, k] = base_logits[b, k] + e1 . w2^T       (w2 stored [vocab, rank])
 *   tokens[b, k] = argmax_v logits[b, k, v]            (equal maxima: the lowest index)
 *   conf[b, k]   = sigmoid([block[b, k], e1] . conf_w + conf_b)
 *   prev         = tokens[b, k]
 * The base logits are the target model's LM head applied to the draft block
 * (#baseLogits); they are an input here. The logits are float32: the bias
 * products multiply the stored w1 and w2 values and accumulate in float32.
 *   block        [A, gamma, d] float32: the draft block (the output norm applied)
 *   base_logits  [A, gamma, vocab] float32
 *   anchor       [A] int32 device: the token each block continues (clamped to [0, vocab))
 *   w1           [vocab, rank] dims->dtype: row v is token v's Markov embedding
 *   w2           [vocab, rank] dims->dtype: row v holds the weights of logit v ([out, in])
 *   conf_w       [d + rank] float32;  conf_b  [1] float32 (device)
 *   tokens       out [A, gamma] int32;  conf  out [A, gamma] float32
 *   draft_logits out [A, gamma, vocab] float32 (the logits of every position)
 *   ws, ws_bytes dspark_markov_workspace_size(dims, A, vocab, rank) bytes
 * Sizes: vocab a multiple of 8 (gamma * vocab < 2^31), rank a multiple of 64
 * up to 16256, A * gamma <= 1024. Uses dims->d, gamma and dtype only. */
size_t dspark_markov_workspace_size(const dspark_dims* dims, int32_t A, int32_t vocab, int32_t rank);
dspark_status dspark_markov_draft(const dspark_dims* dims, int32_t A, int32_t vocab, int32_t rank,
                                  const float* block, const float* base_logits, const int32_t* anchor,
                                  const void* w1, const void* w2, const float* conf_w,
                                  const float* conf_b, int32_t* tokens, float* conf,
                                  float* draft_logits, void* ws, size_t ws_bytes, void* stream);

/* Message for the last non-OK status on this thread ("" if none). */
const char* dspark_last_error(void);

/* Library version string. */
const char* dspark_version(void);

/* ---- measurement support: per-kernel HIP-event timing -------------------
 * Kernel kinds are numbered 0 .. dspark_kernel_kinds()-1 and named by
 * dspark_kernel_name(). dspark_trace_begin(mask) makes every later launch of
 * a kind whose bit is set in `mask` record a HIP event pair on its stream
 * (at most `capacity` launches). dspark_trace_end() waits for those events,
 * writes per-kind totals (milliseconds) and launch counts into the caller's
 * arrays of length n_kinds, and stops tracing. Not for concurrent use. */
int32_t dspark_kernel_kinds(void);
const char* dspark_kernel_name(int32_t kind);
dspark_status dspark_trace_begin(uint64_t mask, int32_t capacity);
dspark_status dspark_trace_end(double* total_ms, int64_t* launches, int32_t n_kinds);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
