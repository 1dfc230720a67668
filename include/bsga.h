/*
 * libbsga — block-sparse global attention for VGGT-style multi-view geometry
 * transformers, as hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the page "Block-Sparse Global Attention for Efficient
 * Multi-View Geometry Transformers" (cited below as [BSGA]): its overall
 * framework flowchart, key design 1 (block-mask prediction; equations
 * "Attention" and "SparseAttn"), key design 2 (Top-K + CDF two-threshold
 * block selection) and key design 3 (special tokens take a dense path).
 * Per-head budgets follow "HeSS: Head Sensitivity Score for Sparsity
 * Redistribution in VGGT" (cited as [HeSS]), proposed method.
 *
 * Conventions for every call
 * --------------------------
 * Tensors (batch 1, heads outermost):
 *   Q, K, V, O   [H][N][64] bfloat16, passed as raw bits (uint16_t), row
 *                stride 128 bytes, 16-byte aligned device pointers.
 *   LSE          [H][N] float32, natural log of the softmax denominator.
 *   probs        [H][B][B] float32 row-major (block-importance distribution).
 *   row_ptr      [H*B + 1] int32; rows are ordered head-major, then query
 *                block; col_idx[row_ptr[r] .. row_ptr[r+1]) are the kept key
 *                blocks of row r in ascending order.
 * Token order: frame-major; every frame holds `special_per_frame` special
 * tokens (camera, then registers) followed by `patches_per_frame` patch
 * tokens in raster order.  N = frames * (patches_per_frame +
 * special_per_frame).  Patch p (0 <= p < N_p = frames * patches_per_frame)
 * is token (p / P) * (P + S) + S + p % P.  Patch block i holds patches
 * [i*b, min((i+1)*b, N_p)); B = ceil(N_p / b); the last block may be partial.
 *
 * Ownership: the caller owns and allocates every buffer, including the
 * workspace (size from bsga_workspace_bytes).  The library never allocates
 * and never synchronises the host; every call only enqueues kernels on
 * `stream` (a hipStream_t; NULL = the null stream) and returns.  Inputs are
 * read-only.  No state outlives a call, except the fixed device array of
 * bsga_select_static (described there).
 *
 * Errors: every call returns a bsga_status.  All arguments are validated on
 * the host before anything is enqueued, so an error means nothing was
 * launched.  BSGA_ERR_HIP reports a launch failure seen after enqueueing.
 */
#ifndef BSGA_H
#define BSGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSGA_VERSION 3
#define BSGA_MAX_HEADS 256     /* per-head budget table size */
#define BSGA_MAX_BLOCKS 4096   /* largest B accepted by bsga_select */

typedef enum bsga_status {
  BSGA_OK = 0,
  BSGA_ERR_INVALID_ARG = 1, /* null pointer, bad size, rho/tau out of range */
  BSGA_ERR_UNSUPPORTED = 2, /* head_dim != 64, block not 64/128, too large
                               (N + 256 >= 2^24 tokens, or a select limit) */
  BSGA_ERR_MISALIGNED = 3,  /* bf16 tensors not 16-byte aligned, others 4 */
  BSGA_ERR_WORKSPACE = 4,   /* workspace missing, misaligned or too small */
  BSGA_ERR_HIP = 5          /* a kernel launch failed */
} bsga_status;

/* Operations, for bsga_workspace_bytes. */
typedef enum bsga_op {
  BSGA_OP_PREDICT_MASK = 0,
  BSGA_OP_SELECT = 1,
  BSGA_OP_SPARSE_ATTN = 2,
  BSGA_OP_SPECIAL_DENSE = 3,
  BSGA_OP_DENSE_ATTN = 4,
  BSGA_OP_LAYER = 5,
  BSGA_OP_SPECIAL_DENSE_PACKED = 6,
  BSGA_OP_PROBE_SELECT = 7,
  BSGA_OP_NMSE = 8,
  BSGA_OP_BACKWARD = 9,
  BSGA_OP_PATCH_ROWS_PACKED = 10
} bsga_op;

/* Shape of one global-attention layer.  head_dim must be 64; block (b) must
 * be 64 or 128; frames, patches_per_frame, heads >= 1;
 * special_per_frame >= 0. */
typedef struct bsga_shape {
  int32_t frames;
  int32_t patches_per_frame;
  int32_t special_per_frame;
  int32_t heads;
  int32_t head_dim;
  int32_t block;
} bsga_shape;

/* Library version (BSGA_VERSION). */
int bsga_version(void);

/* Static description of a status code; never NULL. */
const char* bsga_status_string(int status);

/* B = ceil(N_p / b), the number of patch blocks ([BSGA] key design 1). */
int bsga_num_blocks(const bsga_shape* shape, int32_t* n_blocks);

/* k = floor(B (1 - rho)) ([BSGA] key design 2), evaluated exactly with rho
 * read as a decimal on a 1e-6 grid, so that e.g. B = 2140, rho = 0.9 gives
 * 214.  rho must lie in [0, 1]. */
int bsga_keep_count(int32_t n_blocks, double rho, int32_t* k);

/* Head-wise budget redistribution ([HeSS] proposed method: the layer's total
 * attention budget is reallocated across heads by iterative capping, denser
 * attention for more sensitive heads).  With keep fractions
 * kappa_h = 1 - rho_h, the result is the unique solution of
 *   kappa_h = clamp(lambda * weights[h], 1 - rho_max, 1 - rho_min),
 *   mean_h kappa_h = 1 - mean_rho,
 * i.e. keep fractions proportional to the weights, clipped at both bounds,
 * with the budget a clipped head cannot take spread over the others.
 *   weights: HOST array of `heads` finite values > 0 (e.g. per-head
 *     sensitivity scores; they are not computed here).
 *   0 <= rho_min <= mean_rho <= rho_max <= 1; 1 <= heads <= BSGA_MAX_HEADS.
 *   rho_out: HOST array of `heads` values, the per-head rho for bsga_select.
 * Host-only computation (no GPU work, no allocation); O(heads log heads).
 * Returns BSGA_ERR_INVALID_ARG for null pointers, a bad count, a weight that
 * is not finite and positive, or bounds out of order. */
int bsga_redistribute(int32_t heads, const double* weights, double mean_rho,
                      double rho_min, double rho_max, double* rho_out);

/* Entries col_idx must be able to hold: H * B * B (every block kept). */
int bsga_csr_capacity(const bsga_shape* shape, int64_t* entries);

/* Workspace bytes needed by operation `op` (a bsga_op).  The workspace must
 * be a device buffer aligned to 256 bytes; its contents on entry do not
 * matter and are clobbered. */
int bsga_workspace_bytes(const bsga_shape* shape, int op, size_t* bytes);

/* Block-mask prediction ([BSGA] key design 1).
 *   Qbar[h][i] = mean of the patch rows of block i of Q (likewise Kbar),
 *   S = Qbar Kbar^T / sqrt(64), probs[h][i][:] = softmax of S[h][i][:].
 * q, k: [H][N][64] bf16.  probs: [H][B][B] float32 (output).
 * scores: optional [H][B][B] float32 output of S itself (NULL to skip).
 * qbar, kbar: optional [H][B][64] float32 outputs (NULL to skip).
 * Pooling accumulates in float32; the pooled-score product runs on bf16
 * MFMA on a three-way bf16 split of the float32 means (x = x1 + x2 + x3, six
 * cross products of exact float32 terms accumulated in float32: error near
 * that of a float32 dot product); the softmax is float32.  The optional
 * outputs must be 4-byte aligned and must not overlap probs. */
int bsga_predict_mask(const bsga_shape* shape, const uint16_t* q,
                      const uint16_t* k, float* probs, float* scores,
                      float* qbar, float* kbar, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Two-threshold block selection ([BSGA] key design 2; [HeSS] per-head
 * budget).  For every row (h, i) of probs: rank the B key blocks by
 * probability descending (ties: lower block index first), let
 * k_h = floor(B (1 - rho_h)) and n_tau the smallest n whose cumulative
 * probability of the n top-ranked blocks is >= tau (float64 sum; tau <= 0
 * gives 0; tau >= 1 gives B; B if never reached), and keep the first
 * max(k_h, n_tau) ranked blocks, emitted in ascending block order.
 *   probs: [H][B][B] float32, non-negative (device).
 *   rho_per_head: NULL (use rho for all heads) or a HOST array of H values
 *     in [0, 1] (requires H <= BSGA_MAX_HEADS).
 *   rho in [0, 1]; tau any finite value.
 *   row_ptr: [H*B+1] int32 output; col_idx: output of capacity
 *   col_capacity >= H*B*B entries.  Requires B <= BSGA_MAX_BLOCKS. */
int bsga_select(const bsga_shape* shape, const float* probs,
                const double* rho_per_head, double rho, double tau,
                int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                void* workspace, size_t workspace_bytes, void* stream);

/* bsga_select without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, semantics and results
 * as bsga_select (bit-identical CSR).  Its scratch (per-row counts and
 * thresholds) is a 1 MiB array the library holds in device memory, one copy
 * per GPU, kept until the process ends; the call allocates nothing.  Every
 * such call on one GPU shares that array, so calls that may overlap on one
 * GPU (other streams, other host threads) race and must be serialised by
 * the caller; a call leaves the array's contents behind, and the next call
 * never reads them.  Limit: H * B <= BSGA_SELECT_STATIC_MAX_ROWS rows
 * (BSGA_ERR_UNSUPPORTED beyond it, checked before anything is launched);
 * BSGA_ERR_HIP if the array's device address cannot be found. */
#define BSGA_SELECT_STATIC_MAX_ROWS 65536
int bsga_select_static(const bsga_shape* shape, const float* probs,
                       const double* rho_per_head, double rho, double tau,
                       int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                       void* stream);

/* Query-probe Top-K block selection ("SAF3R: Dynamic Sparse Attention for
 * Feed-Forward 3D Reconstruction Transformers", cited as [SAF3R], section 4:
 * the query-probe Top-K kernel for heads whose queries share a few dominant
 * keys, with its O(N) online estimate).  Per head h:
 *   qbar = (1/N) sum over all N tokens of Q[h][t]           (the probe),
 *   r_p  = qbar . K[h][patch p] / sqrt(64)   for every patch key p,
 * which equals the mean over all queries of their score with key p.  The
 * `topk` patch keys with the largest r_p (ties: lower patch index first) are
 * taken, and every query block of the head keeps the patch blocks holding at
 * least one of them, in ascending order (same CSR layout as bsga_select, all
 * rows of a head equal).  Special keys are not ranked: they stay dense in the
 * attention calls.
 *   q, k: [H][N][64] bf16.  topk >= 0 (0 keeps no block; >= N_p keeps all).
 *   scores: optional [H][N_p] float32 output of r (patch order), or NULL.
 *   row_ptr [H*B+1], col_idx (capacity >= H*B*B) as for bsga_select.
 *   workspace: bsga_workspace_bytes(BSGA_OP_PROBE_SELECT).  Requires
 *   B <= BSGA_MAX_BLOCKS.  Float32 mean and dot products; the ranking uses the
 *   float32 r exactly as written to `scores`. */
int bsga_probe_select(const bsga_shape* shape, const uint16_t* q,
                      const uint16_t* k, int32_t topk, float* scores,
                      int32_t* row_ptr, int32_t* col_idx,
                      int64_t col_capacity, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Block-sparse attention of the patch queries over their kept patch blocks
 * ([BSGA] equation SparseAttn, masked entries excluded from the softmax):
 * for patch query q in block i of head h,
 *   O[h][q] = sum_t softmax_t(Q[q].K[t] / 8) V[t],  LSE[h][q] = log sum_t e^..
 * over the patch tokens t of the blocks col_idx[row_ptr[h*B+i] ..).  Writes
 * only the patch rows of o and lse (special rows untouched).  An empty row
 * gives O = 0, LSE = -inf.  MFMA products with float32 accumulation and a
 * float32 online softmax: Q K^T in bf16; P enters the P V product as
 * float16 (11 significant bits; weights never exceed 2^15), V as float16
 * scaled per head by a power of two (exact for bf16 values; see
 * bsga_pack_kv). */
int bsga_sparse_attn(const bsga_shape* shape, const uint16_t* q,
                     const uint16_t* k, const uint16_t* v,
                     const int32_t* row_ptr, const int32_t* col_idx,
                     uint16_t* o, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Dense part for the special tokens ([BSGA] key design 3 and framework
 * flowchart): special queries attend to all N tokens (their rows of o/lse
 * are written), and patch queries attend to all special tokens; the latter
 * result is merged in place with the patch rows already in o/lse (from
 * bsga_sparse_attn) by log-sum-exp, giving one softmax over the union of
 * keys.  Must follow bsga_sparse_attn on the same stream. */
int bsga_special_dense(const bsga_shape* shape, const uint16_t* q,
                       const uint16_t* k, const uint16_t* v, uint16_t* o,
                       float* lse, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Dense softmax attention of every token over every token ([BSGA] equation
 * Attention): the library's own dense path, for comparison. */
int bsga_dense_attn(const bsga_shape* shape, const uint16_t* q,
                    const uint16_t* k, const uint16_t* v, uint16_t* o,
                    float* lse, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Normalised mean squared error per head ([SAF3R] section 4, offline head
 * profiling):  nmse[h] = ||o_ref[h] - o[h]||^2 / ||o_ref[h]||^2  over all N
 * rows and 64 dims of the head (0 when both are zero, +inf when only the
 * reference is).  o_ref, o: [H][N][64] bf16 (e.g. the dense and a sparse
 * output).  nmse: DEVICE array of H doubles (output).  Float32 sums per
 * chunk of 1024 rows, float64 across chunks, in a fixed order
 * (deterministic).  Workspace: bsga_workspace_bytes(BSGA_OP_NMSE).
 *
 * Ablation without the dense special path ([BSGA] ablation of the special-
 * token design): pass every call the shape {frames = 1, patches_per_frame =
 * N, special_per_frame = 0}; blocks then run over the whole token sequence,
 * so the special tokens are pooled and selected together with the patches. */
int bsga_nmse(const bsga_shape* shape, const uint16_t* o_ref, const uint16_t* o,
              double* nmse, void* workspace, size_t workspace_bytes,
              void* stream);

/* Backward of the layer's attention for a fixed mask ([BSGA] outlook:
 * sparse attention inside training; the block selection is not
 * differentiated).  For the output O of bsga_layer (patch queries over their
 * kept patch blocks and every special key, special queries over every key),
 * given dO = dL/dO, writes dQ, dK, dV = dL/dQ, dL/dK, dL/dV:
 *   P = exp(q.k / 8 - LSE),  dS = P (dO.v - dO.O),
 *   dQ = sum_k dS k / 8,  dK = sum_q dS q / 8,  dV = sum_q P dO.
 *   q, k, v, o, d_o: [H][N][64] bf16 (o and lse as written by the forward
 *     with this mask); lse: [H][N] float32; row_ptr/col_idx: the mask (as
 *     returned by bsga_select or bsga_probe_select).
 *   dq, dk, dv: [H][N][64] float32 outputs, 16-byte aligned, fully written.
 *   workspace: bsga_workspace_bytes(BSGA_OP_BACKWARD) (packed operands,
 *     row statistics and the transposed mask).
 * MFMA products with float32 accumulation: S, dP and the dQ, dK products in
 * bf16, with dS entering as a bf16 pair hi + lo; dV = P^T dO in float16, with
 * P (times 2^15) rounded once to float16 and dO times a per-head power of two
 * (exact for bf16 values), so each weight of dV carries a relative rounding of
 * at most 2^-11.  D = dO . O is recomputed as sum_k P dP from the same float32
 * P and dP (the stored bf16 O is not used for it).  No atomics: dQ
 * is accumulated per query tile over the mask's rows, dK and dV per key tile
 * over its transpose (deterministic). */
int bsga_attn_backward(const bsga_shape* shape, const uint16_t* q,
                       const uint16_t* k, const uint16_t* v, const uint16_t* o,
                       const float* lse, const uint16_t* d_o,
                       const int32_t* row_ptr, const int32_t* col_idx,
                       float* dq, float* dk, float* dv, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Packed K/V: the layout the attention kernels stream.  Keys are listed in
 * "packed order" — the N_p patch tokens in patch order, zero rows up to the
 * next multiple of 128, then the N_s special tokens, zero rows up to the next
 * multiple of 128 (Ntot_pad keys in all) — and stored as
 *   K rows   [H][Ntot_pad][64] bf16, followed by
 *   V^T      [H][64][Ntot_pad] float16 (V transposed: keys contiguous),
 *            holding V[h] * 2^sigma_h, where sigma_h puts the head's largest
 *            |V| in [2^14, 2^15) (clamped to [-100, 100]; 0 when the head has
 *            no finite nonzero value), followed by
 *   sigma    [H] int32 (256-byte aligned), and a per-head scratch table the
 *            packing uses to find each head's largest |V|.
 * A bf16 value times a power of two is exact in float16 inside its normal
 * range, so the scaled copy loses nothing but values more than 2^28 below the
 * head's largest |V| (absolute error below 2^-39 of it).  Packing (two
 * kernels: the per-head maximum, then the copy) once per layer lets the
 * sparse, special and dense calls share it.  kv_packed must be a 256-byte
 * aligned device buffer of at least bsga_packed_kv_bytes bytes. */
int bsga_packed_kv_bytes(const bsga_shape* shape, size_t* bytes);
int bsga_pack_kv(const bsga_shape* shape, const uint16_t* k, const uint16_t* v,
                 void* kv_packed, size_t kv_bytes, void* stream);

/* bsga_sparse_attn, bsga_special_dense and bsga_dense_attn on K/V already
 * packed by bsga_pack_kv (same semantics; no packing inside).  The special
 * call needs a workspace of bsga_workspace_bytes(BSGA_OP_SPECIAL_DENSE_PACKED)
 * for its split-K partial results. */
int bsga_sparse_attn_packed(const bsga_shape* shape, const uint16_t* q,
                            const void* kv_packed, size_t kv_bytes,
                            const int32_t* row_ptr, const int32_t* col_idx,
                            uint16_t* o, float* lse, void* stream);
int bsga_special_dense_packed(const bsga_shape* shape, const uint16_t* q,
                              const void* kv_packed, size_t kv_bytes,
                              uint16_t* o, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream);
int bsga_dense_attn_packed(const bsga_shape* shape, const uint16_t* q,
                           const void* kv_packed, size_t kv_bytes, uint16_t* o,
                           float* lse, void* stream);

/* The layer's final rows in two calls on packed K/V, the way bsga_layer
 * computes them ([BSGA] framework flowchart and key design 3, one softmax per
 * query over its whole key set):
 *   bsga_patch_rows_packed: every patch query attends to the patch tokens of
 *     its kept blocks AND to every special token, in one online softmax, and
 *     writes its final row of o/lse (equal to bsga_sparse_attn followed by the
 *     merge in bsga_special_dense, without the intermediate bf16 rounding).
 *     Optional workspace (NULL, or bsga_workspace_bytes(
 *     BSGA_OP_PATCH_ROWS_PACKED) bytes; at b = 64 it is 0 when B > 8192).
 *     At b = 64 (B <= 8192) a workspace lets the call run query blocks in
 *     aligned pairs: query blocks 2I, 2I + 1 form a
 *     128-query tile that walks the 128-key tiles (key blocks 2J, 2J + 1)
 *     holding a block either of them keeps, each wave skipping the 32-key
 *     sub-tiles its query block does not keep (the same softmax; the lists
 *     are built on the device into the workspace); without one, 64-query
 *     tiles walk 64-key tiles.  With it, at b = 128 (and for the pairs) the
 *     query blocks left for the last, partial round of workgroups are split into
 *     pieces of consecutive key tiles (as many per block as let them all run
 *     at once when that round is at most half full; for a fuller round the
 *     count, at most 16, whose pieces finish first, if that is under 0.8 of
 *     a block's time) whose float32 partials are merged by log-sum-exp
 *     afterwards, which balances that round; the result is the same softmax
 *     (it may differ from the unsplit rows in the last bit).  At b = 128
 *     with B <= 4096 the workspace also holds an order of each head's query
 *     blocks, longest kept list first (ties by block index), which the
 *     workgroups follow: concurrent workgroups then hold rows of similar
 *     length and the split last round the shortest rows (every row's result
 *     is the same as in natural order, the split rows aside).  The plan uses
 *     the compute-unit count of the current device: size and use the
 *     workspace with the same device current;
 *   bsga_special_rows_packed: every special query attends to all N tokens
 *     (split over key ranges, partial results combined by log-sum-exp in a
 *     workspace of bsga_workspace_bytes(BSGA_OP_SPECIAL_DENSE_PACKED)) and
 *     writes its row of o/lse.
 * Precision as in bsga_sparse_attn (P enters the P V product as float16).
 * The two calls write disjoint rows and may run in either order (with
 * different workspaces if they overlap). */
int bsga_patch_rows_packed(const bsga_shape* shape, const uint16_t* q,
                           const void* kv_packed, size_t kv_bytes,
                           const int32_t* row_ptr, const int32_t* col_idx,
                           uint16_t* o, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream);
int bsga_special_rows_packed(const bsga_shape* shape, const uint16_t* q,
                             const void* kv_packed, size_t kv_bytes,
                             uint16_t* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* One replaced global-attention layer ([BSGA] framework flowchart):
 * bsga_predict_mask, bsga_select, bsga_pack_kv, bsga_patch_rows_packed and
 * bsga_special_rows_packed in that order on `stream` (so each output row is
 * one softmax over its key set, rounded to bf16 once).  probs, row_ptr and
 * col_idx receive the intermediate mask (same layouts as above). */
int bsga_layer(const bsga_shape* shape, const uint16_t* q, const uint16_t* k,
               const uint16_t* v, const double* rho_per_head, double rho,
               double tau, float* probs, int32_t* row_ptr, int32_t* col_idx,
               int64_t col_capacity, uint16_t* o, float* lse,
               void* workspace, size_t workspace_bytes, void* stream);

/* Training mode of bsga_layer ([BSGA] outlook: sparse attention inside
 * training): the same mask and softmax, except that P enters the P V
 * products as a float16 pair hi + lo (hi = fp16(w), lo = fp16(w - hi):
 * about 22 significant bits of every weight, against 11 for hi alone), and
 * every final row is also written as float32 to o32 ([H][N][64], 16-byte
 * aligned, fully written); o holds bf16(o32), element for element.  o32 is
 * what bsga_attn_backward_o32 takes to form D = dO . O without recomputing
 * the softmax.  The P V products cost twice the matrix-core work and the
 * split about half again the softmax's vector work.  Same arguments and
 * workspace (BSGA_OP_LAYER) as bsga_layer; BSGA_ERR_UNSUPPORTED at b = 64
 * with B > 8192 (the unpaired 64-row kernel has no training mode). */
int bsga_layer_train(const bsga_shape* shape, const uint16_t* q,
                     const uint16_t* k, const uint16_t* v,
                     const double* rho_per_head, double rho, double tau,
                     float* probs, int32_t* row_ptr, int32_t* col_idx,
                     int64_t col_capacity, uint16_t* o, float* lse,
                     float* o32, void* workspace, size_t workspace_bytes,
                     void* stream);

/* bsga_attn_backward with D = dO . O taken from the float32 rows o32 of
 * bsga_layer_train (accurate to about 2^-22 of each weight) instead of
 * recomputed as sum_k P dP by a first sweep of the dQ kernel over every
 * kept key: the dQ kernel then runs its gradient sweep only.  Same
 * arguments, layouts, precision (otherwise) and workspace as
 * bsga_attn_backward, with o32 ([H][N][64] float32, 16-byte aligned) in
 * place of o. */
int bsga_attn_backward_o32(const bsga_shape* shape, const uint16_t* q,
                           const uint16_t* k, const uint16_t* v,
                           const float* o32, const float* lse,
                           const uint16_t* d_o, const int32_t* row_ptr,
                           const int32_t* col_idx, float* dq, float* dk,
                           float* dv, void* workspace, size_t workspace_bytes,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSGA_H */
