/*
 * llatte.h -- C ABI of the MI355X (gfx950) library for the forward pass of
 * LLaTTE's target-aware sequence transformer with Multi-head Latent Attention.
 *
 * Sources, cited by page title and section:
 *   [LLaTTE] "LLaTTE: Scaling Laws for Multi-Stage Sequence Modeling in
 *            Large-Scale Ads Recommendation" (annotated translation):
 *            section 1.3.2 (the five steps of the sequence module),
 *            Appendix A.2 (query tokens and fusion; layer equations; the
 *            pyramidal schedule, its cost and the three attention modes;
 *            sequence summaries), Appendix A.3 (MLA and its absorbed form).
 *   [Repro]  "LLaTTE: Multi-stage sequence scaling" (reproduction note),
 *            core formula: target-aware query q = W_Q [x; c].
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless marked "host". Buffers are
 *     caller-owned, contiguous and row-major; matrices are [in, out] so that
 *     y = x W. Activation/weight matrices use the descriptor's dtype (F32 or
 *     BF16); gains, residual-stream inputs and all outputs are float32.
 *   - Alignment: every device pointer must be 16-byte aligned.
 *   - The library never allocates, frees or retains a pointer after it
 *     returns. Scratch memory is passed in as a caller-owned workspace whose
 *     size the matching *_workspace_size function returns.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns without synchronising. Inputs must stay
 *     alive until the stream work completes.
 *   - Errors: every function returns LLATTE_OK (0) or a negative status.
 *     Host-side validation happens before anything is enqueued; on a
 *     validation error nothing is launched. llatte_last_error() gives a
 *     message for the last failing call on the calling thread. Malformed
 *     device-side offsets (non-monotone, or inconsistent with the host
 *     totals) are undefined behaviour.
 *   - Re-entrant; no global mutable state besides the per-thread message.
 */
#ifndef LLATTE_H
#define LLATTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t llatte_status;
#define LLATTE_OK 0
#define LLATTE_ERR_INVALID_ARG (-1) /* bad pointer, size or shape          */
#define LLATTE_ERR_UNSUPPORTED (-2) /* valid but not implemented (e.g. r)  */
#define LLATTE_ERR_WORKSPACE (-3)   /* workspace too small                 */
#define LLATTE_ERR_HIP (-4)         /* a HIP runtime call or launch failed */

#define LLATTE_F32 0
#define LLATTE_BF16 1

#define LLATTE_NORM_PRE 0  /* pre-norm layer (default)                     */
#define LLATTE_NORM_POST 1 /* post-norm, as written in [LLaTTE] A.2        */

#define LLATTE_PYR_FIXED 0     /* values[l] per layer, capped by layer l-1  */
#define LLATTE_PYR_HALVING 1   /* max(min(floor, L_u), L_u >> l)            */
#define LLATTE_PYR_GEOMETRIC 2 /* start -> end geometric, rounded half up   */

/* The readout returns Flatten(Z_raw) itself in out_emb (seed-major,
 * [B, n_seeds*d]; d_out must equal n_seeds*d and W_p is not used), as the
 * input of llatte_summaries. */
#define LLATTE_FLAG_RAW_READOUT 1u

/* Opt-in device check of hist_offsets before anything else runs (the S_u of
 * [LLaTTE] A.2 are ordered, non-empty action sequences): offsets[0] == 0,
 * every L_u = offsets[u+1] - offsets[u] in [1, max_len], offsets[B] ==
 * total_rows. One small kernel reads only the offsets and writes an error
 * word; the call then synchronises the stream and returns
 * LLATTE_ERR_INVALID_ARG (with the first failing user in the message) if the
 * check failed, before any other kernel is launched. Without the flag such
 * offsets are undefined behaviour. For tests and debugging; it costs a sync. */
#define LLATTE_FLAG_VALIDATE 2u

/* Per-layer dump for localising a parity failure: the output rows of every
 * layer (and of the readout layer), float32, written to desc->debug_dump.
 * Layer l's section starts at row llatte_mla_forward_debug_layout(...)[l]
 * (element offset row * d) and holds the layer's B*n_q candidate (or seed)
 * rows, then its kept history rows, user-major, oldest first, i.e. the layer's
 * query rows; the section ends at the next offset (upper bound; the rows past
 * the layer's actual count are left untouched). */
#define LLATTE_FLAG_DEBUG_DUMP 4u

#define LLATTE_MAX_LAYERS 64

/* Pyramidal schedule ([LLaTTE] A.2): how many of the most recent history rows
 * stay as queries/outputs at each layer. The count for user u at layer l
 * (0-based) is capped by the count at layer l-1 (layer -1 = L_u). A count of
 * 0 is cross-attention mode (only the query tokens stay), allowed only at
 * the last layer of the stack. */
typedef struct {
  int32_t kind;                       /* LLATTE_PYR_*                        */
  int32_t floor;                      /* HALVING: the floor (>= 1)           */
  int32_t start, end;                 /* GEOMETRIC: endpoints (>= 1)         */
  int32_t values[LLATTE_MAX_LAYERS];  /* FIXED: per-layer counts (>= 0)      */
} llatte_pyramid_rule;

/* Model shape and options. d_ff must be 4*d. head_dim*n_heads is the query
 * width. rank is the latent width r of C = H W_dkv ([LLaTTE] A.3).
 * q_rank selects the query path of [LLaTTE] A.3: 0 = one full-rank W_uq
 * [d, h*dk]; > 0 = the low-rank path q = RMSNorm(H W_dq) g_q W_uq with
 * W_dq [d, q_rank] and W_uq [q_rank, h*dk] (q_rank a multiple of 8 on the
 * bf16 path, of 4 on the fp32 path, at most 1024). */
typedef struct {
  int32_t d;           /* model width                                       */
  int32_t n_heads;     /* h                                                 */
  int32_t head_dim;    /* d_k; the softmax scale is 1/sqrt(d_k)             */
  int32_t rank;        /* r                                                 */
  int32_t d_ff;        /* FFN hidden width (= 4d)                           */
  int32_t n_layers;    /* N, 1 .. LLATTE_MAX_LAYERS - 1 (the readout takes
                          the last plan slot)                              */
  int32_t n_q;         /* candidate query tokens per user (>= 0)            */
  int32_t d_ctx;       /* per-user context width d_c (>= 0)                 */
  int32_t dtype;       /* LLATTE_F32 or LLATTE_BF16                         */
  int32_t norm_mode;   /* LLATTE_NORM_PRE or LLATTE_NORM_POST               */
  int32_t latent_norm; /* 1: RMSNorm on the latent C ([LLaTTE] A.3); 0: off */
  float eps;           /* RMSNorm epsilon, inside the square root           */
  llatte_pyramid_rule pyramid;
  int32_t n_seeds;     /* readout seed queries (0 = no readout)             */
  int32_t d_out;       /* readout embedding width                           */
  uint32_t flags;      /* 0 or LLATTE_FLAG_RAW_READOUT | LLATTE_FLAG_VALIDATE
                          | LLATTE_FLAG_DEBUG_DUMP                          */
  int32_t q_rank;      /* 0: full-rank queries; > 0: low-rank query width   */
  float* debug_dump;   /* device, with LLATTE_FLAG_DEBUG_DUMP: float32
                          [llatte_mla_forward_debug_layout()[N_plans], d]   */
  size_t debug_dump_bytes;  /* its size in bytes                            */
} llatte_model_desc;

/* Weights of one layer (device pointers). g* are float32 gains; the
 * matrices have the descriptor's dtype:
 *   W_dkv [d, r], W_uq [d, h*dk] (q_rank = 0) or [q_rank, h*dk],
 *   W_uk [r, h*dk], W_uv [r, h*dk], W_o [h*dk, d], W1 [d, d_ff], W2 [d_ff, d];
 *   with q_rank > 0 also W_dq [d, q_rank] and g_q [q_rank] (NULL otherwise).
 * Head j of W_uk / W_uv is the column slice j*dk .. (j+1)*dk-1. */
typedef struct {
  const float* g1;
  const void* W_dkv;
  const float* g_c;
  const void* W_uq;
  const void* W_uk;
  const void* W_uv;
  const void* W_o;
  const float* g2;
  const void* W1;
  const void* W2;
  const void* W_dq;    /* low-rank query path only */
  const float* g_q;
} llatte_layer_weights;

/* All weights. `layers` is a HOST array of n_layers structs.
 *   W_q   [d + d_ctx, d]  fusion projection of [x_j ; c_u] (needed if n_q>0)
 *   seeds [n_seeds, d]    float32 learned readout queries   (if n_seeds>0)
 *   readout               weights of the readout layer       (if n_seeds>0)
 *   W_p   [n_seeds*d, d_out] readout projection              (if n_seeds>0,
 *         unused with LLATTE_FLAG_RAW_READOUT) */
typedef struct {
  const llatte_layer_weights* layers;
  const void* W_q;
  const float* seeds;
  llatte_layer_weights readout;
  const void* W_p;
} llatte_weights;

/* ------------------------------------------------------------------------
 * llatte_mla_forward -- the whole sequence-module forward ([LLaTTE] 1.3.2):
 * fusion of the query tokens, N layers of MLA with the pyramidal schedule,
 * then the optional readout.
 *
 * Per user u the history is rows hist_offsets[u] .. hist_offsets[u+1]-1 of
 * hist_values (oldest first, L_u >= 1 rows). The n_q candidate tokens of
 * user u are rows u*n_q .. of cand_x, each fused with the user's context as
 * Q0 = [x_j ; c_u] W_q ([Repro] core formula; [LLaTTE] A.2 fusion).
 * Layer l (0-based) takes K = n_{l-1}(u) history rows as keys/values
 * (n_{-1} = L_u) and the last n_l(u) of them plus the candidates as queries.
 * History queries attend causally; candidates attend every history key.
 * Each layer is (PRE) R1 = R + MLA(RMSNorm(R)); R2 = R1 + FFN(RMSNorm(R1))
 * or (POST) R1 = RMSNorm(R + MLA(R)); R2 = RMSNorm(R1 + FFN(R1)), with
 * FFN(x) = GELU(x W1) W2 (exact erf GELU) ([LLaTTE] A.2, A.3).
 * The readout runs one more layer with n = 0 whose queries are the seeds,
 * then emb_u = flatten(seed outputs of u, seed-major) W_p ([LLaTTE] A.2
 * sequence summaries, with a linear map).
 *
 * Precision of the BF16 path: matrices and activations entering matrix
 * products are bf16 with fp32 accumulation, except inside the attention core
 * where the latent C, the latent queries (times scale * log2 e), the softmax
 * weights and the latent output are fp16 (more mantissa than bf16 at the
 * same rate); the residual stream, norms and softmax statistics are fp32.
 * Range precondition of that choice: every element of C and of the scaled
 * latent queries must stay below 65504 in magnitude (fp16's largest finite
 * value), else the outputs hold inf/NaN. With latent_norm = 1 (the
 * default, [LLaTTE] A.3) C is RMS-normalised, |C_j| <= sqrt(r) max|g_c|, so
 * this holds for any gains below 65504 / sqrt(r); with latent_norm = 0 it
 * is the caller's to ensure (|RMSNorm(R) W_dkv| and |q W_uk^T| / sqrt(d_k)
 * * 1.443 below 65504). llatte_mla_attention itself has no such limit (it
 * rescales its inputs by powers of two). The F32 path has none.
 *
 *   desc               host pointer
 *   w                  host pointer to device weights; may be NULL when
 *                      packed_weights is given
 *   packed_weights     NULL, or a blob written by llatte_pack_weights for
 *                      this desc (saves re-packing the weights every call)
 *   hist_values        [total_rows, d] float32
 *   hist_offsets       [B+1] int32, hist_offsets[0] = 0, strictly increasing
 *   B                  users (>= 1)
 *   total_rows         host copy of hist_offsets[B]
 *   max_len            host upper bound of every L_u
 *   cand_x             [B*n_q, d] float32 (NULL iff n_q == 0)
 *   ctx                [B, d_ctx] float32 (NULL iff d_ctx == 0 or n_q == 0)
 *   out_cand           [B*n_q, d] float32 (NULL iff n_q == 0)
 *   out_hist           [sum_u n_{N-1}(u), d] float32, or NULL; rows ordered
 *                      by user, oldest first; llatte_pyramid_counts_host
 *                      gives the row count
 *   out_hist_offsets   [B+1] int32 or NULL: offsets of out_hist
 *   out_emb            [B, d_out] float32 (NULL iff n_seeds == 0)
 *   workspace          >= llatte_mla_forward_workspace_size(...) bytes,
 *                      256-byte aligned
 * BF16 requires rank in {64, 128, 256} and head_dim in {32, 64, 128};
 * d and rank must be <= 1024.
 * ---------------------------------------------------------------------- */
llatte_status llatte_mla_forward(
    const llatte_model_desc* desc, const llatte_weights* w,
    const void* packed_weights, const float* hist_values,
    const int32_t* hist_offsets, int32_t B, int32_t total_rows,
    int32_t max_len, const float* cand_x, const float* ctx, float* out_cand,
    float* out_hist, int32_t* out_hist_offsets, float* out_emb,
    void* workspace, size_t workspace_bytes, void* stream);

/* Packed weights: every matrix of `w` transposed into the layout the kernels
 * read (K-contiguous), W_uv per head in fp16 on the BF16 path, gains and
 * seeds copied. The blob depends only on desc and w; write it once and pass
 * it to every llatte_mla_forward call. `packed` is device memory of at least
 * llatte_packed_weights_size(desc) bytes (0 = invalid desc). */
size_t llatte_packed_weights_size(const llatte_model_desc* desc);
llatte_status llatte_pack_weights(const llatte_model_desc* desc,
                                  const llatte_weights* w, void* packed,
                                  size_t packed_bytes, void* stream);

/* Workspace bytes needed by llatte_mla_forward for these sizes (host only;
 * returns 0 if the arguments are invalid). */
size_t llatte_mla_forward_workspace_size(const llatte_model_desc* desc,
                                         int32_t B, int32_t total_rows,
                                         int32_t max_len);

/* Row layout of the LLATTE_FLAG_DEBUG_DUMP buffer (host only): writes
 * n_layers + 2 (with a readout; n_layers + 1 without) int64 row offsets
 * to row_offsets (host array): section l = rows row_offsets[l] ..
 * row_offsets[l+1] - 1, each row d floats. Returns the number of offsets
 * written, 0 if the arguments are invalid. The buffer needs
 * row_offsets[last] * d * 4 bytes. */
int32_t llatte_mla_forward_debug_layout(const llatte_model_desc* desc,
                                        int32_t B, int32_t total_rows,
                                        int32_t max_len, int64_t* row_offsets);

/* ------------------------------------------------------------------------
 * llatte_mla_attention -- the attention core of the absorbed MLA form
 * ([LLaTTE] A.3, "MQA on the latent"): queries already moved into latent
 * space score against the shared latent C and average C itself.
 *
 *   out[i, j, :] = sum_k softmax_k(scale * q_lat[i, j, :] . C_k) * C_k
 *   lse[i, j]    = log(sum_k exp(scale * q_lat[i, j, :] . C_k))  (natural log)
 * over the keys k allowed to query row i (head j).
 *
 * Rows of q_lat / out: first the candidate rows, user-major
 * (user u's candidates are rows u*n_cand .. u*n_cand+n_cand-1), then the
 * history query rows: user u's are rows B*n_cand + hq_offsets[u] ..
 * B*n_cand + hq_offsets[u+1]-1. With n_u = hq_offsets[u+1]-hq_offsets[u]
 * <= K_u = kv_offsets[u+1]-kv_offsets[u], history row t sits at key position
 * K_u - n_u + t and attends keys 0 .. K_u - n_u + t (causal, [LLaTTE] A.2);
 * candidate rows attend all K_u keys. Every user needs K_u >= 1.
 *
 *   a                  host descriptor
 *   q_lat              [Mtot, h, r] dtype
 *   c_lat              [Ktot, r] dtype, user u's keys at kv_offsets[u]..
 *   kv_offsets         [B+1] int32;  hq_offsets [B+1] int32 (device)
 *   Mtot               host: B*n_cand + hq_offsets[B]
 *   Ktot               host: kv_offsets[B]
 *   out                [Mtot, h, r] float32 (normalised output)
 *   lse                [Mtot, h] float32 or NULL
 *   workspace          >= llatte_mla_attention_workspace_size(...) bytes
 * BF16 requires r in {64, 128, 256}; F32 accepts 1 <= r <= 256.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t n_heads; /* h                                      */
  int32_t rank;    /* r                                      */
  int32_t n_cand;  /* candidate rows per user (>= 0)         */
  int32_t dtype;   /* LLATTE_F32 or LLATTE_BF16              */
  float scale;     /* softmax scale, e.g. 1/sqrt(head_dim)   */
} llatte_attn_desc;

llatte_status llatte_mla_attention(
    const llatte_attn_desc* a, const void* q_lat, const void* c_lat,
    const int32_t* kv_offsets, const int32_t* hq_offsets, int32_t B,
    int32_t Mtot, int32_t Ktot, void* out, float* lse, void* workspace,
    size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * llatte_mla_attention_noalloc -- llatte_mla_attention for callers that
 * cannot allocate device memory or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, semantics and results as llatte_mla_attention, without
 * workspace / workspace_bytes: the attention plan lives in a fixed device
 * array of llatte_mla_attention_noalloc_max_scratch() bytes (8 MiB) inside
 * the library, one per GPU, held until the process ends. The call allocates
 * nothing. Sizes whose plan exceeds the array (llatte_mla_attention_
 * workspace_size(a, B, Mtot, Ktot) > 8 MiB, about 600 K query rows) return
 * LLATTE_ERR_WORKSPACE before anything is enqueued. Every call on a GPU uses
 * that GPU's one array, which keeps the last call's plan: calls that overlap
 * on one GPU (concurrent streams, or threads that do not serialise their
 * launches) race and must not be issued. The array's device address is
 * looked up on the first call on each device (that device current).
 * ---------------------------------------------------------------------- */
llatte_status llatte_mla_attention_noalloc(
    const llatte_attn_desc* a, const void* q_lat, const void* c_lat,
    const int32_t* kv_offsets, const int32_t* hq_offsets, int32_t B,
    int32_t Mtot, int32_t Ktot, void* out, float* lse, void* stream);

/* Bytes of the fixed scratch of llatte_mla_attention_noalloc. */
size_t llatte_mla_attention_noalloc_max_scratch(void);

/* ------------------------------------------------------------------------
 * llatte_mla_attention_backward -- gradients of llatte_mla_attention's
 * output with respect to q_lat and c_lat: the training backward of the
 * attention core of [LLaTTE] A.3 (C is both key and value), i.e. the
 * derivative of the definition above:
 *   p_k   = exp(scale q_lat[i,j,:] . C_k - lse[i,j])      (allowed keys)
 *   D     = d_out[i,j,:] . out[i,j,:]
 *   ds_k  = p_k (d_out[i,j,:] . C_k - D)
 *   d_q[i,j,:] = scale sum_k ds_k C_k
 *   d_c[k,:]   = sum over rows i and heads j that see key k of
 *                (p_k d_out[i,j,:] + scale ds_k q_lat[i,j,:])
 * Rows, masks, q_lat, c_lat, offsets, B, Mtot and Ktot as in
 * llatte_mla_attention; out and lse are that call's outputs (lse required);
 * d_out [Mtot, h, r] float32; d_q [Mtot, h, r] and d_c [Ktot, r] float32
 * are overwritten (d_c rows of every user, d_q rows of every query row).
 * max_len (host) must be >= every K_u: a smaller value leaves part of d_q
 * and d_c unwritten (no access outside the buffers). The softmax is
 * recomputed from lse. workspace: device memory of at least
 * llatte_mla_attention_backward_workspace_size(a, Mtot) bytes, caller-owned
 * (it holds D and d_out split into two bf16 parts between the two kernels).
 * With Mtot = 0, d_c is zeroed and q_lat, out, lse, d_out, d_q and workspace
 * may be NULL. Device pointers 16-byte aligned. Errors:
 * LLATTE_ERR_UNSUPPORTED unless dtype is BF16 and r is 64 or 128;
 * LLATTE_ERR_INVALID_ARG for NULL or misaligned pointers or bad sizes;
 * LLATTE_ERR_WORKSPACE if workspace_bytes is too small; LLATTE_ERR_HIP if a
 * launch fails. Nothing is enqueued on an argument error.
 * ---------------------------------------------------------------------- */
llatte_status llatte_mla_attention_backward(
    const llatte_attn_desc* a, const void* q_lat, const void* c_lat,
    const int32_t* kv_offsets, const int32_t* hq_offsets, int32_t B,
    int32_t Mtot, int32_t Ktot, int32_t max_len, const float* out,
    const float* lse, const float* d_out, float* d_q, float* d_c,
    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of llatte_mla_attention_backward (host only; 0 if the
 * descriptor is invalid). */
size_t llatte_mla_attention_backward_workspace_size(const llatte_attn_desc* a,
                                                    int32_t Mtot);

/* ------------------------------------------------------------------------
 * llatte_ffn_backward -- gradients of the pre-norm FFN sublayer of the
 * [LLaTTE] A.2 layer equation (pre-norm reading), row-wise over M rows:
 *   R2 = R1 + GELU(RMSNorm(R1) * g2 . W1) . W2     (exact-erf GELU, no bias)
 * Given d_out = dL/dR2 it writes
 *   d_r1 = dL/dR1 [M, d] (residual plus the path through norm and FFN),
 *   d_g2 [d], d_w1 [d, d_ff], d_w2 [d_ff, d]        (all float32),
 * recomputing RMSNorm(R1) and the pre-activation. The five products take
 * bf16 operands with fp32 accumulation: r1 and d_out are rounded to bf16
 * where they enter a product (the norm backward itself runs in fp32).
 *   f            host descriptor: d (multiple of 8, <= 1024), d_ff
 *                (multiple of 8), dtype (LLATTE_BF16 only), eps
 *   r1, d_out    [M, d] float32;  g2 [d] float32
 *   w1           [d, d_ff] bf16 row-major;  w2 [d_ff, d] bf16 row-major
 *   workspace    >= llatte_ffn_backward_workspace_size(f, M) bytes,
 *                caller-owned (recomputed activations, their transposes and
 *                the split-K scratch)
 * With M = 0 the weight and gain gradients are zeroed and r1, d_out, d_r1
 * and workspace may be NULL. Device pointers 16-byte aligned. Errors:
 * LLATTE_ERR_UNSUPPORTED for a dtype other than BF16; LLATTE_ERR_INVALID_ARG
 * for bad sizes or NULL / misaligned pointers; LLATTE_ERR_WORKSPACE if the
 * workspace is too small; LLATTE_ERR_HIP if a launch fails. Nothing is
 * enqueued on an argument error.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t d;      /* model width                  */
  int32_t d_ff;   /* FFN hidden width (4d)        */
  int32_t dtype;  /* LLATTE_BF16                  */
  float eps;      /* RMSNorm epsilon              */
} llatte_ffn_desc;

llatte_status llatte_ffn_backward(const llatte_ffn_desc* f, const float* r1,
                                  const float* g2, const void* w1,
                                  const void* w2, const float* d_out,
                                  int32_t M, float* d_r1, float* d_g2,
                                  float* d_w1, float* d_w2, void* workspace,
                                  size_t workspace_bytes, void* stream);
size_t llatte_ffn_backward_workspace_size(const llatte_ffn_desc* f,
                                          int32_t M);

/* ------------------------------------------------------------------------
 * llatte_attn_sublayer_backward -- gradients of the attention sublayer of
 * one pre-norm MLA layer ([LLaTTE] A.3 MLA with full-rank queries; A.2
 * layer equation, pre-norm reading), over a jagged batch of B users:
 *   H  = RMSNorm(R) g1 (every history row of the layer input, and the
 *        candidate rows),  C = RMSNorm(H W_dkv) g_c (or H W_dkv with
 *        latent_norm = 0),  q = H_q W_uq (the query rows),
 *   per head: K = C W_uk, V = C W_uv, o = softmax(q K^T / sqrt(d_k)) V
 *        (the masks of llatte_mla_attention),
 *   R1 = R_q + o W_o.
 * Given d_out = dL/dR1 for the query rows it writes the gradients of the
 * layer-input rows (history and candidate) and of g1, W_dkv, g_c, W_uq,
 * W_uk, W_uv, W_o. The forward is recomputed (in the absorbed form, on the
 * same kernels as llatte_mla_attention and llatte_mla_attention_backward);
 * products take bf16 operands with fp32 accumulation.
 *   d            host descriptor; BF16 only; rank 64 or 128; d and head_dim
 *                multiples of 8, d <= 1024
 *   w            host struct of device pointers: g1 [d], g_c [r] float32;
 *                w_dkv [d, r], w_uq [d, h*dk], w_uk [r, h*dk],
 *                w_uv [r, h*dk], w_o [h*dk, d] bf16 row-major (head j's
 *                columns of w_uq / w_uk / w_uv are j*dk .. j*dk+dk-1)
 *   r_kv         [Ktot, d] float32: user u's history rows at
 *                kv_offsets[u] .. kv_offsets[u+1]-1 (oldest first)
 *   r_cand       [B*n_cand, d] float32 (NULL if n_cand = 0)
 *   hq_offsets   [B+1]: user u's query rows are its last n_u history rows
 *   d_out        [Mtot, d] float32 in the attention row order (candidates
 *                u*n_cand.., then history query rows B*n_cand + hq_offsets[u]..)
 *   d_r_kv       [Ktot, d], d_r_cand [B*n_cand, d] float32 (overwritten)
 *   g            host struct of device pointers to the float32 gradients,
 *                overwritten, laid out as the weights (g_c ignored with
 *                latent_norm = 0)
 *   max_len      host: >= every K_u
 *   workspace    >= llatte_attn_sublayer_backward_workspace_size(...) bytes
 * With Mtot = 0 (no query rows) every gradient is zeroed. Device pointers
 * 16-byte aligned. Errors: LLATTE_ERR_UNSUPPORTED (dtype, rank, latent
 * norm flag), LLATTE_ERR_INVALID_ARG (sizes, NULL or misaligned pointers),
 * LLATTE_ERR_WORKSPACE, LLATTE_ERR_HIP. Nothing is enqueued on an argument
 * error.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t d, n_heads, head_dim, rank, n_cand, dtype, latent_norm;
  float eps;
} llatte_attn_sublayer_desc;

typedef struct {
  const float* g1;
  const void* w_dkv;
  const float* g_c;
  const void* w_uq;
  const void* w_uk;
  const void* w_uv;
  const void* w_o;
} llatte_attn_sublayer_weights;

typedef struct {
  float* g1;
  float* w_dkv;
  float* g_c;
  float* w_uq;
  float* w_uk;
  float* w_uv;
  float* w_o;
} llatte_attn_sublayer_grads;

llatte_status llatte_attn_sublayer_backward(
    const llatte_attn_sublayer_desc* d, const llatte_attn_sublayer_weights* w,
    const float* r_kv, const float* r_cand, const int32_t* kv_offsets,
    const int32_t* hq_offsets, int32_t B, int32_t Mtot, int32_t Ktot,
    int32_t max_len, const float* d_out, float* d_r_kv, float* d_r_cand,
    const llatte_attn_sublayer_grads* g, void* workspace,
    size_t workspace_bytes, void* stream);
size_t llatte_attn_sublayer_backward_workspace_size(
    const llatte_attn_sublayer_desc* d, int32_t B, int32_t Mtot,
    int32_t Ktot);

size_t llatte_mla_attention_workspace_size(const llatte_attn_desc* a,
                                           int32_t B, int32_t Mtot,
                                           int32_t Ktot);

/* ------------------------------------------------------------------------
 * llatte_mla_backward -- the training backward of the whole sequence module
 * of llatte_mla_forward (fusion, N layers with the pyramidal schedule, the
 * readout; [LLaTTE] 1.3.2, trained end to end as in 1.5.1): given the
 * gradients of a loss with respect to the forward's outputs, it writes the
 * gradients with respect to every weight and to the inputs. The forward
 * runs again on the same kernels as llatte_mla_forward, keeping each
 * layer's output rows and its rows after the attention sublayer (R1); then
 * the layers are walked back with llatte_ffn_backward and
 * llatte_attn_sublayer_backward ([LLaTTE] A.2 layer equation, pre-norm
 * reading; A.3 MLA):
 *   - layer l's output rows are its query rows (the candidates, then the
 *     last n_l(u) history rows of each user, oldest first); their gradient
 *     gives the gradient of all of layer l's input rows, which are layer
 *     l-1's output rows (the pyramid keeps the most recent rows), so rows
 *     that layer l does not keep get only its key/value terms;
 *   - the readout layer (queries = the seeds, keys = the last layer's
 *     history outputs, n = 0) adds its key gradient to the last layer's
 *     history output gradient; the seeds' gradient is summed over users;
 *     emb = flatten(Z) W_p gives dZ = d_emb W_p^T and dW_p = flatten(Z)^T
 *     d_emb (with LLATTE_FLAG_RAW_READOUT dZ = d_emb);
 *   - the fusion Q0 = [x ; c] W_q gives dW_q = [x ; c]^T dQ0 and
 *     d[x ; c] = dQ0 W_q^T, the context part summed over each user's
 *     candidates.
 * Products take bf16 operands with fp32 accumulation; gradients are fp32.
 *   desc               as llatte_mla_forward; supported: dtype BF16,
 *                      norm_mode PRE, q_rank 0, rank 64 or 128, d_out a
 *                      multiple of 8 (W_p readout); flags 0 or
 *                      LLATTE_FLAG_RAW_READOUT
 *   w                  host pointer to the device weights (raw layout, as
 *                      llatte_mla_forward's w; packed weights are not
 *                      accepted: the backward reads the raw matrices)
 *   hist_values, hist_offsets, B, total_rows, max_len, cand_x, ctx
 *                      as llatte_mla_forward
 *   hist_offsets_host  host copy of hist_offsets (B+1): the per-layer row
 *                      counts are sized on the host
 *   d_out_cand         [B*n_q, d] float32 (NULL iff n_q == 0): dL/d out_cand
 *   d_out_hist         rows of out_hist, float32, or NULL (zero)
 *   d_out_emb          [B, d_out] float32 (NULL iff n_seeds == 0); with
 *                      LLATTE_FLAG_RAW_READOUT [B, n_seeds*d]
 *   g                  host pointer to the gradients (device float32,
 *                      each laid out as its weight, overwritten): layers
 *                      (host array of n_layers), W_q (n_q > 0), seeds,
 *                      readout and W_p (n_seeds > 0; W_p not with
 *                      LLATTE_FLAG_RAW_READOUT); g_c is not written with
 *                      latent_norm = 0
 *   d_hist             [total_rows, d] float32, overwritten
 *   d_cand_x           [B*n_q, d] float32 (NULL iff n_q == 0), overwritten
 *   d_ctx              [B, d_ctx] float32 (NULL iff d_ctx == 0 or n_q == 0)
 *   workspace          >= llatte_mla_backward_workspace_size(...) bytes,
 *                      256-byte aligned
 * Errors: LLATTE_ERR_UNSUPPORTED outside the supported set above;
 * LLATTE_ERR_INVALID_ARG for NULL or misaligned pointers, bad sizes or host
 * offsets that disagree with total_rows / max_len; LLATTE_ERR_WORKSPACE;
 * LLATTE_ERR_HIP. Nothing is enqueued on an argument error.
 * ---------------------------------------------------------------------- */
typedef struct {
  float* g1;
  float* W_dkv;
  float* g_c;
  float* W_uq;
  float* W_uk;
  float* W_uv;
  float* W_o;
  float* g2;
  float* W1;
  float* W2;
} llatte_layer_grads;

typedef struct {
  const llatte_layer_grads* layers;  /* HOST array of n_layers */
  float* W_q;
  float* seeds;
  llatte_layer_grads readout;
  float* W_p;
} llatte_grads;

llatte_status llatte_mla_backward(
    const llatte_model_desc* desc, const llatte_weights* w,
    const float* hist_values, const int32_t* hist_offsets,
    const int32_t* hist_offsets_host, int32_t B, int32_t total_rows,
    int32_t max_len, const float* cand_x, const float* ctx,
    const float* d_out_cand, const float* d_out_hist, const float* d_out_emb,
    const llatte_grads* g, float* d_hist, float* d_cand_x, float* d_ctx,
    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of llatte_mla_backward (host only; 0 if the descriptor is
 * invalid or outside the supported set). */
size_t llatte_mla_backward_workspace_size(const llatte_model_desc* desc,
                                          int32_t B, int32_t total_rows,
                                          int32_t max_len);

/* ------------------------------------------------------------------------
 * llatte_pyramid_compact -- keep the last keep[u] rows of every user's
 * segment, in order ([LLaTTE] A.2: the next layer works on
 * X[:, -T_{l+1}:, :]).
 *
 *   values             [total_rows, row_elems] of dtype dt (F32 or BF16)
 *   offsets_in         [B+1] int32 (device); total_rows = offsets_in[B] (host)
 *   keep               [B] int32, 0 <= keep[u] <= L_u
 *   values_out         [>= sum keep, row_elems]
 *   offsets_out        [B+1] int32: exclusive scan of keep
 *   src_index          [sum keep] int32 or NULL: global source row of each
 *                      kept row, offsets_in[u] + L_u - keep[u] + t
 * Integer-exact; rows are copied bit for bit.
 * ---------------------------------------------------------------------- */
llatte_status llatte_pyramid_compact(const void* values, int32_t row_elems,
                                     int32_t dt, const int32_t* offsets_in,
                                     int32_t B, int32_t total_rows,
                                     const int32_t* keep, void* values_out,
                                     int32_t* offsets_out, int32_t* src_index,
                                     void* stream);

/* ------------------------------------------------------------------------
 * llatte_pyramid_counts -- evaluate a pyramid rule on the device:
 * keep_out[l*B + u] = n_l(u) for l < n_layers ([LLaTTE] A.2).
 *   rule (host), offsets_in [B+1] (device), keep_out [n_layers*B] (device)
 * llatte_pyramid_counts_host is the same on host arrays (lengths [B]).
 * ---------------------------------------------------------------------- */
llatte_status llatte_pyramid_counts(const llatte_pyramid_rule* rule,
                                    int32_t n_layers,
                                    const int32_t* offsets_in, int32_t B,
                                    int32_t* keep_out, void* stream);

llatte_status llatte_pyramid_counts_host(const llatte_pyramid_rule* rule,
                                         int32_t n_layers,
                                         const int32_t* lengths, int32_t B,
                                         int32_t* keep_out);

/* ------------------------------------------------------------------------
 * llatte_token_embed -- event tokens from a hashed-ID table plus a
 * projected semantic vector ([LLaTTE] section 1.3 features: sparse-ID
 * embeddings and dense content embeddings per event):
 *   out[i, :] = table[rows[i], :] + sem[i, :] W_s
 *
 *   table [V, d] dtype; rows [n] int32 in [0, V); sem [n, d_sem] dtype;
 *   W_s [d_sem, d] dtype; out [n, d] float32.
 *   workspace >= llatte_token_embed_workspace_size(d, d_sem, dt) bytes.
 * ---------------------------------------------------------------------- */
llatte_status llatte_token_embed(const void* table, int32_t V,
                                 const int32_t* rows, const void* sem,
                                 const void* W_s, int32_t n, int32_t d,
                                 int32_t d_sem, int32_t dt, float* out,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

size_t llatte_token_embed_workspace_size(int32_t d, int32_t d_sem,
                                         int32_t dt);

/* ------------------------------------------------------------------------
 * llatte_action_tokenize -- one d-wide token per user action ([LLaTTE]
 * Appendix A.2, Sequence Module item 1): each action (timestamp tau, type,
 * item, surface, meta) is embedded per field, the five embeddings pass
 * through MLP_act, and additive timestamp encodings go on a subset of the
 * hidden dimensions:
 *   age   = max(0, t_req[u] - tau[i])               (u = the row's user)
 *   U[i]  = [E_type[type_i] | E_item[item_i] | E_surf[surf_i]
 *            | E_time[min(floor(log2(1 + age)), n_buckets - 1)]
 *            | meta[i] W_meta]                        (d_in wide)
 *   out[i] = GELU(U[i] W_a) W_b + enc(age)            (exact-erf GELU)
 *   enc(age)[2j], [2j+1] = sin, cos of (age / 3600) 10000^(-2j / d_enc)
 *   for 2j < d_enc; 0 beyond.
 * The page fixes none of the field embeddings, MLP_act or the encoding;
 * these are the readings the library implements (one hidden layer, no
 * biases, log-bucketed age table, linear meta embedding, sinusoidal
 * encoding of the age in hours on the leading d_enc dimensions).
 *
 *   offsets [B+1] int32 (exclusive scan; user u owns rows offsets[u] ..
 *   offsets[u+1]-1, n = offsets[B]); t_req [B] int32 request time (s);
 *   tau, type_id, item_id, surf_id [n] int32; meta [n, d_meta] dtype.
 *   Tables E_type [V_type, d_type], E_item [V_item, d_item],
 *   E_surf [V_surf, d_surf], E_time [n_buckets, d_time], W_meta
 *   [d_meta, d_meta_emb], W_a [d_in, d_hidden], W_b [d_hidden, d], all in
 *   dtype, d_in = d_type + d_item + d_surf + d_time + d_meta_emb.
 *   out [n, d] float32.
 *   Widths: d_type, d_item, d_surf, d_time, d_meta_emb, d_hidden, d and
 *   d_meta are multiples of 8 (BF16) or 4 (F32); d_enc is even, <= d.
 *   Ids outside their table are clamped into it (no out-of-bounds read);
 *   timestamps after the request give age 0. n = 0 is valid and enqueues
 *   nothing (the per-row pointers may then be NULL).
 *   workspace >= llatte_action_tokenize_workspace_size(desc, n) bytes.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t d, d_hidden, d_enc;
  int32_t d_type, d_item, d_surf, d_time, d_meta, d_meta_emb;
  int32_t V_type, V_item, V_surf, n_buckets;
  int32_t dtype; /* LLATTE_F32 or LLATTE_BF16 */
} llatte_action_desc;

typedef struct {
  const void *E_type, *E_item, *E_surf, *E_time, *W_meta, *W_a, *W_b;
} llatte_action_weights;

llatte_status llatte_action_tokenize(const llatte_action_desc* desc /* host */,
                                     const llatte_action_weights* w /* host */,
                                     const int32_t* offsets, int32_t B, int32_t n,
                                     const int32_t* t_req, const int32_t* tau,
                                     const int32_t* type_id, const int32_t* item_id,
                                     const int32_t* surf_id, const void* meta,
                                     float* out, void* workspace,
                                     size_t workspace_bytes, void* stream);

size_t llatte_action_tokenize_workspace_size(const llatte_action_desc* desc,
                                             int32_t n);

/* ------------------------------------------------------------------------
 * Sequence summaries ([LLaTTE] Appendix A.2 item 4): K fixed-size summaries
 * of the flattened readout z = Flatten(Z_raw), each a low-rank adapted MLP.
 * The page gives no internals; the library implements one hidden layer with
 * the exact-erf GELU and no biases, base weights shared by the summaries and
 * rank-`rank` adapters per summary on both matrices:
 *   out[k] = GELU(z (W1 + A1[k] B1[k])) (W2 + A2[k] B2[k])
 *
 *   W1 [d_z, d_hidden], W2 [d_hidden, d_seq], A1 [K, d_z, rank],
 *   B1 [K, rank, d_hidden], A2 [K, d_hidden, rank], B2 [K, rank, d_seq],
 *   all in dtype. z [B, d_z] float32 (for instance out_emb of
 *   llatte_mla_forward with LLATTE_FLAG_RAW_READOUT); out [K, B, d_seq]
 *   float32. d_z, d_hidden and d_seq are multiples of 8 (BF16) or 4 (F32);
 *   1 <= rank <= 256; 1 <= n_summaries <= 64.
 *
 *   llatte_summary_pack merges the adapters into the base weights once (in
 *   dtype, transposed for the products) into caller memory of
 *   llatte_summary_packed_size(desc) bytes; llatte_summaries then needs a
 *   workspace of llatte_summaries_workspace_size(desc, B) bytes. B = 0 is
 *   valid and enqueues nothing.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t d_z, d_hidden, d_seq, rank, n_summaries;
  int32_t dtype; /* LLATTE_F32 or LLATTE_BF16 */
} llatte_summary_desc;

typedef struct {
  const void *W1, *W2, *A1, *B1, *A2, *B2;
} llatte_summary_weights;

size_t llatte_summary_packed_size(const llatte_summary_desc* desc);
llatte_status llatte_summary_pack(const llatte_summary_desc* desc /* host */,
                                  const llatte_summary_weights* w /* host */,
                                  void* packed, size_t packed_bytes, void* stream);
size_t llatte_summaries_workspace_size(const llatte_summary_desc* desc, int32_t B);
llatte_status llatte_summaries(const llatte_summary_desc* desc /* host */,
                               const void* packed, const float* z, int32_t B,
                               float* out, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * Diagnostics.
 *   llatte_last_error   message of the last non-OK status on this thread
 *   llatte_version      library version (major*10000 + minor*100 + patch)
 *   llatte_kernel_timing_enable(1) makes later calls on this thread record
 *   HIP events around every kernel launch; llatte_kernel_timing_read then
 *   synchronises those events and fills, per kernel name (up to `cap`
 *   entries), the launch count and summed milliseconds. Returns the number
 *   of entries. Timing adds one event pair per launch; leave it off for
 *   throughput runs.
 * ---------------------------------------------------------------------- */
const char* llatte_last_error(void);
int32_t llatte_version(void);
void llatte_kernel_timing_enable(int32_t on);
int32_t llatte_kernel_timing_read(char* names, int32_t name_stride,
                                  int32_t* counts, double* ms, int32_t cap);
void llatte_kernel_timing_reset(void);

/* Phase breakdown of the bf16 attention kernel (a diagnostic; the absorbed
 * form's three parts, [LLaTTE] App. A.3: the W_uk absorption of the queries,
 * the key-tile loop of latent flash attention, the W_uv map of the output).
 *   llatte_attention_phases_enable(max_workgroups) allocates room for that
 *   many workgroups' stamps on the current device (0 frees and turns the
 *   diagnostic off; LLATTE_ERR_HIP if the allocation fails). While it is on,
 *   every bf16 attention launch of this thread (forward layers, standalone
 *   calls, the backward's recomputed forward) runs an instrumented copy of
 *   the kernel whose workgroups stamp the 100 MHz real-time clock at their
 *   start, after the prologue, after the key loop and after their last
 *   store; the library then synchronises the stream and reduces the stamps.
 *   Launches with more workgroups than the room are not instrumented. Not
 *   for throughput runs, and not with llatte_mla_attention_noalloc (it
 *   allocates).
 *   llatte_attention_phases_read(out, cap) writes up to cap records of
 *   LLATTE_ATTN_PHASE_FIELDS doubles to out (host), one per instrumented
 *   launch in launch order: workgroups; summed prologue, key-loop and
 *   epilogue microseconds over those workgroups; the launch span (first
 *   start to last end, us); the longest workgroup (us). Returns the number
 *   of records taken since the last enable (out may be NULL to count). */
#define LLATTE_ATTN_PHASE_FIELDS 6
llatte_status llatte_attention_phases_enable(int32_t max_workgroups);
int32_t llatte_attention_phases_read(double* out, int32_t cap);

/* Phase breakdown of the bf16 matrix products on the 128 x 128 tile staged
 * by LDS DMA (a diagnostic; the products of [LLaTTE] App. A.2's layer
 * equation and App. A.3's projections that run on it: the large W_dkv,
 * W_uq, W_o, W1 and W2 launches).
 *   llatte_gemm_phases_enable(max_workgroups) allocates room for that many
 *   workgroups' stamps on the current device (0 frees and turns the
 *   diagnostic off; LLATTE_ERR_HIP if the allocation fails). While it is on,
 *   every such product of this thread whose K is not split runs an
 *   instrumented copy of the kernel whose workgroups stamp the 100 MHz
 *   real-time clock at their start, once their first operands have landed,
 *   once their last products have landed and after their last store; the
 *   library then synchronises the stream and reduces the stamps. Launches
 *   with more workgroups than the room, and the other tiles, are not
 *   instrumented. Not for throughput runs.
 *   llatte_gemm_phases_read(out, cap) writes up to cap records of
 *   LLATTE_GEMM_PHASE_FIELDS doubles to out (host), one per instrumented
 *   launch in launch order: workgroups with rows; the row bound M, N and K
 *   of the product; summed wait for the first operands, K loop and
 *   epilogue microseconds over those workgroups; the launch span (us); the
 *   longest workgroup (us). Returns the number of records taken since the
 *   last enable (out may be NULL to count). */
#define LLATTE_GEMM_PHASE_FIELDS 9
llatte_status llatte_gemm_phases_enable(int32_t max_workgroups);
int32_t llatte_gemm_phases_read(double* out, int32_t cap);

#ifdef __cplusplus
}
#endif
#endif /* LLATTE_H */
