// Internal launcher interfaces between the C-ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace llatte {

// ------------------------------------------------------------------ timing
// Optional per-launch HIP-event timing (off by default). `name` must be a
// string literal.
void timing_begin(const char* name, hipStream_t s);
void timing_end(hipStream_t s);

// ------------------------------------------------------------------ GEMM
// Element kinds of buffers whose type is chosen at run time.
enum Kind { K_F32 = 0, K_BF16 = 1, K_F16 = 2 };

// C[m, n] = sum_k A[m, k] * B[n, k]  (A row-major [M, K], B row-major [N, K],
// i.e. both operands K-contiguous), fp32 accumulation, then an epilogue.
enum GemmEpi {
  EPI_STORE = 0,       // C (dtype) = alpha * acc
  EPI_STORE_F32 = 1,   // C (float) = alpha * acc
  EPI_GELU = 2,        // C (dtype) = gelu(acc)
  EPI_RESID_F32 = 3,   // C (float) = acc + res.row(res_rows ? res_rows[m] : m)
  EPI_GATHER_ADD_F32 = 4,  // C (float) = acc + table[g_rows[m]]
  EPI_ROWNORM = 5,     // C (out_kind) = gain ? RMSNorm(acc) * gain : acc;
                       // with a gain the tile must span all N columns
  EPI_GELU_BWD = 6,    // with a = table[m][n] (dtype): C (dtype) = acc GELU'(a),
                       // cast_out (dtype) = GELU(a)  (exact erf)
};

// Fused RMSNorm of the A rows. A holds the rows x unscaled (cast to the
// compute dtype) and the gain is folded into B; since the norm's row scale
// commutes with the product, the epilogue multiplies acc by
//   1 / sqrt(sum_p ss[p * ld + row] / n + eps),  row = a_rows ? a_rows[m] : m,
// where ss holds partial sums of squares of x written by the producer,
// slot-major so that consecutive rows are consecutive addresses.
struct RowScale {
  const float* ss = nullptr;
  int np = 0;
  long long ld = 0;
  int n = 0;
  float eps = 0.f;
};

struct GemmParams {
  const void* A = nullptr;
  int lda = 0;
  const int* a_rows = nullptr;  // optional gather: A row m is A[a_rows[m]]
  const void* B = nullptr;
  int ldb = 0;
  int M_cap = 0;
  const int* M_dev = nullptr;   // optional device-side row count (<= M_cap)
  int N = 0, K = 0;
  int batch = 1;                // grid.z; operands advance by the strides
  long long sA = 0, sB = 0, sC = 0;
  int epi = EPI_STORE;
  const char* name = "gemm";    // label for the optional kernel timing
  void* C = nullptr;
  int ldc = 0;
  float alpha = 1.f;
  RowScale rs{};                // optional, applied before the epilogue
  RowSrc res{};                 // EPI_RESID_F32
  const int* res_rows = nullptr;
  // EPI_RESID_F32 extras for a following fused RMSNorm: the result cast to
  // the dtype ([M, ld_cast]) and per-row partial sums of its squares,
  // ss_out[slot * ss_ld + m], one slot per wave column strip
  // (gemm_ss_slots() of them).
  void* cast_out = nullptr;
  int ld_cast = 0;
  float* ss_out = nullptr;
  long long ss_ld = 0;
  const void* table = nullptr;  // EPI_GATHER_ADD_F32 (dtype of A)
  int ld_table = 0;
  const int* g_rows = nullptr;
  const float* gain = nullptr;  // EPI_ROWNORM
  float eps = 0.f;
  int out_kind = K_BF16;
  // Non-temporal output stores (EPI_STORE, EPI_GELU, and the float result
  // of EPI_RESID_F32; its cast copy, read by the next GEMM, stays cached): a
  // large output streams to HBM without displacing the operands the tiles
  // still read from the caches.
  bool nt = false;
  // EPI_STORE_F32 extra (timestamp encoding of the action tokens): columns
  // 2i, 2i+1 < enc_dims of row m get sin / cos of
  // (enc_age[m] / 3600) * 10000^(-2i / enc_dims), computed in fp64.
  const int* enc_age = nullptr;
  int enc_dims = 0;
  // Split-K scratch (optional, sk_part_cap floats): with it, launches that
  // leave the GPU short of workgroups split K into sk_splits parts (set by
  // the launcher); a first launch stores each split's fp32 tile, a second
  // sums them in split order and runs the epilogue.
  float* sk_part = nullptr;
  long long sk_part_cap = 0;
  int sk_splits = 1;
  // Phase stamps of the diagnostic kernel copy (gemm_phases_enable): four
  // 64-bit clock values per workgroup, in launch order.
  unsigned long long* clk = nullptr;
};

// Partial sums of squares per row that an EPI_RESID_F32 launch with these
// parameters writes to ss_out.
int gemm_ss_slots(const GemmParams& p, bool bf16);
hipError_t gemm(const GemmParams& p, bool bf16, hipStream_t s);
// Phase diagnostic of the 128 x 128 LDS-staged tile (llatte_gemm_phases_*).
hipError_t gemm_phases_enable(int max_wg);
int gemm_phases_read(double* out, int cap);
constexpr int kGemmPhaseFields = 9;

// ------------------------------------------------------------------ actions
// U[row] = [E_type(type) | E_item(item) | E_surf(surf) | E_time(bucket) |
// meta W_meta] in the dtype, and age[row] (seconds, >= 0), for n actions of
// B users (rows offsets[u] .. offsets[u+1]-1 belong to user u). Field widths
// are multiples of 16 bytes of the dtype.
struct ActionConcat {
  const int* offsets = nullptr;
  int B = 0, n = 0;
  const int* t_req = nullptr;
  const int* tau = nullptr;
  const int* type_id = nullptr;
  const int* item_id = nullptr;
  const int* surf_id = nullptr;
  const void* meta = nullptr;
  const void* E_type = nullptr;
  const void* E_item = nullptr;
  const void* E_surf = nullptr;
  const void* E_time = nullptr;
  const void* W_meta = nullptr;
  int d_type = 0, d_item = 0, d_surf = 0, d_time = 0, d_meta = 0, d_meta_emb = 0, d_in = 0;
  int V_type = 0, V_item = 0, V_surf = 0, n_buckets = 0;
  void* U = nullptr;
  int* age = nullptr;
};
hipError_t action_concat(const ActionConcat& p, bool bf16, hipStream_t s);

// ------------------------------------------------------------------ summaries
// out[k] = (W + A[k] Bm[k])^T in the dtype: W [rows, cols], A [K, rows,
// rank], Bm [K, rank, cols], out [K, cols, rows].
hipError_t lora_merge(const void* W, const void* A, const void* Bm, int rows, int cols,
                      int rank, int K, void* out, bool bf16, hipStream_t s);
// dst (dtype) = src (float32), n elements.
hipError_t cast_f32(const float* src, void* dst, long long n, bool bf16, hipStream_t s);

// ------------------------------------------------------------------ row ops
// One wave per row (d <= 1024): out = gain ? x / sqrt(mean(x^2) + eps) * gain : x, where
// x = src.row(i); written as float to out_f32 (may alias the source) and/or
// as `t_kind` to out_t; ss_out (optional) receives sum(x^2) of each row.
// Rows i >= *rows_dev (if given) are skipped.
hipError_t norm_rows(RowSrc src, int rows_cap, const int* rows_dev,
                     const float* gain, float eps, float* out_f32, int ld_f32,
                     void* out_t, int ld_t, int d, int t_kind, hipStream_t s,
                     float* ss_out = nullptr);

// dst [cols, rows] = transpose(src [rows, cols]) for a batch of `batch`
// matrices laid out with the given element strides; src has kind s_kind,
// dst kind d_kind (bf16 -> f16 and same-kind copies).
// row_scale (optional, float [src_rows]) multiplies source row i first.
hipError_t transpose(const void* src, int src_rows, int src_cols, int ld_src,
                     long long s_src, void* dst, int ld_dst, long long s_dst,
                     int batch, int s_kind, int d_kind, hipStream_t s,
                     const float* row_scale = nullptr);

// xc (dtype) [B*n_q, d + d_c]: row u*n_q + j = [cand[u*n_q+j] ; ctx[u]].
hipError_t concat_queries(const float* cand, const float* ctx, int B, int n_q,
                          int d, int d_c, void* xc, bool bf16, hipStream_t s);

// out (float) [B*n_s, d]: row u*n_s + j = seeds[j].
hipError_t broadcast_rows(const float* seeds, int n_s, int d, int B,
                          float* out, hipStream_t s);

// Copy float rows [row0, row0 + count) of src into dst (count from device if
// count_dev is given, else count_cap).
hipError_t copy_rows_f32(const float* src, int ld, float* dst, int count_cap,
                         const int* count_dev, int d, hipStream_t s);

// out [na, width] (float): out[a][c] = sum over b < nb of
// src[(a sa + b sb) ld + col0 + c], added in increasing b.
hipError_t group_sum_rows(const float* src, int ld, int col0, int na, int sa, int nb, int sb,
                          int width, float* out, hipStream_t s);
// dst[i] += src[i], i < n (float).
hipError_t add_f32(float* dst, const float* src, long long n, hipStream_t s);

// ------------------------------------------------------------------ plan
// Per-layer device plan built from the history offsets.
struct LayerPlan {
  int* kv_len;     // [B]   keys per user at this layer (K_u)
  int* keep;       // [B]   history queries per user (n_u)
  int* kv_off;     // [B+1] exclusive scan of kv_len
  int* hq_off;     // [B+1] exclusive scan of keep
  int* counts;     // [4]   {sum K, sum n, rows = nc + sum K, M = nc + sum n}
  int* qmap;       // [qcap] query row -> row of the layer's row space
  int2* qinfo;     // [qcap] query row -> {kv base row, key position}
  i32x4* items;    // [icap] attention work items, heaviest first
  int* n_items;    // [1]
};

// All layers' plans in one block of device memory with fixed strides.
struct PlanBase {
  int* kv_len;   // [n_plans][B]
  int* keep;     // [n_plans][B]
  int* kv_off;   // [n_plans][ostride]: B+1 offsets, rows 16-byte aligned
  int* hq_off;   // [n_plans][ostride]
  int* counts;   // [n_plans][4]
  int* qmap;     // [n_plans][qcap]
  int2* qinfo;   // [n_plans][qcap]
  i32x4* items;  // [n_plans][icap]
  int* n_items;  // [n_plans]
  int B, qcap, icap;
  int ostride;   // B+1 rounded up to a multiple of 4
  __host__ __device__ static int offsets_stride(int B) { return (B + 4) & ~3; }
  __host__ __device__ LayerPlan layer(int l) const {
    LayerPlan p;
    p.kv_len = kv_len + (size_t)l * B;
    p.keep = keep + (size_t)l * B;
    p.kv_off = kv_off + (size_t)l * ostride;
    p.hq_off = hq_off + (size_t)l * ostride;
    p.counts = counts + (size_t)l * 4;
    p.qmap = qmap + (size_t)l * qcap;
    p.qinfo = qinfo + (size_t)l * qcap;
    p.items = items + (size_t)l * icap;
    p.n_items = n_items + l;
    return p;
  }
  // bytes of device memory for n_plans layers
  static size_t bytes(int n_plans, int B, int qcap, int icap) {
    size_t n = (size_t)n_plans;
    return n * (2 * (size_t)B + 2 * (size_t)offsets_stride(B) + 4 + 1) * sizeof(int) +
           n * (size_t)qcap * (sizeof(int) + sizeof(int2)) +
           n * (size_t)icap * sizeof(i32x4) + 64 * 9;
  }
};

// A pyramid rule with the per-layer list already expanded on the host
// (FIXED and GEOMETRIC: kind 0 with values; HALVING: kind 1 with floor).
struct RuleDev {
  int kind;
  int floor;
  int n_layers;
  int values[64];
};

// Builds the plans of layers 0..rule.n_layers-1, plus one readout plan
// (no history queries, n_seeds query tokens) when n_plans > n_layers.
// bq/bn: query rows and keys per attention tile (bq = 0: no work items).
// hq_copy (optional, device, B + 1 ints) receives a copy of plan
// copy_plan's history query offsets.
hipError_t build_plan(const int* offsets, int B, const RuleDev& rule, int n_q,
                      int n_seeds, const PlanBase& base, int n_plans, int bq,
                      int bn, hipStream_t s, int* hq_copy = nullptr, int copy_plan = -1);

// One-layer plan for the standalone attention entry from given offsets.
hipError_t build_attn_plan(const int* kv_off, const int* hq_off, int B,
                           int n_cand, int bq, int bn, const PlanBase& base,
                           hipStream_t s);

hipError_t pyramid_counts_dev(const RuleDev& rule, const int* offsets, int B,
                              int* keep_out, hipStream_t s);

// err[0..1] = {kind, user} of the first malformed history offset (0 when
// every L_u is in [1, max_len], offsets[0] == 0 and offsets[B] == total).
hipError_t validate_offsets(const int* offsets, int B, int total, int max_len, int* err,
                            hipStream_t s);

hipError_t pyramid_compact(const void* values, int row_bytes,
                           const int* offsets_in, int B, int total_rows,
                           const int* keep, void* values_out,
                           int* offsets_out, int* src_index, hipStream_t s);

// ------------------------------------------------------------------ attention
struct AttnParams {
  // fused (forward pass): q = query projection [M, h*dk] bf16, c = latent
  //   [Ktot, r] f16, w_uk [r, h*dk] bf16, w_uv_t [h][dk][r] f16,
  //   out = o [M, h*dk] bf16.
  // standalone (bf16): q = latent queries [M, h, r] bf16, c [Ktot, r] bf16,
  //   out [M, h, r] float32, lse [M, h] float32 or null.
  // f32 kernel: q [M, h, r], c [Ktot, r], out [M, h, r], all float32.
  const void* q;
  const void* c;
  void* out;
  float* lse;
  bool fused;
  const void* w_uk;
  const void* w_uv_t;
  int dk;
  int h, r;
  float scale;
  const i32x4* items; // bf16 path
  const int* n_items;
  int items_cap;
  const int2* qinfo;  // f32 path: per query row {kv base, key position}
  int M_cap;
  const int* M_dev;
  // standalone bf16 path: {max |q| * scale * log2 e, max |c|} as float bits
  // (attn_absmax); the kernel scales both by powers of two into fp16 range
  // and undoes the scaling exactly. nullptr: no scaling.
  const unsigned* amax = nullptr;
  // standalone bf16 path: also the output as bf16 ([M, h, r]), or nullptr
  bf16* out_bf16 = nullptr;
  // diagnostics only (attn_phases_enable): four real-time clock stamps per
  // workgroup, at [(blockIdx.y * gridDim.x + blockIdx.x) * 4]; nullptr in
  // normal operation.
  unsigned long long* clk = nullptr;
};

// LDS layout of the latent rows in the MFMA attention kernel: within each
// 32-element block of r, the 4-element chunk q (r = 4q .. 4q+3) is stored at
// chunk position slot(q) = 2q (q < 4) or 2(q-4) + 1 (q >= 4), so that chunks
// g and 4 + g (one lane group's k values of a 32-wide MFMA step) sit side by
// side. The kernel's output rows come in this stored order; the W_uv
// fragments (attn_pack_weights) take r in the same order.
__host__ __device__ constexpr int attn_chunk_slot(int q) { return q < 4 ? 2 * q : 2 * (q - 4) + 1; }
__host__ __device__ constexpr int attn_slot_chunk(int c) { return (c & 1) ? 4 + (c >> 1) : c >> 1; }

// Query rows per work item for the bf16 kernel at these sizes (0 if the
// shape is not supported by the MFMA kernel).
int attn_bq(int h, int r);
bool attn_fused_supported(int h, int r, int dk);
constexpr int kAttnBN = 64;
hipError_t attention(const AttnParams& p, bool bf16, hipStream_t s);
// Packs W_uk ([r, h*dk] bf16) and W_uv ([r, h*dk] bf16) for the fused bf16
// kernel in fragment order: per head, per 16-row block and 32-wide k step
// of the MFMA operand, the 64 lanes' eight values in lane order (one
// 16-byte load per lane, 1 KB per wave). uk_frag: bf16, A operand of the
// W_uk product (rows r, k over the head's dk). uv_frag: fp16, A operand of
// the W_uv product (rows dk, k over r in the kernel's stored latent order).
// Both hold r * h * dk values; needs dk % 32 == 0 and r % 32 == 0.
hipError_t attn_pack_weights(const void* W_uk, const void* W_uv, int r, int h, int dk,
                             void* uk_frag, void* uv_frag, hipStream_t s);
// Phase diagnostics of the bf16 attention kernel, per calling thread:
// enable with room for max_wg workgroups (allocates on the current device;
// 0 frees and disables). While enabled, each bf16 attention launch runs the
// instrumented kernel copy, synchronises and appends one record of
// kAttnPhaseFields doubles: workgroups, summed prologue / key-loop /
// epilogue microseconds over workgroups, the launch span from the first
// start to the last end, and the longest workgroup.
constexpr int kAttnPhaseFields = 6;
hipError_t attn_phases_enable(int max_wg);
int attn_phases_read(double* out, int cap);
// amax[0] = max |q| * scale * log2 e, amax[1] = max |c| (bf16 inputs, float
// bits), followed by two words per scan block for the partial maxima: the
// buffer holds kAbsmaxWords unsigned, all written by this call (two launches,
// no memset, no atomics).
constexpr int kAbsmaxBlocks = 2048;
constexpr int kAbsmaxWords = 2 + 2 * kAbsmaxBlocks;
hipError_t attn_absmax(const void* q, long long nq, const void* c, long long nc, float scale,
                       unsigned* amax, hipStream_t s);

}  // namespace llatte
