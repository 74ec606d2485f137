// C ABI of the library: argument validation, workspace layout, and the
// composition of the forward pass from the kernels.
//
// Forward pass of one layer (LLaTTE Appendix A.2 layer equation and A.3
// MLA, absorbed form), rows of the layer's row space ordered as
// [candidate/seed rows (B*n_q) ; history rows (sum_u K_u, user-major)] and
// query rows as [candidates ; last n_u history rows of each user]:
//   H   = RMSNorm(R) (pre) or R (post), as the compute dtype
//   C   = H_hist W_dkv, then RMSNorm(C) g_c          (latent, [sum K, r])
//   q   = H[qmap] W_uq                               ([M, h*dk])
//   ql  = q_j W_uk_j^T per head j                    ([M, h, r], absorbed)
//   ol  = latent attention(ql, C)                    ([M, h, r])
//   o   = ol_j W_uv_j per head                       ([M, h*dk])
//   R1  = R[qmap] + o W_o              (post: then RMSNorm with g1)
//   R2  = R1 + GELU(RMSNorm(R1) W1) W2 (post: GELU(R1 W1) W2, then RMSNorm g2)
// The output rows are exactly the next layer's row space, so the pyramidal
// output extraction costs no copy.
//
// bf16 pre-norm path: the three RMSNorms run inside the GEMMs. A norm's row
// scale s(x) = 1/sqrt(mean(x^2) + eps) commutes with the product that
// follows it, RMSNorm(x) g W = s(x) * (x (diag(g) W)), so the gains are
// folded into W_dkv, W_uq (g1) and W1 (g2) at packing, the producer of x (the
// residual epilogues) also writes x as bf16 with per-row partial sums of
// squares, and the consumer GEMM scales its rows in the epilogue. The latent
// norm is the down-projection's epilogue (one tile spans the r columns).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/llatte.h"
#include "backward.hpp"

namespace llatte {

// ------------------------------------------------------------------ errors
static thread_local std::string t_err;

static llatte_status fail(llatte_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  t_err = buf;
  return code;
}

#define HIP_TRY(expr)                                                        \
  do {                                                                       \
    hipError_t e_ = (expr);                                                  \
    if (e_ != hipSuccess)                                                    \
      return fail(LLATTE_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// ------------------------------------------------------------------ timing
struct PendingEv {
  const char* name;
  hipEvent_t a, b;
};
static thread_local bool t_timing = false;
static thread_local std::vector<PendingEv> t_pending;
static thread_local std::map<std::string, std::pair<int, double>> t_acc;

void timing_begin(const char* name, hipStream_t s) {
  if (!t_timing) return;
  PendingEv p{name, nullptr, nullptr};
  if (hipEventCreate(&p.a) != hipSuccess || hipEventCreate(&p.b) != hipSuccess) return;
  hipEventRecord(p.a, s);
  t_pending.push_back(p);
}
void timing_end(hipStream_t s) {
  if (!t_timing || t_pending.empty()) return;
  hipEventRecord(t_pending.back().b, s);
}

static void timing_collect() {
  for (auto& p : t_pending) {
    float ms = 0.f;
    hipEventSynchronize(p.b);
    if (hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      auto& e = t_acc[p.name];
      e.first += 1;
      e.second += ms;
    }
    hipEventDestroy(p.a);
    hipEventDestroy(p.b);
  }
  t_pending.clear();
}

// ------------------------------------------------------------------ workspace
// Bump allocator: a dry run (base == nullptr) measures, a real run carves.
struct Arena {
  char* base;
  size_t off = 0;
  explicit Arena(void* b) : base((char*)b) {}
  template <typename T> T* take(size_t count) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

static PlanBase carve_plan(Arena& ar, int n_plans, int B, int qcap, int icap) {
  PlanBase pb;
  pb.B = B;
  pb.qcap = qcap;
  pb.icap = icap;
  pb.ostride = PlanBase::offsets_stride(B);
  pb.kv_len = ar.take<int>((size_t)n_plans * B);
  pb.keep = ar.take<int>((size_t)n_plans * B);
  pb.kv_off = ar.take<int>((size_t)n_plans * pb.ostride);
  pb.hq_off = ar.take<int>((size_t)n_plans * pb.ostride);
  pb.counts = ar.take<int>((size_t)n_plans * 4);
  pb.qmap = ar.take<int>((size_t)n_plans * qcap);
  pb.qinfo = ar.take<int2>((size_t)n_plans * qcap);
  pb.items = ar.take<i32x4>((size_t)n_plans * icap);
  pb.n_items = ar.take<int>((size_t)n_plans);
  return pb;
}

// ------------------------------------------------------------------ shapes
struct Shapes {
  int B, total, max_len;
  int d, h, dk, hd, r, dff, N, nq, dc, ns, dout;
  int rq, qin;                // query rank (0: full rank) and W_uq input width
  bool bf16, pre, lnorm;
  bool fnorm;                 // norms fused into the GEMMs (bf16, pre-norm)
  bool raw = false;           // readout returns Flatten(Z_raw) (no W_p)
  bool validate = false;      // device check of the history offsets first
  bool dump = false;          // per-layer output rows into desc->debug_dump
  float eps;
  int NP;                     // plans: N layers (+ readout)
  RuleDev rule;
  std::vector<long long> UBn, UBK, UBM, UBrows;
  int qcap = 0, icap = 1, bq = 0;
  size_t esz;                 // bytes per dtype element
};

static long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

static llatte_status expand_rule(const llatte_pyramid_rule* pr, int N,
                                 RuleDev* out) {
  memset(out, 0, sizeof *out);
  out->n_layers = N;
  if (pr->kind == LLATTE_PYR_HALVING) {
    if (pr->floor < 1) return fail(LLATTE_ERR_INVALID_ARG, "halving floor must be >= 1");
    out->kind = 1;
    out->floor = pr->floor;
    return LLATTE_OK;
  }
  out->kind = 0;
  if (pr->kind == LLATTE_PYR_FIXED) {
    for (int l = 0; l < N; ++l) {
      if (pr->values[l] < 0) return fail(LLATTE_ERR_INVALID_ARG, "pyramid count < 0 at layer %d", l);
      if (pr->values[l] == 0 && l != N - 1)
        return fail(LLATTE_ERR_INVALID_ARG, "a pyramid count of 0 is allowed only at the last layer");
      out->values[l] = pr->values[l];
    }
    return LLATTE_OK;
  }
  if (pr->kind == LLATTE_PYR_GEOMETRIC) {
    if (pr->start < 1 || pr->end < 1)
      return fail(LLATTE_ERR_INVALID_ARG, "geometric endpoints must be >= 1");
    for (int l = 0; l < N; ++l) {
      double v = N == 1 ? (double)pr->start
                        : (double)pr->start *
                              pow((double)pr->end / (double)pr->start, (double)l / (N - 1));
      out->values[l] = (int)floor(v + 0.5);
    }
    return LLATTE_OK;
  }
  return fail(LLATTE_ERR_INVALID_ARG, "unknown pyramid kind %d", pr->kind);
}

static llatte_status make_shapes(const llatte_model_desc* dsc, int B, int total,
                                 int max_len, Shapes* S) {
  if (!dsc) return fail(LLATTE_ERR_INVALID_ARG, "desc is NULL");
  if (dsc->flags & ~(LLATTE_FLAG_RAW_READOUT | LLATTE_FLAG_VALIDATE | LLATTE_FLAG_DEBUG_DUMP))
    return fail(LLATTE_ERR_INVALID_ARG, "unknown flags 0x%x", dsc->flags);
  if (B < 1 || total < B || max_len < 1 || (long long)max_len * B < total)
    return fail(LLATTE_ERR_INVALID_ARG, "need B >= 1, total_rows >= B, max_len*B >= total_rows");
  if (dsc->dtype != LLATTE_F32 && dsc->dtype != LLATTE_BF16)
    return fail(LLATTE_ERR_UNSUPPORTED, "dtype %d", dsc->dtype);
  if (dsc->norm_mode != LLATTE_NORM_PRE && dsc->norm_mode != LLATTE_NORM_POST)
    return fail(LLATTE_ERR_INVALID_ARG, "norm_mode %d", dsc->norm_mode);
  if (dsc->n_layers < 1 || dsc->n_layers > LLATTE_MAX_LAYERS - 1)
    return fail(LLATTE_ERR_INVALID_ARG, "n_layers must be in [1, %d]", LLATTE_MAX_LAYERS - 1);
  S->B = B;
  S->total = total;
  S->max_len = max_len;
  S->d = dsc->d;
  S->h = dsc->n_heads;
  S->dk = dsc->head_dim;
  S->hd = S->h * S->dk;
  S->r = dsc->rank;
  S->dff = dsc->d_ff;
  S->N = dsc->n_layers;
  S->nq = dsc->n_q;
  S->dc = dsc->d_ctx;
  S->ns = dsc->n_seeds;
  S->dout = dsc->d_out;
  S->raw = (dsc->flags & LLATTE_FLAG_RAW_READOUT) != 0;
  S->validate = (dsc->flags & LLATTE_FLAG_VALIDATE) != 0;
  S->dump = (dsc->flags & LLATTE_FLAG_DEBUG_DUMP) != 0;
  S->rq = dsc->q_rank;
  S->qin = S->rq > 0 ? S->rq : dsc->d;
  S->bf16 = dsc->dtype == LLATTE_BF16;
  S->pre = dsc->norm_mode == LLATTE_NORM_PRE;
  S->lnorm = dsc->latent_norm != 0;
  S->fnorm = S->bf16 && S->pre;
  S->eps = dsc->eps;
  S->esz = S->bf16 ? 2 : 4;
  const int al = S->bf16 ? 8 : 4;  // 16-byte vectors of the dtype
  if (S->d < al || S->h < 1 || S->dk < 1 || S->r < 1 || S->nq < 0 || S->dc < 0 ||
      S->ns < 0)
    return fail(LLATTE_ERR_INVALID_ARG, "bad model dimensions");
  if (S->d % al || S->dk % al || S->r % al || (S->d + S->dc) % al)
    return fail(LLATTE_ERR_UNSUPPORTED, "d, head_dim, rank and d+d_ctx must be multiples of %d", al);
  if (S->d > 1024 || S->r > 1024)
    return fail(LLATTE_ERR_UNSUPPORTED, "d and rank must be <= 1024");
  if (S->rq < 0 || S->rq > 1024 || S->rq % al)
    return fail(LLATTE_ERR_UNSUPPORTED, "q_rank must be 0 or a multiple of %d up to 1024", al);
  if (S->dff != 4 * S->d) return fail(LLATTE_ERR_INVALID_ARG, "d_ff must be 4*d");
  if (!(S->eps >= 0.f)) return fail(LLATTE_ERR_INVALID_ARG, "eps must be >= 0");
  if (S->nq == 0 && S->dc != 0) return fail(LLATTE_ERR_INVALID_ARG, "d_ctx needs n_q > 0");
  if (S->ns > 0 && (S->dout < 1 || S->dout % 4))
    return fail(LLATTE_ERR_INVALID_ARG, "d_out must be a positive multiple of 4");
  if (S->raw && S->ns > 0 && S->dout != S->ns * S->d)
    return fail(LLATTE_ERR_INVALID_ARG, "with LLATTE_FLAG_RAW_READOUT d_out must be n_seeds*d");
  if (S->bf16) {
    if (!attn_fused_supported(S->h, S->r, S->dk))
      return fail(LLATTE_ERR_UNSUPPORTED,
                  "bf16 path needs rank in {64, 128, 256} and head_dim in {32, 64, 128}");
  } else if (S->r > 256) {
    return fail(LLATTE_ERR_UNSUPPORTED, "f32 path needs rank <= 256");
  }
  llatte_status st = expand_rule(&dsc->pyramid, S->N, &S->rule);
  if (st) return st;
  if (S->ns > 0 && S->rule.kind == 0 && S->rule.values[S->N - 1] == 0)
    return fail(LLATTE_ERR_INVALID_ARG, "the readout needs history rows after the last layer");
  S->NP = S->N + (S->ns > 0 ? 1 : 0);
  S->bq = S->bf16 ? attn_bq(S->h, S->r) : 0;
  S->UBn.assign(S->NP, 0);
  S->UBK.assign(S->NP, 0);
  S->UBM.assign(S->NP, 0);
  S->UBrows.assign(S->NP, 0);
  long long prev = total;
  long long icap = 1, qcap = 0;
  for (int l = 0; l < S->NP; ++l) {
    long long n;
    if (l >= S->N)
      n = 0;
    else if (S->rule.kind == 1)
      n = std::min<long long>(std::min<long long>((long long)B * S->rule.floor, total) +
                                  ((long long)total >> std::min(l, 62)),
                              total);
    else
      n = std::min<long long>((long long)B * S->rule.values[l], total);
    n = std::min(n, prev);
    const int nql = l < S->N ? S->nq : S->ns;
    S->UBK[l] = prev;
    S->UBn[l] = n;
    S->UBM[l] = (long long)B * nql + n;
    S->UBrows[l] = (long long)B * nql + prev;
    qcap = std::max(qcap, S->UBM[l]);
    if (S->bq > 0)
      icap = std::max(icap, cdiv(n, S->bq) + B + (long long)B * cdiv(nql, S->bq));
    prev = n;
  }
  if (qcap >= (1LL << 31) || S->UBrows[0] >= (1LL << 31))
    return fail(LLATTE_ERR_UNSUPPORTED, "row counts exceed int32");
  S->qcap = (int)qcap;
  S->icap = (int)icap;
  return LLATTE_OK;
}

// Packed weights: matrices transposed to K-contiguous layout (the GEMM's
// B operand), W_uv per head transposed and in fp16 for the fused attention
// epilogue on the bf16 path, gains and seeds copied. One blob, written by
// llatte_pack_weights (or into the workspace by every forward call).
struct PackedLayer {
  float *g1, *g_c, *g2, *g_q;
  void *Wdkv, *Wuq, *Wuk, *Wuv, *Wo, *W1, *W2, *Wdq;
};
struct Packed {
  std::vector<PackedLayer> L;  // N layers (+ readout)
  void *WqT, *WpT;
  float* seeds;
};

static size_t layout_packed(const Shapes& S, void* base, Packed* P) {
  Arena ar(base);
  const size_t e = S.esz;
  P->L.resize(S.NP);
  for (int l = 0; l < S.NP; ++l) {
    PackedLayer& q = P->L[l];
    q.g1 = ar.take<float>(S.d);
    q.g_c = ar.take<float>(S.r);
    q.g2 = ar.take<float>(S.d);
    q.Wdkv = ar.take<char>((size_t)S.d * S.r * e);
    q.Wuq = ar.take<char>((size_t)S.qin * S.hd * e);
    q.Wdq = S.rq ? ar.take<char>((size_t)S.d * S.rq * e) : nullptr;
    q.g_q = S.rq ? ar.take<float>(S.rq) : nullptr;
    q.Wuk = ar.take<char>((size_t)S.r * S.hd * e);
    q.Wuv = ar.take<char>((size_t)S.r * S.hd * e);   // f16 on the bf16 path
    q.Wo = ar.take<char>((size_t)S.hd * S.d * e);
    q.W1 = ar.take<char>((size_t)S.d * S.dff * e);
    q.W2 = ar.take<char>((size_t)S.dff * S.d * e);
  }
  P->WqT = S.nq ? ar.take<char>((size_t)(S.d + S.dc) * S.d * e) : nullptr;
  P->WpT = S.ns ? ar.take<char>((size_t)S.ns * S.d * S.dout * e) : nullptr;
  P->seeds = S.ns ? ar.take<float>((size_t)S.ns * S.d) : nullptr;
  return ar.off + 256;
}

// Partial sums of squares per row written by a residual epilogue over d
// columns (one per 32-column strip at most).
static int kMaxSlots(const Shapes& S) { return (S.d + 31) / 32; }

// Workspace layout of the forward pass.
struct FwdWS {
  PlanBase plan;
  Packed pk;    // used when the caller passes no packed weights
  void* H;      // [max rows, d]
  float* Cf;    // [max K, r] latent before its norm
  void* Cl;     // [max K, r] (f16 on the bf16 path)
  void* q;      // [qcap, hd]
  void* Hq;     // [qcap, rq]  low-rank query path: RMSNorm(H W_dq) g_q
  float* Qf;    // [qcap, rq]  its fp32 input when the norm is a separate pass
  void* ql;     // [qcap, h, r]   (f32 path)
  void* ol;     // [qcap, h, r]   (f32 path)
  void* o;      // [qcap, hd]
  float* R1;    // [qcap, d]
  void* H2;     // [qcap, d]
  void* F;      // [qcap, dff]
  float* Rb[2]; // [qcap, d]
  float* SSin;  // [kMaxSlots, ss_ld_in] partial sums of squares, layer input
  long long ss_ld_in;  // max rows
  float* SS2;   // [kMaxSlots, qcap] partial sums of squares of R1
  float* Q0;    // [B*nq, d]
  void* XC;     // [B*nq, d+dc]
  float* S;     // [B*ns, d]
  void* E;      // [B*ns*d]
  float* sk_part;  // split-K tiles of the GEMMs (kSkPart floats)
  int* vcheck;     // [2] result of the offsets check (LLATTE_FLAG_VALIDATE)
};

// Split-K scratch of the GEMMs that leave the GPU short of workgroups (late
// pyramid layers, readout, summaries).
constexpr long long kSkPart = 8ll << 20;

static void with_sk(GemmParams& g, float* part) {
  g.sk_part = part;
  g.sk_part_cap = kSkPart;
}

static size_t layout_forward(const Shapes& S, void* base, FwdWS* w) {
  Arena ar(base);
  const size_t e = S.esz;
  long long maxrows = 0, maxK = 0;
  for (int l = 0; l < S.NP; ++l) {
    maxrows = std::max(maxrows, S.UBrows[l]);
    maxK = std::max(maxK, S.UBK[l]);
  }
  w->plan = carve_plan(ar, S.NP, S.B, S.qcap, S.icap);
  {
    Packed tmp;
    const size_t pb = layout_packed(S, nullptr, &tmp);
    char* blob = ar.take<char>(pb);
    layout_packed(S, blob, &w->pk);
  }
  w->H = ar.take<char>((size_t)maxrows * S.d * e);
  w->Cf = S.fnorm ? nullptr : ar.take<float>((size_t)maxK * S.r);
  w->Cl = ar.take<char>((size_t)maxK * S.r * e);
  w->q = ar.take<char>((size_t)S.qcap * S.hd * e);
  w->Hq = S.rq ? ar.take<char>((size_t)S.qcap * S.rq * e) : nullptr;
  w->Qf = S.rq && !(S.fnorm && S.rq <= 256) ? ar.take<float>((size_t)S.qcap * S.rq) : nullptr;
  w->ql = S.bf16 ? nullptr : ar.take<char>((size_t)S.qcap * S.h * S.r * e);
  w->ol = S.bf16 ? nullptr : ar.take<char>((size_t)S.qcap * S.h * S.r * e);
  w->o = ar.take<char>((size_t)S.qcap * S.hd * e);
  w->R1 = ar.take<float>((size_t)S.qcap * S.d);
  w->H2 = ar.take<char>((size_t)S.qcap * S.d * e);
  w->F = ar.take<char>((size_t)S.qcap * S.dff * e);
  w->Rb[0] = ar.take<float>((size_t)S.qcap * S.d);
  w->Rb[1] = ar.take<float>((size_t)S.qcap * S.d);
  w->ss_ld_in = maxrows;
  w->SSin = S.fnorm ? ar.take<float>((size_t)maxrows * kMaxSlots(S)) : nullptr;
  w->SS2 = S.fnorm ? ar.take<float>((size_t)S.qcap * kMaxSlots(S)) : nullptr;
  w->Q0 = S.nq ? ar.take<float>((size_t)S.B * S.nq * S.d) : nullptr;
  w->XC = S.nq ? ar.take<char>((size_t)S.B * S.nq * (S.d + S.dc) * e) : nullptr;
  w->S = S.ns ? ar.take<float>((size_t)S.B * S.ns * S.d) : nullptr;
  w->E = S.ns ? ar.take<char>((size_t)S.B * S.ns * S.d * e) : nullptr;
  w->sk_part = ar.take<float>((size_t)kSkPart);
  w->vcheck = ar.take<int>(2);
  return ar.off + 256;
}

// First row of each layer's section of the debug dump (N layers, the readout
// if any, then the end): the sections hold the layers' query rows.
static std::vector<long long> dump_rows(const Shapes& S) {
  std::vector<long long> off(S.NP + 1, 0);
  for (int l = 0; l < S.NP; ++l) off[l + 1] = off[l] + S.UBM[l];
  return off;
}

static llatte_status check_layer(const Shapes& S, const llatte_layer_weights* L, int l) {
  if (!L->g1 || !L->W_dkv || !L->W_uq || !L->W_uk || !L->W_uv || !L->W_o ||
      !L->g2 || !L->W1 || !L->W2)
    return fail(LLATTE_ERR_INVALID_ARG, "layer %d: NULL weight pointer", l);
  if (S.rq > 0 && (!L->W_dq || !L->g_q))
    return fail(LLATTE_ERR_INVALID_ARG, "layer %d: q_rank > 0 needs W_dq and g_q", l);
  return LLATTE_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Packs one layer's weights into the packed layout.
static hipError_t pack_layer(const Shapes& S, const llatte_layer_weights* L,
                             const PackedLayer& T, hipStream_t s) {
  const int k = S.bf16 ? K_BF16 : K_F32;
  const size_t e = S.esz;
  hipError_t err;
  if ((err = hipMemcpyAsync(T.g1, L->g1, S.d * 4, hipMemcpyDeviceToDevice, s))) return err;
  if ((err = hipMemcpyAsync(T.g_c, L->g_c, S.r * 4, hipMemcpyDeviceToDevice, s))) return err;
  if ((err = hipMemcpyAsync(T.g2, L->g2, S.d * 4, hipMemcpyDeviceToDevice, s))) return err;
  // bf16: W_uk and W_uv in the fused attention kernel's fragment order
  if (S.bf16) {
    if ((err = attn_pack_weights(L->W_uk, L->W_uv, S.r, S.h, S.dk, T.Wuk, T.Wuv, s))) return err;
  } else if ((err = hipMemcpyAsync(T.Wuk, L->W_uk, (size_t)S.r * S.hd * e,
                                   hipMemcpyDeviceToDevice, s))) {
    return err;
  }
  // fused norms: diag(g1) W_dkv, diag(g1) W_uq (or W_dq), diag(g2) W1
  const float* g1 = S.fnorm ? L->g1 : nullptr;
  const float* g2 = S.fnorm ? L->g2 : nullptr;
  if ((err = transpose(L->W_dkv, S.d, S.r, S.r, 0, T.Wdkv, S.d, 0, 1, k, k, s, g1))) return err;
  if ((err = transpose(L->W_uq, S.qin, S.hd, S.hd, 0, T.Wuq, S.qin, 0, 1, k, k, s,
                       S.rq ? nullptr : g1)))
    return err;
  if (S.rq) {
    if ((err = transpose(L->W_dq, S.d, S.rq, S.rq, 0, T.Wdq, S.d, 0, 1, k, k, s, g1))) return err;
    if ((err = hipMemcpyAsync(T.g_q, L->g_q, S.rq * 4, hipMemcpyDeviceToDevice, s))) return err;
  }
  // fp32: per head W_uv[:, j*dk:(j+1)*dk] ([r, dk]) -> [dk, r]
  if (!S.bf16 && (err = transpose(L->W_uv, S.r, S.dk, S.hd, S.dk, T.Wuv, S.r,
                                  (long long)S.dk * S.r, S.h, k, K_F32, s)))
    return err;
  if ((err = transpose(L->W_o, S.hd, S.d, S.d, 0, T.Wo, S.hd, 0, 1, k, k, s))) return err;
  if ((err = transpose(L->W1, S.d, S.dff, S.dff, 0, T.W1, S.d, 0, 1, k, k, s, g2))) return err;
  if ((err = transpose(L->W2, S.dff, S.d, S.d, 0, T.W2, S.dff, 0, 1, k, k, s))) return err;
  return hipSuccess;
}

static hipError_t pack_all(const Shapes& S, const llatte_weights* w,
                           const Packed& P, hipStream_t s) {
  const int k = S.bf16 ? K_BF16 : K_F32;
  hipError_t err;
  for (int l = 0; l < S.N; ++l)
    if ((err = pack_layer(S, &w->layers[l], P.L[l], s))) return err;
  if (S.ns) {
    if ((err = pack_layer(S, &w->readout, P.L[S.N], s))) return err;
    if ((err = hipMemcpyAsync(P.seeds, w->seeds, (size_t)S.ns * S.d * 4,
                              hipMemcpyDeviceToDevice, s)))
      return err;
    if (!S.raw &&
        (err = transpose(w->W_p, S.ns * S.d, S.dout, S.dout, 0, P.WpT, S.ns * S.d,
                         0, 1, k, k, s)))
      return err;
  }
  if (S.nq &&
      (err = transpose(w->W_q, S.d + S.dc, S.d, S.d, 0, P.WqT, S.d + S.dc, 0, 1, k, k, s)))
    return err;
  return hipSuccess;
}

// Hand-over between layers on the fused-norm path.
struct LayerIO {
  bool in_ready = false;  // w.H / w.SSin hold this layer's rows as bf16 and
                          // their partial sums of squares
  int np_in = 0;          // slots per row in w.SSin
  bool next = false;      // write them for the next layer (from the FFN)
  int np_out = 0;         // slots written
  bf16* cast_to = nullptr;  // otherwise (fused norms): the output rows as bf16
};

// One layer (plan index l) from row space `src` into `out` ([UBM, d] float).
static hipError_t run_layer(const Shapes& S, const FwdWS& w, int l,
                            const PackedLayer& L, RowSrc src, float* out,
                            LayerIO& io, hipStream_t s) {
  const LayerPlan P = w.plan.layer(l);
  const bool b = S.bf16;
  const int tk = b ? K_BF16 : K_F32;
  const int nql = l < S.N ? S.nq : S.ns;
  const long long nc = (long long)S.B * nql;
  const int UBrows = (int)S.UBrows[l], UBK = (int)S.UBK[l], UBM = (int)S.UBM[l];
  const size_t e = S.esz;
  hipError_t err;
  int np2 = 0;
  auto gemm_base = [&](const char* name) {
    GemmParams g;
    g.name = name;
    g.M_cap = UBM;
    g.M_dev = P.counts + 3;
    with_sk(g, w.sk_part);
    return g;
  };

  // 1. H = RMSNorm(R) g1 (pre) or R (post), all rows of the row space.
  //    Fused norms: H = R as bf16 plus sum(R^2) per row, unless the previous
  //    layer's FFN epilogue has written them already.
  if (!S.fnorm) {
    if ((err = norm_rows(src, UBrows, P.counts + 2, S.pre ? L.g1 : nullptr, S.eps,
                         nullptr, 0, w.H, S.d, S.d, tk, s)))
      return err;
  } else if (!io.in_ready) {
    if ((err = norm_rows(src, UBrows, P.counts + 2, nullptr, 0.f, nullptr, 0, w.H,
                         S.d, S.d, K_BF16, s, w.SSin)))
      return err;
    io.np_in = 1;
  }
  const RowScale rs_in{w.SSin, io.np_in, w.ss_ld_in, S.d, S.eps};
  // 2. latent C = H_hist W_dkv, then RMSNorm(C) g_c (f16 on the bf16 path)
  {
    GemmParams g;
    g.name = "gemm_down";
    with_sk(g, w.sk_part);
    g.A = (const char*)w.H + (size_t)nc * S.d * e;
    g.lda = S.d;
    g.B = L.Wdkv;
    g.ldb = S.d;
    g.M_cap = UBK;
    g.M_dev = P.counts + 0;
    g.N = S.r;
    g.K = S.d;
    if (S.fnorm) {
      g.rs = rs_in;
      g.rs.ss = w.SSin + nc;
      g.epi = EPI_ROWNORM;
      g.gain = S.lnorm ? L.g_c : nullptr;
      g.eps = S.eps;
      g.out_kind = K_F16;
      g.C = w.Cl;
      g.ldc = S.r;
      if ((err = gemm(g, b, s))) return err;
    } else {
      g.epi = EPI_STORE_F32;
      g.C = w.Cf;
      g.ldc = S.r;
      if ((err = gemm(g, b, s))) return err;
      if ((err = norm_rows(RowSrc{w.Cf, w.Cf, 0, S.r}, UBK, P.counts + 0,
                           S.lnorm ? L.g_c : nullptr, S.eps, nullptr, 0, w.Cl, S.r,
                           S.r, b ? K_F16 : K_F32, s)))
        return err;
    }
  }
  // 3. q = H[qmap] W_uq, or the low-rank path q = RMSNorm(H[qmap] W_dq) g_q W_uq
  if (S.rq) {
    GemmParams g = gemm_base("gemm_qdown");
    if (S.fnorm) g.rs = rs_in;
    g.A = w.H;
    g.lda = S.d;
    g.a_rows = P.qmap;
    g.B = L.Wdq;
    g.ldb = S.d;
    g.N = S.rq;
    g.K = S.d;
    if (!w.Qf) {  // the query norm in the epilogue (one tile spans q_rank)
      g.epi = EPI_ROWNORM;
      g.gain = L.g_q;
      g.eps = S.eps;
      g.out_kind = tk;
      g.C = w.Hq;
      g.ldc = S.rq;
      if ((err = gemm(g, b, s))) return err;
    } else {
      g.epi = EPI_STORE_F32;
      g.C = w.Qf;
      g.ldc = S.rq;
      if ((err = gemm(g, b, s))) return err;
      if ((err = norm_rows(RowSrc{w.Qf, w.Qf, 0, S.rq}, UBM, P.counts + 3, L.g_q, S.eps,
                           nullptr, 0, w.Hq, S.rq, S.rq, tk, s)))
        return err;
    }
  }
  {
    GemmParams g = gemm_base("gemm_q");
    if (S.rq) {
      g.A = w.Hq;
      g.lda = S.rq;
    } else {
      if (S.fnorm) g.rs = rs_in;
      g.A = w.H;
      g.lda = S.d;
      g.a_rows = P.qmap;
    }
    g.B = L.Wuq;
    g.ldb = S.qin;
    g.N = S.hd;
    g.K = S.qin;
    g.C = w.q;
    g.ldc = S.hd;
    if ((err = gemm(g, b, s))) return err;
  }
  AttnParams a;
  a.c = w.Cl;
  a.lse = nullptr;
  a.h = S.h;
  a.r = S.r;
  a.dk = S.dk;
  a.scale = 1.f / sqrtf((float)S.dk);
  a.items = P.items;
  a.n_items = P.n_items;
  // the grid: this layer's item bound (the plan's buffer holds S.icap per
  // layer, the largest layer's); late layers launch far fewer workgroups
  a.items_cap = S.bq > 0 ? (int)std::min<long long>(cdiv(S.UBn[l], S.bq) + S.B +
                                                        (long long)S.B * cdiv(nql, S.bq),
                                                    S.icap)
                         : S.icap;
  a.qinfo = P.qinfo;
  a.M_cap = UBM;
  a.M_dev = P.counts + 3;
  if (b) {
    // 4-6. o = attention with q_lat = q W_uk^T formed in the prologue and
    //      o_j = o_lat_j W_uv_j applied in the epilogue
    a.fused = true;
    a.q = w.q;
    a.w_uk = L.Wuk;
    a.w_uv_t = L.Wuv;
    a.out = w.o;
    if ((err = attention(a, true, s))) return err;
  } else {
    // 4. latent queries per head: ql_j = q_j W_uk_j^T
    GemmParams g = gemm_base("gemm_absorb_uk");
    g.A = w.q;
    g.lda = S.hd;
    g.sA = S.dk;
    g.B = L.Wuk;
    g.ldb = S.hd;
    g.sB = S.dk;
    g.batch = S.h;
    g.N = S.r;
    g.K = S.dk;
    g.C = w.ql;
    g.ldc = S.h * S.r;
    g.sC = S.r;
    if ((err = gemm(g, b, s))) return err;
    // 5. attention in latent space
    a.fused = false;
    a.q = w.ql;
    a.out = w.ol;
    if ((err = attention(a, false, s))) return err;
    // 6. o_j = ol_j W_uv_j
    GemmParams g2 = gemm_base("gemm_absorb_uv");
    g2.A = w.ol;
    g2.lda = S.h * S.r;
    g2.sA = S.r;
    g2.B = L.Wuv;
    g2.ldb = S.r;
    g2.sB = (long long)S.dk * S.r;
    g2.batch = S.h;
    g2.N = S.dk;
    g2.K = S.r;
    g2.C = w.o;
    g2.ldc = S.hd;
    g2.sC = S.dk;
    if ((err = gemm(g2, b, s))) return err;
  }
  // 7. R1 = R[qmap] + o W_o
  {
    GemmParams g = gemm_base("gemm_out");
    g.nt = true;  // the fp32 result is next read by the FFN epilogue
    g.A = w.o;
    g.lda = S.hd;
    g.B = L.Wo;
    g.ldb = S.hd;
    g.N = S.d;
    g.K = S.hd;
    g.epi = EPI_RESID_F32;
    g.C = w.R1;
    g.ldc = S.d;
    g.res = src;
    g.res_rows = P.qmap;
    if (S.fnorm) {  // H2 = R1 as bf16, sum(R1^2) per row
      g.cast_out = w.H2;
      g.ld_cast = S.d;
      g.ss_out = w.SS2;
      g.ss_ld = S.qcap;
      np2 = gemm_ss_slots(g, b);
    }
    if ((err = gemm(g, b, s))) return err;
  }
  // 8. H2 = RMSNorm(R1) g2 (pre); post: R1 = RMSNorm(R1) g1, H2 = R1
  if (S.fnorm)
    err = hipSuccess;
  else if (S.pre)
    err = norm_rows(RowSrc{w.R1, w.R1, 0, S.d}, UBM, P.counts + 3, L.g2, S.eps,
                    nullptr, 0, w.H2, S.d, S.d, tk, s);
  else
    err = norm_rows(RowSrc{w.R1, w.R1, 0, S.d}, UBM, P.counts + 3, L.g1, S.eps,
                    w.R1, S.d, w.H2, S.d, S.d, tk, s);
  if (err) return err;
  // 9. F = GELU(H2 W1)
  {
    GemmParams g = gemm_base("gemm_ffn1");
    if (S.fnorm) g.rs = RowScale{w.SS2, np2, S.qcap, S.d, S.eps};
    g.A = w.H2;
    g.lda = S.d;
    g.B = L.W1;
    g.ldb = S.d;
    g.N = S.dff;
    g.K = S.d;
    g.epi = EPI_GELU;
    g.C = w.F;
    g.ldc = S.dff;
    g.nt = true;  // the layer's largest tensor (M x d_ff): streamed, it keeps W1 and H2 cached
    if ((err = gemm(g, b, s))) return err;
  }
  // 10. out = R1 + F W2 (post: then RMSNorm g2)
  {
    GemmParams g = gemm_base("gemm_ffn2");
    g.nt = true;  // the fp32 result is next read as a residual, much later
    g.A = w.F;
    g.lda = S.dff;
    g.B = L.W2;
    g.ldb = S.dff;
    g.N = S.d;
    g.K = S.dff;
    g.epi = EPI_RESID_F32;
    g.C = out;
    g.ldc = S.d;
    g.res = RowSrc{w.R1, w.R1, 0, S.d};
    if (S.fnorm && io.next) {  // the next layer's H and sums of squares
      g.cast_out = w.H;
      g.ld_cast = S.d;
      g.ss_out = w.SSin;
      g.ss_ld = w.ss_ld_in;
      io.np_out = gemm_ss_slots(g, b);
    } else if (S.fnorm && io.cast_to) {
      g.cast_out = io.cast_to;
      g.ld_cast = S.d;
    }
    if ((err = gemm(g, b, s))) return err;
  }
  if (!S.pre &&
      (err = norm_rows(RowSrc{out, out, 0, S.d}, UBM, P.counts + 3, L.g2, S.eps,
                       out, S.d, nullptr, 0, S.d, tk, s)))
    return err;
  return hipSuccess;
}

}  // namespace llatte

using namespace llatte;

extern "C" {

const char* llatte_last_error(void) { return t_err.c_str(); }
int32_t llatte_version(void) { return 100; }

void llatte_kernel_timing_enable(int32_t on) { t_timing = on != 0; }

void llatte_kernel_timing_reset(void) {
  timing_collect();
  t_acc.clear();
}

int32_t llatte_kernel_timing_read(char* names, int32_t name_stride,
                                  int32_t* counts, double* ms, int32_t cap) {
  timing_collect();
  int32_t i = 0;
  for (auto& kv : t_acc) {
    if (i >= cap) break;
    if (names && name_stride > 0) {
      strncpy(names + (size_t)i * name_stride, kv.first.c_str(), name_stride - 1);
      names[(size_t)i * name_stride + name_stride - 1] = 0;
    }
    if (counts) counts[i] = kv.second.first;
    if (ms) ms[i] = kv.second.second;
    ++i;
  }
  return i;
}

llatte_status llatte_attention_phases_enable(int32_t max_workgroups) {
  static_assert(LLATTE_ATTN_PHASE_FIELDS == kAttnPhaseFields, "phase record size");
  HIP_TRY(attn_phases_enable(max_workgroups));
  return LLATTE_OK;
}

int32_t llatte_attention_phases_read(double* out, int32_t cap) {
  return attn_phases_read(out, cap < 0 ? 0 : cap);
}

llatte_status llatte_gemm_phases_enable(int32_t max_workgroups) {
  static_assert(kGemmPhaseFields == LLATTE_GEMM_PHASE_FIELDS, "record width");
  HIP_TRY(gemm_phases_enable(max_workgroups));
  return LLATTE_OK;
}

int32_t llatte_gemm_phases_read(double* out, int32_t cap) {
  return gemm_phases_read(out, cap < 0 ? 0 : cap);
}

size_t llatte_mla_forward_workspace_size(const llatte_model_desc* desc,
                                         int32_t B, int32_t total_rows,
                                         int32_t max_len) {
  Shapes S;
  if (make_shapes(desc, B, total_rows, max_len, &S) != LLATTE_OK) return 0;
  FwdWS w;
  return layout_forward(S, nullptr, &w);
}

int32_t llatte_mla_forward_debug_layout(const llatte_model_desc* desc, int32_t B,
                                        int32_t total_rows, int32_t max_len,
                                        int64_t* row_offsets) {
  Shapes S;
  if (!row_offsets || make_shapes(desc, B, total_rows, max_len, &S) != LLATTE_OK) return 0;
  const std::vector<long long> off = dump_rows(S);
  for (size_t i = 0; i < off.size(); ++i) row_offsets[i] = off[i];
  return (int32_t)off.size();
}

size_t llatte_packed_weights_size(const llatte_model_desc* desc) {
  Shapes S;
  if (make_shapes(desc, 1, 1, 1, &S) != LLATTE_OK) return 0;
  Packed P;
  return layout_packed(S, nullptr, &P);
}

static llatte_status check_weights(const Shapes& S, const llatte_weights* wts) {
  llatte_status st;
  if (!wts || !wts->layers) return fail(LLATTE_ERR_INVALID_ARG, "weights are NULL");
  for (int l = 0; l < S.N; ++l)
    if ((st = check_layer(S, &wts->layers[l], l))) return st;
  if (S.nq > 0 && !wts->W_q) return fail(LLATTE_ERR_INVALID_ARG, "n_q > 0 needs W_q");
  if (S.ns > 0) {
    if (!wts->seeds || (!wts->W_p && !S.raw))
      return fail(LLATTE_ERR_INVALID_ARG, "readout needs seeds and W_p");
    if ((st = check_layer(S, &wts->readout, -1))) return st;
  }
  return LLATTE_OK;
}

llatte_status llatte_pack_weights(const llatte_model_desc* desc,
                                  const llatte_weights* wts, void* packed,
                                  size_t packed_bytes, void* stream) {
  Shapes S;
  llatte_status st = make_shapes(desc, 1, 1, 1, &S);
  if (st) return st;
  if ((st = check_weights(S, wts))) return st;
  if (!packed || !aligned16(packed)) return fail(LLATTE_ERR_INVALID_ARG, "packed must be 16-byte aligned");
  Packed P;
  const size_t need = layout_packed(S, nullptr, &P);
  if (packed_bytes < need)
    return fail(LLATTE_ERR_WORKSPACE, "packed buffer %zu bytes < %zu needed", packed_bytes, need);
  layout_packed(S, packed, &P);
  HIP_TRY(pack_all(S, wts, P, (hipStream_t)stream));
  return LLATTE_OK;
}

llatte_status llatte_mla_forward(
    const llatte_model_desc* desc, const llatte_weights* wts,
    const void* packed_weights, const float* hist_values,
    const int32_t* hist_offsets, int32_t B, int32_t total_rows,
    int32_t max_len, const float* cand_x, const float* ctx, float* out_cand,
    float* out_hist, int32_t* out_hist_offsets, float* out_emb,
    void* workspace, size_t workspace_bytes, void* stream) {
  Shapes S;
  llatte_status st = make_shapes(desc, B, total_rows, max_len, &S);
  if (st) return st;
  if (!packed_weights && (st = check_weights(S, wts))) return st;
  if (!hist_values || !hist_offsets)
    return fail(LLATTE_ERR_INVALID_ARG, "hist_values/hist_offsets are NULL");
  if (S.nq > 0 && (!cand_x || !out_cand))
    return fail(LLATTE_ERR_INVALID_ARG, "n_q > 0 needs cand_x and out_cand");
  if (S.nq > 0 && S.dc > 0 && !ctx)
    return fail(LLATTE_ERR_INVALID_ARG, "d_ctx > 0 needs ctx");
  if (S.ns > 0 && !out_emb) return fail(LLATTE_ERR_INVALID_ARG, "readout needs out_emb");
  const void* ptrs[] = {hist_values, cand_x, ctx, out_cand, out_hist, out_emb,
                        workspace, packed_weights};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(LLATTE_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (!workspace) return fail(LLATTE_ERR_INVALID_ARG, "workspace is NULL");
  FwdWS w;
  const size_t need = layout_forward(S, nullptr, &w);
  if (workspace_bytes < need)
    return fail(LLATTE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  std::vector<long long> dsec;
  if (S.dump) {
    dsec = dump_rows(S);
    const size_t need_dump = (size_t)dsec.back() * S.d * sizeof(float);
    if (!desc->debug_dump || !aligned16(desc->debug_dump))
      return fail(LLATTE_ERR_INVALID_ARG, "LLATTE_FLAG_DEBUG_DUMP needs a 16-byte aligned debug_dump");
    if (desc->debug_dump_bytes < need_dump)
      return fail(LLATTE_ERR_WORKSPACE, "debug_dump %zu bytes < %zu needed", desc->debug_dump_bytes,
                  need_dump);
  }
  layout_forward(S, workspace, &w);
  hipStream_t s = (hipStream_t)stream;
  if (S.validate) {
    // the only launch before the offsets are known to be well formed
    int h[2] = {0, 0};
    HIP_TRY(validate_offsets(hist_offsets, B, total_rows, max_len, w.vcheck, s));
    HIP_TRY(hipMemcpyAsync(h, w.vcheck, sizeof h, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    static const char* what[] = {"", "hist_offsets[0] != 0", "an empty history (L_u < 1)",
                                 "a history longer than max_len", "hist_offsets[B] != total_rows"};
    if (h[0] != 0)
      return fail(LLATTE_ERR_INVALID_ARG, "LLATTE_FLAG_VALIDATE: %s at user %d",
                  what[h[0] >= 1 && h[0] <= 4 ? h[0] : 0], h[1]);
  }
  const bool b = S.bf16;
  Packed PK;
  if (packed_weights) {
    layout_packed(S, (void*)packed_weights, &PK);
  } else {
    PK = w.pk;
    HIP_TRY(pack_all(S, wts, PK, s));
  }

  // out_hist_offsets: the last layer's history query offsets, written by the plan
  HIP_TRY(build_plan(hist_offsets, B, S.rule, S.nq, S.ns, w.plan, S.NP, S.bq,
                     kAttnBN, s, out_hist_offsets, S.N - 1));
  if (S.nq) {
    HIP_TRY(concat_queries(cand_x, ctx, B, S.nq, S.d, S.dc, w.XC, b, s));
    GemmParams g;
    g.name = "gemm_fusion";
    with_sk(g, w.sk_part);
    g.A = w.XC;
    g.lda = S.d + S.dc;
    g.B = PK.WqT;
    g.ldb = S.d + S.dc;
    g.M_cap = B * S.nq;
    g.N = S.d;
    g.K = S.d + S.dc;
    g.epi = EPI_STORE_F32;
    g.C = w.Q0;
    g.ldc = S.d;
    HIP_TRY(gemm(g, b, s));
  }
  const long long nc = (long long)B * S.nq;
  float* last = nullptr;
  LayerIO io;
  for (int l = 0; l < S.N; ++l) {
    RowSrc src;
    if (l == 0)
      src = RowSrc{w.Q0, hist_values, (int)nc, S.d};
    else
      src = RowSrc{last, last + nc * S.d, (int)nc, S.d};
    // with no candidate rows ahead of them, the last layer's rows are the
    // caller's history rows: written there directly (only the W2 product
    // and the post-norm pass write a layer's output, both within the
    // device-side row count, which out_hist holds)
    float* out = (l == S.N - 1 && out_hist && nc == 0) ? out_hist : w.Rb[l & 1];
    io.next = S.fnorm && l + 1 < S.N;
    HIP_TRY(run_layer(S, w, l, PK.L[l], src, out, io, s));
    if (S.dump)
      HIP_TRY(copy_rows_f32(out, S.d, desc->debug_dump + (size_t)dsec[l] * S.d, (int)S.UBM[l],
                            w.plan.layer(l).counts + 3, S.d, s));
    io.in_ready = io.next;
    io.np_in = io.np_out;
    last = out;
  }
  const LayerPlan PN = w.plan.layer(S.N - 1);
  if (S.nq) HIP_TRY(copy_rows_f32(last, S.d, out_cand, (int)nc, nullptr, S.d, s));
  if (out_hist && last != out_hist)
    HIP_TRY(copy_rows_f32(last + nc * S.d, S.d, out_hist, (int)S.UBn[S.N - 1],
                          PN.counts + 1, S.d, s));
  if (S.ns) {
    HIP_TRY(broadcast_rows(PK.seeds, S.ns, S.d, B, w.S, s));
    float* ro = w.Rb[S.N & 1];
    RowSrc src{w.S, last + nc * S.d, B * S.ns, S.d};
    LayerIO rio;
    // the readout rows as the W_p operand: bf16 straight from the FFN's
    // epilogue on the fused-norm path, else a cast pass
    if (!S.raw && S.fnorm) rio.cast_to = (bf16*)w.E;
    HIP_TRY(run_layer(S, w, S.N, PK.L[S.N], src, ro, rio, s));
    if (S.dump)
      HIP_TRY(copy_rows_f32(ro, S.d, desc->debug_dump + (size_t)dsec[S.N] * S.d, (int)S.UBM[S.N],
                            w.plan.layer(S.N).counts + 3, S.d, s));
    if (S.raw) {  // Flatten(Z_raw): the readout rows are already seed-major per user
      HIP_TRY(copy_rows_f32(ro, S.d, out_emb, B * S.ns, nullptr, S.d, s));
      return LLATTE_OK;
    }
    if (!rio.cast_to)
      HIP_TRY(norm_rows(RowSrc{ro, ro, 0, S.d}, B * S.ns, nullptr, nullptr, 0.f,
                        nullptr, 0, w.E, S.d, S.d, b ? K_BF16 : K_F32, s));
    GemmParams g;
    g.name = "gemm_readout";
    with_sk(g, w.sk_part);
    g.A = w.E;
    g.lda = S.ns * S.d;
    g.B = PK.WpT;
    g.ldb = S.ns * S.d;
    g.M_cap = B;
    g.N = S.dout;
    g.K = S.ns * S.d;
    g.epi = EPI_STORE_F32;
    g.C = out_emb;
    g.ldc = S.dout;
    HIP_TRY(gemm(g, b, s));
  }
  return LLATTE_OK;
}

size_t llatte_mla_attention_workspace_size(const llatte_attn_desc* a,
                                           int32_t B, int32_t Mtot,
                                           int32_t Ktot) {
  if (!a || B < 1 || Mtot < 0 || Ktot < B) return 0;
  const bool b = a->dtype == LLATTE_BF16;
  const int bq = b ? attn_bq(a->n_heads, a->rank) : 0;
  const long long nh = (long long)Mtot - (long long)B * a->n_cand;
  if (nh < 0) return 0;
  const long long icap =
      bq > 0 ? cdiv(nh, bq) + B + (long long)B * cdiv(a->n_cand, bq) : 1;
  Arena ar(nullptr);
  carve_plan(ar, 1, B, std::max(Mtot, 1), (int)icap);
  ar.take<unsigned>(kAbsmaxWords);  // max magnitudes of q_lat and c_lat (bf16 range scaling)
  return ar.off + 256;
}

}  // extern "C"

namespace llatte {
static llatte_status scratch_ptr(void** out);
constexpr size_t kAttnScratchBytes = (size_t)8 << 20;

// Validation and launch of the attention core. The plan goes into the
// caller's workspace, or (fixed_scratch) into the library's fixed scratch,
// whose address is fetched only after every host-side check has passed.
static llatte_status mla_attention_impl(
    const llatte_attn_desc* a, const void* q_lat, const void* c_lat,
    const int32_t* kv_offsets, const int32_t* hq_offsets, int32_t B,
    int32_t Mtot, int32_t Ktot, void* out, float* lse, void* workspace,
    size_t workspace_bytes, void* stream, bool fixed_scratch, bf16* out_bf16 = nullptr) {
  if (!a) return fail(LLATTE_ERR_INVALID_ARG, "desc is NULL");
  if (a->dtype != LLATTE_F32 && a->dtype != LLATTE_BF16)
    return fail(LLATTE_ERR_UNSUPPORTED, "dtype %d", a->dtype);
  const bool b = a->dtype == LLATTE_BF16;
  if (a->n_heads < 1 || a->rank < 1 || a->n_cand < 0 || B < 1 || Ktot < B ||
      Mtot < (long long)B * a->n_cand)
    return fail(LLATTE_ERR_INVALID_ARG, "bad sizes");
  if (b && attn_bq(a->n_heads, a->rank) == 0)
    return fail(LLATTE_ERR_UNSUPPORTED, "bf16 attention needs rank in {64, 128, 256}");
  if (!b && a->rank > 256) return fail(LLATTE_ERR_UNSUPPORTED, "f32 attention needs rank <= 256");
  if (!(a->scale > 0.f)) return fail(LLATTE_ERR_INVALID_ARG, "scale must be > 0");
  if (!q_lat || !c_lat || !kv_offsets || !hq_offsets || !out || (!fixed_scratch && !workspace))
    return fail(LLATTE_ERR_INVALID_ARG, "NULL pointer");
  const void* ptrs[] = {q_lat, c_lat, out, lse, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(LLATTE_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const size_t need = llatte_mla_attention_workspace_size(a, B, Mtot, Ktot);
  if (fixed_scratch) {
    if (need > kAttnScratchBytes)
      return fail(LLATTE_ERR_WORKSPACE,
                  "these sizes need %zu bytes of plan scratch; the fixed scratch holds %zu "
                  "(use llatte_mla_attention with a workspace)",
                  need, kAttnScratchBytes);
  } else if (workspace_bytes < need) {
    return fail(LLATTE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  }
  if (Mtot == 0) return LLATTE_OK;
  if (fixed_scratch) {
    const llatte_status st = scratch_ptr(&workspace);
    if (st != LLATTE_OK) return st;
  }
  const int bq = b ? attn_bq(a->n_heads, a->rank) : 0;
  const long long nh = (long long)Mtot - (long long)B * a->n_cand;
  const int icap = bq > 0 ? (int)(cdiv(nh, bq) + B + (long long)B * cdiv(a->n_cand, bq)) : 1;
  Arena ar(workspace);
  PlanBase pb = carve_plan(ar, 1, B, Mtot, icap);
  unsigned* amax = ar.take<unsigned>(kAbsmaxWords);
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(build_attn_plan(kv_offsets, hq_offsets, B, a->n_cand, bq, kAttnBN, pb, s));
  // bf16: the kernel computes in fp16 after power-of-two scalings chosen from
  // the inputs' largest magnitudes, so any finite input stays in range
  if (b)
    HIP_TRY(attn_absmax(q_lat, (long long)Mtot * a->n_heads * a->rank, c_lat,
                        (long long)Ktot * a->rank, a->scale, amax, s));
  const LayerPlan P = pb.layer(0);
  AttnParams ap;
  ap.q = q_lat;
  ap.c = c_lat;
  ap.out = out;
  ap.out_bf16 = a->dtype == LLATTE_BF16 ? out_bf16 : nullptr;
  ap.lse = lse;
  ap.fused = false;
  ap.w_uk = nullptr;
  ap.w_uv_t = nullptr;
  ap.dk = 0;
  ap.h = a->n_heads;
  ap.r = a->rank;
  ap.scale = a->scale;
  ap.items = P.items;
  ap.n_items = P.n_items;
  ap.items_cap = icap;
  ap.qinfo = P.qinfo;
  ap.M_cap = Mtot;
  ap.M_dev = P.counts + 3;
  ap.amax = b ? amax : nullptr;
  HIP_TRY(attention(ap, b, s));
  return LLATTE_OK;
}

// Fixed scratch of llatte_mla_attention_noalloc (the attention plan), one
// copy per device, held until the process ends. In host code the array's
// name is only a stand-in: the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) char scratch[kAttnScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static llatte_status scratch_ptr(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(LLATTE_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return fail(LLATTE_ERR_HIP, "hipGetSymbolAddress returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LLATTE_OK;
}
}  // namespace llatte

extern "C" {

llatte_status llatte_mla_attention(
    const llatte_attn_desc* a, const void* q_lat, const void* c_lat,
    const int32_t* kv_offsets, const int32_t* hq_offsets, int32_t B,
    int32_t Mtot, int32_t Ktot, void* out, float* lse, void* workspace,
    size_t workspace_bytes, void* stream) {
  return mla_attention_impl(a, q_lat, c_lat, kv_offsets, hq_offsets, B, Mtot, Ktot, out, lse,
                            workspace, workspace_bytes, stream, false);
}

size_t llatte_mla_attention_noalloc_max_scratch(void) { return kAttnScratchBytes; }

llatte_status llatte_mla_attention_noalloc(
    const llatte_attn_desc* a, const void* q_lat, const void* c_lat,
    const int32_t* kv_offsets, const int32_t* hq_offsets, int32_t B,
    int32_t Mtot, int32_t Ktot, void* out, float* lse, void* stream) {
  return mla_attention_impl(a, q_lat, c_lat, kv_offsets, hq_offsets, B, Mtot, Ktot, out, lse,
                            nullptr, 0, stream, true);
}

llatte_status llatte_pyramid_compact(const void* values, int32_t row_elems,
                                     int32_t dt, const int32_t* offsets_in,
                                     int32_t B, int32_t total_rows,
                                     const int32_t* keep, void* values_out,
                                     int32_t* offsets_out, int32_t* src_index,
                                     void* stream) {
  if (dt != LLATTE_F32 && dt != LLATTE_BF16) return fail(LLATTE_ERR_UNSUPPORTED, "dtype %d", dt);
  if (B < 1 || total_rows < 0 || row_elems < 1)
    return fail(LLATTE_ERR_INVALID_ARG, "bad sizes");
  if (!values || !offsets_in || !keep || !values_out || !offsets_out)
    return fail(LLATTE_ERR_INVALID_ARG, "NULL pointer");
  const int row_bytes = row_elems * (dt == LLATTE_BF16 ? 2 : 4);
  if ((row_bytes & 3) || !aligned16(values) || !aligned16(values_out))
    return fail(LLATTE_ERR_INVALID_ARG, "rows must be a multiple of 4 bytes, pointers 16-byte aligned");
  HIP_TRY(pyramid_compact(values, row_bytes, offsets_in, B, total_rows, keep,
                          values_out, offsets_out, src_index, (hipStream_t)stream));
  return LLATTE_OK;
}

llatte_status llatte_pyramid_counts(const llatte_pyramid_rule* rule,
                                    int32_t n_layers,
                                    const int32_t* offsets_in, int32_t B,
                                    int32_t* keep_out, void* stream) {
  if (!rule || !offsets_in || !keep_out || B < 1 || n_layers < 1 ||
      n_layers > LLATTE_MAX_LAYERS)
    return fail(LLATTE_ERR_INVALID_ARG, "bad arguments");
  RuleDev rd;
  llatte_status st = expand_rule(rule, n_layers, &rd);
  if (st) return st;
  HIP_TRY(pyramid_counts_dev(rd, offsets_in, B, keep_out, (hipStream_t)stream));
  return LLATTE_OK;
}

llatte_status llatte_pyramid_counts_host(const llatte_pyramid_rule* rule,
                                         int32_t n_layers,
                                         const int32_t* lengths, int32_t B,
                                         int32_t* keep_out) {
  if (!rule || !lengths || !keep_out || B < 1 || n_layers < 1 ||
      n_layers > LLATTE_MAX_LAYERS)
    return fail(LLATTE_ERR_INVALID_ARG, "bad arguments");
  RuleDev rd;
  llatte_status st = expand_rule(rule, n_layers, &rd);
  if (st) return st;
  for (int u = 0; u < B; ++u) {
    const int L = lengths[u];
    if (L < 1) return fail(LLATTE_ERR_INVALID_ARG, "length of user %d is < 1", u);
    int prev = L;
    for (int l = 0; l < n_layers; ++l) {
      int k = rd.kind == 1 ? std::max(std::min(rd.floor, L), L >> std::min(l, 30))
                           : rd.values[l];
      prev = std::min(k, prev);
      keep_out[(size_t)l * B + u] = prev;
    }
  }
  return LLATTE_OK;
}

size_t llatte_token_embed_workspace_size(int32_t d, int32_t d_sem, int32_t dt) {
  if (d < 1 || d_sem < 1) return 0;
  return (size_t)d * d_sem * (dt == LLATTE_BF16 ? 2 : 4) + 256;
}

llatte_status llatte_token_embed(const void* table, int32_t V,
                                 const int32_t* rows, const void* sem,
                                 const void* W_s, int32_t n, int32_t d,
                                 int32_t d_sem, int32_t dt, float* out,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (dt != LLATTE_F32 && dt != LLATTE_BF16) return fail(LLATTE_ERR_UNSUPPORTED, "dtype %d", dt);
  const bool b = dt == LLATTE_BF16;
  const int al = b ? 8 : 4;
  if (V < 1 || n < 0 || d < 1 || d_sem < 1) return fail(LLATTE_ERR_INVALID_ARG, "bad sizes");
  if (d % al || d_sem % al)
    return fail(LLATTE_ERR_UNSUPPORTED, "d and d_sem must be multiples of %d", al);
  if (!table || !rows || !sem || !W_s || !out || !workspace)
    return fail(LLATTE_ERR_INVALID_ARG, "NULL pointer");
  const void* ptrs[] = {table, sem, W_s, out, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(LLATTE_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (workspace_bytes < llatte_token_embed_workspace_size(d, d_sem, dt))
    return fail(LLATTE_ERR_WORKSPACE, "workspace too small");
  if (n == 0) return LLATTE_OK;
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(transpose(W_s, d_sem, d, d, 0, workspace, d_sem, 0, 1,
                    b ? K_BF16 : K_F32, b ? K_BF16 : K_F32, s));
  GemmParams g;
  g.name = "gemm_token_embed";
  g.A = sem;
  g.lda = d_sem;
  g.B = workspace;
  g.ldb = d_sem;
  g.M_cap = n;
  g.N = d;
  g.K = d_sem;
  g.epi = EPI_GATHER_ADD_F32;
  g.C = out;
  g.ldc = d;
  g.table = table;
  g.ld_table = d;
  g.g_rows = rows;
  HIP_TRY(gemm(g, b, s));
  return LLATTE_OK;
}


// ---------------------------------------------------------------- actions
// Workspace: U [n, d_in], H [n, d_hidden], age [n], W_a^T, W_b^T (the
// products' K-contiguous operands), each 256-byte aligned.
struct ActionWs {
  size_t U, H, age, WaT, WbT, total;
};
static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
static ActionWs action_ws(const llatte_action_desc* a, int32_t n) {
  const size_t es = a->dtype == LLATTE_BF16 ? 2 : 4;
  const size_t d_in = (size_t)a->d_type + a->d_item + a->d_surf + a->d_time + a->d_meta_emb;
  ActionWs w;
  w.U = 0;
  w.H = w.U + al256((size_t)n * d_in * es);
  w.age = w.H + al256((size_t)n * a->d_hidden * es);
  w.WaT = w.age + al256((size_t)n * 4);
  w.WbT = w.WaT + al256((size_t)a->d_hidden * d_in * es);
  w.total = w.WbT + al256((size_t)a->d * a->d_hidden * es) + 256;
  return w;
}

static llatte_status check_action_desc(const llatte_action_desc* a) {
  if (!a) return fail(LLATTE_ERR_INVALID_ARG, "NULL descriptor");
  if (a->dtype != LLATTE_F32 && a->dtype != LLATTE_BF16)
    return fail(LLATTE_ERR_UNSUPPORTED, "dtype %d", a->dtype);
  const int al = a->dtype == LLATTE_BF16 ? 8 : 4;
  const int32_t widths[] = {a->d, a->d_hidden, a->d_type, a->d_item, a->d_surf,
                            a->d_time, a->d_meta, a->d_meta_emb};
  for (int32_t v : widths) {
    if (v < 1 || v > (1 << 16)) return fail(LLATTE_ERR_INVALID_ARG, "field width %d out of range", v);
    if (v % al) return fail(LLATTE_ERR_UNSUPPORTED, "field widths must be multiples of %d", al);
  }
  if (a->d_enc < 0 || a->d_enc > a->d || a->d_enc % 2)
    return fail(LLATTE_ERR_INVALID_ARG, "d_enc must be even and within [0, d]");
  if (a->V_type < 1 || a->V_item < 1 || a->V_surf < 1 || a->n_buckets < 1 || a->n_buckets > 64)
    return fail(LLATTE_ERR_INVALID_ARG, "table sizes must be >= 1 (n_buckets <= 64)");
  return LLATTE_OK;
}

size_t llatte_action_tokenize_workspace_size(const llatte_action_desc* desc, int32_t n) {
  if (!desc || n < 0 || check_action_desc(desc) != LLATTE_OK) return 0;
  return action_ws(desc, n).total;
}

llatte_status llatte_action_tokenize(const llatte_action_desc* desc,
                                     const llatte_action_weights* w,
                                     const int32_t* offsets, int32_t B, int32_t n,
                                     const int32_t* t_req, const int32_t* tau,
                                     const int32_t* type_id, const int32_t* item_id,
                                     const int32_t* surf_id, const void* meta,
                                     float* out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  llatte_status st = check_action_desc(desc);
  if (st) return st;
  if (!w) return fail(LLATTE_ERR_INVALID_ARG, "NULL weights");
  if (B < 1 || n < 0) return fail(LLATTE_ERR_INVALID_ARG, "B must be >= 1 and n >= 0");
  if (n == 0) return LLATTE_OK;  // nothing to read or write; row arrays may be NULL
  const void* ptrs[] = {offsets, t_req, tau, type_id, item_id, surf_id, meta, out, workspace,
                        w->E_type, w->E_item, w->E_surf, w->E_time, w->W_meta, w->W_a, w->W_b};
  for (const void* p : ptrs) {
    if (!p) return fail(LLATTE_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(p)) return fail(LLATTE_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  }
  const ActionWs ws = action_ws(desc, n);
  if (workspace_bytes < ws.total) return fail(LLATTE_ERR_WORKSPACE, "workspace too small");
  const bool b = desc->dtype == LLATTE_BF16;
  const int kind = b ? K_BF16 : K_F32;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  const int d_in = desc->d_type + desc->d_item + desc->d_surf + desc->d_time + desc->d_meta_emb;

  ActionConcat c;
  c.offsets = offsets;
  c.B = B;
  c.n = n;
  c.t_req = t_req;
  c.tau = tau;
  c.type_id = type_id;
  c.item_id = item_id;
  c.surf_id = surf_id;
  c.meta = meta;
  c.E_type = w->E_type;
  c.E_item = w->E_item;
  c.E_surf = w->E_surf;
  c.E_time = w->E_time;
  c.W_meta = w->W_meta;
  c.d_type = desc->d_type;
  c.d_item = desc->d_item;
  c.d_surf = desc->d_surf;
  c.d_time = desc->d_time;
  c.d_meta = desc->d_meta;
  c.d_meta_emb = desc->d_meta_emb;
  c.d_in = d_in;
  c.V_type = desc->V_type;
  c.V_item = desc->V_item;
  c.V_surf = desc->V_surf;
  c.n_buckets = desc->n_buckets;
  c.U = base + ws.U;
  c.age = (int*)(base + ws.age);
  HIP_TRY(transpose(w->W_a, d_in, desc->d_hidden, desc->d_hidden, 0, base + ws.WaT, d_in, 0, 1,
                    kind, kind, s));
  HIP_TRY(transpose(w->W_b, desc->d_hidden, desc->d, desc->d, 0, base + ws.WbT, desc->d_hidden,
                    0, 1, kind, kind, s));
  HIP_TRY(action_concat(c, b, s));
  {  // H = GELU(U W_a)
    GemmParams g;
    g.name = "gemm_act_a";
    g.A = c.U;
    g.lda = d_in;
    g.B = base + ws.WaT;
    g.ldb = d_in;
    g.M_cap = n;
    g.N = desc->d_hidden;
    g.K = d_in;
    g.epi = EPI_GELU;
    g.C = base + ws.H;
    g.ldc = desc->d_hidden;
    HIP_TRY(gemm(g, b, s));
  }
  {  // out = H W_b + enc(age)
    GemmParams g;
    g.name = "gemm_act_b";
    g.A = base + ws.H;
    g.lda = desc->d_hidden;
    g.B = base + ws.WbT;
    g.ldb = desc->d_hidden;
    g.M_cap = n;
    g.N = desc->d;
    g.K = desc->d_hidden;
    g.epi = EPI_STORE_F32;
    g.C = out;
    g.ldc = desc->d;
    g.enc_age = c.age;
    g.enc_dims = desc->d_enc;
    HIP_TRY(gemm(g, b, s));
  }
  return LLATTE_OK;
}


// ---------------------------------------------------------------- summaries
static llatte_status check_summary_desc(const llatte_summary_desc* a) {
  if (!a) return fail(LLATTE_ERR_INVALID_ARG, "NULL descriptor");
  if (a->dtype != LLATTE_F32 && a->dtype != LLATTE_BF16)
    return fail(LLATTE_ERR_UNSUPPORTED, "dtype %d", a->dtype);
  const int al = a->dtype == LLATTE_BF16 ? 8 : 4;
  const int32_t widths[] = {a->d_z, a->d_hidden, a->d_seq};
  for (int32_t v : widths) {
    if (v < 1 || v > (1 << 16)) return fail(LLATTE_ERR_INVALID_ARG, "width %d out of range", v);
    if (v % al) return fail(LLATTE_ERR_UNSUPPORTED, "widths must be multiples of %d", al);
  }
  if (a->rank < 1 || a->rank > 256) return fail(LLATTE_ERR_INVALID_ARG, "rank must be in [1, 256]");
  if (a->n_summaries < 1 || a->n_summaries > 64)
    return fail(LLATTE_ERR_INVALID_ARG, "n_summaries must be in [1, 64]");
  return LLATTE_OK;
}

// packed: W1^T merged [K, d_hidden, d_z], then W2^T merged [K, d_seq, d_hidden]
static size_t summary_w2_offset(const llatte_summary_desc* a) {
  const size_t es = a->dtype == LLATTE_BF16 ? 2 : 4;
  return al256((size_t)a->n_summaries * a->d_hidden * a->d_z * es);
}

size_t llatte_summary_packed_size(const llatte_summary_desc* desc) {
  if (check_summary_desc(desc) != LLATTE_OK) return 0;
  const size_t es = desc->dtype == LLATTE_BF16 ? 2 : 4;
  return summary_w2_offset(desc) + al256((size_t)desc->n_summaries * desc->d_seq * desc->d_hidden * es);
}

llatte_status llatte_summary_pack(const llatte_summary_desc* desc,
                                  const llatte_summary_weights* w,
                                  void* packed, size_t packed_bytes, void* stream) {
  llatte_status st = check_summary_desc(desc);
  if (st) return st;
  if (!w || !w->W1 || !w->W2 || !w->A1 || !w->B1 || !w->A2 || !w->B2 || !packed)
    return fail(LLATTE_ERR_INVALID_ARG, "NULL pointer");
  const void* ptrs[] = {w->W1, w->W2, w->A1, w->B1, w->A2, w->B2, packed};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(LLATTE_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (packed_bytes < llatte_summary_packed_size(desc))
    return fail(LLATTE_ERR_WORKSPACE, "packed buffer too small");
  const bool b = desc->dtype == LLATTE_BF16;
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(lora_merge(w->W1, w->A1, w->B1, desc->d_z, desc->d_hidden, desc->rank,
                     desc->n_summaries, packed, b, s));
  HIP_TRY(lora_merge(w->W2, w->A2, w->B2, desc->d_hidden, desc->d_seq, desc->rank,
                     desc->n_summaries, (char*)packed + summary_w2_offset(desc), b, s));
  return LLATTE_OK;
}

size_t llatte_summaries_workspace_size(const llatte_summary_desc* desc, int32_t B) {
  if (B < 0 || check_summary_desc(desc) != LLATTE_OK) return 0;
  const size_t es = desc->dtype == LLATTE_BF16 ? 2 : 4;
  return al256((size_t)B * desc->d_z * es) +
         al256((size_t)desc->n_summaries * B * desc->d_hidden * es) +
         al256((size_t)kSkPart * 4) + 256;
}

llatte_status llatte_summaries(const llatte_summary_desc* desc, const void* packed,
                               const float* z, int32_t B, float* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  llatte_status st = check_summary_desc(desc);
  if (st) return st;
  if (B < 0) return fail(LLATTE_ERR_INVALID_ARG, "B must be >= 0");
  if (B == 0) return LLATTE_OK;
  const void* ptrs[] = {packed, z, out, workspace};
  for (const void* p : ptrs) {
    if (!p) return fail(LLATTE_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(p)) return fail(LLATTE_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  }
  if (workspace_bytes < llatte_summaries_workspace_size(desc, B))
    return fail(LLATTE_ERR_WORKSPACE, "workspace too small");
  const bool b = desc->dtype == LLATTE_BF16;
  const size_t es = b ? 2 : 4;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  void* zc = base;
  void* H = base + al256((size_t)B * desc->d_z * es);
  const int K = desc->n_summaries;
  float* sk_part = (float*)((char*)H + al256((size_t)K * B * desc->d_hidden * es));
  HIP_TRY(cast_f32(z, zc, (long long)B * desc->d_z, b, s));
  {  // H[k] = GELU(z W1_k), all summaries in one batched launch
    GemmParams g;
    g.name = "gemm_summary_1";
    with_sk(g, sk_part);
    g.A = zc;
    g.lda = desc->d_z;
    g.sA = 0;
    g.B = packed;
    g.ldb = desc->d_z;
    g.sB = (long long)desc->d_hidden * desc->d_z;
    g.M_cap = B;
    g.N = desc->d_hidden;
    g.K = desc->d_z;
    g.batch = K;
    g.epi = EPI_GELU;
    g.C = H;
    g.ldc = desc->d_hidden;
    g.sC = (long long)B * desc->d_hidden;
    HIP_TRY(gemm(g, b, s));
  }
  {  // out[k] = H[k] W2_k
    GemmParams g;
    g.name = "gemm_summary_2";
    with_sk(g, sk_part);
    g.A = H;
    g.lda = desc->d_hidden;
    g.sA = (long long)B * desc->d_hidden;
    g.B = (const char*)packed + summary_w2_offset(desc);
    g.ldb = desc->d_hidden;
    g.sB = (long long)desc->d_seq * desc->d_hidden;
    g.M_cap = B;
    g.N = desc->d_seq;
    g.K = desc->d_hidden;
    g.batch = K;
    g.epi = EPI_STORE_F32;
    g.C = out;
    g.ldc = desc->d_seq;
    g.sC = (long long)B * desc->d_seq;
    HIP_TRY(gemm(g, b, s));
  }
  return LLATTE_OK;
}


// ---------------------------------------------------------------- attention backward
// d_q goes to d_q (fp32) or, when d_q_bf16 is given, there rounded to bf16.
static llatte_status attention_backward_call(
    const llatte_attn_desc* a, const void* q_lat, const void* c_lat,
    const int32_t* kv_offsets, const int32_t* hq_offsets, int32_t B,
    int32_t Mtot, int32_t Ktot, int32_t max_len, const float* out,
    const float* lse, const float* d_out, float* d_q, bf16* d_q_bf16, float* d_c, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (!a) return fail(LLATTE_ERR_INVALID_ARG, "NULL descriptor");
  if (a->dtype != LLATTE_BF16) return fail(LLATTE_ERR_UNSUPPORTED, "the backward is BF16 only");
  if (a->rank != 64 && a->rank != 128)
    return fail(LLATTE_ERR_UNSUPPORTED, "the backward needs rank 64 or 128");
  if (a->n_heads < 1 || a->n_cand < 0 || B < 1 || Ktot < B || max_len < 1 || Mtot < 0)
    return fail(LLATTE_ERR_INVALID_ARG, "bad sizes");
  // with no query rows only d_C is written (zeros): the row buffers may be NULL
  const void* dq_out = d_q_bf16 ? (const void*)d_q_bf16 : (const void*)d_q;
  const void* ptrs[] = {c_lat, kv_offsets, hq_offsets, d_c, q_lat, out, lse, d_out, dq_out, workspace};
  const int nreq = Mtot == 0 ? 4 : 10;
  for (int i = 0; i < 10; ++i) {
    if (!ptrs[i]) {
      if (i < nreq) return fail(LLATTE_ERR_INVALID_ARG, "NULL pointer");
      continue;
    }
    if (!aligned16(ptrs[i])) return fail(LLATTE_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  }
  AttnBwdParams p;
  p.q = q_lat;
  p.c = c_lat;
  p.out = out;
  p.lse = lse;
  p.dout = d_out;
  p.dq = d_q;
  p.dq_bf16 = d_q_bf16;
  p.dc = d_c;
  p.kv_off = kv_offsets;
  p.hq_off = hq_offsets;
  p.B = B;
  p.n_cand = a->n_cand;
  p.h = a->n_heads;
  p.r = a->rank;
  p.Mtot = Mtot;
  p.scale = a->scale;
  if (workspace_bytes < attention_backward_workspace(Mtot, a->n_heads, a->rank))
    return fail(LLATTE_ERR_WORKSPACE, "backward workspace too small");
  HIP_TRY(attention_backward(p, max_len, workspace, (hipStream_t)stream));
  return LLATTE_OK;
}

llatte_status llatte_mla_attention_backward(
    const llatte_attn_desc* a, const void* q_lat, const void* c_lat,
    const int32_t* kv_offsets, const int32_t* hq_offsets, int32_t B,
    int32_t Mtot, int32_t Ktot, int32_t max_len, const float* out,
    const float* lse, const float* d_out, float* d_q, float* d_c, void* workspace,
    size_t workspace_bytes, void* stream) {
  return attention_backward_call(a, q_lat, c_lat, kv_offsets, hq_offsets, B, Mtot, Ktot, max_len, out,
                                 lse, d_out, d_q, nullptr, d_c, workspace, workspace_bytes, stream);
}

size_t llatte_mla_attention_backward_workspace_size(const llatte_attn_desc* a, int32_t Mtot) {
  if (!a || a->n_heads < 1 || a->rank < 1 || Mtot < 0) return 0;
  return attention_backward_workspace(Mtot, a->n_heads, a->rank);
}

// ------------------------------------------------------------------ attention sublayer backward
static const char* check_sublayer_desc(const llatte_attn_sublayer_desc* D, int* code) {
  *code = LLATTE_ERR_INVALID_ARG;
  if (!D) return "NULL descriptor";
  *code = LLATTE_ERR_UNSUPPORTED;
  if (D->dtype != LLATTE_BF16) return "the sublayer backward is BF16 only";
  if (D->rank != 64 && D->rank != 128) return "the sublayer backward needs rank 64 or 128";
  if (D->latent_norm != 0 && D->latent_norm != 1) return "latent_norm must be 0 or 1";
  *code = LLATTE_ERR_INVALID_ARG;
  if (D->d < 8 || D->d > 1024 || D->d % 8) return "d must be a multiple of 8 in [8, 1024]";
  if (D->n_heads < 1 || D->head_dim < 8 || D->head_dim % 8) return "bad heads";
  if (D->n_cand < 0) return "n_cand must be >= 0";
  if (!(D->eps >= 0.f)) return "eps must be >= 0";
  return nullptr;
}

constexpr long long kSubSkPart = 1ll << 23;  // split-K scratch (floats)

// Carves the workspace and, with launch set, enqueues the whole backward.
// Returns the workspace bytes through *bytes when launch is false.
static llatte_status sublayer_backward_run(
    const llatte_attn_sublayer_desc* D, const llatte_attn_sublayer_weights* W, const float* r_kv,
    const float* r_cand, const int32_t* kv_off, const int32_t* hq_off, int32_t B, int32_t Mtot,
    int32_t Ktot, int32_t max_len, const float* d_out, float* d_r_kv, float* d_r_cand,
    const llatte_attn_sublayer_grads* G, void* workspace, size_t* bytes, bool launch,
    hipStream_t s) {
  const int d = D->d, h = D->n_heads, dk = D->head_dim, r = D->rank, hd = h * dk, hr = h * r;
  const long long M = Mtot, K = Ktot, nc = (long long)B * D->n_cand;
  const bool ln = D->latent_norm != 0;
  const float eps = D->eps;
  llatte_attn_desc ad{h, r, D->n_cand, LLATTE_BF16, 1.f / sqrtf((float)dk)};
  const size_t aws = llatte_mla_attention_workspace_size(&ad, B, Mtot, Ktot);
  const size_t bws = llatte_mla_attention_backward_workspace_size(&ad, Mtot);
  const int pk = rmsnorm_backward_parts(K), pc = rmsnorm_backward_parts(nc);
  Arena ar(workspace);
  bf16* H = ar.take<bf16>(K * d);
  float* ss_kv = ar.take<float>(K);
  bf16* Hc = ar.take<bf16>(nc * d);
  float* ss_c = ar.take<float>(nc);
  bf16* WdkvT = ar.take<bf16>((size_t)r * d);
  float* C0 = ar.take<float>(K * r);
  bf16* Cb = ar.take<bf16>(K * r);
  float* ss_C = ar.take<float>(K);
  bf16* Hq = ar.take<bf16>(M * d);
  int* qmap = ar.take<int>(K);
  bf16* WuqT = ar.take<bf16>((size_t)hd * d);
  bf16* q = ar.take<bf16>(M * hd);
  bf16* qt = ar.take<bf16>(M * hr);
  char* attn_ws = ar.take<char>(aws);
  float* ot = ar.take<float>(M * hr);
  float* lse = ar.take<float>(M * h);
  bf16* otb = ar.take<bf16>(M * hr);
  bf16* WuvT = ar.take<bf16>((size_t)hd * r);
  bf16* WukT = ar.take<bf16>((size_t)hd * r);
  bf16* o = ar.take<bf16>(M * hd);
  bf16* dRb = ar.take<bf16>(M * d);
  bf16* dob = ar.take<bf16>(M * hd);
  float* dot_ = ar.take<float>(M * hr);
  char* abw_ws = ar.take<char>(bws);
  bf16* dqtb = ar.take<bf16>(M * hr);
  bf16* dq = ar.take<bf16>(M * hd);
  float* dHq = ar.take<float>(M * d);
  float* dC = ar.take<float>(K * r);
  float* dC0 = ln ? ar.take<float>(K * r) : dC;
  bf16* dC0b = ar.take<bf16>(K * r);
  float* dH = ar.take<float>(K * d);
  float* dg_part = ar.take<float>((size_t)std::max((long long)(pk + pc) * d, (long long)pk * r));
  float* sk = ar.take<float>(kSubSkPart);
  if (!launch) {
    *bytes = ar.off;
    return LLATTE_OK;
  }
  if (M == 0) {  // no query rows: every gradient is zero
    HIP_TRY(zero_f32(d_r_kv, K * d, s));
    if (nc) HIP_TRY(zero_f32(d_r_cand, nc * d, s));
    HIP_TRY(zero_f32(G->g1, d, s));
    HIP_TRY(zero_f32(G->w_dkv, (long long)d * r, s));
    if (ln) HIP_TRY(zero_f32(G->g_c, r, s));
    HIP_TRY(zero_f32(G->w_uq, (long long)d * hd, s));
    HIP_TRY(zero_f32(G->w_uk, (long long)r * hd, s));
    HIP_TRY(zero_f32(G->w_uv, (long long)r * hd, s));
    HIP_TRY(zero_f32(G->w_o, (long long)hd * d, s));
    return LLATTE_OK;
  }
  // C = A B^T with A [Mr, Kc] (lda), B [N, Kc] (ldb), optional head batch
  auto mm = [&](const void* A, int lda, long long sA, const void* Bm, int ldb, long long sB, long long Mr,
                int N, int Kc, void* C, int ldc, long long sC, int batch, bool f32, bool split,
                const char* name) {
    GemmParams g;
    g.A = A;
    g.lda = lda;
    g.sA = sA;
    g.B = Bm;
    g.ldb = ldb;
    g.sB = sB;
    g.M_cap = (int)Mr;
    g.N = N;
    g.K = Kc;
    g.batch = batch;
    g.epi = f32 ? EPI_STORE_F32 : EPI_STORE;
    g.C = C;
    g.ldc = ldc;
    g.sC = sC;
    g.name = name;
    if (split) {
      g.sk_part = sk;
      g.sk_part_cap = kSubSkPart;
    }
    return gemm(g, true, s);
  };
  // ---- forward recompute
  HIP_TRY(norm_rows(RowSrc{r_kv, r_kv, 0, d}, (int)K, nullptr, W->g1, eps, nullptr, 0, H, d, d, K_BF16,
                    s, ss_kv));
  if (nc)
    HIP_TRY(norm_rows(RowSrc{r_cand, r_cand, 0, d}, (int)nc, nullptr, W->g1, eps, nullptr, 0, Hc, d, d,
                      K_BF16, s, ss_c));
  HIP_TRY(transpose(W->w_dkv, d, r, r, 0, WdkvT, d, 0, 1, K_BF16, K_BF16, s));
  HIP_TRY(mm(H, d, 0, WdkvT, d, 0, K, r, d, C0, r, 0, 1, true, false, "gemm_sub_c0"));
  HIP_TRY(norm_rows(RowSrc{C0, C0, 0, r}, (int)K, nullptr, ln ? W->g_c : nullptr, eps, nullptr, 0, Cb,
                    r, r, K_BF16, s, ln ? ss_C : nullptr));
  HIP_TRY(gather_query_rows(Hc, H, kv_off, hq_off, B, D->n_cand, d, Hq, qmap, s));
  HIP_TRY(transpose(W->w_uq, d, hd, hd, 0, WuqT, d, 0, 1, K_BF16, K_BF16, s));
  HIP_TRY(mm(Hq, d, 0, WuqT, d, 0, M, hd, d, q, hd, 0, 1, false, false, "gemm_sub_q"));
  HIP_TRY(mm(q, hd, dk, W->w_uk, hd, dk, M, r, dk, qt, hr, r, h, false, false, "gemm_sub_qlat"));
  {
    // õ in fp32 (the core backward's D) and as bf16 (the operand of its products)
    const llatte_status st = mla_attention_impl(&ad, qt, Cb, kv_off, hq_off, B, Mtot, Ktot, ot, lse,
                                                attn_ws, aws, s, false, otb);
    if (st != LLATTE_OK) return st;
  }
  HIP_TRY(transpose(W->w_uv, r, hd, hd, 0, WuvT, r, 0, 1, K_BF16, K_BF16, s));
  HIP_TRY(transpose(W->w_uk, r, hd, hd, 0, WukT, r, 0, 1, K_BF16, K_BF16, s));
  HIP_TRY(mm(otb, hr, r, WuvT, r, (long long)dk * r, M, dk, r, o, hd, dk, h, false, false, "gemm_sub_o"));
  // ---- backward
  // weight gradients over the rows: C [n1, n2] (+ head batch) = X^T Y
  auto wg = [&](const bf16* X, int ldx, long long sX, int n1, const bf16* Y, int ldy, long long sY,
                int n2, long long rows, float* C, int ldc, long long sC, int batch, const char* name) {
    WgradParams g;
    g.X = X;
    g.ldx = ldx;
    g.sX = sX;
    g.Y = Y;
    g.ldy = ldy;
    g.sY = sY;
    g.M = rows;
    g.N1 = n1;
    g.N2 = n2;
    g.batch = batch;
    g.C = C;
    g.ldc = ldc;
    g.sC = sC;
    g.part = sk;
    g.part_cap = kSubSkPart;
    g.name = name;
    return wgrad(g, s);
  };
  HIP_TRY(cast_f32(d_out, dRb, M * d, true, s));
  HIP_TRY(wg(o, hd, 0, hd, dRb, d, 0, d, M, G->w_o, d, 0, 1, "gemm_sub_dwo"));
  HIP_TRY(mm(dRb, d, 0, W->w_o, d, 0, M, hd, d, dob, hd, 0, 1, false, false, "gemm_sub_do"));
  HIP_TRY(wg(otb, hr, r, r, dob, hd, dk, dk, M, G->w_uv, hd, dk, h, "gemm_sub_dwuv"));
  HIP_TRY(mm(dob, hd, dk, W->w_uv, hd, dk, M, r, dk, dot_, hr, r, h, true, false, "gemm_sub_dolat"));
  {
    // dq̃ leaves the attention core as bf16, the operand of its two products
    const llatte_status st = attention_backward_call(&ad, qt, Cb, kv_off, hq_off, B, Mtot, Ktot,
                                                     max_len, ot, lse, dot_, nullptr, dqtb, dC, abw_ws,
                                                     bws, s);
    if (st != LLATTE_OK) return st;
  }
  HIP_TRY(mm(dqtb, hr, r, WukT, r, (long long)dk * r, M, dk, r, dq, hd, dk, h, false, false, "gemm_sub_dq"));
  HIP_TRY(wg(dqtb, hr, r, r, q, hd, dk, dk, M, G->w_uk, hd, dk, h, "gemm_sub_dwuk"));
  HIP_TRY(wg(Hq, d, 0, d, dq, hd, 0, hd, M, G->w_uq, hd, 0, 1, "gemm_sub_dwuq"));
  HIP_TRY(mm(dq, hd, 0, W->w_uq, hd, 0, M, d, hd, dHq, d, 0, 1, true, false, "gemm_sub_dhq"));
  if (ln) {
    HIP_TRY(rmsnorm_backward(C0, ss_C, dC, W->g_c, nullptr, eps, K, r, dC0, dg_part, s));
    HIP_TRY(column_sum(dg_part, pk, r, G->g_c, s));
  }
  HIP_TRY(cast_f32(dC0, dC0b, K * r, true, s));
  HIP_TRY(wg(H, d, 0, d, dC0b, r, 0, r, K, G->w_dkv, r, 0, 1, "gemm_sub_dwdkv"));
  HIP_TRY(mm(dC0b, r, 0, W->w_dkv, r, 0, K, d, r, dH, d, 0, 1, true, false, "gemm_sub_dh"));
  // the query rows' dH and residual gradient join their history rows
  HIP_TRY(rmsnorm_backward(r_kv, ss_kv, dH, W->g1, nullptr, eps, K, d, d_r_kv, dg_part, s, qmap, dHq,
                           d_out));
  if (nc)
    HIP_TRY(rmsnorm_backward(r_cand, ss_c, dHq, W->g1, d_out, eps, nc, d, d_r_cand,
                             dg_part + (size_t)pk * d, s));
  HIP_TRY(column_sum(dg_part, pk + pc, d, G->g1, s));
  return LLATTE_OK;
}

size_t llatte_attn_sublayer_backward_workspace_size(const llatte_attn_sublayer_desc* D, int32_t B,
                                                    int32_t Mtot, int32_t Ktot) {
  int code;
  if (check_sublayer_desc(D, &code) || B < 1 || Mtot < 0 || Ktot < B) return 0;
  size_t bytes = 0;
  llatte_attn_sublayer_grads g{};
  sublayer_backward_run(D, nullptr, nullptr, nullptr, nullptr, nullptr, B, Mtot, Ktot, 1, nullptr,
                        nullptr, nullptr, &g, nullptr, &bytes, false, nullptr);
  return bytes;
}

llatte_status llatte_attn_sublayer_backward(
    const llatte_attn_sublayer_desc* D, const llatte_attn_sublayer_weights* W, const float* r_kv,
    const float* r_cand, const int32_t* kv_offsets, const int32_t* hq_offsets, int32_t B,
    int32_t Mtot, int32_t Ktot, int32_t max_len, const float* d_out, float* d_r_kv,
    float* d_r_cand, const llatte_attn_sublayer_grads* G, void* workspace, size_t workspace_bytes,
    void* stream) {
  int code;
  if (const char* why = check_sublayer_desc(D, &code)) return fail(code, "%s", why);
  if (!W || !G) return fail(LLATTE_ERR_INVALID_ARG, "NULL weights or gradients");
  if (B < 1 || Ktot < B || max_len < 1 || Mtot < (long long)B * D->n_cand)
    return fail(LLATTE_ERR_INVALID_ARG, "bad sizes");
  const bool ln = D->latent_norm != 0, cand = D->n_cand > 0;
  const void* need[] = {W->g1, W->w_dkv, W->w_uq, W->w_uk, W->w_uv, W->w_o, r_kv, kv_offsets,
                        hq_offsets, d_r_kv, G->g1, G->w_dkv, G->w_uq, G->w_uk, G->w_uv, G->w_o,
                        workspace, ln ? W->g_c : W->g1, ln ? G->g_c : G->g1,
                        cand ? r_cand : r_kv, cand ? d_r_cand : d_r_kv,
                        Mtot > 0 ? d_out : r_kv};
  for (const void* p : need) {
    if (!p) return fail(LLATTE_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(p)) return fail(LLATTE_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  }
  const size_t bytes = llatte_attn_sublayer_backward_workspace_size(D, B, Mtot, Ktot);
  if (workspace_bytes < bytes)
    return fail(LLATTE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, bytes);
  return sublayer_backward_run(D, W, r_kv, r_cand, kv_offsets, hq_offsets, B, Mtot, Ktot, max_len,
                               d_out, d_r_kv, d_r_cand, G, workspace, nullptr, true,
                               (hipStream_t)stream);
}

static const char* check_ffn_desc(const llatte_ffn_desc* f) {
  if (!f) return "NULL descriptor";
  if (f->dtype != LLATTE_BF16) return "the FFN backward is BF16 only";
  if (f->d < 8 || f->d > 1024 || f->d % 8) return "d must be a multiple of 8 in [8, 1024]";
  if (f->d_ff < 8 || f->d_ff % 8) return "d_ff must be a positive multiple of 8";
  if (!(f->eps >= 0.f)) return "eps must be >= 0";
  return nullptr;
}

size_t llatte_ffn_backward_workspace_size(const llatte_ffn_desc* f, int32_t M) {
  if (check_ffn_desc(f) || M < 0) return 0;
  return ffn_backward_workspace(M, f->d, f->d_ff);
}

llatte_status llatte_ffn_backward(const llatte_ffn_desc* f, const float* r1, const float* g2,
                                  const void* w1, const void* w2, const float* d_out, int32_t M,
                                  float* d_r1, float* d_g2, float* d_w1, float* d_w2,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (const char* why = check_ffn_desc(f))
    return fail(f && f->dtype != LLATTE_BF16 ? LLATTE_ERR_UNSUPPORTED : LLATTE_ERR_INVALID_ARG, "%s", why);
  if (M < 0) return fail(LLATTE_ERR_INVALID_ARG, "M must be >= 0");
  // with no rows only the weight and gain gradients (zeros) are written
  const void* ptrs[] = {g2, w1, w2, d_g2, d_w1, d_w2, r1, d_out, d_r1, workspace};
  const int nreq = M == 0 ? 6 : 10;
  for (int i = 0; i < 10; ++i) {
    if (!ptrs[i]) {
      if (i < nreq) return fail(LLATTE_ERR_INVALID_ARG, "NULL pointer");
      continue;
    }
    if (!aligned16(ptrs[i])) return fail(LLATTE_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  }
  if (M > 0 && workspace_bytes < ffn_backward_workspace(M, f->d, f->d_ff))
    return fail(LLATTE_ERR_WORKSPACE, "FFN backward workspace too small");
  FfnBwdParams p;
  p.r1 = r1;
  p.g2 = g2;
  p.w1 = w1;
  p.w2 = w2;
  p.dout = d_out;
  p.dr1 = d_r1;
  p.dg2 = d_g2;
  p.dW1 = d_w1;
  p.dW2 = d_w2;
  p.M = M;
  p.d = f->d;
  p.F = f->d_ff;
  p.eps = f->eps;
  HIP_TRY(ffn_backward(p, workspace, (hipStream_t)stream));
  return LLATTE_OK;
}

}  // extern "C"

namespace llatte {

// ------------------------------------------------------------------ stack backward
// Workspace of llatte_mla_backward: the forward's own, then every plan's
// output rows and R1 rows (kept from the forward), two output-row gradient
// buffers, the readout / fusion temporaries and one region that the
// sublayer backward calls share (they run one after the other on the stream).
struct StackBwdWS {
  FwdWS fw;
  std::vector<float*> Rout, R1;  // per plan: [UBM, d] in the layer's query-row order
  float* gA = nullptr;           // [max rows of a layer's row space, d]
  float* gB = nullptr;
  float* dR1 = nullptr;          // [max UBM, d]
  bf16* demb_b = nullptr;        // [B, d_out]
  bf16* E = nullptr;             // [B*ns, d] the readout rows as bf16
  float* dS = nullptr;           // [B*ns, d]
  bf16* dq0_b = nullptr;         // [B*nq, d]
  float* dxc = nullptr;          // [B*nq, d+dc]
  char* sub = nullptr;
  size_t sub_bytes = 0;
};

static llatte_attn_sublayer_desc stack_sub_desc(const Shapes& S, int n_cand) {
  llatte_attn_sublayer_desc D;
  D.d = S.d;
  D.n_heads = S.h;
  D.head_dim = S.dk;
  D.rank = S.r;
  D.n_cand = n_cand;
  D.dtype = LLATTE_BF16;
  D.latent_norm = S.lnorm ? 1 : 0;
  D.eps = S.eps;
  return D;
}

static const char* stack_bwd_unsupported(const Shapes& S) {
  if (!S.bf16) return "the stack backward is BF16 only";
  if (!S.pre) return "the stack backward follows the pre-norm layer";
  if (S.rq) return "the stack backward follows the full-rank query path (q_rank = 0)";
  if (S.r != 64 && S.r != 128) return "the stack backward needs rank 64 or 128";
  if (S.validate || S.dump) return "the stack backward takes no VALIDATE or DEBUG_DUMP flag";
  if (S.ns > 0 && !S.raw && S.dout % 8) return "the stack backward needs d_out a multiple of 8";
  return nullptr;
}

static size_t layout_stack_bwd(const Shapes& S, void* base, StackBwdWS* b) {
  const size_t fwd = (layout_forward(S, base, &b->fw) + 255) & ~(size_t)255;
  Arena ar(base ? (char*)base + fwd : nullptr);
  b->Rout.assign(S.NP, nullptr);
  b->R1.assign(S.NP, nullptr);
  long long maxM = 1, maxG = 1;
  size_t sub = 0;
  const llatte_ffn_desc fd{S.d, S.dff, LLATTE_BF16, S.eps};
  for (int l = 0; l < S.NP; ++l) {
    const int nql = l < S.N ? S.nq : S.ns;
    b->Rout[l] = ar.take<float>((size_t)S.UBM[l] * S.d);
    b->R1[l] = ar.take<float>((size_t)S.UBM[l] * S.d);
    maxM = std::max(maxM, S.UBM[l]);
    maxG = std::max(maxG, S.UBrows[l]);
    const llatte_attn_sublayer_desc D = stack_sub_desc(S, nql);
    sub = std::max(sub, llatte_attn_sublayer_backward_workspace_size(&D, S.B, (int)S.UBM[l],
                                                                     (int)S.UBK[l]));
    sub = std::max(sub, llatte_ffn_backward_workspace_size(&fd, (int)S.UBM[l]));
  }
  b->gA = ar.take<float>((size_t)maxG * S.d);
  b->gB = ar.take<float>((size_t)maxG * S.d);
  b->dR1 = ar.take<float>((size_t)maxM * S.d);
  const size_t nq_rows = (size_t)S.B * S.nq, ns_rows = (size_t)S.B * S.ns;
  if (S.ns) {
    b->demb_b = ar.take<bf16>((size_t)S.B * std::max(S.dout, 1));
    b->E = ar.take<bf16>(ns_rows * S.d);
    b->dS = ar.take<float>(ns_rows * S.d);
  }
  if (S.nq) {
    b->dq0_b = ar.take<bf16>(nq_rows * S.d);
    b->dxc = ar.take<float>(nq_rows * (S.d + S.dc));
  }
  b->sub = ar.take<char>(sub);
  b->sub_bytes = sub;
  return fwd + ar.off + 256;
}

}  // namespace llatte

extern "C" {

size_t llatte_mla_backward_workspace_size(const llatte_model_desc* desc, int32_t B,
                                          int32_t total_rows, int32_t max_len) {
  Shapes S;
  if (make_shapes(desc, B, total_rows, max_len, &S) != LLATTE_OK || stack_bwd_unsupported(S))
    return 0;
  StackBwdWS b;
  return layout_stack_bwd(S, nullptr, &b);
}

llatte_status llatte_mla_backward(
    const llatte_model_desc* desc, const llatte_weights* wts, const float* hist_values,
    const int32_t* hist_offsets, const int32_t* hist_offsets_host, int32_t B, int32_t total_rows,
    int32_t max_len, const float* cand_x, const float* ctx, const float* d_out_cand,
    const float* d_out_hist, const float* d_out_emb, const llatte_grads* g, float* d_hist,
    float* d_cand_x, float* d_ctx, void* workspace, size_t workspace_bytes, void* stream) {
  Shapes S;
  llatte_status st = make_shapes(desc, B, total_rows, max_len, &S);
  if (st) return st;
  if (const char* why = stack_bwd_unsupported(S)) return fail(LLATTE_ERR_UNSUPPORTED, "%s", why);
  if ((st = check_weights(S, wts))) return st;
  if (!g || !g->layers) return fail(LLATTE_ERR_INVALID_ARG, "gradients are NULL");
  if (!hist_values || !hist_offsets || !hist_offsets_host || !d_hist || !workspace)
    return fail(LLATTE_ERR_INVALID_ARG, "hist_values, hist_offsets, hist_offsets_host, d_hist and "
                                        "workspace must be given");
  const bool cand = S.nq > 0, ctxp = S.nq > 0 && S.dc > 0, ro = S.ns > 0;
  if (cand && (!cand_x || !d_out_cand || !d_cand_x || !g->W_q))
    return fail(LLATTE_ERR_INVALID_ARG, "n_q > 0 needs cand_x, d_out_cand, d_cand_x and g->W_q");
  if (ctxp && (!ctx || !d_ctx)) return fail(LLATTE_ERR_INVALID_ARG, "d_ctx > 0 needs ctx and d_ctx");
  if (ro && (!d_out_emb || !g->seeds || (!S.raw && !g->W_p)))
    return fail(LLATTE_ERR_INVALID_ARG, "the readout needs d_out_emb, g->seeds and g->W_p");
  std::vector<const void*> ptrs = {hist_values, d_hist, workspace, cand_x, ctx, d_out_cand,
                                   d_out_hist, d_out_emb, d_cand_x, d_ctx, g->W_q, g->seeds,
                                   g->W_p};
  auto layer_ptrs = [&](const llatte_layer_grads& G, const char* what) -> llatte_status {
    const float* need[] = {G.g1, G.W_dkv, S.lnorm ? G.g_c : G.g1, G.W_uq, G.W_uk, G.W_uv,
                           G.W_o, G.g2, G.W1, G.W2};
    for (const float* p : need)
      if (!p) return fail(LLATTE_ERR_INVALID_ARG, "NULL gradient pointer (%s)", what);
    ptrs.insert(ptrs.end(), std::begin(need), std::end(need));
    return LLATTE_OK;
  };
  for (int l = 0; l < S.N; ++l)
    if ((st = layer_ptrs(g->layers[l], "layer"))) return st;
  if (ro && (st = layer_ptrs(g->readout, "readout"))) return st;
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(LLATTE_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  // per-plan row totals from the host offsets
  if (hist_offsets_host[0] != 0 || hist_offsets_host[B] != total_rows)
    return fail(LLATTE_ERR_INVALID_ARG, "hist_offsets_host must start at 0 and end at total_rows");
  std::vector<int> len(B);
  for (int u = 0; u < B; ++u) {
    len[u] = hist_offsets_host[u + 1] - hist_offsets_host[u];
    if (len[u] < 1 || len[u] > max_len)
      return fail(LLATTE_ERR_INVALID_ARG, "user %d: history length %d outside [1, max_len]", u, len[u]);
  }
  std::vector<int> keep((size_t)S.N * B);
  if ((st = llatte_pyramid_counts_host(&desc->pyramid, S.N, len.data(), B, keep.data()))) return st;
  std::vector<long long> Ksum(S.NP, 0), nsum(S.NP, 0);
  std::vector<int> maxK(S.NP, 1);
  for (int l = 0; l < S.NP; ++l)
    for (int u = 0; u < B; ++u) {
      const int K = l == 0 ? len[u] : keep[(size_t)(l - 1) * B + u];
      const int n = l < S.N ? keep[(size_t)l * B + u] : 0;
      Ksum[l] += K;
      nsum[l] += n;
      maxK[l] = std::max(maxK[l], K);
    }
  StackBwdWS b;
  const size_t need = layout_stack_bwd(S, nullptr, &b);
  if (workspace_bytes < need)
    return fail(LLATTE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  layout_stack_bwd(S, workspace, &b);
  hipStream_t s = (hipStream_t)stream;
  FwdWS& w = b.fw;
  const int d = S.d;
  const long long nc = (long long)B * S.nq;

  // ---- the forward again, keeping each layer's output rows and R1
  const Packed PK = w.pk;
  HIP_TRY(pack_all(S, wts, PK, s));
  HIP_TRY(build_plan(hist_offsets, B, S.rule, S.nq, S.ns, w.plan, S.NP, S.bq, kAttnBN, s));
  if (cand) {
    HIP_TRY(concat_queries(cand_x, ctx, B, S.nq, d, S.dc, w.XC, true, s));
    GemmParams gp;
    gp.name = "gemm_fusion";
    with_sk(gp, w.sk_part);
    gp.A = w.XC;
    gp.lda = d + S.dc;
    gp.B = PK.WqT;
    gp.ldb = d + S.dc;
    gp.M_cap = (int)nc;
    gp.N = d;
    gp.K = d + S.dc;
    gp.epi = EPI_STORE_F32;
    gp.C = w.Q0;
    gp.ldc = d;
    HIP_TRY(gemm(gp, true, s));
  }
  LayerIO io;
  for (int l = 0; l < S.N; ++l) {
    const RowSrc src = l == 0 ? RowSrc{w.Q0, hist_values, (int)nc, d}
                              : RowSrc{b.Rout[l - 1], b.Rout[l - 1] + nc * d, (int)nc, d};
    FwdWS wl = w;
    wl.R1 = b.R1[l];
    io.next = S.fnorm && l + 1 < S.N;
    HIP_TRY(run_layer(S, wl, l, PK.L[l], src, b.Rout[l], io, s));
    io.in_ready = io.next;
    io.np_in = io.np_out;
  }
  const float* last_hist = b.Rout[S.N - 1] + nc * d;
  if (ro) {
    HIP_TRY(broadcast_rows(PK.seeds, S.ns, d, B, w.S, s));
    FwdWS wl = w;
    wl.R1 = b.R1[S.N];
    LayerIO rio;
    HIP_TRY(run_layer(S, wl, S.N, PK.L[S.N], RowSrc{w.S, last_hist, B * S.ns, d}, b.Rout[S.N],
                      rio, s));
  }

  // ---- back through the stack
  const llatte_ffn_desc fd{d, S.dff, LLATTE_BF16, S.eps};
  auto layer_backward = [&](int l, const llatte_layer_weights& L, const llatte_layer_grads& G,
                            int n_cand, const float* r_kv, const float* r_c, const float* dout,
                            float* d_kv, float* d_c) -> llatte_status {
    const long long M = (long long)B * n_cand + nsum[l];
    llatte_status e = llatte_ffn_backward(&fd, b.R1[l], L.g2, L.W1, L.W2, dout, (int)M, b.dR1,
                                          G.g2, G.W1, G.W2, b.sub, b.sub_bytes, s);
    if (e) return e;
    const llatte_attn_sublayer_desc D = stack_sub_desc(S, n_cand);
    const llatte_attn_sublayer_weights W{L.g1, L.W_dkv, L.g_c, L.W_uq, L.W_uk, L.W_uv, L.W_o};
    const llatte_attn_sublayer_grads Gs{G.g1, G.W_dkv, G.g_c, G.W_uq, G.W_uk, G.W_uv, G.W_o};
    const LayerPlan P = w.plan.layer(l);
    return llatte_attn_sublayer_backward(&D, &W, r_kv, n_cand ? r_c : nullptr, P.kv_off, P.hq_off,
                                         B, (int)M, (int)Ksum[l], maxK[l], b.dR1, d_kv,
                                         n_cand ? d_c : nullptr, &Gs, b.sub, b.sub_bytes, s);
  };
  auto wgrad_call = [&](const bf16* X, int n1, const bf16* Y, int n2, long long rows, float* C,
                        const char* name) {
    WgradParams p;
    p.X = X;
    p.ldx = n1;
    p.Y = Y;
    p.ldy = n2;
    p.M = rows;
    p.N1 = n1;
    p.N2 = n2;
    p.C = C;
    p.ldc = n2;
    p.part = w.sk_part;
    p.part_cap = kSkPart;
    p.name = name;
    return wgrad(p, s);
  };
  float* cur = b.gA;  // gradient of the current layer's output rows
  float* nxt = b.gB;
  const long long nh_last = nsum[S.N - 1];
  if (ro) {
    // dZ: the readout rows' gradient
    const long long nsr = (long long)B * S.ns;
    const float* dZ = d_out_emb;
    if (!S.raw) {
      HIP_TRY(cast_f32(d_out_emb, b.demb_b, (long long)B * S.dout, true, s));
      GemmParams gp;
      gp.name = "gemm_bwd_readout";
      with_sk(gp, w.sk_part);
      gp.A = b.demb_b;
      gp.lda = S.dout;
      gp.B = wts->W_p;  // [ns*d, d_out] row-major: its rows are the products' columns
      gp.ldb = S.dout;
      gp.M_cap = B;
      gp.N = S.ns * d;
      gp.K = S.dout;
      gp.epi = EPI_STORE_F32;
      gp.C = b.dS;
      gp.ldc = S.ns * d;
      HIP_TRY(gemm(gp, true, s));
      HIP_TRY(cast_f32(b.Rout[S.N], b.E, nsr * d, true, s));
      HIP_TRY(wgrad_call(b.E, S.ns * d, b.demb_b, S.dout, B, g->W_p, "wgrad_readout"));
      dZ = b.dS;
    }
    // the readout layer: keys = the last layer's history outputs, queries =
    // the seeds; its key gradient is the last layer's history output
    // gradient (plus d_out_hist), the seed rows' gradient sums into the seeds
    if ((st = layer_backward(S.N, wts->readout, g->readout, S.ns, last_hist, w.S, dZ,
                             cur + nc * d, nxt)))
      return st;
    HIP_TRY(group_sum_rows(nxt, d, 0, S.ns, 1, B, S.ns, d, g->seeds, s));
    if (d_out_hist) HIP_TRY(add_f32(cur + nc * d, d_out_hist, nh_last * d, s));
  } else if (d_out_hist) {
    HIP_TRY(hipMemcpyAsync(cur + nc * d, d_out_hist, (size_t)nh_last * d * sizeof(float),
                           hipMemcpyDeviceToDevice, s));
  } else {
    HIP_TRY(zero_f32(cur + nc * d, nh_last * d, s));
  }
  if (cand)
    HIP_TRY(hipMemcpyAsync(cur, d_out_cand, (size_t)nc * d * sizeof(float),
                           hipMemcpyDeviceToDevice, s));
  for (int l = S.N - 1; l >= 0; --l) {
    // layer l's input rows are layer l-1's output rows: candidates, then
    // the history rows user by user
    const float* r_kv = l == 0 ? hist_values : b.Rout[l - 1] + nc * d;
    const float* r_c = l == 0 ? w.Q0 : b.Rout[l - 1];
    if ((st = layer_backward(l, wts->layers[l], g->layers[l], S.nq, r_kv, r_c, cur,
                             l == 0 ? d_hist : nxt + nc * d, nxt)))
      return st;
    std::swap(cur, nxt);
  }
  if (cand) {
    // Q0 = [x ; c] W_q: cur holds dQ0
    HIP_TRY(cast_f32(cur, b.dq0_b, nc * d, true, s));
    HIP_TRY(wgrad_call((const bf16*)w.XC, d + S.dc, b.dq0_b, d, nc, g->W_q, "wgrad_fusion"));
    GemmParams gp;
    gp.name = "gemm_bwd_fusion";
    with_sk(gp, w.sk_part);
    gp.A = b.dq0_b;
    gp.lda = d;
    gp.B = wts->W_q;  // [d+dc, d] row-major
    gp.ldb = d;
    gp.M_cap = (int)nc;
    gp.N = d + S.dc;
    gp.K = d;
    gp.epi = EPI_STORE_F32;
    gp.C = b.dxc;
    gp.ldc = d + S.dc;
    HIP_TRY(gemm(gp, true, s));
    HIP_TRY(copy_rows_f32(b.dxc, d + S.dc, d_cand_x, (int)nc, nullptr, d, s));
    if (ctxp) HIP_TRY(group_sum_rows(b.dxc, d + S.dc, d, B, S.nq, S.nq, 1, S.dc, d_ctx, s));
  }
  return LLATTE_OK;
}

}  // extern "C"
