// Device-side planning of the jagged, pyramidal layer stack.
//
// Everything that depends on the per-user history lengths is computed on the
// GPU from the offsets, so the forward pass never waits for the host: per
// layer the key and query counts of every user (pyramidal schedule of
// LLaTTE, Appendix A.2), their exclusive scans, the query-row gather map,
// and the attention work items sorted by decreasing cost (longest-processing-
// time order, so that the heaviest query blocks start first and the tail of
// the grid holds the light ones).
#include "kernels.hpp"

namespace llatte {

constexpr int kPlanThreads = 1024;
constexpr int kMaxBuckets = 4096;  // cost buckets: KV tiles per work item
constexpr unsigned kCandFlag = 0x80000000u;

// Count of user u at layer l (0-based) under the rule, capped by `prev`
// (the count at layer l-1, or L_u at layer 0).
__device__ __forceinline__ int rule_eval(const RuleDev& r, int l, int L,
                                         int prev) {
  int k;
  if (r.kind == 1)  // halving with floor
    k = max(min(r.floor, L), L >> min(l, 30));
  else
    k = r.values[l];
  return min(k, prev);
}

// Exclusive scan of one pair of values per thread over a block of
// kPlanThreads = 1024 threads (16 waves): inclusive scans inside each wave
// by lane shifts, then the 16 wave totals scanned by the first wave through
// LDS; two barriers, plus one at the end so that sh (64 ints) may be reused.
// Returns the thread's exclusive prefixes; tot receives the block totals.
static_assert(kPlanThreads == 1024, "the scan assumes 16 waves");
__device__ __forceinline__ int2 block_exclusive_scan2(int2 v, int* sh, int2& tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int a = v.x, b = v.y;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ya = __shfl_up(a, o, 64), yb = __shfl_up(b, o, 64);
    if (lane >= o) {
      a += ya;
      b += yb;
    }
  }
  if (lane == 63) {
    sh[w] = a;
    sh[16 + w] = b;
  }
  __syncthreads();
  if (w == 0) {
    int ta = lane < 16 ? sh[lane] : 0, tb = lane < 16 ? sh[16 + lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int ya = __shfl_up(ta, o, 64), yb = __shfl_up(tb, o, 64);
      if (lane >= o) {
        ta += ya;
        tb += yb;
      }
    }
    if (lane < 16) {
      sh[32 + lane] = ta;  // inclusive prefixes of the wave totals
      sh[48 + lane] = tb;
    }
  }
  __syncthreads();
  const int pa = w > 0 ? sh[32 + w - 1] : 0, pb = w > 0 ? sh[48 + w - 1] : 0;
  tot = int2{sh[47], sh[63]};
  __syncthreads();
  return int2{pa + a - v.x, pb + b - v.y};
}

// Exclusive scan of in[0..B) into out[0..B], out[B] = total, by one block of
// kPlanThreads threads; each thread owns a contiguous chunk of users.
__device__ void block_scan(const int* in, int* out, int B, int* sh) {
  const int t = threadIdx.x;
  const int chunk = (B + kPlanThreads - 1) / kPlanThreads;
  const int u0 = min(B, t * chunk), u1 = min(B, u0 + chunk);
  int s = 0;
  for (int u = u0; u < u1; ++u) s += in[u];
  int2 tot;
  int run = block_exclusive_scan2(int2{s, 0}, sh, tot).x;
  for (int u = u0; u < u1; ++u) {
    out[u] = run;
    run += in[u];
  }
  if (t == kPlanThreads - 1) out[B] = tot.x;
  __syncthreads();
}

// Keys K and kept query rows n of a user with L history rows at layer l:
// layer 0 sees all L rows, layer i + 1 the rows layer i kept; plans past the
// stack (the readout) keep none.
__device__ __forceinline__ int2 layer_counts(const RuleDev& rule, int n_layers, int l, int L) {
  int K = L, n = 0;
  for (int i = 0; i <= l; ++i) {
    n = i < n_layers ? rule_eval(rule, i, L, K) : 0;
    if (i < l) K = n;
  }
  return int2{K, n};
}

struct PlanArgs {
  PlanBase base;
  int n_plans;
  int n_layers;      // layers of the stack (plans beyond are the readout)
  int nq[65];        // query tokens per user, per plan
  int* hq_copy = nullptr;  // optional second copy of plan copy_plan's hq_off
  int copy_plan = -1;
};

// Attention work items of plan P, counting-sorted by cost (KV tiles) in
// decreasing order, by the whole block (hist: kMaxBuckets ints of LDS,
// zeroed by the caller before a barrier). Item = {first query row, kv base
// row, rows | candidate flag, key position of the first row}. Lane = user
// (users 64 k + lane), wave w = the query blocks b = w, w + 16, ... of each
// user. When the active lanes of a wave fall in the same bucket (equal
// history lengths: block b of every user costs the same), one atomic
// reserves their slots and they take them in lane order, so within a bucket
// the items are in user order: the workgroups dealt to one XCD
// (round-robin) keep to the same users' latent rows, and the atomics of a
// wave do not collide on one address.
__device__ __forceinline__ int bucket_add(int* hist, int bucket) {
  const unsigned long long act = __ballot(1);
  const int first = __builtin_amdgcn_readfirstlane(bucket);
  if (__ballot(bucket == first) == act) {
    const int lane = threadIdx.x & 63;
    const unsigned lo = (unsigned)act, hi = (unsigned)(act >> 32);
    const int rank = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0));
    int base = 0;
    if (lane == __ffsll((long long)act) - 1) base = atomicAdd(&hist[bucket], __popcll(act));
    return __builtin_amdgcn_readfirstlane(base) + rank;
  }
  return atomicAdd(&hist[bucket], 1);
}

__device__ void plan_items(const LayerPlan& P, int nq, int B, int bq, int bn, int items_cap,
                           int* hist, int* sh) {
  const int nc = B * nq;
  const int ncb = (nq + bq - 1) / bq;
  constexpr int kWaves = kPlanThreads / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // pass 0 counts items per cost bucket, pass 1 places them
  for (int pass = 0; pass < 2; ++pass) {
    for (int u = lane; u < B; u += 64) {
      const int K = P.kv_len[u], n = P.keep[u];
      const int kvb = P.kv_off[u];
      const int nhb = (n + bq - 1) / bq;
      for (int b = w; b < nhb + ncb; b += kWaves) {
        i32x4 it;
        int cost;
        if (b < nhb) {
          const int t0 = b * bq, nr = min(bq, n - t0);
          const int pos0 = K - n + t0;
          it = i32x4{nc + P.hq_off[u] + t0, kvb, nr, pos0};
          cost = (pos0 + nr + bn - 1) / bn;
        } else {
          const int j0 = (b - nhb) * bq, nr = min(bq, nq - j0);
          it = i32x4{u * nq + j0, kvb, (int)(kCandFlag | (unsigned)nr), K - 1};
          cost = (K + bn - 1) / bn;
        }
        const int bucket = kMaxBuckets - 1 - min(cost, kMaxBuckets - 1);
        const int slot = bucket_add(hist, bucket);
        if (pass == 1 && slot < items_cap) P.items[slot] = it;
      }
    }
    __syncthreads();
    if (pass == 0) {
      // exclusive scan of the bucket counts (buckets ordered heaviest first)
      const int per = kMaxBuckets / kPlanThreads;
      int s = 0;
      for (int i = 0; i < per; ++i) s += hist[threadIdx.x * per + i];
      int2 tot;
      int run = block_exclusive_scan2(int2{s, 0}, sh, tot).x;
      for (int i = 0; i < per; ++i) {
        const int c = hist[threadIdx.x * per + i];
        hist[threadIdx.x * per + i] = run;
        run += c;
      }
      if (threadIdx.x == kPlanThreads - 1) *P.n_items = min(tot.x, items_cap);
      __syncthreads();
    }
  }
}

// Counts, offsets and (bq > 0) attention work items of layer blockIdx.x. A
// user's counts at a layer follow from its history length alone, so every
// layer is a block of its own; the items read back the counts this block
// wrote (visible to the block after the barrier).
__global__ __launch_bounds__(kPlanThreads) void plan_layer_kernel(
    const int* offsets, int B, RuleDev rule, PlanArgs a, int bq, int bn, int items_cap) {
  __shared__ int sh[64];
  __shared__ int hist[kMaxBuckets];
  const int l = blockIdx.x, t = threadIdx.x;
  const LayerPlan P = a.base.layer(l);
  for (int i = t; i < kMaxBuckets; i += kPlanThreads) hist[i] = 0;
  const int chunk = (B + kPlanThreads - 1) / kPlanThreads;
  const int u0 = min(B, t * chunk), u1 = min(B, u0 + chunk);
  int2 sum{0, 0};
  for (int u = u0; u < u1; ++u) {
    const int2 c = layer_counts(rule, a.n_layers, l, offsets[u + 1] - offsets[u]);
    P.kv_len[u] = c.x;
    P.keep[u] = c.y;
    sum.x += c.x;
    sum.y += c.y;
  }
  int2 tot;
  int2 run = block_exclusive_scan2(sum, sh, tot);
  for (int u = u0; u < u1; ++u) {
    const int2 c = layer_counts(rule, a.n_layers, l, offsets[u + 1] - offsets[u]);
    P.kv_off[u] = run.x;
    P.hq_off[u] = run.y;
    if (l == a.copy_plan) a.hq_copy[u] = run.y;
    run.x += c.x;
    run.y += c.y;
  }
  if (t == kPlanThreads - 1) {
    const int nc = B * a.nq[l];
    P.kv_off[B] = tot.x;
    P.hq_off[B] = tot.y;
    if (l == a.copy_plan) a.hq_copy[B] = tot.y;
    P.counts[0] = tot.x;
    P.counts[1] = tot.y;
    P.counts[2] = nc + tot.x;
    P.counts[3] = nc + tot.y;
  }
  if (bq <= 0) return;
  __syncthreads();
  plan_items(P, a.nq[l], B, bq, bn, items_cap, hist, sh);
}

// Work items of plan blockIdx.x from counts already in place (the
// standalone attention's plan).
__global__ __launch_bounds__(kPlanThreads) void plan_items_kernel(
    PlanArgs a, int B, int bq, int bn, int items_cap) {
  __shared__ int sh[64];
  __shared__ int hist[kMaxBuckets];
  const int l = blockIdx.x;
  for (int i = threadIdx.x; i < kMaxBuckets; i += kPlanThreads) hist[i] = 0;
  __syncthreads();
  plan_items(a.base.layer(l), a.nq[l], B, bq, bn, items_cap, hist, sh);
}

// Query gather map and per-row attention info; grid (B, n_plans).
__global__ void plan_qmap_kernel(PlanArgs a, int B) {
  const int u = blockIdx.x, l = blockIdx.y;
  const LayerPlan P = a.base.layer(l);
  const int nq = a.nq[l];
  const int nc = B * nq;
  const int K = P.kv_len[u], n = P.keep[u];
  const int kvb = P.kv_off[u];
  for (int j = threadIdx.x; j < nq; j += blockDim.x) {
    const int i = u * nq + j;
    P.qmap[i] = i;
    P.qinfo[i] = int2{kvb, K - 1};
  }
  for (int t = threadIdx.x; t < n; t += blockDim.x) {
    const int i = nc + P.hq_off[u] + t;
    P.qmap[i] = nc + kvb + K - n + t;
    P.qinfo[i] = int2{kvb, K - n + t};
  }
}

hipError_t build_plan(const int* offsets, int B, const RuleDev& rule, int n_q,
                      int n_seeds, const PlanBase& base, int n_plans, int bq,
                      int bn, hipStream_t s, int* hq_copy, int copy_plan) {
  PlanArgs a;
  a.base = base;
  a.n_plans = n_plans;
  a.n_layers = rule.n_layers;
  if (hq_copy) {
    a.hq_copy = hq_copy;
    a.copy_plan = copy_plan;
  }
  for (int l = 0; l < n_plans; ++l) a.nq[l] = l < rule.n_layers ? n_q : n_seeds;
  timing_begin("plan", s);
  hipLaunchKernelGGL(plan_layer_kernel, dim3(n_plans), dim3(kPlanThreads), 0, s,
                     offsets, B, rule, a, bq, bn, base.icap);
  hipLaunchKernelGGL(plan_qmap_kernel, dim3(B, n_plans), dim3(256), 0, s, a, B);
  timing_end(s);
  return hipGetLastError();
}

// ------------------------------------------------------------------ counts
__global__ __launch_bounds__(256) void pyramid_counts_kernel(
    RuleDev rule, const int* offsets, int B, int* keep_out) {
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= B) return;
  const int L = offsets[u + 1] - offsets[u];
  int prev = L;
  for (int l = 0; l < rule.n_layers; ++l) {
    prev = rule_eval(rule, l, L, prev);
    keep_out[(size_t)l * B + u] = prev;
  }
}

hipError_t pyramid_counts_dev(const RuleDev& rule, const int* offsets, int B,
                              int* keep_out, hipStream_t s) {
  hipLaunchKernelGGL(pyramid_counts_kernel, dim3((B + 255) / 256), dim3(256), 0,
                     s, rule, offsets, B, keep_out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ validation
// Check of the history offsets (the opt-in LLATTE_FLAG_VALIDATE): every
// user's L_u = offsets[u+1] - offsets[u] in [1, max_len], offsets[0] == 0,
// offsets[B] == total. One block; each thread scans a chunk of users and the
// block keeps the smallest failing index. err[0] = kind (0: valid; 1:
// offsets[0] != 0; 2: L_u < 1; 3: L_u > max_len; 4: offsets[B] != total),
// err[1] = the user (or B for kind 4). Written whatever the outcome, so the
// words need no clearing before the launch.
__global__ __launch_bounds__(kPlanThreads) void validate_offsets_kernel(
    const int* offsets, int B, int total, int max_len, int* err) {
  __shared__ int first[2];
  const int t = threadIdx.x;
  if (t == 0) {
    first[0] = 0x7fffffff;  // smallest failing user (kinds 2, 3)
    first[1] = 0;           // its kind
  }
  __syncthreads();
  const int chunk = (B + kPlanThreads - 1) / kPlanThreads;
  const int u0 = min(B, t * chunk), u1 = min(B, u0 + chunk);
  for (int u = u0; u < u1; ++u) {
    const int L = offsets[u + 1] - offsets[u];
    if (L < 1 || L > max_len) {
      atomicMin(&first[0], u);
      break;
    }
  }
  __syncthreads();
  if (t == 0) {
    int kind = 0, who = 0;
    if (offsets[0] != 0) {
      kind = 1;
    } else if (first[0] != 0x7fffffff) {
      who = first[0];
      const int L = offsets[who + 1] - offsets[who];
      kind = L < 1 ? 2 : 3;
    } else if (offsets[B] != total) {
      kind = 4;
      who = B;
    }
    err[0] = kind;
    err[1] = who;
  }
}

hipError_t validate_offsets(const int* offsets, int B, int total, int max_len, int* err,
                            hipStream_t s) {
  hipLaunchKernelGGL(validate_offsets_kernel, dim3(1), dim3(kPlanThreads), 0, s, offsets, B, total,
                     max_len, err);
  return hipGetLastError();
}

// ------------------------------------------------------------------ compaction
__global__ __launch_bounds__(kPlanThreads) void compact_scan_kernel(
    const int* keep, int B, int* offsets_out) {
  __shared__ int sh[64];
  block_scan(keep, offsets_out, B, sh);
}

// One wave per output row: find the user by binary search over offsets_out,
// copy the row's bytes in 16-byte (or 4-byte) units, record the source row.
__global__ __launch_bounds__(256) void compact_rows_kernel(
    const char* values, int row_bytes, const int* offsets_in, int B,
    const int* keep, const int* offsets_out, char* values_out, int* src_index,
    int rows_cap) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= rows_cap || i >= offsets_out[B]) return;
  int lo = 0, hi = B - 1;  // largest u with offsets_out[u] <= i
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets_out[mid] <= i) lo = mid; else hi = mid - 1;
  }
  const int u = lo;
  const int t = i - offsets_out[u];
  const int src = offsets_in[u + 1] - keep[u] + t;
  if (lane == 0 && src_index) src_index[i] = src;
  const char* s = values + (size_t)src * row_bytes;
  char* d = values_out + (size_t)i * row_bytes;
  if ((row_bytes & 15) == 0) {
    for (int b = lane * 16; b < row_bytes; b += 64 * 16)
      *(i32x4*)(d + b) = *(const i32x4*)(s + b);
  } else {
    for (int b = lane * 4; b < row_bytes; b += 64 * 4)
      *(int*)(d + b) = *(const int*)(s + b);
  }
}

hipError_t pyramid_compact(const void* values, int row_bytes,
                           const int* offsets_in, int B, int total_rows,
                           const int* keep, void* values_out, int* offsets_out,
                           int* src_index, hipStream_t s) {
  timing_begin("pyramid_compact", s);
  hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(kPlanThreads), 0, s,
                     keep, B, offsets_out);
  if (total_rows > 0)
    hipLaunchKernelGGL(compact_rows_kernel, dim3((total_rows + 3) / 4),
                       dim3(256), 0, s, (const char*)values, row_bytes,
                       offsets_in, B, keep, offsets_out, (char*)values_out,
                       src_index, total_rows);
  timing_end(s);
  return hipGetLastError();
}

// ------------------------------------------------------------------ standalone
// Items and row info for llatte_mla_attention from given offsets.
__global__ __launch_bounds__(kPlanThreads) void attn_lens_kernel(
    const int* kv_off, const int* hq_off, int B, int* kv_len, int* keep,
    int* kvo, int* hqo, int* counts, int n_cand) {
  for (int u = threadIdx.x; u < B; u += kPlanThreads) {
    kv_len[u] = kv_off[u + 1] - kv_off[u];
    keep[u] = hq_off[u + 1] - hq_off[u];
    kvo[u] = kv_off[u];
    hqo[u] = hq_off[u];
  }
  if (threadIdx.x == 0) {
    kvo[B] = kv_off[B];
    hqo[B] = hq_off[B];
    counts[0] = kv_off[B];
    counts[1] = hq_off[B];
    counts[2] = B * n_cand + kv_off[B];
    counts[3] = B * n_cand + hq_off[B];
  }
}

hipError_t build_attn_plan(const int* kv_off, const int* hq_off, int B,
                           int n_cand, int bq, int bn, const PlanBase& base,
                           hipStream_t s) {
  const LayerPlan P = base.layer(0);
  PlanArgs a;
  a.base = base;
  a.n_plans = 1;
  a.n_layers = 1;
  a.nq[0] = n_cand;
  timing_begin("plan", s);
  hipLaunchKernelGGL(attn_lens_kernel, dim3(1), dim3(kPlanThreads), 0, s,
                     kv_off, hq_off, B, P.kv_len, P.keep, P.kv_off, P.hq_off,
                     P.counts, n_cand);
  if (bq > 0)
    hipLaunchKernelGGL(plan_items_kernel, dim3(1), dim3(kPlanThreads), 0, s, a,
                       B, bq, bn, base.icap);
  hipLaunchKernelGGL(plan_qmap_kernel, dim3(B, 1), dim3(256), 0, s, a, B);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace llatte
