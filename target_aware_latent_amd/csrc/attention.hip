// Attention in latent space: the core of the absorbed MLA form (LLaTTE,
// Appendix A.3: MLA equals multi-query attention on the latent). Every head
// scores its latent query against the same latent rows C and averages C
// itself, so one C tile in LDS serves all heads of a query block.
//
// MFMA kernel: one workgroup per work item (a block of BQ query rows of one
// user) and group of HG heads. Each wave owns EPW (head, query row) pairs,
// "effective rows", all of one head. For r <= 128 a workgroup has four
// waves and two workgroups share a CU (register budget: two waves per
// SIMD), so one workgroup's prologue, epilogue and barrier waits overlap
// the other's matrix work; for r = 256 eight waves fill the CU (LDS). Per
// 64-key tile of C:
//   S^T = C_tile . Qlat^T        v_mfma_f32_16x16x32_f16; A = C rows (LDS),
//                                B = latent queries held in registers
//   online softmax per column    fp32, exp2 (the softmax scale and log2(e)
//                                are folded into the latent queries); the
//                                column max over the four lane groups with
//                                two permlane swaps, the column sums on the
//                                matrix cores (ones operand)
//   O^T += C_tile^T . P^T        A = C^T from a transposed LDS copy, B = P^T
//                                straight from the S^T accumulators
// Working on the transposed products keeps each lane's softmax column and
// output column the same effective row: the rescale needs no shuffles and P
// never goes through LDS. The tile is staged once, row-major and
// double-buffered; the C^T operand is read from it with the gfx950 transpose
// load (ds_read_b64_tr_b16: within each 16-lane group, lane i receives column
// i of the 4x16 block whose rows the group's lanes address). The 8-byte
// chunks of each tile row are XOR-swizzled by a function of the key's low
// nibble, chosen so that with 64 four-byte LDS banks every 32-lane pass of
// the three access patterns (S^T reads: 16 keys x 2 chunks; transpose reads:
// 8 keys x 4 chunks; staging writes) touches 32 distinct 8-byte bank slots
// (for r = 256 the staging writes keep a 2-way conflict). The swizzled
// offsets are lane constants, computed once. Operand k-order: both MFMA operands of a product
// use the same permutation of the contraction index (lane group g holds
// k = 4g..4g+3 and 16+4g..16+4g+3 of each 32-wide step), which is what the
// S^T accumulator layout hands to the P^T operand.
//
// Operands are fp16 (the latent C and queries are RMS-normalised, well
// inside fp16 range, and P lies in [0, 1]): 11 mantissa bits instead of 8,
// at the same MFMA rate. Accumulation and softmax are fp32.
//
// Fused mode (the forward pass): the prologue forms the latent queries from
// the query projection, q_lat_j = q_j W_uk_j^T (bf16 MFMA), and the epilogue
// maps the normalised output back, o_j = o_lat_j W_uv_j (fp16 MFMA), writing
// o [M, h*dk] in bf16 for the output projection. Neither q_lat nor o_lat
// touches HBM.
//
// Masks: history rows see keys up to their own position (causal, LLaTTE
// Appendix A.2); candidate rows see every key of their user.
//
// fp32 kernel: one wave per (query row, head), keys 64 at a time, plain
// online softmax. It serves the fp32 path only.
#include <algorithm>
#include <type_traits>
#include <vector>

#include "kernels.hpp"

namespace llatte {

// Work-item and workgroup ids from the compiler's intrinsics. This file is
// built with IEEE mode off, and the device library's id functions, built
// with it on, are then not inlined: threadIdx / blockIdx would stay calls,
// whose results the compiler must treat as per-lane values (vector
// registers and vector loads for what is uniform).
__device__ __forceinline__ int lid_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int gid_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int gid_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;  // running-max slack, log2 units

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}
// IEEE-754 maximum (gfx950 v_maximum3_f32): three-way trees fuse into one
// instruction, and no quieting pass over operands the compiler cannot prove
// canonical (MFMA results, permlane outputs) is needed whatever the NaN mode
// the file is built with. Scores here are finite or -inf, where it equals
// fmaxf.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }
// Max of a lane's 16 scores of one accumulator column block (4 blocks of 4).
__device__ __forceinline__ float max16(const f32x4& a, const f32x4& b, const f32x4& c, const f32x4& d) {
  const float x = vmax3(a[0], a[1], a[2]), y = vmax3(a[3], b[0], b[1]), z = vmax3(b[2], b[3], c[0]);
  const float u = vmax3(c[1], c[2], c[3]), w = vmax3(d[0], d[1], d[2]);
  return vmax(vmax3(x, y, z), vmax3(u, w, d[3]));
}
// Max over the four lanes l, l^16, l^32, l^48 (a column of an MFMA
// accumulator block spans the four 16-lane groups). Each permlane swap hands
// a lane its own value and its partner's, in an order that differs between
// the two lanes of a pair; the max of the two is order-free. Runs on the VALU,
// no LDS round trip.
__device__ __forceinline__ float max_across_groups(float x) {
  const unsigned u = __float_as_uint(x);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = vmax(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
  const unsigned w = __float_as_uint(x);
  const auto p32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return vmax(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Values k = 4g..4g+3 and 16+4g..16+4g+3 of two 16-wide accumulator blocks.
__device__ __forceinline__ f16x8 pack8(f32x4 lo, f32x4 hi, float s) {
  return f16x8{(f16)(lo[0] * s), (f16)(lo[1] * s), (f16)(lo[2] * s), (f16)(lo[3] * s),
               (f16)(hi[0] * s), (f16)(hi[1] * s), (f16)(hi[2] * s), (f16)(hi[3] * s)};
}
__device__ __forceinline__ f16x8 pack8(f32x4 lo, f32x4 hi) {
  return f16x8{(f16)lo[0], (f16)lo[1], (f16)lo[2], (f16)lo[3],
               (f16)hi[0], (f16)hi[1], (f16)hi[2], (f16)hi[3]};
}
__device__ __forceinline__ f16x8 cat(f16x4 lo, f16x4 hi) {
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// Eight stored values as fp16; bf16 input is scaled by `mul` (a power of
// two, exact) before the conversion.
__device__ __forceinline__ f16x8 to_f16x8(i32x4 raw, bool is_bf16, float mul) {
  if (!is_bf16) return __builtin_bit_cast(f16x8, raw);
  const bf16x8 b = __builtin_bit_cast(bf16x8, raw);
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (f16)(from_bf16(b[i]) * mul);
  return r;
}

typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 hx4_t;
typedef __attribute__((address_space(3))) hx4_t lds_hx4;
typedef __attribute__((address_space(3))) f16 lds_f16;

// Transposed 4x16 read (see the header comment); p points into LDS.
__device__ __forceinline__ f16x4 lds_read_tr(const f16* p) {
  auto q = (lds_hx4*)((lds_f16*)(f16*)p);
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(q));
}

// XOR mask of the 8-byte chunks of tile row `key` (physical = stored ^ mask).
// Even, so the two halves of a score operand (stored chunks 2g, 2g+1) stay
// one aligned 16-byte read. The LDS serves a 16-byte read in four cycles of
// 16 lanes, grouped by lane >> 5 and the parity of lane bits 2..4, over 64
// four-byte banks; an 8-byte read in two cycles of 32 consecutive lanes over
// the 64 banks; an 8-byte write in four cycles of 16 consecutive lanes over
// 32 banks (lane groups found from the bank-conflict counter with two active
// lanes). With mask 4 (key & 7) + 2 (key & 1) (r >= 128) or 2 (key & 7)
// (r = 64, whose rows hold 16 chunks) and the staging order below, the
// score reads, the transposed reads and the staging writes each hit every
// bank of a cycle at most once (checked exhaustively on the host against
// that model).
template <int R>
__device__ __forceinline__ int swz_key(int key) {
  if constexpr (R == 64) return 2 * (key & 7);
  else return 4 * (key & 7) + 2 * (key & 1);
}

struct AttnCfg {
  int HG;  // heads per workgroup
  int BQ;  // query rows per workgroup (multiple of 16)
};

// Waves per workgroup.
__host__ __device__ constexpr int attn_waves(int r) { return r == 256 ? 8 : 4; }

// PH: the diagnostic copy. Each workgroup stamps the 100 MHz real-time clock
// at its start, once its latent queries are packed (the prologue), once the
// key loop's last products have landed, and after its last store; wave 0
// writes the four stamps to p.clk. Stamps follow register dependencies of
// the phase results, so the compiler cannot move a phase's work past them.
template <int R, int EPW, int DK, bool FUSED, typename CT, bool PH = false>
__global__ __launch_bounds__(64 * attn_waves(R), 2) void attn_mfma_kernel(AttnParams p, AttnCfg cfg) {
  constexpr int kAttnThreads = 64 * attn_waves(R);
  constexpr int BN = kAttnBN;        // keys per tile
  constexpr int NEB = EPW / 16;      // effective-row blocks per wave
  constexpr int NKS = R / 32;        // 32-wide steps over r
  constexpr int NRB = R / 16;        // 16-wide blocks over r
  constexpr int NLD = BN * R / 8 / kAttnThreads;  // 16-byte chunks per thread and tile
  static_assert(NLD >= 1, "tile too small for the staging map");
  constexpr bool C_BF16 = __is_same(CT, bf16);

  __shared__ __attribute__((aligned(16))) f16 Cs[2][BN * R];

  unsigned long long clk0 = 0, clk1 = 0, clk2 = 0;
  if constexpr (PH) clk0 = __builtin_amdgcn_s_memrealtime();
  const int tid = lid_x();
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;
  // Work item and head group from the workgroup's place in dispatch order:
  // workgroups go to the eight XCDs in turn, so in each run of 8 x nhg
  // workgroups the head groups of the same eight items sit eight apart, on
  // one XCD and close in time, and the latent tiles one group stages are
  // still in that XCD's L2 for the other. Items keep their (longest-first)
  // order; a last run with fewer than eight items is laid out the same way.
  const int nhg = (int)__builtin_amdgcn_readfirstlane(p.h / cfg.HG);
  int item, hgrp;
  {
    const int lin = gid_x() + p.items_cap * gid_y();
    const int full = (p.items_cap / 8) * 8;  // items in complete runs of eight
    if (lin < full * nhg) {
      item = (lin / (8 * nhg)) * 8 + lin % 8;
      hgrp = (lin / 8) % nhg;
    } else {
      const int r = lin - full * nhg, tail = p.items_cap - full;
      item = full + r % tail;
      hgrp = r / tail;
    }
  }
  const int h0 = hgrp * cfg.HG;
  // The item count and the work item come in one round trip of scalar
  // loads (constant address space; the workgroup index is below items_cap, so the item is in
  // bounds either way, and both were written by an earlier launch).
  // Workgroups past the count then leave with no vector load outstanding:
  // every launch's grid covers the largest layer's item bound, so late
  // layers have thousands of such workgroups.
  using cint = __attribute__((address_space(4))) const int;
  using ci32x4 = __attribute__((address_space(4))) const i32x4;
  const int nitems_raw = *(cint*)p.n_items;
  const i32x4 it = ((ci32x4*)p.items)[item];
  // the item is read here, with the count: one wait for both scalar loads
  // (the branch needs the count anyway), not a second round trip after it
  asm volatile("" ::"s"(it[0]), "s"(it[1]), "s"(it[2]), "s"(it[3]));
  if (item >= min(nitems_raw, p.items_cap)) return;
  constexpr int KD = DK / 32;
  constexpr int NRB_ = R / 16;
  constexpr int RBC = NRB_ * KD <= 16 ? NRB_ : 16 / KD;
  const int hd = p.h * DK;
  const int head_w = h0 + (wave * EPW) / cfg.BQ;  // every block of a wave: one head
  // W_uk in fragment order (attn_pack_weights): fragment (rb, kd) of the
  // wave's head is 512 values, this lane's eight at lane * 8
  const bf16* wp = FUSED ? (const bf16*)p.w_uk + (size_t)head_w * NRB_ * KD * 512 + lane * 8 : nullptr;
  bf16x8 wa0[FUSED ? RBC : 1][KD];
  if constexpr (FUSED) {
#pragma unroll
    for (int r = 0; r < RBC; ++r)
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) wa0[r][kd] = *(const bf16x8*)(wp + (size_t)(r * KD + kd) * 512);
  }
  const int qrow0 = it[0], kvb = it[1];
  const bool cand = it[2] < 0;
  const int nr = it[2] & 0x7fffffff;
  const int pos0 = it[3];
  const int max_pos = cand ? pos0 : pos0 + nr - 1;
  const int nkeys = max_pos + 1;
  const int ntiles = (nkeys + BN - 1) / BN;

  const float sc = p.scale * kLog2e;   // scores in log2 units
  const CT* Cg = (const CT*)p.c + (size_t)kvb * R;
  // Standalone path: C and the scaled latent queries enter fp16 as C 2^-ec
  // and q sc 2^-eq (powers of two: exact). Preferred is eq = -ec, where the
  // MFMAs give the scores themselves: ec (0 where possible) puts both
  // largest magnitudes in [2^-3, 2^14), below fp16's overflow (65504) and,
  // for all values within 2^-11 of the largest, above its subnormals. Where
  // no such ec exists (the two maxima's product below about 2^-6 or above
  // 2^28), each exponent puts its largest magnitude in [2^13, 2^14) and the
  // scores are scaled back by 2^(ec+eq) before the softmax. The output is
  // scaled by 2^ec at the end. For values that fp16 represents either way
  // the results equal the unscaled computation's. Exponents are clamped to
  // +-60 (all-zero inputs).
  int ec = 0, eq = 0;
  if constexpr (!FUSED) {
    if (p.amax) {
      const auto e_of = [](unsigned bits) {  // x < 2^e for finite x > 0
        return (int)((bits >> 23) & 0xff) - 126;
      };
      const int e_q = e_of(p.amax[0]), e_c = e_of(p.amax[1]);
      const int lo = max(e_c - 14, -2 - e_q), hi = min(14 - e_q, e_c + 2);
      if (lo <= hi) {
        ec = min(max(0, lo), hi);
        eq = -ec;
      } else {
        eq = min(max(-60, e_q - 14), 60);
        ec = min(max(-60, e_c - 14), 60);
      }
    }
  }
  const float c_pre = __builtin_ldexpf(1.f, -ec);       // applied to C on staging
  const float s_post = __builtin_ldexpf(1.f, ec + eq);  // undoes both on the scores
  const bool rescale = ec + eq != 0;

  // this lane's effective rows: one per block (head uniform per block)
  int head[NEB], qrow[NEB], pos[NEB];
  bool valid[NEB];
  int pmin = 0x7fffffff;
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) {
    const int e0 = wave * EPW + eb * 16;
    const int ql = e0 % cfg.BQ + l16;
    head[eb] = h0 + e0 / cfg.BQ;
    valid[eb] = ql < nr;
    const int qc = min(ql, nr - 1);
    qrow[eb] = qrow0 + qc;
    pos[eb] = cand ? pos0 : pos0 + qc;
    pmin = min(pmin, pos[eb]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) pmin = min(pmin, __shfl_xor(pmin, o, 64));

  // C tile staging: chunk idx covers one 16-byte piece j (r 8j .. 8j+7, i.e.
  // the 4-element r-chunks 2j and 2j+1) of a key row, stored at
  // attn_chunk_slot() of its 32-element block and XOR-swizzled. Chunks go to
  // rows in pairs: of each 2 R/8 consecutive chunks, groups of eight
  // alternate between the two rows, so the 16 lanes of one write cycle cover
  // eight pieces of each of two rows (distinct banks with the row masks).
  // Global offsets and LDS offsets (in halves) are fixed per thread.
  i32x4 ld[NLD];
  int ld_src[NLD], st_off[NLD], st_off2[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int idx = tid + i * kAttnThreads;
    const int w = idx % (R / 4);
    const int key = 2 * (idx / (R / 4)) + ((w >> 3) & 1), j = (w & 7) + 8 * (w >> 4);
    const int blk = 8 * (j / 4), kv = swz_key<R>(key);
    ld_src[i] = key * R + j * 8;
    st_off[i] = key * R + ((blk + attn_chunk_slot(2 * (j % 4))) ^ kv) * 4;
    st_off2[i] = key * R + ((blk + attn_chunk_slot(2 * (j % 4) + 1)) ^ kv) * 4;
  }
  // Chunk i of tile t. Keys past the end read the last key's row instead
  // (finite data; their scores are masked to -inf, so P = 0 there): no
  // branch, and a tile past the last one is a harmless load.
  auto load_chunk = [&](int t, int i) {
    const int key = min(t * BN + ld_src[i] / R, nkeys - 1);
    ld[i] = *(const i32x4*)(Cg + (size_t)key * R + ld_src[i] % R);
  };
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) load_chunk(t, i);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const f16x8 v = to_f16x8(ld[i], C_BF16, c_pre);
      *(f16x4*)&Cs[buf][st_off[i]] = f16x4{v[0], v[1], v[2], v[3]};
      *(f16x4*)&Cs[buf][st_off2[i]] = f16x4{v[4], v[5], v[6], v[7]};
    }
  };

  // the first key tile is in flight during the prologue; fused, it is
  // issued after the query rows (below), so that the W_uk products, which
  // wait for those rows, do not also wait for it (loads retire in order)
  if constexpr (!FUSED) load_tile(0);

  // latent queries, B operand of S^T, scaled into log2 units
  f16x8 qf[NEB][NKS];
  if constexpr (FUSED) {
    // q_lat^T[r][e] = sum_k W_uk[r][head*DK + k] * q[e][head*DK + k]. All
    // blocks of a wave belong to one head: each W_uk fragment is loaded once
    // per wave, in batches of at most 16 fragments all in flight together
    // (the first batch was issued at the start).
    static_assert(NRB_ == NRB, "r blocks");
    bf16x8 bq[NEB][KD];
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) {
      const bf16* qp = (const bf16*)p.q + (size_t)qrow[eb] * hd + head_w * DK + g * 8;
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) bq[eb][kd] = *(const bf16x8*)(qp + kd * 32);
    }
    load_tile(0);
    f32x4 acc[NEB][NRB];
#pragma unroll
    for (int rb0 = 0; rb0 < NRB; rb0 += RBC) {
      bf16x8 a[RBC][KD];
#pragma unroll
      for (int r = 0; r < RBC; ++r)
#pragma unroll
        for (int kd = 0; kd < KD; ++kd)
          a[r][kd] = rb0 == 0 ? wa0[r][kd]
                              : *(const bf16x8*)(wp + (size_t)((rb0 + r) * KD + kd) * 512);
#pragma unroll
      for (int r = 0; r < RBC; ++r)
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
          for (int kd = 0; kd < KD; ++kd)
            acc[eb][rb0 + r] = mfma_bf16(a[r][kd], bq[eb][kd],
                                         kd == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[eb][rb0 + r]);
    }
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[eb][ks] = pack8(acc[eb][2 * ks], acc[eb][2 * ks + 1], sc);
  } else {
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) {
      const bf16* qp = (const bf16*)p.q + ((size_t)qrow[eb] * p.h + head[eb]) * R + g * 4;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x4 lo = *(const bf16x4*)(qp + ks * 32);
        const bf16x4 hi = *(const bf16x4*)(qp + ks * 32 + 16);
        qf[eb][ks] = pack8(f32x4{from_bf16(lo[0]), from_bf16(lo[1]), from_bf16(lo[2]), from_bf16(lo[3])},
                           f32x4{from_bf16(hi[0]), from_bf16(hi[1]), from_bf16(hi[2]), from_bf16(hi[3])},
                           __builtin_ldexpf(sc, -eq));
      }
    }
  }

  if constexpr (PH) {
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) asm volatile("" ::"v"(qf[eb][ks]));
    clk1 = __builtin_amdgcn_s_memrealtime();
  }

  // S^T operand reads: row kb*16 + l16; lane group g takes the r-chunks g
  // and 4 + g of k step ks, stored side by side in chunks 2g, 2g + 1 of the
  // step's 32-element block: one 16-byte read. The mask depends on l16 only
  // and is below 32, so blocks 32 elements apart differ by a constant: four
  // lane-constant offsets cover every k step.
  constexpr int NOS = NKS < 4 ? NKS : 4;
  int offS[NOS];
  {
    const int kv = swz_key<R>(l16);
#pragma unroll
    for (int x = 0; x < NOS; ++x) offS[x] = l16 * R + ((8 * x + 2 * g) ^ kv) * 4;
  }
  auto off_s = [&](int ks) { return offS[ks % 4] + (ks / 4) * 128; };
  // transpose reads: rows kk*32 (+16) + 4g + (l16 >> 2), chunk rb*4 + (l16 & 3);
  // with the mask kt below 32, (4rb + j) ^ kt = 4 (rb ^ (kt >> 2)) + (j ^ (kt & 3))
  const int tk = 4 * g + (l16 >> 2);
  const int kt = swz_key<R>(tk);
  const int baseT = tk * R + 4 * ((l16 & 3) ^ (kt & 3));
  const int maskT = 16 * (kt >> 2);
  auto off_t = [&](int rb) { return baseT + (((rb % 8) * 16) ^ maskT) + (rb / 8) * 128; };

  f32x4 acc_o[NRB][NEB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) acc_o[rb][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NEB];
  f32x4 acc_l[NEB];   // every element holds the row sum of P
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) {
    m_run[eb] = -INFINITY;
    acc_l[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const f16x8 kOnes = f16x8{(f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f,
                            (f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f};

  // LDS operands run kPre steps ahead of the MFMAs that use them, so each
  // MFMA waits only for reads issued kPre steps earlier.
  constexpr int kPre = 3;
  constexpr int NSS = 4 * NKS;   // score steps (kb, ks), NEB MFMAs each
  constexpr int NPS = 2 * NRB;   // PV steps (rb, kk), NEB MFMAs each

  // A operand of score step i: rows kb*16.. of the tile, r = 32 ks.. (k
  // step outermost: an accumulator's next step comes 4 * NEB MFMAs later)
  auto rd_s = [&](const f16* cs, int i) {
    const f16* rowb = cs + (i % 4) * 16 * R;
    const int ks = i / 4;
    return *(const f16x8*)&rowb[off_s(ks)];
  };
  // A operand of PV step j: C^T rows rb*16.., keys 32 kk.. (transpose load;
  // key half outermost: an accumulator's second step comes NRB * NEB MFMAs
  // after its first)
  auto rd_pv = [&](const f16* cs, int j) {
    const int rb = j % NRB, kk = j / NRB;
    return cat(lds_read_tr(cs + kk * 32 * R + off_t(rb)),
               lds_read_tr(cs + (kk * 32 + 16) * R + off_t(rb)));
  };

  // S^T[key][e] of the 64-key tile in LDS buffer cs; the first k step of
  // each block starts from a zero accumulator
  // The global loads of tile tn are spread over the score steps, one chunk
  // every NSS / NLD steps, so that the waves of the CU do not issue them in
  // one burst after the barrier.
  constexpr int kLdEvery = NSS / NLD > 0 ? NSS / NLD : 1;
  // The accumulators start at -m_run (m0[eb], 0 on an item's first tile), so
  // the MFMAs produce s - m_run directly.
  auto scores = [&](const f16* cs, f32x4 (&sc)[4][NEB], int tn, const float (&m0)[NEB]) {
    f16x8 a[NSS];
#pragma unroll
    for (int i = 0; i < kPre; ++i) a[i] = rd_s(cs, i);
#pragma unroll
    for (int i = 0; i < NSS; ++i) {
      if (i % kLdEvery == 0 && i / kLdEvery < NLD) load_chunk(tn, i / kLdEvery);
      if (i + kPre < NSS) a[i + kPre] = rd_s(cs, i + kPre);
      const int kb = i % 4, ks = i / 4;
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
        sc[kb][eb] = mfma_f16(a[i], qf[eb][ks],
                              ks == 0 ? f32x4{-m0[eb], -m0[eb], -m0[eb], -m0[eb]} : sc[kb][eb]);
    }
#pragma unroll
    for (int i = NSS / kLdEvery; i < NLD; ++i) load_chunk(tn, i);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPre, 0);
#pragma unroll
    for (int i = 0; i < NSS; ++i) {
      if (i % kLdEvery == 0 && i / kLdEvery < NLD)
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load
      __builtin_amdgcn_sched_group_barrier(0x008, NEB, 0);
      if (i + kPre < NSS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // Online softmax of tile t's scores (this lane's column of S^T per block),
  // into the fp16 P^T operands. The running max only moves when a tile's max
  // exceeds it by more than kLazy (log2 units): P = exp2(s - m_run) then
  // stays <= 2^kLazy, exact enough in fp16, and the accumulators are
  // rescaled only on those tiles.
  // The scores arrive shifted by the running max (s - m_run; on the first
  // tile s itself, m_run then starts at that tile's max).
  auto softmax = [&](int t, f32x4 (&sc)[4][NEB], f16x8 (&pf)[2][NEB]) {
    const bool need_mask = t * BN + BN - 1 > pmin;
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) {
      if (need_mask) {
        // key t*BN + 16kb + 4g + v is masked past pos: compare the in-tile
        // offset 16kb + v (an inline constant) with one per-lane limit
        const int lim = pos[eb] - t * BN - g * 4;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (kb * 16 + v > lim) sc[kb][eb][v] = -INFINITY;
      }
      float mx = max16(sc[0][eb], sc[1][eb], sc[2][eb], sc[3][eb]);
      mx = max_across_groups(mx);
      if (t == 0) {
        // first tile: m_run = its max (the first key is never masked)
        m_run[eb] = mx;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sc[kb][eb] -= mx;
      } else {
        const bool bump = mx > kLazy;
        if (__ballot(bump)) {
          const float dm = bump ? mx : 0.f;
          const float alpha = fast_exp2(-dm);
          m_run[eb] += dm;
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) acc_o[rb][eb] *= alpha;
          acc_l[eb] *= alpha;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) sc[kb][eb] -= dm;
        }
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[kb][eb][v] = fast_exp2(sc[kb][eb][v]);
      pf[0][eb] = pack8(sc[0][eb], sc[1][eb]);
      pf[1][eb] = pack8(sc[2][eb], sc[3][eb]);
    }
  };

  // O^T[r][e] += sum over keys of C^T[r][key] * P^T[key][e]; the C^T operand
  // comes from the row-major tile through the transpose load, its first
  // kPre steps already in flight (pa). Row sums of the fp16 P are
  // accumulated on the matrix cores with an all-ones A operand.
  auto pv = [&](const f16* cs, f16x8 (&pa)[kPre], const f16x8 (&pf)[2][NEB]) {
    f16x8 a[NPS];
#pragma unroll
    for (int j = 0; j < kPre; ++j) a[j] = pa[j];
#pragma unroll
    for (int j = 0; j < NPS; ++j) {
      if (j + kPre < NPS) a[j + kPre] = rd_pv(cs, j + kPre);
      const int rb = j % NRB, kk = j / NRB;
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) acc_o[rb][eb] = mfma_f16(a[j], pf[kk][eb], acc_o[rb][eb]);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) acc_l[eb] = mfma_f16(kOnes, pf[kk][eb], acc_l[eb]);
#pragma unroll
    for (int j = 0; j < NPS; ++j) {
      if (j + kPre < NPS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, NEB, 1);
    }
  };

  // Double-buffered tiles: the next tile's global loads are in flight while
  // this one is computed; one barrier per tile.
  // (two iterations per loop trip, so that each LDS buffer's address is a
  // constant folded into the instructions' offsets)
  f32x4 st[4][NEB];
  store_tile(0);
  __syncthreads();
  auto iter = [&](int t, auto cur) {
    constexpr int CUR = decltype(cur)::value;
    const f16* cs = &Cs[CUR][0];
    float m0[NEB];
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) m0[eb] = t == 0 ? 0.f : m_run[eb];
    if constexpr (!FUSED) {
      if (rescale) {
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb) m0[eb] /= s_post;
      }
    }
    scores(cs, st, t + 1, m0);
    if constexpr (!FUSED) {
      if (rescale) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int eb = 0; eb < NEB; ++eb) st[kb][eb] *= s_post;
      }
    }
    f16x8 pa[kPre];
#pragma unroll
    for (int j = 0; j < kPre; ++j) pa[j] = rd_pv(cs, j);
    f16x8 pf[2][NEB];
    softmax(t, st, pf);
    pv(cs, pa, pf);
    if (t + 1 < ntiles) store_tile(CUR ^ 1);
    __syncthreads();
  };
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    iter(t, std::integral_constant<int, 0>{});
    iter(t + 1, std::integral_constant<int, 1>{});
  }
  if (t < ntiles) iter(t, std::integral_constant<int, 0>{});
  if constexpr (PH) {
    // a read of the last products' results waits for them to land
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) {
      float d;
      asm volatile("v_mov_b32 %0, %1" : "=v"(d) : "v"(acc_l[eb][0]));
      asm volatile("" ::"v"(d));
    }
    clk2 = __builtin_amdgcn_s_memrealtime();
  }

  if constexpr (FUSED) {
    // o^T[k][e] = sum_r W_uv^T[head][k][r] * o_lat^T[r][e]: the head's W_uv^T
    // fragments once per wave, in batches of at most 16 in flight together
    constexpr int NB = DK / 16;
    constexpr int NBC = NB * NKS <= 16 ? NB : 16 / NKS;
    // W_uv in fragment order (attn_pack_weights): fragment (nb, kk) of the
    // head is 512 values, this lane's eight at lane * 8
    const f16* wv = (const f16*)p.w_uv_t + (size_t)head[0] * NB * NKS * 512 + lane * 8;
    f16x8 ob[NEB][NKS];
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) {
      const float inv = 1.f / acc_l[eb][0];
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk)
        ob[eb][kk] = pack8(acc_o[2 * kk][eb], acc_o[2 * kk + 1][eb], inv);
    }
#pragma unroll
    for (int nb0 = 0; nb0 < NB; nb0 += NBC) {
      f16x8 w[NBC][NKS];
#pragma unroll
      for (int n = 0; n < NBC; ++n)
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          w[n][kk] = *(const f16x8*)(wv + (size_t)((nb0 + n) * NKS + kk) * 512);
        }
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) {
        bf16* op = (bf16*)p.out + (size_t)qrow[eb] * (p.h * DK) + head[eb] * DK + g * 4;
#pragma unroll
        for (int n = 0; n < NBC; ++n) {
          f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKS; ++kk) o = mfma_f16(w[n][kk], ob[eb][kk], o);
          if (valid[eb])
            *(bf16x4*)(op + (nb0 + n) * 16) = bf16x4{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
        }
      }
    }
  } else {
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) {
      if (!valid[eb]) continue;
      const float inv = __builtin_ldexpf(1.f / acc_l[eb][0], ec);
      const size_t orow = (size_t)qrow[eb] * p.h + head[eb];
      float* op = (float*)p.out + orow * R;
      // O^T rows come in stored order: rows 16 rb + 4g .. +3 hold the chunk
      // attn_slot_chunk(4 (rb % 2) + g) of the 32-element block rb / 2
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int col = 32 * (rb / 2) + 4 * attn_slot_chunk(4 * (rb % 2) + g);
        const f32x4 v = acc_o[rb][eb] * inv;
        *(f32x4*)(op + col) = v;
        if (p.out_bf16)
          *(bf16x4*)(p.out_bf16 + orow * R + col) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
      }
      if (p.lse && g == 0) p.lse[orow] = (m_run[eb] + log2f(acc_l[eb][0])) * kLn2;
    }
  }
  if constexpr (PH) {
    const unsigned long long clk3 = __builtin_amdgcn_s_memrealtime();
    if (tid == 0) {
      // the grid is items_cap workgroups wide
      unsigned long long* o = p.clk + ((size_t)gid_y() * p.items_cap + gid_x()) * 4;
      o[0] = clk0;
      o[1] = clk1;
      o[2] = clk2;
      o[3] = clk3;
    }
  }
}

// fp32: one wave per (query row, head).
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnParams p) {
  constexpr int RV = 4;  // r <= 256
  __shared__ float sq[256];
  __shared__ float sp[64];
  const int i = gid_x(), hh = gid_y(), lane = lid_x();
  if (i >= dev_count(p.M_dev, p.M_cap)) return;
  const int r = p.r;
  const int2 info = p.qinfo[i];
  const int kvb = info.x, nkeys = info.y + 1;
  const float* q = (const float*)p.q + ((size_t)i * p.h + hh) * r;
  const float* C = (const float*)p.c + (size_t)kvb * r;
  for (int k = lane; k < r; k += 64) sq[k] = q[k];
  __syncthreads();
  float m = -INFINITY, l = 0.f;
  float o[RV] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < nkeys; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j < nkeys) {
      const float* c = C + (size_t)j * r;
      float acc = 0.f;
      for (int k = 0; k < r; ++k) acc += sq[k] * c[k];
      s = acc * p.scale;
    }
    const float m_new = fmaxf(m, wave_max(s));
    const float alpha = expf(m - m_new);
    const float pj = j < nkeys ? expf(s - m_new) : 0.f;
    l = l * alpha + wave_sum(pj);
    m = m_new;
#pragma unroll
    for (int v = 0; v < RV; ++v) o[v] *= alpha;
    sp[lane] = pj;
    __syncthreads();
    const int nj = min(64, nkeys - j0);
    for (int jj = 0; jj < nj; ++jj) {
      const float w = sp[jj];
      const float* c = C + (size_t)(j0 + jj) * r;
#pragma unroll
      for (int v = 0; v < RV; ++v) {
        const int k = lane + 64 * v;
        if (k < r) o[v] += w * c[k];
      }
    }
    __syncthreads();
  }
  float* out = (float*)p.out + ((size_t)i * p.h + hh) * r;
  const float inv = 1.f / l;
#pragma unroll
  for (int v = 0; v < RV; ++v) {
    const int k = lane + 64 * v;
    if (k < r) out[k] = o[v] * inv;
  }
  if (p.lse && lane == 0) p.lse[(size_t)i * p.h + hh] = m + logf(l);
}

// Effective rows per wave: register budget of the O accumulator.
static int attn_epw(int r) { return r == 256 ? 16 : 32; }

static AttnCfg attn_cfg(int h, int r) {
  const int nw = attn_waves(r);
  const int eff = nw * attn_epw(r);  // effective rows per workgroup
  int hg = 1;  // power-of-two divisor of h, BQ >= 16, at most one head per wave
  while (h % (hg * 2) == 0 && eff / (hg * 2) >= 16 && hg * 2 <= nw) hg *= 2;
  return AttnCfg{hg, eff / hg};
}

int attn_bq(int h, int r) {
  if (r != 64 && r != 128 && r != 256) return 0;
  return attn_cfg(h, r).BQ;
}

bool attn_fused_supported(int h, int r, int dk) {
  return attn_bq(h, r) > 0 && (dk == 32 || dk == 64 || dk == 128);
}

template <int R, int EPW, int DK, bool FUSED, typename CT>
static void launch_mfma(const AttnParams& p, hipStream_t s) {
  const AttnCfg c = attn_cfg(p.h, R);
  dim3 grid(p.items_cap, p.h / c.HG);
  if (p.clk)
    hipLaunchKernelGGL((attn_mfma_kernel<R, EPW, DK, FUSED, CT, true>), grid,
                       dim3(64 * attn_waves(R)), 0, s, p, c);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<R, EPW, DK, FUSED, CT>), grid, dim3(64 * attn_waves(R)),
                       0, s, p, c);
}

template <int R, int EPW>
static hipError_t launch_r(const AttnParams& p, hipStream_t s) {
  if (!p.fused) {
    launch_mfma<R, EPW, 64, false, bf16>(p, s);
    return hipSuccess;
  }
  switch (p.dk) {
    case 32: launch_mfma<R, EPW, 32, true, f16>(p, s); break;
    case 64: launch_mfma<R, EPW, 64, true, f16>(p, s); break;
    case 128: launch_mfma<R, EPW, 128, true, f16>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

// Largest magnitude of bf16 arrays (float bits of non-negative values order
// like unsigned integers). Pass 1: a grid-stride max per thread (arrays on a
// 16-byte boundary read eight values per load, two loads in flight; the tail,
// and any other array, one value at a time), a block max through LDS, one
// plain store per array per block. Pass 2: one block folds the partials.
// Thousands of atomics on the same two words would serialise at the memory
// side and cost far more than the scan itself.
__device__ __forceinline__ float absmax8(float m, const bf16x8& v) {
#pragma unroll
  for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(from_bf16(v[k])));
  return m;
}
__device__ __forceinline__ float absmax_scan(const bf16* p, long long n, long long t,
                                             long long stride) {
  float m = 0.f;
  const long long n8 = ((size_t)p & 15) == 0 ? n / 8 : 0;
  const bf16x8* p8 = (const bf16x8*)p;
  long long i = t;
  for (; i + stride < n8; i += 2 * stride) {
    const bf16x8 v0 = p8[i], v1 = p8[i + stride];
    m = absmax8(absmax8(m, v0), v1);
  }
  if (i < n8) m = absmax8(m, p8[i]);
  for (long long j = n8 * 8 + t; j < n; j += stride) m = fmaxf(m, fabsf(from_bf16(p[j])));
  return m;
}
__global__ __launch_bounds__(256) void attn_absmax_kernel(const bf16* q, long long nq,
                                                          const bf16* c, long long nc,
                                                          unsigned* part) {
  __shared__ float red[2][4];
  const int tid = lid_x(), b = gid_x();
  const long long stride = (long long)__builtin_amdgcn_grid_size_x();
  const long long t = b * 256ll + tid;
  float mq = wave_max(absmax_scan(q, nq, t, stride));
  float mc = wave_max(absmax_scan(c, nc, t, stride));
  const int w = tid >> 6;
  if ((tid & 63) == 0) {
    red[0][w] = mq;
    red[1][w] = mc;
  }
  __syncthreads();
  if (tid < 2) {
    const float* r = red[tid];
    part[2 * b + tid] = __float_as_uint(fmaxf(fmaxf(r[0], r[1]), fmaxf(r[2], r[3])));
  }
}
__global__ __launch_bounds__(256) void attn_absmax_fold(const unsigned* part, int nb, float sc,
                                                        unsigned* amax) {
  __shared__ float red[2][4];
  const int tid = lid_x();
  float mq = 0.f, mc = 0.f;
  for (int b = tid; b < nb; b += 256) {
    mq = fmaxf(mq, __uint_as_float(part[2 * b]));
    mc = fmaxf(mc, __uint_as_float(part[2 * b + 1]));
  }
  mq = wave_max(mq);
  mc = wave_max(mc);
  const int w = tid >> 6;
  if ((tid & 63) == 0) {
    red[0][w] = mq;
    red[1][w] = mc;
  }
  __syncthreads();
  if (tid < 2) {
    const float* r = red[tid];
    const float m = fmaxf(fmaxf(r[0], r[1]), fmaxf(r[2], r[3]));
    amax[tid] = __float_as_uint(tid == 0 ? m * sc : m);
  }
}

hipError_t attn_absmax(const void* q, long long nq, const void* c, long long nc, float scale,
                       unsigned* amax, hipStream_t s) {
  // two 16-byte loads per thread and iteration at the least
  const long long n = std::max(nq, nc) / 16;
  const int blocks = (int)std::max<long long>(1, std::min<long long>((n + 255) / 256, kAbsmaxBlocks));
  unsigned* part = amax + 2;
  hipLaunchKernelGGL(attn_absmax_kernel, dim3(blocks), dim3(256), 0, s, (const bf16*)q, nq,
                     (const bf16*)c, nc, part);
  hipLaunchKernelGGL(attn_absmax_fold, dim3(1), dim3(256), 0, s, (const unsigned*)part, blocks,
                     scale * kLog2e, amax);
  return hipGetLastError();
}

// Fragment-order weight packing (attn_pack_weights). Output index o =
// ((head * nrb + rb) * nks + ks) * 512 + lane * 8 + e, with lane = 16 g + l16:
//   W_uk: row rb * 16 + l16 of r, column head * dk + 32 ks + 8 g + e (the
//         prologue's A operand: 16 rows of r, 8 consecutive k per lane);
//   W_uv: row rb * 16 + l16 of the head's dk, stored latent position 32 ks +
//         4 g + e (e < 4) or 32 ks + 16 + 4 g + (e - 4) (e >= 4), i.e. the
//         r-chunks g and 4 + g of the step, mapped back to the original r
//         index through attn_slot_chunk (the epilogue's A operand).
__global__ void attn_pack_uk_kernel(const bf16* W, int r, int h, int dk, bf16* out) {
  const long long n = (long long)r * h * dk;
  const int nks = dk / 32, nrb = r / 16;
  for (long long o = (long long)gid_x() * 256 + lid_x(); o < n;
       o += (long long)__builtin_amdgcn_grid_size_x()) {
    const int e = (int)(o & 7), lane = (int)((o >> 3) & 63);
    long long t = o >> 9;
    const int ks = (int)(t % nks);
    t /= nks;
    const int rb = (int)(t % nrb), head = (int)(t / nrb);
    const int row = rb * 16 + (lane & 15);
    const int col = head * dk + ks * 32 + (lane >> 4) * 8 + e;
    out[o] = W[(size_t)row * h * dk + col];
  }
}
__global__ void attn_pack_uv_kernel(const bf16* W, int r, int h, int dk, f16* out) {
  const long long n = (long long)r * h * dk;
  const int nks = r / 32, nrb = dk / 16;
  for (long long o = (long long)gid_x() * 256 + lid_x(); o < n;
       o += (long long)__builtin_amdgcn_grid_size_x()) {
    const int e = (int)(o & 7), lane = (int)((o >> 3) & 63);
    long long t = o >> 9;
    const int ks = (int)(t % nks);
    t /= nks;
    const int rb = (int)(t % nrb), head = (int)(t / nrb);
    const int k = rb * 16 + (lane & 15), g = lane >> 4;
    const int sp = ks * 32 + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));  // stored position
    const int rr = (sp & ~31) + 4 * attn_slot_chunk((sp & 31) >> 2) + (sp & 3);
    out[o] = (f16)from_bf16(W[(size_t)rr * h * dk + head * dk + k]);
  }
}

hipError_t attn_pack_weights(const void* W_uk, const void* W_uv, int r, int h, int dk,
                             void* uk_frag, void* uv_frag, hipStream_t s) {
  if (dk % 32 || r % 32 || r <= 0 || h <= 0) return hipErrorInvalidValue;
  const long long n = (long long)r * h * dk;
  const int blocks = (int)std::min<long long>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(attn_pack_uk_kernel, dim3(blocks), dim3(256), 0, s, (const bf16*)W_uk, r,
                     h, dk, (bf16*)uk_frag);
  hipLaunchKernelGGL(attn_pack_uv_kernel, dim3(blocks), dim3(256), 0, s, (const bf16*)W_uv, r,
                     h, dk, (f16*)uv_frag);
  return hipGetLastError();
}

// Phase diagnostics (attn_phases_enable): the stamp buffer of this thread's
// device and the records taken so far.
struct PhaseState {
  unsigned long long* buf = nullptr;
  int cap = 0;
  std::vector<double> rec;
};
static thread_local PhaseState t_phase;

hipError_t attn_phases_enable(int max_wg) {
  if (t_phase.buf) {
    hipError_t e = hipFree(t_phase.buf);
    t_phase.buf = nullptr;
    t_phase.cap = 0;
    if (e != hipSuccess) return e;
  }
  t_phase.rec.clear();
  if (max_wg <= 0) return hipSuccess;
  hipError_t e = hipMalloc(&t_phase.buf, (size_t)max_wg * 4 * sizeof(unsigned long long));
  if (e != hipSuccess) {
    t_phase.buf = nullptr;
    return e;
  }
  t_phase.cap = max_wg;
  return hipSuccess;
}

int attn_phases_read(double* out, int cap) {
  const int n = (int)(t_phase.rec.size() / kAttnPhaseFields);
  if (out)
    for (int i = 0; i < std::min(n, cap) * kAttnPhaseFields; ++i) out[i] = t_phase.rec[i];
  return n;
}

// The stamps of one instrumented launch, reduced on the host (clock ticks
// are 10 ns).
static hipError_t phase_collect(int nwg, hipStream_t s) {
  std::vector<unsigned long long> h((size_t)nwg * 4);
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(h.data(), t_phase.buf, h.size() * sizeof(h[0]), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  double wg = 0, pro = 0, loop = 0, epi = 0, longest = 0;
  unsigned long long first = ~0ull, last = 0;
  for (int i = 0; i < nwg; ++i) {
    const unsigned long long* c = &h[(size_t)i * 4];
    if (c[0] == 0) continue;  // workgroup without a work item
    wg += 1;
    pro += (double)(c[1] - c[0]);
    loop += (double)(c[2] - c[1]);
    epi += (double)(c[3] - c[2]);
    longest = std::max(longest, (double)(c[3] - c[0]));
    first = std::min(first, c[0]);
    last = std::max(last, c[3]);
  }
  const double us = 0.01;
  const double rec[kAttnPhaseFields] = {wg, pro * us, loop * us, epi * us,
                                        wg > 0 ? (double)(last - first) * us : 0.0, longest * us};
  t_phase.rec.insert(t_phase.rec.end(), rec, rec + kAttnPhaseFields);
  return hipSuccess;
}

hipError_t attention(const AttnParams& p, bool is_bf16, hipStream_t s) {
  if (p.M_cap <= 0) return hipSuccess;
  hipError_t e = hipSuccess;
  timing_begin(is_bf16 ? "attention_mfma" : "attention_f32", s);
  if (is_bf16) {
    if (p.items_cap > 0) {
      AttnParams q = p;
      int nwg = 0;
      if (t_phase.buf && (p.r == 64 || p.r == 128 || p.r == 256)) {
        nwg = p.items_cap * (p.h / attn_cfg(p.h, p.r).HG);
        if (nwg <= t_phase.cap) {
          q.clk = t_phase.buf;
          e = hipMemsetAsync(q.clk, 0, (size_t)nwg * 4 * sizeof(unsigned long long), s);
          if (e != hipSuccess) return e;
        }
      }
      switch (p.r) {
        case 64: e = launch_r<64, 32>(q, s); break;
        case 128: e = launch_r<128, 32>(q, s); break;
        case 256: e = launch_r<256, 16>(q, s); break;
        default: e = hipErrorInvalidValue;
      }
      if (e == hipSuccess && q.clk) {
        e = hipGetLastError();
        if (e == hipSuccess) e = phase_collect(nwg, s);
      }
    }
  } else {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(p.M_cap, p.h), dim3(64), 0, s, p);
  }
  timing_end(s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace llatte
