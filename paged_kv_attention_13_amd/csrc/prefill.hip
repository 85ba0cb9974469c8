// Causal prefill-chunk attention over a paged KV cache on gfx950 MFMA.
//
// What is computed: rows of an in-flight batch that carry a chunk of n new
// prompt tokens (chunked prefill mixed with decode rows in one pass:
// "TensorRT-LLM, in depth", aicassindra.com, section "In-flight batching and
// the scheduler").  The chunk's own K/V are already in the cache, so with L
// cached tokens the new token i (0-based) sits at position L - n + i and
// attends to every cached token up to and including itself ("How does
// TensorRT-LLM work", outcomeschool.com, section "Custom attention
// kernels": attention looks back at all earlier words).  Prefill is the
// compute-bound phase ("Introduction to TensorRT-LLM", dileepadev.github.io,
// section "The LLM Inference Bottleneck: Prefill vs. Decode"), so the two
// contractions run on the matrix cores.
//
// Tiling.  A workgroup owns one (row, kv head, block of query heads, query
// tile) unit -- or, when the launch has few units, one kv piece of it (the
// unit's tiles cut into up to 8 pieces whose partials the merge kernel
// combines); query tiles are dispatched longest first.  Each wave owns 32
// query positions of one query head.  Two workgroup shapes, chosen by the host
// plan: 4 waves staging 64-token kv tiles (two workgroups per CU), or 8 waves
// staging 128-token tiles (one per CU; each staged tile and each barrier serve
// twice the queries, for launches of prefill rows alone).
// K/V are staged through two LDS buffers in tiles gathered page by page
// through the block table: while tile j is computed, tile j+1 sits in the
// other buffer and tile j+2's global loads are in flight; one barrier per
// tile.  Each loading thread holds 4 consecutive tokens of 8 head-dim
// elements, so V^T is formed in registers (byte permutes) and written with
// 8-byte LDS stores.  FP8-E4M3 pools (the per-head-scaled codes of "TensorRT-LLM,
// in depth", section "Quantization: fewer bytes per weight and per cached token")
// load 8 codes per token and thread and widen them exactly to bf16 before the
// same staging; the K scale joins the softmax scale and the V scale multiplies
// the output.  Per 64-token sub-tile and wave:
//   S^T = K Q^T   : 32 x v_mfma_f32_16x16x32_bf16  (A = K rows from LDS,
//                   B = Q^T held in registers for the whole row)
//   online softmax in fp32 (log2 domain, lazy rescale as in the decode kernel;
//                   the scale folded into one fused multiply-add per weight)
//   O^T += V^T P^T: 32 x v_mfma_f32_16x16x32_bf16  (A = V^T from LDS,
//                   B = P^T straight from the S^T accumulators)
//   denominators  : v_dot2_f32_bf16 of each packed weight pair with (1, 1), so the
//                   sum takes the same bf16 weights as the product
// Computing S transposed puts each lane's probabilities exactly where the
// B operand of the second product wants them (same lane, same query
// column), so no cross-lane transpose is needed: within one 32-token k step
// the MFMA k index 8q + j (q = lane/16) stands for token 4q + j (j < 4) or
// 16 + 4q + (j - 4) (j >= 4), and V^T is read with the same mapping.
// Tiles after a wave's last query are skipped; the diagonal tiles are masked
// by select, never by multiplication, so NaN in unused pool slots (zeroed on
// the way into LDS) cannot leak.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "checks.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;        // 128
constexpr int ST = 64;             // kv tokens per computed sub-tile
constexpr int QW = 32;             // query positions per wave
constexpr int K_STRIDE = 272;      // bytes per K row in LDS (256 + 16 pad: conflict-free 16-B reads)
// Workgroup shape NW (4 or 8 waves): kv tiles of KT = 16 NW tokens are staged (each thread
// holds 4 tokens x 8 elements of K and of V), V^T rows of KT tokens plus 16 bytes of pad
template <int NW>
struct Shape {
  static constexpr int KT = 16 * NW;
  static constexpr int NT = NW * 64;
  static constexpr int V_STRIDE = 2 * KT + 16;
  static constexpr int CHUNKS = KT * kHeadDim * 2 / 16 / NT;   // 16-byte chunks per thread and tile: 4
};
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;
constexpr float kSlack = 8.0f;
constexpr int kTblLds = 1024;      // block-table entries staged in LDS (longer ranges read global memory)

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}



__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// c + lo(w) + hi(w) for a packed bf16 pair w (products by 1.0 are exact)
__device__ __forceinline__ float dot2_ones(uint32_t w, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3F803F80u), c,
                                         false);
}

// Eight E4M3 codes (FP8 pools) widened to eight bf16 values, exactly: every E4M3 value is a
// bf16 value.  The pool's per-head scales are applied outside the products.
__device__ __forceinline__ u32x4 widen_e4m3x8(u32x2 w) {
  auto pair = [](uint32_t c, bool hi) {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, false));
  };
  return u32x4{pair(w[0], false), pair(w[0], true), pair(w[1], false), pair(w[1], true)};
}

template <bool OUT_BF16>
__device__ __forceinline__ void store4(void *out, size_t idx, f32x4 v) {
  if constexpr (OUT_BF16) {
    u32x2 w = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    *reinterpret_cast<u32x2 *>(static_cast<__bf16 *>(out) + idx) = w;
  } else {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + idx) = v;
  }
}

// Piece length (in kv tiles) of a split launch, the same in every wave of the prefill
// kernel and of its merge: at least ceil(longest row's tiles / splits), so the launch's
// `splits` pieces per unit always cover the unit, and at least the average work per
// resident workgroup, so that a launch whose units are already balanced is not cut
// further.  The work estimate per row takes its query tiles' mean visible length.
template <int QB, int KT>
__device__ int piece_tiles(const PrefillLaunch &p, int lane, int units_per_qtile) {
  if (p.splits <= 1) return 1 << 30;
  int mx = 0;
  int64_t work = 0;                        // tile visits, x 2 (half tiles are counted)
  for (int r0 = 0; r0 < p.num_rows; r0 += 64) {
    const int r = p.first_row + r0 + lane;
    if (r0 + lane < p.num_rows) {
      const int L = checked_len(p.seq_lens[r], p.max_len, p.check_flags);
      const int n = checked_qlen(p.q_start_loc[r + 1] - p.q_start_loc[r], L, p.check_flags);
      const int nq = (n + QB - 1) / QB;
      mx = max(mx, (L + KT - 1) / KT);
      work += (int64_t)nq * ((2 * (int64_t)(L - n) + n + QB) / KT + 2);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mx = max(mx, __shfl_xor(mx, off));
    work += __shfl_xor(work, off);
  }
  const int64_t total = work * units_per_qtile / 2;
  const int64_t slots = p.resident_slots;
  const int balanced = (int)((total + slots - 1) / slots);
  return max(max((mx + p.splits - 1) / p.splits, balanced), kPrefillMinChunkTiles);
}

// The unit of one prefill workgroup.  Workgroups are dispatched to the 8 XCDs round-robin
// (id mod 8), each XCD with its own L2; when the (kv head, head block) pairs come in
// multiples of 8, all workgroups of a pair go to one XCD, so that XCD's L2 serves the K/V
// tiles every query tile of the pair re-reads (8 kv heads: one per XCD).  Then the query
// tile, the longest (last in the row) dispatched first, then (piece, row) with the piece
// slowest, so consecutive workgroups are different units rather than pieces of one unit
// that may have no work.
struct PrefillUnit {
  int qt;          // query tile
  int piece;       // kv piece
  int row_local;   // prefill row, from first_row
  int g;           // kv head
  int hb;          // head block within the kv head
  int hbk;         // (kv head, head block) pair
};

__device__ __forceinline__ PrefillUnit prefill_unit(const PrefillLaunch &p, int hblocks) {
  const int U = p.num_kv_heads * hblocks;
  const int id = (int)blockIdx.x;
  int hbk, rest;
  if (U % 8 == 0) {
    const int k = id >> 3;
    hbk = (id & 7) + 8 * (k % (U >> 3));
    rest = k / (U >> 3);
  } else {
    hbk = id % U;
    rest = id / U;
  }
  PrefillUnit u;
  u.qt = p.max_qtiles - 1 - rest % p.max_qtiles;
  const int zz = rest / p.max_qtiles;
  u.piece = zz / p.num_rows;
  u.row_local = zz % p.num_rows;
  u.g = hbk / hblocks;
  u.hb = hbk % hblocks;
  u.hbk = hbk;
  return u;
}

// HB: query heads per workgroup (1, 2 or 4); the 4 waves cover HB heads x (4/HB) query sub-tiles.
// FP8: E4M3 pools, widened to bf16 as each tile is staged; k_scale[g] joins the softmax scale
// and v_scale[g] multiplies the output (or the piece's unnormalised output).
template <int HB, bool OUT_BF16, int NWP, bool FP8>
__global__ __launch_bounds__(NWP * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillLaunch p) {
  constexpr int QSUB = NWP / HB;
  constexpr int QB = QW * QSUB;            // queries per workgroup
  constexpr int KT = Shape<NWP>::KT;
  constexpr int NTP = Shape<NWP>::NT;
  constexpr int V_STRIDE = Shape<NWP>::V_STRIDE;
  constexpr int CHUNKS = Shape<NWP>::CHUNKS;

  // two LDS buffers: tile j is computed from buffer j&1 while tile j+1 is stored to the other
  __shared__ __attribute__((aligned(16))) char s_k[2][KT * K_STRIDE];
  __shared__ __attribute__((aligned(16))) char s_vt[2][D * V_STRIDE];
  __shared__ int s_tbl[kTblLds];           // block-table entries of the pages this workgroup visits

  const int Hq = p.num_q_heads;
  const int Hkv = p.num_kv_heads;
  const int G = Hq / Hkv;
  const int hblocks = G / HB;              // head blocks per kv head
  const int U = Hkv * hblocks;             // (kv head, head block) pairs
  const PrefillUnit un = prefill_unit(p, hblocks);
  const int qt = un.qt;
  const int piece = un.piece;
  const int row_local = un.row_local;
  const int g = un.g;
  const int hb = un.hb;
  const int hbk = un.hbk;
  const int row = p.first_row + row_local;
  const int q_begin = p.q_start_loc[row];
  const int n = p.q_start_loc[row + 1] - q_begin;
  // a split launch's piece length: its loads go out beside the row's metadata, before any
  // exit, so that the two share one round trip (chunk of 256 after 8,192: 66.5 -> 64.9 us)
  const int C = p.splits > 1 ? __builtin_amdgcn_readfirstlane(piece_tiles<QB, KT>(p, threadIdx.x & 63, Hkv * hblocks))
                             : 1 << 30;
  if (qt * QB >= n) return;                // whole workgroup: past this row's chunk
  const int L = p.seq_lens[row];
  const int prior = L - n;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 15;                // column (query) / row-in-tile index
  const int lg = lane >> 4;                // lane group 0..3
  const int h = g * G + hb * HB + (wave % HB);
  const int q0 = qt * QB + (wave / HB) * QW;              // first query of this wave
  const int blk_last_q = min(qt * QB + QB, n) - 1;
  const int kv_end = prior + blk_last_q + 1;              // tokens the unit visits
  const int ntile = (kv_end + KT - 1) / KT;
  // this workgroup's piece of the unit: tiles [j_begin, j_end)
  const int j_begin = piece * C;
  if (j_begin >= ntile) return;            // whole workgroup: the unit has fewer pieces
  const int j_end = min(ntile, j_begin + C);
  const bool split = ntile > C;
  const int wave_last_pos = prior + min(q0 + QW, n) - 1;  // last position among this wave's queries
  const bool wave_active = q0 < n;

  // Q^T as the B operand: qb[qtile][ks] holds Q[q0 + 16*qtile + lq][32*ks + 8*lg .. +8]
  u32x4 qb[2][4];
#pragma unroll
  for (int qt2 = 0; qt2 < 2; ++qt2) {
    const int qi = q0 + 16 * qt2 + lq;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (qi < n) {
        const __bf16 *qp = static_cast<const __bf16 *>(p.q) + ((size_t)(q_begin + qi) * Hq + h) * D +
                           32 * ks + 8 * lg;
        qb[qt2][ks] = *reinterpret_cast<const u32x4 *>(qp);
      } else {
        qb[qt2][ks] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  float v_scale = 1.f;
  float qk_scale = p.scale * kLog2e;
  if constexpr (FP8) {
    qk_scale *= p.k_scale[g];
    v_scale = p.v_scale[g];
  }

  // cooperative tile loads: thread -> 4 consecutive tokens 4*tq .. 4*tq+3, elements 8*dg .. 8*dg+7,
  // so each load instruction of a wave covers four whole 256-byte token rows
  const int bs = p.block_size;
  const int log2bs = __builtin_ctz(bs);
  const int32_t *trow = p.block_table + (size_t)row * p.max_blocks_per_seq;
  constexpr int EBY = FP8 ? 1 : 2;           // bytes per cached element
  const size_t page_elems = (size_t)bs * D;
  const char *kpool = static_cast<const char *>(p.k_pool) + (size_t)g * page_elems * EBY;
  const char *vpool = static_cast<const char *>(p.v_pool) + (size_t)g * page_elems * EBY;
  const size_t phys_stride = (size_t)Hkv * page_elems;
  // thread -> (token quad c_tq, 16-byte chunk c_dg).  The quad index is a bit permutation of
  // tid >> 4 chosen so that the two 16-lane halves of each 32-lane half-wave take quads that
  // differ in bit 2, i.e. fill opposite 8-byte halves of the V^T pairs below: their 8-byte
  // stores then meet different banks instead of sharing one 16-byte slot
  const int c_dg = tid & 15;
  const int c_u = tid >> 4;                 // 4 * wave + (lane >> 4)
  const int c_tq = ((c_u >> 3) << 3) | ((c_u & 1) << 2) | (((c_u >> 1) & 1) << 1) | ((c_u >> 2) & 1);

  // stage the block-table entries of every page the loads below can touch in LDS, so the
  // pipelined loads depend on one LDS read instead of a global load.  The loads cover
  // every token < L of the workgroup's tiles, which can run past kv_end in the last tile.
  const int page0 = (j_begin * KT) >> log2bs;
  const int npages = ((min(L, j_end * KT) + bs - 1) >> log2bs) - page0;
  const bool tbl_in_lds = npages <= kTblLds;
  if (tbl_in_lds)
    for (int i = tid; i < npages; i += NTP) s_tbl[i] = trow[page0 + i];
  __syncthreads();

  // the next tile in registers until its LDS stores: 8 bf16 elements per register quad, or for
  // FP8 pools the raw codes (widened only by the stores, so that no load is waited for early)
  u32x4 rk[CHUNKS], rv[CHUNKS];
  u32x2 ck[CHUNKS], cv[CHUNKS];
  auto load_regs = [&](int j) {
    // the 4 tokens share one page (4 | bs)
    const int t_first = j * KT + 4 * c_tq;
    const bool any = t_first < L;
    const int page = t_first >> log2bs;
    const int phys = !any ? 0 : (tbl_in_lds ? s_tbl[page - page0] : trow[page]);
    const size_t base = (size_t)phys * phys_stride + (size_t)(t_first & (bs - 1)) * D + 8 * c_dg;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      if constexpr (FP8) {
        if (t_first + i < L) {
          ck[i] = *reinterpret_cast<const u32x2 *>(kpool + base + i * D);
          cv[i] = *reinterpret_cast<const u32x2 *>(vpool + base + i * D);
        } else {
          ck[i] = u32x2{0u, 0u};             // code 0 is +0
          cv[i] = u32x2{0u, 0u};
        }
      } else {
        if (t_first + i < L) {
          rk[i] = *reinterpret_cast<const u32x4 *>(kpool + 2 * (base + i * D));
          rv[i] = *reinterpret_cast<const u32x4 *>(vpool + 2 * (base + i * D));
        } else {
          rk[i] = u32x4{0u, 0u, 0u, 0u};
          rv[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto store_lds = [&](int buf) {
    char *kb = s_k[buf];
    char *vb = s_vt[buf];
    u32x4 tk[CHUNKS], tv[CHUNKS];
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      if constexpr (FP8) {
        tk[i] = widen_e4m3x8(ck[i]);
        tv[i] = widen_e4m3x8(cv[i]);
      } else {
        tk[i] = rk[i];
        tv[i] = rv[i];
      }
    }
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i)
      *reinterpret_cast<u32x4 *>(kb + (4 * c_tq + i) * K_STRIDE + c_dg * 16) = tk[i];
    // V^T: for element d = 8*dg + e, the 4 tokens 4*tq .. +3 become one 8-byte half of row d's
    // 16-byte pair 4*(tq >> 3) + (tq & 3) (low half for tq & 4 clear): a pair holds an MFMA
    // operand's 8 k slots in order, so each operand is one 16-byte read (gfx950 serves
    // 16-byte LDS reads at twice the bytes per clock of 8-byte ones).  Pairs are XOR-ed with
    // (d >> 4) & 7, the operand's 16-row block: conflict-free operand reads, two-way
    // conflicted stores under a 64-bank model.
    // (128-token tiles: the same within each 64-token half of the row)
    const int cq = KT == 64 ? c_tq : c_tq & 15;
    const int vgrp = (KT == 64 ? 0 : 128 * (c_tq >> 4)) + 16 * ((4 * (cq >> 3) + (cq & 3)) ^ ((c_dg >> 1) & 7)) +
                     8 * ((cq >> 2) & 1);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo01 = __builtin_amdgcn_perm(tv[1][w], tv[0][w], 0x05040100u);   // e=2w:   t0 t1
      const uint32_t lo23 = __builtin_amdgcn_perm(tv[3][w], tv[2][w], 0x05040100u);   //         t2 t3
      const uint32_t hi01 = __builtin_amdgcn_perm(tv[1][w], tv[0][w], 0x07060302u);   // e=2w+1: t0 t1
      const uint32_t hi23 = __builtin_amdgcn_perm(tv[3][w], tv[2][w], 0x07060302u);
      *reinterpret_cast<u32x2 *>(vb + (8 * c_dg + 2 * w) * V_STRIDE + vgrp) = u32x2{lo01, lo23};
      *reinterpret_cast<u32x2 *>(vb + (8 * c_dg + 2 * w + 1) * V_STRIDE + vgrp) = u32x2{hi01, hi23};
    }
  };

  float m[2] = {kNegBig, kNegBig};        // running max of the scaled logits (log2 units)
  f32x4 o[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int qt2 = 0; qt2 < 2; ++qt2) o[dt][qt2] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lsum[2] = {0.f, 0.f};              // per-lane partial of the softmax denominator

  // lane parts of the V^T operand addresses: row lq of a 16-row block, pair lg ^ i (see the
  // product below)
  int vt_lane[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) vt_lane[i] = lq * V_STRIDE + 16 * (lg ^ i);

  // sub-tile hs (64 tokens) of staged tile j
  auto compute = [&](int j, int hs) {
    const char *kb = s_k[j & 1] + ST * hs * K_STRIDE;
    const char *vb = s_vt[j & 1] + 2 * ST * hs;
    const int kv0 = j * KT + ST * hs;
    // ---- S^T = K Q^T ----
    f32x4 s[4][2];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int qt2 = 0; qt2 < 2; ++qt2) s[tt][qt2] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K fragments are read one k step ahead of the MFMAs that use them (the scheduling
    // barriers keep the compiler from sinking the LDS reads next to their uses)
    u32x4 ka[2][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      ka[0][tt] = *reinterpret_cast<const u32x4 *>(kb + (16 * tt + lq) * K_STRIDE + (8 * lg) * 2);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          ka[(ks + 1) & 1][tt] = *reinterpret_cast<const u32x4 *>(
              kb + (16 * tt + lq) * K_STRIDE + (32 * (ks + 1) + 8 * lg) * 2);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int qt2 = 0; qt2 < 2; ++qt2) s[tt][qt2] = mfma(ka[ks & 1][tt], qb[qt2][ks], s[tt][qt2]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- causal mask, online softmax (per query column) ----
    // the max is taken over the raw scores (the scale is positive) and the scale enters each
    // weight through one fused multiply-add: p = 2^(s * scale * log2(e) - m)
    const bool diag = kv0 + ST - 1 > prior + q0;          // some element may be masked
    float tmax[2];
#pragma unroll
    for (int qt2 = 0; qt2 < 2; ++qt2) {
      if (diag) {
        // element (tt, i) is token kv0 + 16 tt + 4 lg + i: visible up to the column's position,
        // i.e. while 16 tt + i <= lim (compared with constants: no per-element index arithmetic)
        const int lim = prior + min(q0 + 16 * qt2 + lq, n - 1) - kv0 - 4 * lg;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[tt][qt2][i] = 16 * tt + i <= lim ? s[tt][qt2][i] : -__builtin_inff();
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[tt][qt2][i]);
      tmax[qt2] = mx * qk_scale;           // this lane's part of the column max
    }
    // A column needs rescaling when its max exceeds m by more than the slack, i.e. when
    // one of its lanes' parts does: the vote needs no cross-lane reduction, which the
    // rare rescale path then does (same values as reducing first)
    const bool need = tmax[0] > m[0] + kSlack || tmax[1] > m[1] + kSlack;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int qt2 = 0; qt2 < 2; ++qt2) {
        tmax[qt2] = fmaxf(tmax[qt2], __shfl_xor(tmax[qt2], 16));
        tmax[qt2] = fmaxf(tmax[qt2], __shfl_xor(tmax[qt2], 32));
        const float mn = fmaxf(m[qt2], tmax[qt2]);
        const float a = fast_exp2(m[qt2] - mn);
        m[qt2] = mn;
        lsum[qt2] *= a;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt][qt2] *= a;
      }
    }
    // P^T as the B operand of the second product: pb[qtile][ks2]
    u32x4 pb[2][2];
#pragma unroll
    for (int qt2 = 0; qt2 < 2; ++qt2)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = fast_exp2(__builtin_fmaf(s[2 * ks2][qt2][i], qk_scale, -m[qt2]));
          pv[4 + i] = fast_exp2(__builtin_fmaf(s[2 * ks2 + 1][qt2][i], qk_scale, -m[qt2]));
        }
        pb[qt2][ks2] = u32x4{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                             pack_bf16(pv[6], pv[7])};
        // the denominator sums the same bf16-rounded weights the product uses
#pragma unroll
        for (int w = 0; w < 4; ++w) lsum[qt2] = dot2_ones(pb[qt2][ks2][w], lsum[qt2]);
      }
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        // row d = 16 dt + lq of V^T, pair (4 ks2 + lg) ^ dt: a lane base (four variants, by
        // dt & 3) plus an immediate
        const u32x4 a = *reinterpret_cast<const u32x4 *>(vb + vt_lane[dt & 3] + 16 * dt * V_STRIDE +
                                                          64 * (ks2 ^ (dt >> 2)));
#pragma unroll
        for (int qt2 = 0; qt2 < 2; ++qt2) o[dt][qt2] = mfma(a, pb[qt2][ks2], o[dt][qt2]);
      }
    }
  };

  // pipeline: tile j is computed from LDS while tile j+1 waits in LDS and tile j+2's
  // global loads are in flight; one barrier per tile
  load_regs(j_begin);
  store_lds(j_begin & 1);
  if (j_begin + 1 < j_end) load_regs(j_begin + 1);
  __syncthreads();
  // The next tile goes to LDS (and the global loads of the one after are issued) after this
  // tile's computation -- in the 8-wave shape between its two sub-tiles, which gives those loads
  // half a tile more lead and moves the staging stores away from the barrier (the 8,192-token
  // prompt 520 -> 507 us; staging first in half of the waves gave 510 us).  The buffer written
  // was last read before the previous barrier.
  auto stage = [&](int j) {
    if (j + 1 < j_end) {
      store_lds((j + 1) & 1);
      if (j + 2 < j_end) load_regs(j + 2);
    }
  };
  for (int j = j_begin; j < j_end; ++j) {
    // sub-tiles past a wave's last query are fully masked (written out without a loop: the
    // 4-wave shape's registers come out 15 higher through a one-trip loop)
    if (wave_active && j * KT <= wave_last_pos) compute(j, 0);
    if constexpr (KT == 2 * ST) {
      stage(j);
      if (wave_active && j * KT + ST <= wave_last_pos) compute(j, 1);
    } else {
      stage(j);
    }
    __syncthreads();
  }

  if (!wave_active) return;
  // denominator: sum the four lane groups of each query column
#pragma unroll
  for (int qt2 = 0; qt2 < 2; ++qt2) {
    lsum[qt2] += __shfl_xor(lsum[qt2], 16);
    lsum[qt2] += __shfl_xor(lsum[qt2], 32);
  }
  if (split) {
    // a piece of a cut unit: the unnormalised sum, the running max and the sum of
    // weights go to the piece's slot (a wave that saw no tile of this piece leaves
    // max = -1e30, sum = 0, zeros); the merge kernel combines the pieces
    const size_t slot = ((((size_t)row_local * U + hbk) * p.max_qtiles + qt) * p.splits + piece) * NWP + wave;
    float *po = p.part_o + slot * (QW * D);
    float *pml = p.part_ml + slot * (QW * 2);
#pragma unroll
    for (int qt2 = 0; qt2 < 2; ++qt2) {
      const int ql = 16 * qt2 + lq;
      if (q0 + ql >= n) continue;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<f32x4 *>(po + ql * D + 16 * dt + 4 * lg) = FP8 ? o[dt][qt2] * v_scale : o[dt][qt2];
      if (lg == 0) *reinterpret_cast<float2 *>(pml + 2 * ql) = float2{m[qt2], lsum[qt2]};
    }
    return;
  }
#pragma unroll
  for (int qt2 = 0; qt2 < 2; ++qt2) {
    const int qi = q0 + 16 * qt2 + lq;
    if (qi >= n) continue;
    const size_t base = ((size_t)(q_begin + qi) * Hq + h) * D;
    // o / l as o * (1/l) with one residual correction (l >= 1: the running max is at most
    // 8 below the column's max, so no special values); o = c * l gives exactly c
    const float l = lsum[qt2];
    const float r = __builtin_amdgcn_rcpf(l);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      f32x4 v = o[dt][qt2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float q = v[i] * r;
        v[i] = __builtin_fmaf(__builtin_fmaf(-l, q, v[i]), r, q);
        if constexpr (FP8) v[i] *= v_scale;
      }
      store4<OUT_BF16>(p.out, base + 16 * dt + 4 * lg, v);
    }
  }
}

// Merge of the pieces of every cut unit (same grid as the prefill kernel without the
// piece index): out = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p with M = max_p m_p,
// the rescaling identity of the online softmax applied across pieces.  x = (query tile,
// quarter): a workgroup merges 8 of the 32 query positions of each of the unit's waves,
// so four times as many workgroups keep loads in flight.  Lane c < 8 of a wave first
// forms the normalised piece weights of its c-th position; then lane pairs take one
// position each, 4 consecutive head-dim elements per lane, all four steps unrolled.
template <int HB, bool OUT_BF16, int NWP>
__global__ __launch_bounds__(NWP * 64) void prefill_merge_kernel(PrefillLaunch p) {
  constexpr int KT = Shape<NWP>::KT;
  constexpr int QSUB = NWP / HB;
  constexpr int QB = QW * QSUB;
  const int Hq = p.num_q_heads;
  const int Hkv = p.num_kv_heads;
  const int G = Hq / Hkv;
  const int hblocks = G / HB;
  constexpr int QM = QW / 4;               // positions per wave and workgroup
  const int qt = p.max_qtiles - 1 - (int)blockIdx.x / 4;
  const int quarter = (int)blockIdx.x % 4;
  const int g = blockIdx.y / hblocks;
  const int hb = blockIdx.y % hblocks;
  const int row = p.first_row + blockIdx.z;
  // metadata and piece length in one round trip (their loads issued before any exit)
  const int q_begin = p.q_start_loc[row];
  const int n = p.q_start_loc[row + 1] - q_begin;
  const int L = p.seq_lens[row];
  const int tid = threadIdx.x;
  const int C = __builtin_amdgcn_readfirstlane(piece_tiles<QB, KT>(p, tid & 63, Hkv * hblocks));
  if (qt * QB >= n) return;
  const int prior = L - n;
  const int ntile = (prior + min(qt * QB + QB, n) + KT - 1) / KT;
  if (ntile <= C) return;                  // the prefill kernel stored this unit itself
  const int npieces = (ntile + C - 1) / C;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = g * G + hb * HB + (wave % HB);
  const int q0 = qt * QB + (wave / HB) * QW;
  if (q0 >= n) return;
  const int qm0 = quarter * QM;            // first position (within the wave's 32) merged here
  const int q_lim = min(QW, n - q0);
  if (qm0 >= q_lim) return;
  const size_t slot0 = ((((size_t)blockIdx.z * gridDim.y + blockIdx.y) * p.max_qtiles + qt) * p.splits) * NWP + wave;
  const float *__restrict__ po = p.part_o + slot0 * (QW * D);
  const float *__restrict__ pml = p.part_ml + slot0 * (QW * 2);
  constexpr size_t kPieceO = (size_t)NWP * QW * D;       // floats between pieces of one slot
  constexpr size_t kPieceML = (size_t)NWP * QW * 2;
  // every load of the merge (the pieces' outputs and their (max, sum) pairs) is issued
  // before any use: one round trip
  const int half = lane >> 5;
  const int d = 4 * (lane & 31);
  f32x4 pv[QM / 2][kPrefillMaxSplits];
#pragma unroll
  for (int qq = 0; qq < QM; qq += 2) {
    const int ql = qm0 + qq + half;
#pragma unroll
    for (int s = 0; s < kPrefillMaxSplits; ++s)
      pv[qq / 2][s] = (s < npieces && ql < q_lim) ? *reinterpret_cast<const f32x4 *>(po + s * kPieceO + ql * D + d)
                                                  : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float wt[kPrefillMaxSplits];
  {
    const int c = qm0 + (lane & (QM - 1));
    float mp[kPrefillMaxSplits], lp[kPrefillMaxSplits];
    float M = -__builtin_inff();
#pragma unroll
    for (int s = 0; s < kPrefillMaxSplits; ++s) {
      mp[s] = -__builtin_inff();
      lp[s] = 0.f;
      if (s < npieces && c < q_lim) {
        const float2 ml = *reinterpret_cast<const float2 *>(pml + s * kPieceML + 2 * c);
        mp[s] = ml.x;
        lp[s] = ml.y;
      }
      M = fmaxf(M, mp[s]);
    }
    float den = 0.f;
#pragma unroll
    for (int s = 0; s < kPrefillMaxSplits; ++s) {
      wt[s] = s < npieces && c < q_lim ? fast_exp2(mp[s] - M) : 0.f;
      den += wt[s] * lp[s];
    }
#pragma unroll
    for (int s = 0; s < kPrefillMaxSplits; ++s) wt[s] = c < q_lim ? wt[s] / den : 0.f;
  }
#pragma unroll
  for (int qq = 0; qq < QM; qq += 2) {
    const int ql = qm0 + qq + half;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kPrefillMaxSplits; ++s) {
      const float w = __shfl(wt[s], qq + half);
      if (s < npieces && ql < q_lim) acc += w * pv[qq / 2][s];
    }
    if (ql < q_lim) store4<OUT_BF16>(p.out, ((size_t)(q_begin + q0 + ql) * Hq + h) * D + d, acc);
  }
}

template <int HB, int NW>
int launch_shape(const PrefillLaunch &P, hipStream_t st) {
  constexpr int QB = QW * (NW / HB);
  const int G = P.num_q_heads / P.num_kv_heads;
  if (P.max_qtiles != (P.max_q_len + QB - 1) / QB || P.splits < 1 || P.splits > kPrefillMaxSplits ||
      (P.splits > 1 && (!P.part_o || !P.part_ml)))
    return (int)hipErrorInvalidValue;
  // one-dimensional grid of (query tiles) x (kv head, head block) x (rows x pieces); the
  // kernel decodes its unit from the workgroup id (prefill_unit)
  const int64_t nwg = (int64_t)P.max_qtiles * P.num_kv_heads * (G / HB) * P.num_rows * P.splits;
  if (nwg > INT32_MAX) return (int)hipErrorInvalidValue;
  dim3 grid((unsigned)nwg);
  if (P.kv_dtype == PA_FP8_E4M3) {
    if (!P.k_scale || !P.v_scale) return (int)hipErrorInvalidValue;
    if (P.out_dtype == PA_BF16)
      hipLaunchKernelGGL((prefill_kernel<HB, true, NW, true>), grid, dim3(NW * 64), 0, st, P);
    else
      hipLaunchKernelGGL((prefill_kernel<HB, false, NW, true>), grid, dim3(NW * 64), 0, st, P);
  } else if (P.kv_dtype == PA_BF16) {
    if (P.out_dtype == PA_BF16)
      hipLaunchKernelGGL((prefill_kernel<HB, true, NW, false>), grid, dim3(NW * 64), 0, st, P);
    else
      hipLaunchKernelGGL((prefill_kernel<HB, false, NW, false>), grid, dim3(NW * 64), 0, st, P);
  } else {
    return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

template <int HB, int NW>
int launch_merge_shape(const PrefillLaunch &P, hipStream_t st) {
  constexpr int QB = QW * (NW / HB);
  const int G = P.num_q_heads / P.num_kv_heads;
  if (P.max_qtiles != (P.max_q_len + QB - 1) / QB || P.splits < 2 || P.splits > kPrefillMaxSplits ||
      !P.part_o || !P.part_ml)
    return (int)hipErrorInvalidValue;
  dim3 grid(P.max_qtiles * 4, P.num_kv_heads * (G / HB), P.num_rows);
  if (P.out_dtype == PA_BF16)
    hipLaunchKernelGGL((prefill_merge_kernel<HB, true, NW>), grid, dim3(NW * 64), 0, st, P);
  else
    hipLaunchKernelGGL((prefill_merge_kernel<HB, false, NW>), grid, dim3(NW * 64), 0, st, P);
  return (int)hipGetLastError();
}

template <int HB>
int launch_hb(const PrefillLaunch &P, hipStream_t st) {
  if (P.waves == 8) return launch_shape<HB, 8>(P, st);
  if (P.waves == 4) return launch_shape<HB, 4>(P, st);
  return (int)hipErrorInvalidValue;
}

template <int HB>
int launch_merge_hb(const PrefillLaunch &P, hipStream_t st) {
  if (P.waves == 8) return launch_merge_shape<HB, 8>(P, st);
  if (P.waves == 4) return launch_merge_shape<HB, 4>(P, st);
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_prefill(const PrefillLaunch &P, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int G = P.num_q_heads / P.num_kv_heads;
  switch (G) {
    case 1: return launch_hb<1>(P, st);
    case 2: return launch_hb<2>(P, st);
    case 4: return launch_hb<4>(P, st);
    case 8: return launch_hb<4>(P, st);
  }
  return (int)hipErrorInvalidValue;
}

int launch_prefill_merge(const PrefillLaunch &P, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int G = P.num_q_heads / P.num_kv_heads;
  switch (G) {
    case 1: return launch_merge_hb<1>(P, st);
    case 2: return launch_merge_hb<2>(P, st);
    case 4: return launch_merge_hb<4>(P, st);
    case 8: return launch_merge_hb<4>(P, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace pa
