// Multi-query "verify" rows over a paged KV cache on gfx950 MFMA.
//
// What is computed: rows that carry a handful of new tokens (the draft tokens
// of speculative decoding, all checked by the target model in one pass:
// "How does TensorRT-LLM work", outcomeschool.com, section "Speculative
// decoding"; "TensorRT-LLM, in depth", aicassindra.com, section "Speculative
// decoding").  Their K/V are already in the cache: with L cached tokens and n
// new ones, new token i sits at position L - n + i and attends to every token
// up to and including itself.
//
// Such rows are decode-like -- each reads its whole cache once, so the pass is
// HBM-bound -- but carry n x (Hq/Hkv) query columns per kv head (up to 32),
// too many for the VALU dot products of the decode kernel.  Here the two
// contractions run on the matrix cores and everything else follows the decode
// kernel: the flattened (row, kv head, 32-token tile) work is cut into equal
// ranges, one per worker wave; a unit covered by one wave is finished in
// place, a unit cut by range boundaries leaves one (m, l, acc) partial per
// piece and query column for the log-sum-exp merge kernel.
//
// Per 32-token tile and wave (C = 16 or 32 query columns, column c = query
// c / G, head c % G of the kv head's group):
//   S^T = K Q^T   : 2 x C/16 x 4 v_mfma_f32_16x16x32_bf16.  The A operand
//                   (16 tokens x 32 head-dim elements) is exactly what a lane
//                   loads from the page: 16 contiguous bytes of one token row,
//                   so K goes from HBM straight into MFMA registers.
//   online softmax per column in fp32 (log2 domain, lazy rescale)
//   O^T += V^T P^T: 8 x C/16 v_mfma_f32_16x16x32_bf16, plus C/16 more against
//                   a row of ones for the softmax denominators.  P^T is already in
//                   B-operand order in the S^T accumulators (k slot 8q + j of a
//                   lane group q is token 4q + j, or 16 + 4q + j - 4 for j >= 4).
//                   V^T goes through a wave-private 8 KB LDS tile: each lane
//                   loads 4 consecutive tokens x 8 elements twice, transposes
//                   them with byte permutes and writes 16-byte groups at a
//                   swizzled position (conflict-free for the writes and for
//                   the MFMA-operand reads).
// FP8-E4M3 pools: codes are widened to bf16 in registers with
// v_cvt_scalef32_pk_bf16_fp8 (exact: every E4M3 value is a bf16 value), the
// per-head K scale folded into the softmax scale and the V scale applied to
// the result.  16 code bytes = 16 consecutive head-dim elements of one token
// feed two MFMA k steps; the head-dim order of the contraction is permuted to
// match (and Q^T is read in the same order), which leaves the dot products
// unchanged.  K is loaded as whole 128-byte token rows (8 rows per load
// instruction; in the operand layout an instruction would cover half of 16
// rows) and reaches the operand layout through a wave-private 4 KB LDS tile.
// FP8 V^T has an LDS layout of its own, conflict-free for its 8-byte writes.
// Three register sets keep two tiles' loads in flight while one is computed;
// one wave per SIMD (up to 512 registers).  Tokens at or past the row's end
// are excluded by select and their V zeroed before the transpose, so NaN in
// unused pool slots cannot leak.
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

constexpr int D = kHeadDim;            // 128
constexpr int TILE = kVerifyTile;      // 32 tokens
constexpr int NW = kWavesPerBlock;     // 4 independent waves per workgroup
constexpr int NT = NW * 64;
constexpr int VT_BYTES = D * TILE * 2; // one wave's V^T tile: 8 KB
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;
constexpr float kSlack = 8.0f;

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// two E4M3 codes (byte pair HI of the dword) -> bf16 pair, exact
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t codes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, HI));
}

// Items of a launch.
constexpr int kItemVerify = 0;   // verify rows: q_start_loc gives the queries, causal
constexpr int kItemPrefix = 1;   // groups of decode rows over their shared prefix
constexpr int kItemDecode = 2;   // decode rows: one query each, at the row's own index

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ long long readlane64(long long v, int k) {
  const int lo = __builtin_amdgcn_readlane((int)(v & 0xFFFFFFFFLL), k);
  const int hi = __builtin_amdgcn_readlane((int)(v >> 32), k);
  return ((long long)hi << 32) | (unsigned int)lo;
}

// Byte offset of the 16-byte group gi (k slots 8 gi .. 8 gi + 7) of V^T row d in
// a wave's tile.  Rows are taken four at a time (256 bytes = all 64 banks); within
// such a block the row picks the bank quarter and the group is XOR-ed with the
// block index, so that both the transposing writes (lanes of a pass hold rows
// 8 dg + e for four dg, groups 0..3) and the operand reads (rows 16 db + 0..15,
// one group) touch 16 distinct quarters x groups.
__device__ __forceinline__ int vt_offset(int d, int gi) {
  const int blk = d >> 2;
  const int quarter = ((d & 3) + (blk >> 1)) & 3;
  return blk * 256 + (4 * quarter + (gi ^ (blk & 3))) * 16;
}

// V^T layout of FP8 pools, whose transposing writes are 8 bytes wide (4 tokens of one row d):
// row d's 64 bytes sit in quarter ((d & 3) + d / 16) mod 4 of 256-byte block d / 4, its
// 16-byte groups XOR-ed with (d / 4 + d / 16) mod 4.  Under a 64-bank model each half-wave of
// writes (rows 16 dg + 4 w + e for four dg, all groups and halves) and each 16-lane operand
// read (rows 16 db + 0..15, one group) touch distinct banks (the bf16 layout above leaves the
// 8-byte writes two-way conflicted).
__device__ __forceinline__ int vt_offset8(int d, int gi) {
  const int r = d >> 4;
  const int quarter = ((d & 3) + r) & 3;
  return (d >> 2) * 256 + 64 * quarter + 16 * (gi ^ (((d >> 2) + r) & 3));
}

// Keeps the compiler from moving this wave's LDS accesses across the point;
// the LDS itself serves one wave's accesses in issue order.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

// KV: PA_BF16 or PA_FP8_E4M3 pools.  NCB: 16-column blocks of query columns (1: up to
// 16 columns, 2: up to 32).  ITEM: kItemVerify, kItemDecode, or kItemPrefix (the query
// columns are the group rows' queries, nothing is masked inside the prefix, and every
// piece is left as a partial for the final merge).
// Waves per SIMD: one (up to 512 registers) -- except FP8 pools with 16 columns, whose
// smaller tiles fit 256 registers: two waves per SIMD keep twice the bytes in flight.
template <int KV, int NCB>
constexpr int mq_waves_per_simd() { return (KV == PA_FP8_E4M3 && NCB == 1) ? 2 : 1; }

template <int KV, int ITEM, int NCB, bool OUT_BF16>
__global__ __launch_bounds__(NT)
__attribute__((amdgpu_waves_per_eu(mq_waves_per_simd<KV, NCB>(), mq_waves_per_simd<KV, NCB>())))
void verify_kernel(VerifyLaunch p) {
  constexpr bool FP8 = KV == PA_FP8_E4M3;
  constexpr bool PREFIX = ITEM == kItemPrefix;
  constexpr int EB = FP8 ? 1 : 2;          // bytes per element
  constexpr int KR = FP8 ? 4 : 8;          // 16-byte K registers per tile and lane
  constexpr int VR = FP8 ? 4 : 8;          // 16-byte V registers per tile and lane
  __shared__ __attribute__((aligned(16))) char s_vt[NW][VT_BYTES];
  // FP8 K tile (32 tokens x 128 code bytes) of each wave: loaded as whole 128-byte token
  // rows, read back in the MFMA operand layout
  constexpr int KQ_BYTES = FP8 ? TILE * D : 16;
  __shared__ __attribute__((aligned(16))) char s_kq[NW][KQ_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int worker = blockIdx.x * NW + wave;
  const int nworkers = p.num_workers;
  if (worker >= nworkers) return;
  const int R = p.num_rows;
  const int Hq = p.num_q_heads;
  const int Hkv = p.num_kv_heads;
  const int G = Hq / Hkv;
  const int log2G = __builtin_ctz(G);
  const int lq = lane & 15;                // MFMA row / column index
  const int lg = lane >> 4;                // MFMA lane group
  // V loads: bf16 -- token quad tqa (+ 4 per 16-token half) and 8-element group dg;
  //          fp8  -- token quad tq8 (of 8) and 16-element group dg8
  const int tqa = lane & 3;
  const int dg = lane >> 2;
  const int tq8 = lane & 7;
  const int dg8 = lane >> 3;
  char *vt = s_vt[wave];
  char *kq = s_kq[wave];

  // tokens each item covers (a group's shared prefix may be empty: no tiles)
  auto len_of = [&](int r) -> int {
    if constexpr (PREFIX) return p.shared_len[p.group_start[r]];
    else return checked_len(p.seq_lens[p.first_row + r], p.max_len, p.check_flags);
  };

  // Each unit counts unit_cost extra virtual tiles ahead of its real ones: starting a
  // unit (query and block-table loads, filling the load pipeline) costs about that much
  // time, so a worker given many short units gets fewer tiles.  Virtual tiles are
  // never loaded; a worker whose range holds only a unit's virtual tiles skips it.
  const int C = p.unit_cost;
  auto vtiles = [&](int len) -> int {
    const int t = (len + TILE - 1) / TILE;
    return t > 0 ? t + C : 0;
  };

  // ---- this worker's share of the flattened (item, kv head, virtual tile) space ----
  long long W = 0;
  int n_first = 0, incl_first = 0;         // the first 64 rows' counts, kept for the search below
  for (int base = 0; base < R; base += 64) {
    const int r = base + lane;
    const int n = r < R ? vtiles(len_of(r)) : 0;
    const int incl = wave_inclusive_scan(n, lane);
    if (base == 0) {
      n_first = n;
      incl_first = incl;
    }
    W += __builtin_amdgcn_readlane(incl, 63);
  }
  W *= Hkv;
  // the plan sized the launch for items of max_seq_len; shorter items get fewer workers
  int nwk = nworkers;
  if (p.workers_auto) nwk = (int)min((long long)nwk, max(1LL, W / p.min_tiles));
  const int nw = (int)min((long long)nwk, W);
  if (worker >= nw) return;
  const long long x0 = (long long)worker * W / nw;
  const long long x1 = (long long)(worker + 1) * W / nw;
  auto worker_of = [&](long long x) { return (int)(((x + 1) * nw - 1) / W); };

  int rb = 0;
  long long rowstart = 0;
  {
    long long before = 0;
    for (int base = 0; base < R; base += 64) {
      const int r = base + lane;
      const int n = base == 0 ? n_first : (r < R ? vtiles(len_of(r)) : 0);
      const int incl = base == 0 ? incl_first : wave_inclusive_scan(n, lane);
      const long long lo = before + (long long)(incl - n) * Hkv;
      const long long hi = before + (long long)incl * Hkv;
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(x0 >= lo && x0 < hi && n > 0);
      if (hit != 0) {
        const int k = __builtin_ctzll(hit);
        rb = base + k;
        rowstart = readlane64(lo, k);
        break;
      }
      before += (long long)__builtin_amdgcn_readlane(incl, 63) * Hkv;
    }
  }

  const int bs = p.block_size;
  const int log2bs = __builtin_ctz(bs);
  const size_t page_bytes = (size_t)bs * D * EB;
  const size_t phys_stride = (size_t)Hkv * page_bytes;

  int L = len_of(rb);
  int nb = (L + TILE - 1) / TILE;
  int vnb = nb + C;
  int g = (int)((x0 - rowstart) / vnb);
  int tv = (int)((x0 - rowstart) % vnb);
  long long ustart = rowstart + (long long)g * vnb;
  long long x = x0;
  int tbl0 = 0, tbl0_row = -1;             // the first 64 block-table entries of row tbl0_row

  while (x < x1) {
    const int cntv = (int)min((long long)(vnb - tv), x1 - x);
    // the real tiles [t0, t0 + cnt) of this unit in this worker's range
    const int t0 = max(tv - C, 0);
    const int cnt = tv + cntv - C - t0;
    if (cnt > 0) {
    const int u = rb * Hkv + g;
    // the item's first row: its block-table row, and its first query row
    const int row = PREFIX ? p.group_start[rb] : p.first_row + rb;
    float qk_scale = p.scale * kLog2e;
    float vscale = 1.f;
    if constexpr (FP8) {
      qk_scale *= p.k_scale[g];
      vscale = p.v_scale[g];
    }
    if (t0 == 0 && lane == 0) {
      p.seg_first[u] = worker;
      p.seg_count[u] = worker_of(ustart + C + nb - 1) - worker + 1;
    }
    const bool whole = !PREFIX && t0 == 0 && cnt == nb;
    // decode rows have one query each, at their own row index
#if PA_DEVICE_CHECKS
    int qbase = ITEM == kItemVerify ? p.q_start_loc[row] : row;
    int n = ITEM == kItemVerify ? p.q_start_loc[row + 1] - qbase
          : ITEM == kItemPrefix ? p.group_start[rb + 1] - row : 1;
    if (ITEM == kItemVerify) checked_qrange(qbase, n, L, p.total_q, p.check_flags);
#else
    const int qbase = ITEM == kItemVerify ? p.q_start_loc[row] : row;
    const int n = ITEM == kItemVerify ? p.q_start_loc[row + 1] - qbase
                : ITEM == kItemPrefix ? p.group_start[rb + 1] - row : 1;
#endif
    const int ncols = n << log2G;
    const int tok_begin = t0 * TILE;
    const int tok_end = min((t0 + cnt) * TILE, L);
    const int first_page = tok_begin >> log2bs;
    const int last_page = (tok_end - 1) >> log2bs;
    const int32_t *trow = p.block_table + (size_t)row * p.max_blocks_per_seq;
    const int mb_last = p.max_blocks_per_seq - 1;
    int chunk_base = first_page;
    int tbl = 0;

    // query columns of this lane: Q^T as the B operand, and the last visible position
    u32x4 qb[NCB][4];
    int lim[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int c = 16 * cb + lq;
      const int qi = c >> log2G;
      lim[cb] = (c < ncols && !PREFIX) ? L - n + qi : L - 1;
      const __bf16 *qp = static_cast<const __bf16 *>(p.q) +
                         ((size_t)(qbase + qi) * Hq + g * G + (c & (G - 1))) * D;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        // head-dim elements of k step kk held by lane group lg (the order K is loaded in)
        const int d0 = FP8 ? 16 * (lg + 4 * (kk >> 1)) + 8 * (kk & 1) : 32 * kk + 8 * lg;
        qb[cb][kk] = c < ncols ? *reinterpret_cast<const u32x4 *>(qp + d0) : u32x4{0u, 0u, 0u, 0u};
      }
    }
    const int mask_from = PREFIX ? L - 1 : L - n;   // tiles reaching past this need the mask
    const char *kpool = static_cast<const char *>(p.k_pool) + (size_t)g * page_bytes;
    const char *vpool = static_cast<const char *>(p.v_pool) + (size_t)g * page_bytes;

    // o: O^T blocks; ls: the denominators, accumulated by the same MFMA as O^T from a
    // V^T row of ones (row 0 of the block: lanes 0..15, element 0), so that numerator and
    // denominator see the same rounding (a constant V comes out exact)
    float m[NCB];
    f32x4 o[8][NCB], ls[NCB];
    const uint32_t one = lq == 0 ? 0x3F803F80u : 0u;      // bf16 pairs (1, 1): row 0, every k
    const u32x4 ones = {one, one, one, one};
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      m[cb] = kNegBig;
      ls[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < 8; ++db) o[db][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // bf16: k[4 tb + kk]: token ts + 16 tb + lq, elements 32 kk + 8 lg .. +8 (an MFMA A operand)
    //       v[4 tb + i]:  token ts + 16 tb + 4 tqa + i, elements 8 dg .. +8
    // fp8:  k[2 tb + h]:  token ts + 16 tb + lq, elements 16 (lg + 4 h) .. +16 (two k steps)
    //       v[i]:         token ts + 4 tq8 + i, elements 16 dg8 .. +16
    auto load_tile = [&](int t, u32x4 (&k)[KR], u32x4 (&v)[VR]) {
      const int ts = tok_begin + t * TILE;
      const char *vbase[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int tok0 = ts + 16 * tb;     // 16 tokens inside one page (bs >= 16)
        const int page = min(tok0 >> log2bs, last_page);
        const int phys = checked_block(__builtin_amdgcn_readlane(tbl, page - chunk_base), p.num_blocks, p.check_flags);
        const char *kp = kpool + (size_t)phys * phys_stride;
        vbase[tb] = vpool + (size_t)phys * phys_stride;
        const uint32_t krow = (uint32_t)(((tok0 + lq) & (bs - 1)) * (D * EB));
        if constexpr (FP8) {
          // each load instruction covers 8 whole token rows (lane: token lane/8 + 8h, 16
          // bytes at 16 (lane % 8)); the rows reach the operand layout through LDS
#pragma unroll
          for (int h = 0; h < 2; ++h)
            k[2 * tb + h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                kp + (uint32_t)(((tok0 + (lane >> 3) + 8 * h) & (bs - 1)) * D) + 16 * (lane & 7)));
        } else {
          const uint32_t voff = (uint32_t)(((tok0 + 4 * tqa) & (bs - 1)) * (D * 2) + 16 * dg);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            k[4 * tb + kk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kp + krow + 16 * lg + 64 * kk));
#pragma unroll
          for (int i = 0; i < 4; ++i)
            v[4 * tb + i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(vbase[tb] + voff + (D * 2) * i));
        }
      }
      if constexpr (FP8) {
        // quads 0..3 lie in the first 16 tokens, 4..7 in the second: a per-lane page
        const char *vp = (tq8 >> 2) ? vbase[1] : vbase[0];
        const uint32_t voff = (uint32_t)(((ts + 4 * tq8) & (bs - 1)) * D + 16 * dg8);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vp + voff + D * i));
      }
    };

    // FP8 K rows in this wave's LDS tile: token t's 16-byte group g sits at group
    // g ^ ((t >> 1) & 7) of its 128-byte row, so 16 consecutive lanes of a write (tokens t,
    // t + 1, all 8 groups) or of a read (16 tokens, one group) touch 16 different 16-byte
    // bank groups of a 256-byte bank row
    auto kq_addr = [&](int t, int g) -> int { return t * D + 16 * (g ^ ((t >> 1) & 7)); };
    // MFMA A operand of k step kk for token half tb (bf16 pairs); FP8: kc[tb][kk / 2] holds
    // 16 code bytes of token 16 tb + lq, elements 16 (lg + 4 (kk / 2)) .. +16
    auto k_operand = [&](const u32x4 (&k)[KR], const u32x4 (&kc)[2][2], int tb, int kk) -> u32x4 {
      if constexpr (FP8) {
        const u32x4 c = kc[tb][kk >> 1];
        const uint32_t w0 = (kk & 1) ? c[2] : c[0];
        const uint32_t w1 = (kk & 1) ? c[3] : c[1];
        return u32x4{fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
                     fp8x2_to_bf16x2<true>(w1)};
      } else {
        return k[4 * tb + kk];
      }
    };

    auto compute_tile = [&](int t, const u32x4 (&k)[KR], u32x4 (&v)[VR]) {
      const int ts = tok_begin + t * TILE;
      // ---- V^T into this wave's LDS tile (after the previous tile's operand reads) ----
      if (ts + TILE > L) {
#pragma unroll
        for (int r = 0; r < VR; ++r) {
          const int tok = FP8 ? ts + 4 * tq8 + r : ts + 16 * (r >> 2) + 4 * tqa + (r & 3);
          if (tok >= L) v[r] = u32x4{0u, 0u, 0u, 0u};
        }
      }
      wave_lds_fence();
      if constexpr (FP8) {
        // byte b of dword w of token i is element 16 dg8 + 4 w + b; gather it over the
        // four tokens, widen to bf16 and write 8 bytes (4 k slots) of row d
        const int half = 8 * (tq8 >> 2);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x01 = __builtin_amdgcn_perm(v[1][w], v[0][w], 0x05010400u);   // t0b0 t1b0 t0b1 t1b1
          const uint32_t x23 = __builtin_amdgcn_perm(v[3][w], v[2][w], 0x05010400u);
          const uint32_t y01 = __builtin_amdgcn_perm(v[1][w], v[0][w], 0x07030602u);   // t0b2 t1b2 t0b3 t1b3
          const uint32_t y23 = __builtin_amdgcn_perm(v[3][w], v[2][w], 0x07030602u);
          const int d = 16 * dg8 + 4 * w;
          *reinterpret_cast<u32x2 *>(vt + vt_offset8(d, tq8 & 3) + half) =
              u32x2{fp8x2_to_bf16x2<false>(x01), fp8x2_to_bf16x2<false>(x23)};
          *reinterpret_cast<u32x2 *>(vt + vt_offset8(d + 1, tq8 & 3) + half) =
              u32x2{fp8x2_to_bf16x2<true>(x01), fp8x2_to_bf16x2<true>(x23)};
          *reinterpret_cast<u32x2 *>(vt + vt_offset8(d + 2, tq8 & 3) + half) =
              u32x2{fp8x2_to_bf16x2<false>(y01), fp8x2_to_bf16x2<false>(y23)};
          *reinterpret_cast<u32x2 *>(vt + vt_offset8(d + 3, tq8 & 3) + half) =
              u32x2{fp8x2_to_bf16x2<true>(y01), fp8x2_to_bf16x2<true>(y23)};
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const u32x4 grp = {__builtin_amdgcn_perm(v[1][w], v[0][w], sel),
                             __builtin_amdgcn_perm(v[3][w], v[2][w], sel),
                             __builtin_amdgcn_perm(v[5][w], v[4][w], sel),
                             __builtin_amdgcn_perm(v[7][w], v[6][w], sel)};
          *reinterpret_cast<u32x4 *>(vt + vt_offset(8 * dg + e, tqa)) = grp;
        }
      }
      u32x4 kc[2][2];
      if constexpr (FP8) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            *reinterpret_cast<u32x4 *>(kq + kq_addr(16 * tb + (lane >> 3) + 8 * h, lane & 7)) = k[2 * tb + h];
        wave_lds_fence();
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            kc[tb][h] = *reinterpret_cast<const u32x4 *>(kq + kq_addr(16 * tb + lq, lg + 4 * h));
      }
      // ---- S^T = K Q^T ----
      f32x4 s[2][NCB];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) s[tb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const u32x4 a = k_operand(k, kc, tb, kk);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) s[tb][cb] = mfma(a, qb[cb][kk], s[tb][cb]);
        }
      // ---- scale, mask, online softmax per column ----
      const bool masked = ts + TILE - 1 > mask_from;
      float tmax[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float xv = s[tb][cb][i] * qk_scale;
            if (masked) xv = ts + 16 * tb + 4 * lg + i <= lim[cb] ? xv : -__builtin_inff();
            s[tb][cb][i] = xv;
            mx = fmaxf(mx, xv);
          }
        tmax[cb] = mx;                     // this lane's part of the column max
      }
      // a column needs rescaling when one of its lanes' parts exceeds m by more than the
      // slack: the vote needs no cross-lane reduction, which the rare rescale path does
      bool need = false;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) need |= tmax[cb] > m[cb] + kSlack;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          tmax[cb] = fmaxf(tmax[cb], __shfl_xor(tmax[cb], 16));
          tmax[cb] = fmaxf(tmax[cb], __shfl_xor(tmax[cb], 32));
          const float mn = fmaxf(m[cb], tmax[cb]);
          const float a = fast_exp2(m[cb] - mn);
          m[cb] = mn;
          ls[cb] *= a;
#pragma unroll
          for (int db = 0; db < 8; ++db) o[db][cb] *= a;
        }
      }
      u32x4 pb[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = fast_exp2(s[0][cb][i] - m[cb]);
          pv[4 + i] = fast_exp2(s[1][cb][i] - m[cb]);
        }
        pb[cb] = u32x4{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                       pack_bf16(pv[6], pv[7])};
        ls[cb] = mfma(ones, pb[cb], ls[cb]);
      }
      // ---- O^T += V^T P^T ----
      wave_lds_fence();
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(
            vt + (FP8 ? vt_offset8(16 * db + lq, lg) : vt_offset(16 * db + lq, lg)));
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) o[db][cb] = mfma(a, pb[cb], o[db][cb]);
      }
    };

    // software pipeline over tiles [ta, tb): three register sets, two tiles in flight;
    // look-ahead loads past the last tile are skipped (loading the last tile again
    // would fetch it from HBM again: the loads do not allocate in the caches)
    auto run_tiles = [&](int ta, int tb) {
      u32x4 ka[KR], va[VR], kb2[KR], vb2[VR], kc[KR], vc[VR];
      load_tile(ta, ka, va);
      if (ta + 1 < tb) load_tile(ta + 1, kb2, vb2);
      for (int t = ta; t < tb; t += 3) {
        if (t + 2 < tb) load_tile(t + 2, kc, vc);
        compute_tile(t, ka, va);
        if (t + 3 < tb) load_tile(t + 3, ka, va);
        if (t + 1 < tb) compute_tile(t + 1, kb2, vb2);
        if (t + 4 < tb) load_tile(t + 4, kb2, vb2);
        if (t + 2 < tb) compute_tile(t + 2, kc, vc);
      }
    };
    // chunks of 64 pages share one block-table load (64 * bs tokens: whole tiles); the
    // row's first chunk is kept for the next unit, usually the next kv head of the row
    for (int ta = 0; ta < cnt;) {
      const int tb = min(cnt, (((chunk_base + 64) << log2bs) - tok_begin) / TILE);
      if (chunk_base == 0 && row == tbl0_row) {
        tbl = tbl0;
      } else {
        tbl = trow[min(chunk_base + lane, mb_last)];
        if (chunk_base == 0) {
          tbl0 = tbl;
          tbl0_row = row;
        }
      }
      run_tiles(ta, tb);
      ta = tb;
      chunk_base += 64;
    }

    // ---- denominators: row 0 of the ones product, held by lanes 0..15; write ----
    float lsum[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) lsum[cb] = __shfl(ls[cb][0], lq);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int c = 16 * cb + lq;
      if (c >= ncols) continue;
      if (whole) {
        const size_t base = ((size_t)(qbase + (c >> log2G)) * Hq + g * G + (c & (G - 1))) * D;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const f32x4 v = o[db][cb] * vscale;
          const float l = lsum[cb];
          store4<OUT_BF16>(p.out, base + 16 * db + 4 * lg, f32x4{v[0] / l, v[1] / l, v[2] / l, v[3] / l});
        }
      } else {
        const size_t slot = (size_t)(u + worker) * p.slot_cols + c;
#pragma unroll
        for (int db = 0; db < 8; ++db)
          *reinterpret_cast<f32x4 *>(p.part_acc + slot * D + 16 * db + 4 * lg) = o[db][cb] * vscale;
        if (lg == 0) {
          p.part_m[slot] = m[cb];
          p.part_l[slot] = lsum[cb];
        }
      }
    }

    }  // cnt > 0

    // next unit
    x += cntv;
    tv = 0;
    ustart += vnb;
    if (++g == Hkv) {
      g = 0;
      ++rb;
      if (x < x1) {
        L = len_of(rb);
        nb = (L + TILE - 1) / TILE;
        while (nb == 0) {                  // items without tiles (empty shared prefix)
          L = len_of(++rb);
          nb = (L + TILE - 1) / TILE;
        }
        vnb = nb + C;
      }
    }
  }
}

// Combine the pieces of one (row, kv head, query column) cut across workers.
template <int ITEM, bool OUT_BF16>
__global__ __launch_bounds__(64) void verify_merge_kernel(VerifyLaunch p) {
  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const int lane = threadIdx.x;
  const int Hkv = p.num_kv_heads;
  const int G = p.num_q_heads / Hkv;
  const int rb = u / Hkv;
  const int g = u % Hkv;
  const int row = p.first_row + rb;
#if PA_DEVICE_CHECKS
  int qbase = ITEM == kItemDecode ? row : p.q_start_loc[row];
  int n = ITEM == kItemDecode ? 1 : p.q_start_loc[row + 1] - qbase;
  if (ITEM != kItemDecode)
    checked_qrange(qbase, n, checked_len(p.seq_lens[row], p.max_len, p.check_flags), p.total_q, p.check_flags);
#else
  const int qbase = ITEM == kItemDecode ? row : p.q_start_loc[row];
  const int n = ITEM == kItemDecode ? 1 : p.q_start_loc[row + 1] - qbase;
#endif
  if (c >= n * G) return;
  int cnt = p.seg_count[u];
  if (cnt <= 1) return;                    // written directly by its only worker
  // slots u + w exist for the launch's workers w in [0, num_workers): a record that does
  // not come from the partials launch on this workspace gives wrong numbers, never a read
  // outside it
  const int first = min(max(p.seg_first[u], 0), p.num_workers - 1);
  cnt = min(cnt, p.num_workers - first);
  float n0 = 0.f, n1 = 0.f, den = 0.f;
  if (cnt <= 8) {
    // every piece's (max, sum, two accumulators) in one round trip, then the same
    // arithmetic in the same order as the general path below
    float pm[8], pl[8];
    float2 pa[8];
    float M = kNegBig;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < cnt) {
        const size_t slot = (size_t)(u + first + k) * p.slot_cols + c;
        pm[k] = p.part_m[slot];
        pl[k] = p.part_l[slot];
        pa[k] = *reinterpret_cast<const float2 *>(p.part_acc + slot * D + 2 * lane);
        M = fmaxf(M, pm[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < cnt) {
        const float wt = fast_exp2(pm[k] - M);
        den = __builtin_fmaf(wt, pl[k], den);
        n0 = __builtin_fmaf(wt, pa[k].x, n0);
        n1 = __builtin_fmaf(wt, pa[k].y, n1);
      }
    }
  } else {
  // the pieces' maxima, one per lane: one round trip however many pieces there are
  float M = kNegBig;
  for (int base = 0; base < cnt; base += 64)
    if (base + lane < cnt) M = fmaxf(M, p.part_m[(size_t)(u + first + base + lane) * p.slot_cols + c]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  // then the pieces in order, eight at a time with all their loads issued before use
  for (int base = 0; base < cnt; base += 8) {
    float pm[8], pl[8];
    float2 pa[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (base + k < cnt) {
        const size_t slot = (size_t)(u + first + base + k) * p.slot_cols + c;
        pm[k] = p.part_m[slot];
        pl[k] = p.part_l[slot];
        pa[k] = *reinterpret_cast<const float2 *>(p.part_acc + slot * D + 2 * lane);
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (base + k < cnt) {
        const float wt = fast_exp2(pm[k] - M);
        den = __builtin_fmaf(wt, pl[k], den);
        n0 = __builtin_fmaf(wt, pa[k].x, n0);
        n1 = __builtin_fmaf(wt, pa[k].y, n1);
      }
    }
  }
  }
  const size_t o = ((size_t)(qbase + c / G) * p.num_q_heads + g * G + c % G) * D + 2 * lane;
  if constexpr (OUT_BF16) {
    static_cast<__bf16 *>(p.out)[o] = (__bf16)(n0 / den);
    static_cast<__bf16 *>(p.out)[o + 1] = (__bf16)(n1 / den);
  } else {
    static_cast<float *>(p.out)[o] = n0 / den;
    static_cast<float *>(p.out)[o + 1] = n1 / den;
  }
}

template <int KV, int ITEM, int NCB>
int launch_one(const VerifyLaunch &V, hipStream_t st) {
  dim3 grid((V.num_workers + NW - 1) / NW);
  if (V.out_dtype == PA_BF16)
    hipLaunchKernelGGL((verify_kernel<KV, ITEM, NCB, true>), grid, dim3(NT), 0, st, V);
  else
    hipLaunchKernelGGL((verify_kernel<KV, ITEM, NCB, false>), grid, dim3(NT), 0, st, V);
  return (int)hipGetLastError();
}

template <int KV>
int launch_kv(const VerifyLaunch &V, hipStream_t st) {
  const bool wide = V.slot_cols > 16;
  switch (V.item_kind) {
    case 0: return wide ? launch_one<KV, kItemVerify, 2>(V, st) : launch_one<KV, kItemVerify, 1>(V, st);
    case 1: return wide ? launch_one<KV, kItemPrefix, 2>(V, st) : launch_one<KV, kItemPrefix, 1>(V, st);
    case 2: return wide ? launch_one<KV, kItemDecode, 2>(V, st) : launch_one<KV, kItemDecode, 1>(V, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_verify_partials(const VerifyLaunch &V, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (V.kv_dtype == PA_FP8_E4M3) return launch_kv<PA_FP8_E4M3>(V, st);
  return launch_kv<PA_BF16>(V, st);
}

int launch_verify_merge(const VerifyLaunch &V, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  dim3 grid(V.slot_cols, V.num_rows * V.num_kv_heads);
  const bool dec = V.item_kind == 2;
  if (V.out_dtype == PA_BF16) {
    if (dec) hipLaunchKernelGGL((verify_merge_kernel<kItemDecode, true>), grid, dim3(64), 0, st, V);
    else hipLaunchKernelGGL((verify_merge_kernel<kItemVerify, true>), grid, dim3(64), 0, st, V);
  } else {
    if (dec) hipLaunchKernelGGL((verify_merge_kernel<kItemDecode, false>), grid, dim3(64), 0, st, V);
    else hipLaunchKernelGGL((verify_merge_kernel<kItemVerify, false>), grid, dim3(64), 0, st, V);
  }
  return (int)hipGetLastError();
}

}  // namespace pa
