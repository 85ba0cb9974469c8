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
// Tiling.  A workgroup (4 x wave64) owns one (row, kv head, block of query
// heads, query tile); each wave owns 32 query positions of one query head.
// K/V are staged through LDS in tiles of 64 tokens gathered page by page
// through the block table; the next tile is prefetched into registers while
// the current one is computed.  Per tile and wave:
//   S^T = K Q^T   : 32 x v_mfma_f32_16x16x32_bf16  (A = K rows from LDS,
//                   B = Q^T held in registers for the whole row)
//   online softmax in fp32 (log2 domain, lazy rescale as in the decode kernel)
//   O^T += V^T P^T: 32 x v_mfma_f32_16x16x32_bf16  (A = V^T from LDS,
//                   B = P^T straight from the S^T accumulators)
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

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;        // 128
constexpr int KT = 64;             // kv tokens per tile
constexpr int QW = 32;             // query positions per wave
constexpr int NWP = 4;             // waves per workgroup
constexpr int NTP = NWP * 64;
constexpr int K_STRIDE = 272;      // bytes per K row in LDS (256 + 16 pad: conflict-free 16-B reads)
constexpr int V_STRIDE = 144;      // bytes per V^T row in LDS (128 + 16 pad)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;
constexpr float kSlack = 8.0f;
constexpr int CHUNKS = KT * D * 2 / 16 / NTP;   // 16-byte chunks per thread per tile (K or V): 4

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_round(float x) { return (float)(__bf16)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool OUT_BF16>
__device__ __forceinline__ void store4(void *out, size_t idx, f32x4 v) {
  if constexpr (OUT_BF16) {
    u32x2 w = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    *reinterpret_cast<u32x2 *>(static_cast<__bf16 *>(out) + idx) = w;
  } else {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + idx) = v;
  }
}

// HB: query heads per workgroup (1, 2 or 4); the 4 waves cover HB heads x (4/HB) query sub-tiles.
template <int HB, bool OUT_BF16>
__global__ __launch_bounds__(NTP) void prefill_kernel(PrefillLaunch p) {
  constexpr int QSUB = NWP / HB;
  constexpr int QB = QW * QSUB;            // queries per workgroup

  __shared__ __attribute__((aligned(16))) char s_k[KT * K_STRIDE];
  __shared__ __attribute__((aligned(16))) char s_vt[D * V_STRIDE];

  const int Hq = p.num_q_heads;
  const int Hkv = p.num_kv_heads;
  const int G = Hq / Hkv;
  const int hblocks = G / HB;              // head blocks per kv head
  const int qt = blockIdx.x;
  const int g = blockIdx.y / hblocks;
  const int hb = blockIdx.y % hblocks;
  const int row = p.first_row + blockIdx.z;
  const int q_begin = p.q_start_loc[row];
  const int n = p.q_start_loc[row + 1] - q_begin;
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
  const int kv_end = prior + blk_last_q + 1;              // tokens the workgroup visits
  const int ntile = (kv_end + KT - 1) / KT;
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
  const float qk_scale = p.scale * kLog2e;

  // cooperative tile loads: thread chunk c = tid + 256*i -> token c/16, elements 8*(c%16)..+8
  const int bs = p.block_size;
  const int log2bs = __builtin_ctz(bs);
  const int32_t *trow = p.block_table + (size_t)row * p.max_blocks_per_seq;
  const size_t page_elems = (size_t)bs * D;
  const __bf16 *kpool = static_cast<const __bf16 *>(p.k_pool) + (size_t)g * page_elems;
  const __bf16 *vpool = static_cast<const __bf16 *>(p.v_pool) + (size_t)g * page_elems;
  const size_t phys_stride = (size_t)Hkv * page_elems;
  const int c_tok = tid >> 4;              // + 16 * i
  const int c_d0 = 8 * (tid & 15);

  u32x4 rk[CHUNKS], rv[CHUNKS];
  auto load_regs = [&](int j) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int t = j * KT + c_tok + 16 * i;
      if (t < L) {
        const int phys = trow[t >> log2bs];
        const size_t off = (size_t)phys * phys_stride + (size_t)(t & (bs - 1)) * D + c_d0;
        rk[i] = *reinterpret_cast<const u32x4 *>(kpool + off);
        rv[i] = *reinterpret_cast<const u32x4 *>(vpool + off);
      } else {
        rk[i] = u32x4{0u, 0u, 0u, 0u};
        rv[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_lds = [&]() {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int tk = c_tok + 16 * i;
      *reinterpret_cast<u32x4 *>(s_k + tk * K_STRIDE + c_d0 * 2) = rk[i];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t dw = rv[i][w];
        *reinterpret_cast<uint16_t *>(s_vt + (c_d0 + 2 * w) * V_STRIDE + tk * 2) = (uint16_t)(dw & 0xFFFFu);
        *reinterpret_cast<uint16_t *>(s_vt + (c_d0 + 2 * w + 1) * V_STRIDE + tk * 2) = (uint16_t)(dw >> 16);
      }
    }
  };

  float m[2] = {kNegBig, kNegBig};
  float lsum[2] = {0.f, 0.f};              // per-lane partial of the softmax denominator
  f32x4 o[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int qt2 = 0; qt2 < 2; ++qt2) o[dt][qt2] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_regs(0);
  for (int j = 0; j < ntile; ++j) {
    __syncthreads();                       // every wave is done reading tile j-1
    store_lds();
    __syncthreads();
    if (j + 1 < ntile) load_regs(j + 1);   // in flight while tile j is computed
    const int kv0 = j * KT;
    if (!wave_active || kv0 > wave_last_pos) continue;    // fully masked for this wave

    // ---- S^T = K Q^T ----
    f32x4 s[4][2];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int qt2 = 0; qt2 < 2; ++qt2) s[tt][qt2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(s_k + (16 * tt + lq) * K_STRIDE + (32 * ks + 8 * lg) * 2);
#pragma unroll
        for (int qt2 = 0; qt2 < 2; ++qt2) s[tt][qt2] = mfma(a, qb[qt2][ks], s[tt][qt2]);
      }
    }
    // ---- scale, causal mask, online softmax (per query column) ----
    const bool diag = kv0 + KT - 1 > prior + q0;          // some element may be masked
    float tmax[2];
#pragma unroll
    for (int qt2 = 0; qt2 < 2; ++qt2) {
      const int qi = q0 + 16 * qt2 + lq;
      const int pos = prior + min(qi, n - 1);
      float mx = -__builtin_inff();
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = s[tt][qt2][i] * qk_scale;
          if (diag) {
            const int tok = kv0 + 16 * tt + 4 * lg + i;
            x = tok <= pos ? x : -__builtin_inff();
          }
          s[tt][qt2][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      tmax[qt2] = mx;
    }
    const bool need = tmax[0] > m[0] + kSlack || tmax[1] > m[1] + kSlack;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int qt2 = 0; qt2 < 2; ++qt2) {
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
          pv[i] = fast_exp2(s[2 * ks2][qt2][i] - m[qt2]);
          pv[4 + i] = fast_exp2(s[2 * ks2 + 1][qt2][i] - m[qt2]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) lsum[qt2] += bf16_round(pv[i]);
        pb[qt2][ks2] = u32x4{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                             pack_bf16(pv[6], pv[7])};
      }
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const char *vrow = s_vt + (16 * dt + lq) * V_STRIDE + (32 * ks2 + 4 * lg) * 2;
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow);
        const u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + 32);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int qt2 = 0; qt2 < 2; ++qt2) o[dt][qt2] = mfma(a, pb[qt2][ks2], o[dt][qt2]);
      }
    }
  }

  if (!wave_active) return;
  // denominator: sum the four lane groups of each query column
#pragma unroll
  for (int qt2 = 0; qt2 < 2; ++qt2) {
    lsum[qt2] += __shfl_xor(lsum[qt2], 16);
    lsum[qt2] += __shfl_xor(lsum[qt2], 32);
  }
#pragma unroll
  for (int qt2 = 0; qt2 < 2; ++qt2) {
    const int qi = q0 + 16 * qt2 + lq;
    if (qi >= n) continue;
    const size_t base = ((size_t)(q_begin + qi) * Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      f32x4 v = o[dt][qt2];
      f32x4 r = {v[0] / lsum[qt2], v[1] / lsum[qt2], v[2] / lsum[qt2], v[3] / lsum[qt2]};
      store4<OUT_BF16>(p.out, base + 16 * dt + 4 * lg, r);
    }
  }
}

template <int HB>
int launch_hb(const PrefillLaunch &P, hipStream_t st) {
  constexpr int QB = QW * (NWP / HB);
  const int G = P.num_q_heads / P.num_kv_heads;
  dim3 grid((P.max_q_len + QB - 1) / QB, P.num_kv_heads * (G / HB), P.num_rows);
  if (P.out_dtype == PA_BF16)
    hipLaunchKernelGGL((prefill_kernel<HB, true>), grid, dim3(NTP), 0, st, P);
  else
    hipLaunchKernelGGL((prefill_kernel<HB, false>), grid, dim3(NTP), 0, st, P);
  return (int)hipGetLastError();
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

}  // namespace pa
