// Decode attention over a paged KV cache on gfx950 (CDNA4), VALU path.
//
// What is computed: for every decode row, kv head g and query head h of g's
// group, softmax(scale * q.K^T) V over the row's whole KV cache, with the
// cache reached block by block through the row's block table ("How does
// TensorRT-LLM work", outcomeschool.com, section "The paged KV cache";
// "TensorRT-LLM, in depth", aicassindra.com, section "First principles:
// where the GPU memory goes": each decode step reads the request's entire KV
// cache, so the step is memory-bandwidth-bound).  The long-context split over
// the context with a log-sum-exp merge is the Flash-Decoding idea named in
// "Introduction to TensorRT-LLM" (dileepadev.github.io), section "Core
// Optimization Technologies".
//
// Work decomposition.  One workgroup (4 x wave64) owns one (row b, kv head g,
// partition s) unit: tokens [s*P, min((s+1)*P, L)).  The four waves take
// interleaved tiles of 16 tokens (32 for FP8).  Inside a wave, 8 lanes share
// one token: each lane holds 16 of its 128 elements, loaded with 16-byte
// loads so that one load instruction covers eight whole 128-byte lines of a
// (block, head) page.  The group of Hq/Hkv query heads that shares kv head g
// is processed together, so every K/V byte is read from HBM once per step.
//
// Arithmetic.  Q.K uses v_dot2c_f32_bf16 (bf16 pairs, fp32 accumulate); the
// 8 partial sums of a token are combined with three DPP adds (quad xor 1,
// quad xor 2, half-row mirror).  FP8-E4M3 codes are widened to bf16 in
// registers (exactly: every E4M3 value is a bf16 value) with
// v_cvt_scalef32_pk_bf16_fp8; the per-head K scale is folded into the softmax
// scale and the V scale applied once at the end.  The softmax runs in the
// log2 domain in fp32 registers, one running (max, sum) per 8-lane token
// group, with lazy rescaling: the running max moves only when a tile's max
// exceeds it by more than 2^8, which keeps every exp2 argument <= 8 and makes
// the rescale branch (wave-uniform) rare.  P.V pairs two tokens per
// v_dot2c_f32_bf16 (P rounded to bf16, the softmax denominator summed from the
// same rounded values).  Tokens past the row's end are excluded by select and
// their V registers zeroed, so NaN in unused slots never reaches the result.
//
// Epilogue.  The 32 (wave, token-group) partial states of a workgroup are
// merged with one DPP step and one LDS pass using the log-sum-exp identity;
// one-partition plans write the normalised output directly, otherwise
// (m, l, acc) partials go to the workspace for merge_kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;
constexpr int NW = kWavesPerBlock;
constexpr int NT = NW * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;   // finite start value of running maxima
constexpr float kSlack = 8.0f;        // lazy-rescale threshold, log2 units

// DPP controls (GFX9 encoding)
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror: lane i <-> 7-i within 8
constexpr int kDppRowRor8 = 0x128;    // row_ror:8: lane i <- (i+8) mod 16

template <int KV> struct KvTraits;
template <> struct KvTraits<PA_F32> { static constexpr int EB = 4, TPL = 2; };
template <> struct KvTraits<PA_BF16> { static constexpr int EB = 2, TPL = 2; };
template <> struct KvTraits<PA_FP8_E4M3> { static constexpr int EB = 1, TPL = 4; };

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

// two E4M3 codes (byte pair HI of the dword) -> bf16 pair, exact
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t codes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, HI));
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// element e (0..15) of lane c (0..7) maps to head-dim index d
template <int EB>
__device__ __forceinline__ constexpr int elem_d(int c, int e) {
  return (e / (16 / EB)) * (128 / EB) + c * (16 / EB) + (e % (16 / EB));
}

template <bool OUT_BF16>
__device__ __forceinline__ void store_out(void *out, size_t idx, float v) {
  if constexpr (OUT_BF16) {
    static_cast<__bf16 *>(out)[idx] = (__bf16)v;
  } else {
    static_cast<float *>(out)[idx] = v;
  }
}

template <int KV, int G, bool OUT_BF16>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeLaunch p) {
  constexpr int EB = KvTraits<KV>::EB;
  constexpr int TPL = KvTraits<KV>::TPL;   // tokens per lane per tile
  constexpr int TILE = 8 * TPL;            // tokens per tile
  constexpr int DW = 4 * EB;               // dwords per token per lane
  constexpr bool kBf = KV != PA_F32;

  __shared__ float s_acc[NW][4][G][D];
  __shared__ float s_m[NW][4][G];
  __shared__ float s_l[NW][4][G];

  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int L = p.seq_lens[b];
  const int part_start = s * p.partition_size;
  if (part_start >= L) return;           // whole workgroup: empty partition
  const int end = min(part_start + p.partition_size, L);

  const int lane = threadIdx.x & 63;
  // wave index is uniform across the wave: keep it (and all tile/page arithmetic) scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 7;                  // element slot inside the token row
  const int grp = lane >> 3;               // token group 0..7
  const int bs = p.block_size;
  const int log2bs = __builtin_ctz(bs);
  const int first_page = part_start >> log2bs;
  const int last_page = (end - 1) >> log2bs;
  const int npages = last_page - first_page + 1;   // <= 64 by plan
  const int Hq = p.num_q_heads;
  const int Hkv = p.num_kv_heads;

  // block-table entries of this partition: lane i holds page first_page + i
  const int32_t *trow = p.block_table + (size_t)b * p.max_blocks_per_seq;
  const int tbl = trow[first_page + min(lane, npages - 1)];

  // query group of kv head g, in this lane's element order
  uint32_t qb[G][8];
  float qf[G][16];
  if constexpr (kBf) {
    const uint16_t *q = static_cast<const uint16_t *>(p.q) + ((size_t)b * Hq + g * G) * D;
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        qb[hh][i] = *reinterpret_cast<const uint32_t *>(q + hh * D + elem_d<EB>(c, 2 * i));
  } else {
    const float *q = static_cast<const float *>(p.q) + ((size_t)b * Hq + g * G) * D;
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 16; ++e) qf[hh][e] = q[hh * D + elem_d<EB>(c, e)];
  }

  float qk_scale = p.scale * kLog2e;
  if constexpr (KV == PA_FP8_E4M3) qk_scale *= p.k_scale[g];

  const size_t page_bytes = (size_t)bs * D * EB;
  const char *kpool = static_cast<const char *>(p.k_pool) + (size_t)g * page_bytes;
  const char *vpool = static_cast<const char *>(p.v_pool) + (size_t)g * page_bytes;
  const size_t phys_stride = (size_t)Hkv * page_bytes;
  const int lane_off = c * 16;

  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = kNegBig;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[hh][e] = 0.f;
  }

  const int ntiles = (end - part_start + TILE - 1) / TILE;

  u32x4 kr[TPL][EB], vr[TPL][EB];
  auto load_tile = [&](int t, u32x4 (&k)[TPL][EB], u32x4 (&v)[TPL][EB]) {
#pragma unroll
    for (int r = 0; r < TPL; ++r) {
      const int tok0 = part_start + t * TILE + 8 * r;
      const int page = min(tok0 >> log2bs, last_page);
      const int phys = __builtin_amdgcn_readlane(tbl, page - first_page);
      // scalar page base + 32-bit per-lane offset (global_load ... saddr form)
      const char *kp = kpool + (size_t)phys * phys_stride;
      const char *vp = vpool + (size_t)phys * phys_stride;
      const uint32_t off = (uint32_t)(((tok0 + grp) & (bs - 1)) * (D * EB) + lane_off);
#pragma unroll
      for (int j = 0; j < EB; ++j) {
        k[r][j] = *reinterpret_cast<const u32x4 *>(kp + off + j * 128);
        v[r][j] = *reinterpret_cast<const u32x4 *>(vp + off + j * 128);
      }
    }
  };

  auto compute_tile = [&](int t, const u32x4 (&k)[TPL][EB], u32x4 (&v)[TPL][EB]) {
    const int tile_start = part_start + t * TILE;
    float sc[TPL][G];
#pragma unroll
    for (int r = 0; r < TPL; ++r) {
      uint32_t kd[DW];
#pragma unroll
      for (int i = 0; i < DW; ++i) kd[i] = k[r][i / 4][i % 4];
      if constexpr (kBf) {
        uint32_t kp[8];
        if constexpr (KV == PA_BF16) {
#pragma unroll
          for (int i = 0; i < 8; ++i) kp[i] = kd[i];
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            kp[2 * w] = fp8x2_to_bf16x2<false>(kd[w]);
            kp[2 * w + 1] = fp8x2_to_bf16x2<true>(kd[w]);
          }
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float a = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) a = dot2bf(qb[hh][i], kp[i], a);
          sc[r][hh] = a;
        }
      } else {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) a = __builtin_fmaf(qf[hh][e], __builtin_bit_cast(float, kd[e]), a);
          sc[r][hh] = a;
        }
      }
    }
    // sum the 8 partial dot products of each token
#pragma unroll
    for (int r = 0; r < TPL; ++r)
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float x = sc[r][hh];
        x += dpp<kDppXor1>(x);
        x += dpp<kDppXor2>(x);
        x += dpp<kDppHalfMirror>(x);
        sc[r][hh] = x * qk_scale;
      }
    // tokens at or past `end` take no part
    if (tile_start + TILE > end) {
#pragma unroll
      for (int r = 0; r < TPL; ++r) {
        if (tile_start + 8 * r + grp >= end) {
#pragma unroll
          for (int hh = 0; hh < G; ++hh) sc[r][hh] = -__builtin_inff();
#pragma unroll
          for (int j = 0; j < EB; ++j) v[r][j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    // online softmax with lazy rescaling
    float tmax[G];
    bool need = false;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float x = sc[0][hh];
#pragma unroll
      for (int r = 1; r < TPL; ++r) x = fmaxf(x, sc[r][hh]);
      tmax[hh] = x;
      need |= x > m[hh] + kSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float mn = fmaxf(m[hh], tmax[hh]);
        const float a = fast_exp2(m[hh] - mn);
        m[hh] = mn;
        l[hh] *= a;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[hh][e] *= a;
      }
    }
    float pr[TPL][G];
#pragma unroll
    for (int r = 0; r < TPL; ++r)
#pragma unroll
      for (int hh = 0; hh < G; ++hh) pr[r][hh] = fast_exp2(sc[r][hh] - m[hh]);

    // P.V
    if constexpr (kBf) {
      constexpr uint32_t kOnes = 0x3F803F80u;   // bf16 pair (1, 1)
#pragma unroll
      for (int u = 0; u < TPL / 2; ++u) {
        const int r0 = 2 * u, r1 = 2 * u + 1;
        uint32_t pp[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          pp[hh] = pack_bf16(pr[r0][hh], pr[r1][hh]);
          l[hh] = dot2bf(pp[hh], kOnes, l[hh]);
        }
        if constexpr (KV == PA_BF16) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t A = v[r0][i / 4][i % 4];
            const uint32_t B = v[r1][i / 4][i % 4];
            const uint32_t lo = __builtin_amdgcn_perm(B, A, 0x05040100u);
            const uint32_t hi = __builtin_amdgcn_perm(B, A, 0x07060302u);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
              acc[hh][2 * i] = dot2bf(lo, pp[hh], acc[hh][2 * i]);
              acc[hh][2 * i + 1] = dot2bf(hi, pp[hh], acc[hh][2 * i + 1]);
            }
          }
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t A = v[r0][0][w];
            const uint32_t B = v[r1][0][w];
            const uint32_t X = __builtin_amdgcn_perm(B, A, 0x05010400u);   // a0 b0 a1 b1
            const uint32_t Y = __builtin_amdgcn_perm(B, A, 0x07030602u);   // a2 b2 a3 b3
            const uint32_t v0 = fp8x2_to_bf16x2<false>(X);
            const uint32_t v1 = fp8x2_to_bf16x2<true>(X);
            const uint32_t v2 = fp8x2_to_bf16x2<false>(Y);
            const uint32_t v3 = fp8x2_to_bf16x2<true>(Y);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
              acc[hh][4 * w + 0] = dot2bf(v0, pp[hh], acc[hh][4 * w + 0]);
              acc[hh][4 * w + 1] = dot2bf(v1, pp[hh], acc[hh][4 * w + 1]);
              acc[hh][4 * w + 2] = dot2bf(v2, pp[hh], acc[hh][4 * w + 2]);
              acc[hh][4 * w + 3] = dot2bf(v3, pp[hh], acc[hh][4 * w + 3]);
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < TPL; ++r) {
        // copy out of the vector first: bit-casting a vector element in place is not
        // reliable with this compiler (it reads element 0)
        float vf[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t bits = v[r][e / 4][e % 4];
          vf[e] = __builtin_bit_cast(float, bits);
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          l[hh] += pr[r][hh];
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[hh][e] = __builtin_fmaf(pr[r][hh], vf[e], acc[hh][e]);
        }
      }
    }
  };

  // Double-buffered software pipeline over this wave's tiles t = wave, wave+NW, ...:
  // two register sets, loads for one in flight while the other is computed.  Tile
  // indices past the wave's last tile are clamped to it (an L2-resident reload), so
  // every iteration issues the same loads and the wait counts stay static.
  if (wave < ntiles) {
    const int last = wave + ((ntiles - 1 - wave) / NW) * NW;   // this wave's last tile
    u32x4 kb[TPL][EB], vb[TPL][EB];
    load_tile(wave, kr, vr);
    for (int t = wave; t <= last; t += 2 * NW) {
      const int t1 = min(t + NW, last);
      const int t2 = min(t + 2 * NW, last);
      load_tile(t1, kb, vb);
      compute_tile(t, kr, vr);
      load_tile(t2, kr, vr);
      if (t + NW <= last) compute_tile(t + NW, kb, vb);
    }
  }

  // ---- epilogue: merge token groups k and k^1 of each 16-lane row (DPP) ----
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float mo = dpp<kDppRowRor8>(m[hh]);
    const float mn = fmaxf(m[hh], mo);
    const float a = fast_exp2(m[hh] - mn);
    m[hh] = mn;
    l[hh] *= a;
    l[hh] += dpp<kDppRowRor8>(l[hh]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc[hh][e] *= a;
      acc[hh][e] += dpp<kDppRowRor8>(acc[hh][e]);
    }
  }
  const int row16 = lane >> 4;
  if ((lane & 8) == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 16; ++e) s_acc[wave][row16][hh][elem_d<EB>(c, e)] = acc[hh][e];
    if (c == 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        s_m[wave][row16][hh] = m[hh];
        s_l[wave][row16][hh] = l[hh];
      }
    }
  }
  __syncthreads();

  float vscale = 1.f;
  if constexpr (KV == PA_FP8_E4M3) vscale = p.v_scale[g];
  const int S = p.num_partitions;
  for (int idx = threadIdx.x; idx < G * D; idx += NT) {
    const int hh = idx / D;
    const int d = idx % D;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int k = 0; k < 4; ++k) M = fmaxf(M, s_m[w][k][hh]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float wt = fast_exp2(s_m[w][k][hh] - M);
        num = __builtin_fmaf(wt, s_acc[w][k][hh][d], num);
        den = __builtin_fmaf(wt, s_l[w][k][hh], den);
      }
    num *= vscale;
    const int h = g * G + hh;
    if (S == 1) {
      store_out<OUT_BF16>(p.out, ((size_t)b * Hq + h) * D + d, num / den);
    } else {
      const size_t pi = ((size_t)b * Hq + h) * S + s;
      p.part_acc[pi * D + d] = num;
      if (d == 0) {
        p.part_m[pi] = M;
        p.part_l[pi] = den;
      }
    }
  }
}

// Combine the per-partition partials of one (row, query head): the
// log-sum-exp identity  o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
template <bool OUT_BF16>
__global__ __launch_bounds__(64) void merge_kernel(DecodeLaunch p) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int L = p.seq_lens[b];
  const int S = p.num_partitions;
  const int Sb = (L + p.partition_size - 1) / p.partition_size;
  const size_t base = ((size_t)b * p.num_q_heads + h) * S;
  float M = kNegBig;
  for (int s = 0; s < Sb; ++s) M = fmaxf(M, p.part_m[base + s]);
  float n0 = 0.f, n1 = 0.f, den = 0.f;
  for (int s = 0; s < Sb; ++s) {
    const float wt = fast_exp2(p.part_m[base + s] - M);
    den = __builtin_fmaf(wt, p.part_l[base + s], den);
    const float2 a = *reinterpret_cast<const float2 *>(p.part_acc + (base + s) * D + 2 * lane);
    n0 = __builtin_fmaf(wt, a.x, n0);
    n1 = __builtin_fmaf(wt, a.y, n1);
  }
  const size_t o = ((size_t)b * p.num_q_heads + h) * D + 2 * lane;
  store_out<OUT_BF16>(p.out, o, n0 / den);
  store_out<OUT_BF16>(p.out, o + 1, n1 / den);
}

template <int KV, int G>
int launch_kv_g(const DecodeLaunch &L, hipStream_t st) {
  dim3 grid(L.num_partitions, L.num_kv_heads, L.num_seqs);
  if (L.out_dtype == PA_BF16)
    hipLaunchKernelGGL((decode_kernel<KV, G, true>), grid, dim3(NT), 0, st, L);
  else
    hipLaunchKernelGGL((decode_kernel<KV, G, false>), grid, dim3(NT), 0, st, L);
  return (int)hipGetLastError();
}

template <int KV>
int launch_kv(const DecodeLaunch &L, hipStream_t st) {
  switch (L.num_q_heads / L.num_kv_heads) {
    case 1: return launch_kv_g<KV, 1>(L, st);
    case 2: return launch_kv_g<KV, 2>(L, st);
    case 4: return launch_kv_g<KV, 4>(L, st);
    case 8: return launch_kv_g<KV, 8>(L, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_decode_partials(const DecodeLaunch &L, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (L.kv_dtype) {
    case PA_F32: return launch_kv<PA_F32>(L, st);
    case PA_BF16: return launch_kv<PA_BF16>(L, st);
    case PA_FP8_E4M3: return launch_kv<PA_FP8_E4M3>(L, st);
  }
  return (int)hipErrorInvalidValue;
}

int launch_merge(const DecodeLaunch &L, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  dim3 grid(L.num_q_heads, L.num_seqs);
  if (L.out_dtype == PA_BF16)
    hipLaunchKernelGGL(merge_kernel<true>, grid, dim3(64), 0, st, L);
  else
    hipLaunchKernelGGL(merge_kernel<false>, grid, dim3(64), 0, st, L);
  return (int)hipGetLastError();
}

const char *hip_error_name(int code) { return hipGetErrorName(static_cast<hipError_t>(code)); }

}  // namespace pa
