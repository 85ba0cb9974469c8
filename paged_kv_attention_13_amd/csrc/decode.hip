// Decode attention over a paged KV cache on gfx950 (CDNA4), VALU path (fp32 and bf16
// pools; FP8 pools run on the matrix-core multi-query kernel).
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
// Work decomposition.  Short rows (bounded by 1,024 tokens, worker count left
// to the library) run decode_unit_kernel: one workgroup per (row, kv head),
// its waves merged in LDS, no workspace and no merge launch (and, for
// pa_append_decode, the row's new token appended in the same launch); with
// fewer units than CUs each unit is cut over several workgroups instead, whose
// partials sit in fixed slots for the merge kernel.
// Otherwise the work is the flattened sequence of (row, kv head, 16-token
// tile) units, each unit preceded by a few virtual tiles that stand for its
// start-up cost, cut into equal contiguous ranges, one per worker wave; the
// launch holds about as many waves as the chip keeps resident, so there is
// no tail of late workgroups and no empty workgroup for short rows.  Each
// wave streams its range on its own (no LDS, no barriers).  A unit covered by
// one wave is finished and written directly; a unit cut by a range boundary
// leaves one partial (m, l, acc) per piece, which the merge kernel combines
// with the log-sum-exp identity --
// the split over the context named Flash-Decoding on the dileepadev page.
// Inside a wave, 8 lanes share one token: each lane holds 16 of its 128
// elements, loaded with 16-byte loads so that one load instruction covers
// eight whole 128-byte lines of a (block, head) page; three register sets
// keep two tiles in flight while the third is computed.  The Hq/Hkv query
// heads that share kv head g are processed together, so every K/V byte is
// read from HBM once per step.
//
// Arithmetic.  Q.K uses v_dot2c_f32_bf16 (bf16 pairs, fp32 accumulate); the
// 8 partial sums of a token are combined with three DPP adds (quad xor 1,
// quad xor 2, half-row mirror).  The softmax runs in the
// log2 domain in fp32 registers, one running (max, sum) per 8-lane token
// group, with lazy rescaling: the running max moves only when a tile's max
// exceeds it by more than 2^8, which keeps every exp2 argument <= 8 and makes
// the rescale branch (wave-uniform) rare.  P.V pairs two tokens per
// v_dot2c_f32_bf16 (P rounded to bf16, the softmax denominator summed from the
// same rounded values).  Tokens past the row's end are excluded by select and
// their V registers zeroed, so NaN in unused slots never reaches the result.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "checks.h"
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

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
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

// Inclusive prefix sum across the 64 lanes of a wave.
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

// CASCADE: each row covers only its tokens from kv_start[b] on (the rest of its cache
// is a shared prefix handled elsewhere), and every piece is left as a partial.
template <int KV, int G, bool OUT_BF16, bool CASCADE>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeLaunch p) {
  constexpr int EB = KvTraits<KV>::EB;
  constexpr int TPL = KvTraits<KV>::TPL;   // tokens per lane per tile
  constexpr int TILE = 8 * TPL;            // tokens per tile
  constexpr int DW = 4 * EB;               // dwords per token per lane
  constexpr bool kBf = KV != PA_F32;
  constexpr int NBUF = (KV == PA_F32 || G >= 8) ? 2 : 3;   // tiles held in registers

  const int lane = threadIdx.x & 63;
  // the wave index is uniform across the wave: keep it (and all work arithmetic) scalar
  const int worker = blockIdx.x * NW + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nworkers = p.num_workers;
  if (worker >= nworkers) return;
  const int B = p.num_seqs;
  const int Hq = p.num_q_heads;
  const int Hkv = p.num_kv_heads;
  const int c = lane & 7;                  // element slot inside the token row
  const int grp = lane >> 3;               // token group 0..7
  // tokens of row r this kernel covers
  auto span_of = [&](int r) -> int {
    if constexpr (CASCADE) return p.seq_lens[r] - p.kv_start[r];
    else return checked_len(p.seq_lens[r], p.max_len, p.check_flags);
  };

  // Each unit counts unit_cost extra virtual tiles ahead of its real ones: starting a
  // unit (query and block-table loads, filling and draining the load pipeline, the
  // store) costs about that much time, so a worker given many short units gets fewer
  // tiles.  Virtual tiles are never loaded; a worker whose range holds only a unit's
  // virtual tiles skips it.
  const int C = p.unit_cost;
  auto vtiles = [&](int span) -> int {
    const int t = (span + TILE - 1) / TILE;
    return t > 0 ? t + C : 0;
  };

  // ---- this worker's share of the flattened (row, kv head, virtual tile) space ----
  long long W = 0;
  int n_first = 0, incl_first = 0;         // the first 64 rows' counts, kept for the search below
  for (int base = 0; base < B; base += 64) {
    const int r = base + lane;
    const int n = r < B ? vtiles(span_of(r)) : 0;
    const int incl = wave_inclusive_scan(n, lane);
    if (base == 0) {
      n_first = n;
      incl_first = incl;
    }
    W += __builtin_amdgcn_readlane(incl, 63);
  }
  W *= Hkv;
  int nwk = nworkers;
  // the plan sized the launch for rows of max_seq_len; shorter rows get fewer, longer ranges
  if (p.workers_auto) nwk = (int)min((long long)nwk, max(1LL, W / p.min_tiles));
  // never more workers than tiles, so that every worker's range is non-empty and the
  // workers covering a unit are exactly the consecutive ones from its first to its last
  const int nw = (int)min((long long)nwk, W);
  if (worker >= nw) return;
  const long long x0 = (long long)worker * W / nw;
  const long long x1 = (long long)(worker + 1) * W / nw;
  // worker covering flattened tile index x: the largest w with w*W/nw <= x
  auto worker_of = [&](long long x) { return (int)(((x + 1) * nw - 1) / W); };

  // locate x0: row b whose units span [rowstart, rowstart + Hkv * n_b)
  int b = 0;
  long long rowstart = 0;
  {
    long long before = 0;
    for (int base = 0; base < B; base += 64) {
      const int r = base + lane;
      const int n = base == 0 ? n_first : (r < B ? vtiles(span_of(r)) : 0);
      const int incl = base == 0 ? incl_first : wave_inclusive_scan(n, lane);
      const long long lo = before + (long long)(incl - n) * Hkv;
      const long long hi = before + (long long)incl * Hkv;
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(x0 >= lo && x0 < hi && n > 0);
      if (hit != 0) {
        const int k = __builtin_ctzll(hit);
        b = base + k;
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
  const int lane_off = c * 16;

  int L = span_of(b);
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
    auto next_unit = [&]() {
      x += cntv;
      tv = 0;
      ustart += vnb;
      if (++g == Hkv) {
        g = 0;
        ++b;
        if (x < x1) {
          L = span_of(b);
          nb = (L + TILE - 1) / TILE;
          vnb = nb + C;
        }
      }
    };
    if (cnt <= 0) {
      next_unit();
      continue;
    }
    const int u = b * Hkv + g;
    if (t0 == 0 && lane == 0) {
      p.seg_first[u] = worker;
      p.seg_count[u] = worker_of(ustart + C + nb - 1) - worker + 1;
    }
    const bool whole = !CASCADE && t0 == 0 && cnt == nb;
    const int tok_begin = t0 * TILE;
    const int tok_end = min((t0 + cnt) * TILE, L);
    const int first_page = tok_begin >> log2bs;
    const int last_page = (tok_end - 1) >> log2bs;

    // block-table entries, one per lane, for a chunk of up to 64 pages
    const int skip_pages = CASCADE ? (p.kv_start[b] >> log2bs) : 0;
    const int32_t *trow = p.block_table + (size_t)b * p.max_blocks_per_seq + skip_pages;
    const int mb_last = p.max_blocks_per_seq - 1 - skip_pages;
    int chunk_base = first_page;
    int tbl = 0;

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
    const float qk_scale = p.scale * kLog2e;
    const char *kpool = static_cast<const char *>(p.k_pool) + (size_t)g * page_bytes;
    const char *vpool = static_cast<const char *>(p.v_pool) + (size_t)g * page_bytes;

    float m[G], l[G], acc[G][16];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      m[hh] = kNegBig;
      l[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[hh][e] = 0.f;
    }

    auto load_tile = [&](int t, u32x4 (&k)[TPL][EB], u32x4 (&v)[TPL][EB]) {
#pragma unroll
      for (int r = 0; r < TPL; ++r) {
        const int tok0 = tok_begin + t * TILE + 8 * r;
        const int page = min(tok0 >> log2bs, last_page);
        const int phys = checked_block(__builtin_amdgcn_readlane(tbl, page - chunk_base), p.num_blocks, p.check_flags);
        // scalar page base + 32-bit per-lane offset (global_load ... saddr form); the
        // cache is streamed once per step, so the loads are non-temporal (measured
        // ~10% more HBM bandwidth than cached loads on MI355X)
        const char *kp = kpool + (size_t)phys * phys_stride;
        const char *vp = vpool + (size_t)phys * phys_stride;
        const uint32_t off = (uint32_t)(((tok0 + grp) & (bs - 1)) * (D * EB) + lane_off);
#pragma unroll
        for (int j = 0; j < EB; ++j) {
          k[r][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kp + off + j * 128));
          v[r][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vp + off + j * 128));
        }
      }
    };

    auto compute_tile = [&](int t, const u32x4 (&k)[TPL][EB], u32x4 (&v)[TPL][EB]) {
      const int tile_start = tok_begin + t * TILE;
      float sc[TPL][G];
#pragma unroll
      for (int r = 0; r < TPL; ++r) {
        uint32_t kd[DW];
#pragma unroll
        for (int i = 0; i < DW; ++i) kd[i] = k[r][i / 4][i % 4];
        if constexpr (kBf) {
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) a = dot2bf(qb[hh][i], kd[i], a);
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
          float y = sc[r][hh];
          y += dpp<kDppXor1>(y);
          y += dpp<kDppXor2>(y);
          y += dpp<kDppHalfMirror>(y);
          sc[r][hh] = y * qk_scale;
        }
      // tokens at or past the segment end take no part
      if (tile_start + TILE > tok_end) {
#pragma unroll
        for (int r = 0; r < TPL; ++r) {
          if (tile_start + 8 * r + grp >= tok_end) {
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
        float y = sc[0][hh];
#pragma unroll
        for (int r = 1; r < TPL; ++r) y = fmaxf(y, sc[r][hh]);
        tmax[hh] = y;
        need |= y > m[hh] + kSlack;
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
        for (int w2 = 0; w2 < TPL / 2; ++w2) {
          const int r0 = 2 * w2, r1 = 2 * w2 + 1;
          uint32_t pp[G];
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            pp[hh] = pack_bf16(pr[r0][hh], pr[r1][hh]);
            l[hh] = dot2bf(pp[hh], kOnes, l[hh]);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t A = v[r0][i / 4][i % 4];
            const uint32_t Bv = v[r1][i / 4][i % 4];
            const uint32_t lo = __builtin_amdgcn_perm(Bv, A, 0x05040100u);
            const uint32_t hi = __builtin_amdgcn_perm(Bv, A, 0x07060302u);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
              acc[hh][2 * i] = dot2bf(lo, pp[hh], acc[hh][2 * i]);
              acc[hh][2 * i + 1] = dot2bf(hi, pp[hh], acc[hh][2 * i + 1]);
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

    // Software pipeline over tiles [ta, tb) with NBUF register sets: while one tile
    // is computed, the next NBUF-1 tiles are in flight.  Look-ahead loads past the
    // last tile are skipped: the loads do not allocate in the caches, so re-loading
    // the last tile would fetch it from HBM again.  Nothing else is loaded inside the
    // pipeline: a load there would make the compiler drain every load before each use
    // of the block-table register.
    auto run_tiles = [&](int ta, int tb) {
      u32x4 ka[TPL][EB], va[TPL][EB], kb[TPL][EB], vb[TPL][EB];
      load_tile(ta, ka, va);
      if constexpr (NBUF == 3) {
        u32x4 kc[TPL][EB], vc[TPL][EB];
        if (ta + 1 < tb) load_tile(ta + 1, kb, vb);
        for (int t = ta; t < tb; t += 3) {
          if (t + 2 < tb) load_tile(t + 2, kc, vc);
          compute_tile(t, ka, va);
          if (t + 3 < tb) load_tile(t + 3, ka, va);
          if (t + 1 < tb) compute_tile(t + 1, kb, vb);
          if (t + 4 < tb) load_tile(t + 4, kb, vb);
          if (t + 2 < tb) compute_tile(t + 2, kc, vc);
        }
      } else {
        for (int t = ta; t < tb; t += 2) {
          if (t + 1 < tb) load_tile(t + 1, kb, vb);
          compute_tile(t, ka, va);
          if (t + 2 < tb) load_tile(t + 2, ka, va);
          if (t + 1 < tb) compute_tile(t + 1, kb, vb);
        }
      }
    };
    // walk the segment in chunks of 64 pages (one block-table load per chunk); chunk
    // boundaries fall on multiples of 64 pages, which are tile boundaries.  The row's
    // first chunk is kept across units: the next unit is usually the next kv head of the
    // same row, which then starts without waiting for a table load.
    for (int ta = 0; ta < cnt;) {
      const int tb = min(cnt, (((chunk_base + 64) << log2bs) - tok_begin) / TILE);
      if (chunk_base == 0 && b == tbl0_row) {
        tbl = tbl0;
      } else {
        tbl = trow[min(chunk_base + lane, mb_last)];
        if (chunk_base == 0) {
          tbl0 = tbl;
          tbl0_row = b;
        }
      }
      run_tiles(ta, tb);
      ta = tb;
      chunk_base += 64;
    }

    // ---- merge the 8 token groups of the wave (log-sum-exp), then store ----
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float M = m[hh];
      M = fmaxf(M, dpp<kDppRowRor8>(M));
      M = fmaxf(M, __shfl_xor(M, 16));
      M = fmaxf(M, __shfl_xor(M, 32));
      const float a = fast_exp2(m[hh] - M);
      m[hh] = M;
      float lv = l[hh] * a;
      lv += dpp<kDppRowRor8>(lv);
      lv += __shfl_xor(lv, 16);
      lv += __shfl_xor(lv, 32);
      l[hh] = lv;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float y = acc[hh][e] * a;
        y += dpp<kDppRowRor8>(y);
        y += __shfl_xor(y, 16);
        y += __shfl_xor(y, 32);
        acc[hh][e] = y;
      }
    }
    constexpr float vscale = 1.f;
    // token group hh writes head hh (all 16 of its elements per lane)
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      if (grp != hh) continue;
      const int h = g * G + hh;
      if (whole) {
        const size_t base = ((size_t)b * Hq + h) * D;
#pragma unroll
        for (int e = 0; e < 16; ++e)
          store_out<OUT_BF16>(p.out, base + elem_d<EB>(c, e), acc[hh][e] * vscale / l[hh]);
      } else {
        const size_t slot = (size_t)(u + worker) * G + hh;
#pragma unroll
        for (int e = 0; e < 16; ++e) p.part_acc[slot * D + elem_d<EB>(c, e)] = acc[hh][e] * vscale;
        if (c == 0) {
          p.part_m[slot] = m[hh];
          p.part_l[slot] = l[hh];
        }
      }
    }

    next_unit();
  }
}

// Combine the partials of one (row, query head) whose unit was split across
// workers: o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
template <bool OUT_BF16>
__global__ __launch_bounds__(64) void merge_kernel(DecodeLaunch p) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int g = h / G;
  const int hh = h % G;
  const int u = b * p.num_kv_heads + g;
  // units cut over workgroups have their pieces at fixed slots (no record to read)
  const bool fixed = p.unit_mode && p.unit_pieces > 1;
  int cnt = fixed ? p.unit_pieces : p.seg_count[u];
  if (cnt <= 1) return;                    // written directly by its only worker
  // slots u + w exist for the launch's workers w in [0, num_workers): a record that does
  // not come from the partials launch on this workspace gives wrong numbers, never a read
  // outside it
  const int first = fixed ? u * (cnt - 1) : min(max(p.seg_first[u], 0), p.num_workers - 1);
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
        const size_t slot = (size_t)(u + first + k) * G + hh;
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
    const size_t o = ((size_t)b * p.num_q_heads + h) * D + 2 * lane;
    store_out<OUT_BF16>(p.out, o, n0 / den);
    store_out<OUT_BF16>(p.out, o + 1, n1 / den);
    return;
  }
  // the pieces' maxima, one per lane: one round trip however many pieces there are
  float M = kNegBig;
  for (int base = 0; base < cnt; base += 64)
    if (base + lane < cnt) M = fmaxf(M, p.part_m[(size_t)(u + first + base + lane) * G + hh]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  // then the pieces in order, eight at a time with all their loads issued before use
  for (int base = 0; base < cnt; base += 8) {
    float pm[8], pl[8];
    float2 pa[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (base + k < cnt) {
        const size_t slot = (size_t)(u + first + base + k) * G + hh;
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
  const size_t o = ((size_t)b * p.num_q_heads + h) * D + 2 * lane;
  store_out<OUT_BF16>(p.out, o, n0 / den);
  store_out<OUT_BF16>(p.out, o + 1, n1 / den);
}

// Short rows (at most 64 pages and kUnitMaxTokens tokens, as bounded by max_seq_len):
// one workgroup per (row, kv head) unit.  Its 8 (or 4) waves take consecutive shares of
// the unit's tiles and then combine their (max, sum, output) states in LDS with the same
// log-sum-exp identity as the merge kernel, so there is no workspace and no second
// launch.  The row's length, its block-table entries (all within the first 64) and
// its queries do not depend on each other, so they are loaded together before any
// KV load.  Per-tile arithmetic as in decode_kernel.
// APPEND: also append row b's new token (its K/V rows k_new/v_new[b]) at slot
// new_slots[b] and take position L - 1 from those rows instead of the pool: nothing in
// this launch reads the slot being written, and the values are the ones the slot gets.
template <int KV, int G, bool OUT_BF16, bool APPEND>
__global__ __launch_bounds__(unit_waves(KV, G) * 64) void decode_unit_kernel(DecodeLaunch p) {
  constexpr int NWU = unit_waves(KV, G);   // waves per workgroup
  constexpr int NTU = NWU * 64;
  constexpr int EB = KvTraits<KV>::EB;
  constexpr int TPL = KvTraits<KV>::TPL;
  constexpr int TILE = 8 * TPL;
  constexpr int DW = 4 * EB;
  constexpr bool kBf = KV != PA_F32;
  constexpr int NBUF = (KV == PA_F32 || G >= 8) ? 2 : 3;
  __shared__ float s_ml[NWU][G][2];
  __shared__ float s_acc[NWU][G][D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hq = p.num_q_heads;
  const int Hkv = p.num_kv_heads;
  const int S = p.unit_pieces;                   // workgroups per unit
  const int u = (int)blockIdx.x / S;
  const int piece = (int)blockIdx.x % S;
  const int b = u / Hkv;
  const int g = u % Hkv;
  const int c = lane & 7;
  const int grp = lane >> 3;

  // independent loads first
  const int L = checked_len(p.seq_lens[b], p.max_len, p.check_flags);
  const int tbl = p.block_table[(size_t)b * p.max_blocks_per_seq + min(lane, p.max_blocks_per_seq - 1)];
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

  int new_slot = -1;
  const char *knew = nullptr;
  const char *vnew = nullptr;
  if constexpr (APPEND) {
    new_slot = checked_slot(p.new_slots[b], p.num_blocks, p.block_size, p.check_flags);
    const size_t row_off = ((size_t)b * Hkv + g) * D * EB;
    knew = static_cast<const char *>(p.k_new) + row_off;
    vnew = static_cast<const char *>(p.v_new) + row_off;
  }

  // this workgroup's share of the unit's tiles, then each wave's share of that
  const int nb = (L + TILE - 1) / TILE;
  const int pt0 = piece * nb / S;
  const int pn = (piece + 1) * nb / S - pt0;
  const int t_lo = pt0 + wave * pn / NWU;
  const int t_hi = pt0 + (wave + 1) * pn / NWU;
  const int bs = p.block_size;
  const int log2bs = __builtin_ctz(bs);
  const size_t page_bytes = (size_t)bs * D * EB;
  const size_t phys_stride = (size_t)Hkv * page_bytes;
  const int lane_off = c * 16;
  const float qk_scale = p.scale * kLog2e;
  const char *kpool = static_cast<const char *>(p.k_pool) + (size_t)g * page_bytes;
  const char *vpool = static_cast<const char *>(p.v_pool) + (size_t)g * page_bytes;
  if constexpr (APPEND) {
    // the appended row: 16 bytes per lane of wave 0 of the unit's first workgroup (the
    // workgroup whose tiles reach position L - 1 takes that token from the new rows)
    if (piece == 0 && wave == 0 && new_slot >= 0 && lane < D * EB / 16) {
      const size_t dst = (size_t)(new_slot >> log2bs) * phys_stride + (size_t)g * page_bytes +
                         (size_t)(new_slot & (bs - 1)) * (D * EB) + 16 * lane;
      *reinterpret_cast<u32x4 *>(static_cast<char *>(p.k_pool_w) + dst) =
          *reinterpret_cast<const u32x4 *>(knew + 16 * lane);
      *reinterpret_cast<u32x4 *>(static_cast<char *>(p.v_pool_w) + dst) =
          *reinterpret_cast<const u32x4 *>(vnew + 16 * lane);
    }
  }

  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = kNegBig;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[hh][e] = 0.f;
  }

  if (t_hi > t_lo) {
    const int tok_begin = t_lo * TILE;
    const int tok_end = min(t_hi * TILE, L);
    const int last_page = (tok_end - 1) >> log2bs;

    auto load_tile = [&](int t, u32x4 (&k)[TPL][EB], u32x4 (&v)[TPL][EB]) {
#pragma unroll
      for (int r = 0; r < TPL; ++r) {
        const int tok0 = tok_begin + t * TILE + 8 * r;
        const int page = min(tok0 >> log2bs, last_page);
        const int phys = checked_block(__builtin_amdgcn_readlane(tbl, page), p.num_blocks, p.check_flags);
        const char *kp = kpool + (size_t)phys * phys_stride;
        const char *vp = vpool + (size_t)phys * phys_stride;
        const uint32_t off = (uint32_t)(((tok0 + grp) & (bs - 1)) * (D * EB) + lane_off);
        const char *ka = kp + off;
        const char *va = vp + off;
        if constexpr (APPEND) {
          if (new_slot >= 0 && tok0 + grp == L - 1) {
            ka = knew + lane_off;
            va = vnew + lane_off;
          }
        }
#pragma unroll
        for (int j = 0; j < EB; ++j) {
          k[r][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ka + j * 128));
          v[r][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(va + j * 128));
        }
      }
    };

    auto compute_tile = [&](int t, const u32x4 (&k)[TPL][EB], u32x4 (&v)[TPL][EB]) {
      const int tile_start = tok_begin + t * TILE;
      float sc[TPL][G];
#pragma unroll
      for (int r = 0; r < TPL; ++r) {
        uint32_t kd[DW];
#pragma unroll
        for (int i = 0; i < DW; ++i) kd[i] = k[r][i / 4][i % 4];
        if constexpr (kBf) {
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) a = dot2bf(qb[hh][i], kd[i], a);
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
#pragma unroll
      for (int r = 0; r < TPL; ++r)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float y = sc[r][hh];
          y += dpp<kDppXor1>(y);
          y += dpp<kDppXor2>(y);
          y += dpp<kDppHalfMirror>(y);
          sc[r][hh] = y * qk_scale;
        }
      if (tile_start + TILE > tok_end) {
#pragma unroll
        for (int r = 0; r < TPL; ++r) {
          if (tile_start + 8 * r + grp >= tok_end) {
#pragma unroll
            for (int hh = 0; hh < G; ++hh) sc[r][hh] = -__builtin_inff();
#pragma unroll
            for (int j = 0; j < EB; ++j) v[r][j] = u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
      float tmax[G];
      bool need = false;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float y = sc[0][hh];
#pragma unroll
        for (int r = 1; r < TPL; ++r) y = fmaxf(y, sc[r][hh]);
        tmax[hh] = y;
        need |= y > m[hh] + kSlack;
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
      if constexpr (kBf) {
        constexpr uint32_t kOnes = 0x3F803F80u;
#pragma unroll
        for (int w2 = 0; w2 < TPL / 2; ++w2) {
          const int r0 = 2 * w2, r1 = 2 * w2 + 1;
          uint32_t pp[G];
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            pp[hh] = pack_bf16(pr[r0][hh], pr[r1][hh]);
            l[hh] = dot2bf(pp[hh], kOnes, l[hh]);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t A = v[r0][i / 4][i % 4];
            const uint32_t Bv = v[r1][i / 4][i % 4];
            const uint32_t lo = __builtin_amdgcn_perm(Bv, A, 0x05040100u);
            const uint32_t hi = __builtin_amdgcn_perm(Bv, A, 0x07060302u);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
              acc[hh][2 * i] = dot2bf(lo, pp[hh], acc[hh][2 * i]);
              acc[hh][2 * i + 1] = dot2bf(hi, pp[hh], acc[hh][2 * i + 1]);
            }
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < TPL; ++r) {
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

    const int cnt = t_hi - t_lo;
    u32x4 ka[TPL][EB], va[TPL][EB], kb[TPL][EB], vb[TPL][EB];
    load_tile(0, ka, va);
    if constexpr (NBUF == 3) {
      u32x4 kc[TPL][EB], vc[TPL][EB];
      if (1 < cnt) load_tile(1, kb, vb);
      for (int t = 0; t < cnt; t += 3) {
        if (t + 2 < cnt) load_tile(t + 2, kc, vc);
        compute_tile(t, ka, va);
        if (t + 3 < cnt) load_tile(t + 3, ka, va);
        if (t + 1 < cnt) compute_tile(t + 1, kb, vb);
        if (t + 4 < cnt) load_tile(t + 4, kb, vb);
        if (t + 2 < cnt) compute_tile(t + 2, kc, vc);
      }
    } else {
      for (int t = 0; t < cnt; t += 2) {
        if (t + 1 < cnt) load_tile(t + 1, kb, vb);
        compute_tile(t, ka, va);
        if (t + 2 < cnt) load_tile(t + 2, ka, va);
        if (t + 1 < cnt) compute_tile(t + 1, kb, vb);
      }
    }

    // merge the 8 token groups of the wave
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float M = m[hh];
      M = fmaxf(M, dpp<kDppRowRor8>(M));
      M = fmaxf(M, __shfl_xor(M, 16));
      M = fmaxf(M, __shfl_xor(M, 32));
      const float a = fast_exp2(m[hh] - M);
      m[hh] = M;
      float lv = l[hh] * a;
      lv += dpp<kDppRowRor8>(lv);
      lv += __shfl_xor(lv, 16);
      lv += __shfl_xor(lv, 32);
      l[hh] = lv;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float y = acc[hh][e] * a;
        y += dpp<kDppRowRor8>(y);
        y += __shfl_xor(y, 16);
        y += __shfl_xor(y, 32);
        acc[hh][e] = y;
      }
    }
  }

  // every wave (one with no tiles holds max -1e30, sum 0, zeros) publishes its state;
  // token group hh writes head hh
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    if (grp != hh) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) s_acc[wave][hh][elem_d<EB>(c, e)] = acc[hh][e];
    if (c == 0) {
      s_ml[wave][hh][0] = m[hh];
      s_ml[wave][hh][1] = l[hh];
    }
  }
  __syncthreads();
  // a unit cut over several workgroups: its pieces take the fixed slots u * S + piece, which
  // the merge kernel reads without piece records (a piece without tiles leaves max -1e30,
  // sum 0)
  for (int i = threadIdx.x; i < G * D; i += NTU) {
    const int hh = i / D;
    const int d = i % D;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < NWU; ++w) M = fmaxf(M, s_ml[w][hh][0]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NWU; ++w) {
      const float wt = fast_exp2(s_ml[w][hh][0] - M);
      den = __builtin_fmaf(wt, s_ml[w][hh][1], den);
      num = __builtin_fmaf(wt, s_acc[w][hh][d], num);
    }
    if (S > 1) {
      const size_t slot = (size_t)(u * S + piece) * G + hh;
      p.part_acc[slot * D + d] = num;
      if (d == 0) {
        p.part_m[slot] = M;
        p.part_l[slot] = den;
      }
    } else {
      store_out<OUT_BF16>(p.out, ((size_t)b * Hq + g * G + hh) * D + d, num / den);
    }
  }
}

template <int KV, int G>
int launch_kv_g(const DecodeLaunch &L, hipStream_t st) {
  if (L.unit_mode) {
    if (L.kv_start) return (int)hipErrorInvalidValue;
    if (L.unit_pieces < 1 || (L.unit_pieces > 1 && !L.part_acc)) return (int)hipErrorInvalidValue;
    dim3 ugrid((unsigned)L.num_seqs * L.num_kv_heads * (unsigned)L.unit_pieces);
    dim3 ublock(unit_waves(KV, G) * 64);
    if (L.k_new) {
      if (!L.v_new || !L.new_slots || !L.k_pool_w || !L.v_pool_w) return (int)hipErrorInvalidValue;
      if (L.out_dtype == PA_BF16)
        hipLaunchKernelGGL((decode_unit_kernel<KV, G, true, true>), ugrid, ublock, 0, st, L);
      else
        hipLaunchKernelGGL((decode_unit_kernel<KV, G, false, true>), ugrid, ublock, 0, st, L);
    } else if (L.out_dtype == PA_BF16) {
      hipLaunchKernelGGL((decode_unit_kernel<KV, G, true, false>), ugrid, ublock, 0, st, L);
    } else {
      hipLaunchKernelGGL((decode_unit_kernel<KV, G, false, false>), ugrid, ublock, 0, st, L);
    }
    return (int)hipGetLastError();
  }
  dim3 grid((L.num_workers + NW - 1) / NW);
  if constexpr (KV == PA_BF16) {
    if (L.kv_start) {
      if (L.out_dtype == PA_BF16)
        hipLaunchKernelGGL((decode_kernel<KV, G, true, true>), grid, dim3(NT), 0, st, L);
      else
        hipLaunchKernelGGL((decode_kernel<KV, G, false, true>), grid, dim3(NT), 0, st, L);
      return (int)hipGetLastError();
    }
  }
  if (L.out_dtype == PA_BF16)
    hipLaunchKernelGGL((decode_kernel<KV, G, true, false>), grid, dim3(NT), 0, st, L);
  else
    hipLaunchKernelGGL((decode_kernel<KV, G, false, false>), grid, dim3(NT), 0, st, L);
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
  }
  return (int)hipErrorInvalidValue;
}

int launch_merge(const DecodeLaunch &L, void *stream) {
  if (L.unit_mode && L.unit_pieces == 1) return 0;   // the unit kernel wrote every output itself
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
