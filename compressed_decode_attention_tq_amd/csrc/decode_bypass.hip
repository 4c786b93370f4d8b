// Split-K decode attention over uncompressed (bf16) layers (gfx950).
//
// "tiny-turboquant 0.18.0", "Knobs that actually move the needle": protected
// boundary layers keep full-precision K/V.  They are served by the same split-K
// decode as the compressed layers ("turbo-attn 0.24.0", "Configuration",
// TKV_DECODE_SPLITS): one workgroup per (split, KV head, sequence) serving all
// query heads of the KV head, partials (acc, m, l) merged by the combine launch,
// with plain scores s = scale * q.k.
//
// Page = 16 tokens of one KV head: K [16][128] bf16 token-major, then
// V^T [128][16] bf16 dim-major.  Both products of a page run on the matrix
// cores with the page's tokens as one tile:
//   S^T = K Q^T    16x16x32 bf16, 4 K-steps over the head dim.  A = the key rows
//                  (lane l: token l%16, dims 32s + 8(l/16) .. +7, 16 contiguous
//                  bytes); B = the query heads as columns, 2h the bf16 rounding
//                  of q_h * scale * log2(e) and 2h+1 the bf16 rounding of the
//                  remainder, so the head score is the sum of the column pair.
//   O^T += V^T P^T 16x16x16 bf16, 8 tiles over the head dim.  A = V^T rows
//                  (lane l: dim 16i + l%16, tokens 4(l/16) .. +3, 8 contiguous
//                  bytes); B = the probabilities, which the first product left in
//                  exactly this operand layout (lane l: tokens 4(l/16) + r of
//                  column l%16): column 2h carries p truncated to bf16, column
//                  2h+1 the truncated remainder (|error| < 2^-15 p).
// The softmax runs in base 2 with a lazily raised running max: a page only
// rescales the accumulators when its max exceeds the running max by more than
// kTau (probabilities stay below 2^kTau), which after the first pages of a
// context is rare.
#include <hip/hip_runtime.h>

#include <cmath>

#include "split_items.hpp"
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPart = kDim + 4;        // acc[128], m, l, pad, pad
constexpr unsigned kPageBytes = 8192;  // 16 x 128 bf16 keys + values
constexpr unsigned kValOff = 4096;
constexpr float kTau = 8.0f;           // lazy rescale threshold (log2 units)
// Pages in flight per wave while one is processed.
constexpr int kRing = 2;

struct BypassArgs {
  const unsigned char* pool;
  const int* seq_lens;
  const void* q;  // [B][Hq][128], bf16 or float32
  float* part;    // [B*Hq][n_splits][kPart]
  long long max_blocks;
  int Hq, Hkv, n_splits, split_tokens;
  int batch, work_list;  // item order of the grid (split_items.hpp)
  float qscale;  // softmax scale * log2(e)
};

__device__ __forceinline__ floatx4 mfma_qk(u32x4 k, bf16x8 q, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k), q, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_pv(u32x2 v, short4v p, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, v), p, c, 0, 0, 0);
}

// bf16 round-to-nearest-even of a finite float, as its 16-bit pattern.
__device__ __forceinline__ unsigned bf16_rne(float x) {
  const unsigned u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// x plus x of the other lane of its pair (lanes 2c, 2c+1); both lanes of a pair
// get the same bits.
__device__ __forceinline__ float pair_sum(float x) {
  const int y = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1 /* quad_perm [1,0,3,2] */, 0xF, 0xF,
                                         true);
  return x + __builtin_bit_cast(float, y);
}

// Max / sum over the four 16-lane rows (lanes c, c+16, c+32, c+48); every lane
// of a column gets the same bits.
__device__ __forceinline__ float rows_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__builtin_bit_cast(float, static_cast<unsigned>(a[0])), __builtin_bit_cast(float, static_cast<unsigned>(a[1])));
  const unsigned v = __builtin_bit_cast(unsigned, x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__builtin_bit_cast(float, static_cast<unsigned>(b[0])), __builtin_bit_cast(float, static_cast<unsigned>(b[1])));
}
__device__ __forceinline__ float rows_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __builtin_bit_cast(float, static_cast<unsigned>(a[0])) + __builtin_bit_cast(float, static_cast<unsigned>(a[1]));
  const unsigned v = __builtin_bit_cast(unsigned, x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __builtin_bit_cast(float, static_cast<unsigned>(b[0])) + __builtin_bit_cast(float, static_cast<unsigned>(b[1]));
}

struct Page {
  u32x4 k[4];  // K-step s: token l%16, dims 32s + 8(l/16) .. +7
  u32x2 v[8];  // tile i: dim 16i + l%16, tokens 4(l/16) .. +3
};

// One workgroup of four waves per (split, KV head g, sequence b); wave w takes
// the split's pages w, w + 4, w + 8, ...  The block table comes as its own
// read-only, non-aliased parameter.
template <int NREP, bool QBF16>
__global__ __launch_bounds__(256) void splitk_bypass_kernel(BypassArgs a, const int* __restrict__ btab) {
  const SplitItem item = split_item(a.seq_lens, a.batch, a.Hkv, a.split_tokens, a.n_splits, a.work_list != 0);
  if (item.b < 0) return;  // past the work list (the whole workgroup)
  const int split = item.split, g = item.g, b = item.b;
  const int start = split * a.split_tokens;

  __shared__ __attribute__((aligned(16))) float mbuf[4][NREP][kDim];
  __shared__ float mg_m[4][NREP], mg_l[4][NREP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const int head = col >> 1;
  const bool lo_col = (col & 1) != 0;
  const bool live = head < NREP;

  // Block ids of this wave's pages, one per lane (at most 64: a split spans at
  // most 4096 tokens = 256 pages over four waves), read before the sequence
  // length is known so that the two reads overlap; table entries past the
  // context (the index clamped to the row) are read but never used.
  // (The host launches no split kernel for a table of zero blocks per row.)
  int ids;
  {
    const long long pg = start / kPage + wave + 4 * lane;
    ids = btab[static_cast<long long>(b) * a.max_blocks + (pg < a.max_blocks ? pg : a.max_blocks - 1)];
  }

  // Query operand: K-step s holds dims 32s + 8kg .. +7 of column col (all
  // four K-steps' reads issued, then the sequence length tested, before any is
  // used).
  bf16x8 qb[4];
  int T;
  {
    const size_t qrow = (static_cast<size_t>(b) * a.Hq + g * NREP + (live ? head : 0)) * kDim + 8 * kg;
    constexpr int NW = QBF16 ? 1 : 2;  // 16-byte reads per K-step
    u32x4 raw[4][NW];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < NW; ++u) {
        if constexpr (QBF16)
          raw[s][u] = *reinterpret_cast<const u32x4*>(static_cast<const unsigned short*>(a.q) + qrow + 32 * s);
        else
          raw[s][u] = *reinterpret_cast<const u32x4*>(static_cast<const float*>(a.q) + qrow + 32 * s + 4 * u);
      }
    T = a.seq_lens[b];
    if (start >= T) {
      // the reads above stay ahead of this test (their results are not needed here)
      asm volatile("" ::"v"(ids));
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int u = 0; u < NW; ++u) asm volatile("" ::"v"(raw[s][u]));
      return;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (QBF16) {
          x[2 * e] = __uint_as_float(raw[s][0][e] << 16);
          x[2 * e + 1] = __uint_as_float(raw[s][0][e] & 0xffff0000u);
        } else {
          x[e] = __uint_as_float(raw[s][0][e]);
          x[4 + e] = __uint_as_float(raw[s][NW - 1][e]);
        }
      }
      unsigned h16[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = x[e] * a.qscale;
        const unsigned hi = bf16_rne(v);
        const unsigned lo = bf16_rne(v - __uint_as_float(hi << 16));
        h16[e] = live ? (lo_col ? lo : hi) : 0u;
      }
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = h16[2 * e] | (h16[2 * e + 1] << 16);
      qb[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int end = min(T, start + a.split_tokens);
  const int npg = (end - start + kPage - 1) / kPage;
  const int nj = npg > wave ? (npg - wave + 3) >> 2 : 0;

  const unsigned koff = col * 256 + kg * 16;
  const unsigned voff = kValOff + col * 32 + kg * 8;
  auto load = [&](Page& pg, int j) {
    const int blk = __builtin_amdgcn_readlane(ids, j);
    const unsigned char* base = a.pool + (static_cast<long long>(blk) * a.Hkv + g) * kPageBytes;
#pragma unroll
    for (int s = 0; s < 4; ++s) pg.k[s] = *reinterpret_cast<const u32x4*>(base + koff + 64 * s);
#pragma unroll
    for (int i = 0; i < 8; ++i) pg.v[i] = *reinterpret_cast<const u32x2*>(base + voff + 512 * i);
  };

  float m = -INFINITY, lsum = 0.0f;
  floatx4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  auto process = [&](Page& pg, int j) {
    floatx4 st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) st = mfma_qk(pg.k[s], qb[s], st);
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = pair_sum(st[r]);
    const int lim = end - (start + kPage * (wave + 4 * j));  // valid tokens of this page
    if (lim < kPage) {
      // masked tokens: no score, and their value bits (slots never written may
      // hold anything) replaced by zeros
      unsigned keep[2];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * kg + r >= lim) sc[r] = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        keep[h] = (4 * kg + 2 * h < lim ? 0x0000ffffu : 0u) | (4 * kg + 2 * h + 1 < lim ? 0xffff0000u : 0u);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pg.v[i][0] &= keep[0];
        pg.v[i][1] &= keep[1];
      }
    }
    const float pm = rows_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    if (__builtin_amdgcn_ballot_w64(pm > m + kTau)) {
      const float mn = fmaxf(m, pm);
      const float al = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= al;
      lsum *= al;
      m = mn;
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sc[r] - m);
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    unsigned pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float rem = p[r] - __uint_as_float(__float_as_uint(p[r]) & 0xffff0000u);
      pw[r] = __float_as_uint(lo_col ? rem : p[r]);  // the upper 16 bits are the operand
    }
    u32x2 pb;
    pb[0] = __builtin_amdgcn_perm(pw[1], pw[0], 0x07060302u);
    pb[1] = __builtin_amdgcn_perm(pw[3], pw[2], 0x07060302u);
    const short4v pv = __builtin_bit_cast(short4v, pb);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = mfma_pv(pg.v[i], pv, acc[i]);
  };

  if (nj > 0) {
    // Every step processes one page and loads one (past the wave's last page,
    // the last one again: a cached re-read) so that each wait leaves the
    // younger pages' loads outstanding.
    const int jmax = nj - 1;
    Page ring[kRing];
#pragma unroll
    for (int r = 0; r < kRing; ++r) load(ring[r], r < jmax ? r : jmax);
    int j0 = 0;
    for (; j0 + kRing <= nj; j0 += kRing) {
#pragma unroll
      for (int r = 0; r < kRing; ++r) {
        const int j = j0 + r;
        process(ring[r], j);
        load(ring[r], j + kRing < jmax ? j + kRing : jmax);
      }
    }
#pragma unroll
    for (int r = 0; r < kRing - 1; ++r)
      if (j0 + r < nj) process(ring[r], j0 + r);
  }

  // ---- per-wave results -> LDS, then merge the four waves
  const float ls = rows_sum(lsum);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[i][r] = pair_sum(acc[i][r]);
  if (live && !lo_col) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<floatx4*>(&mbuf[wave][head][16 * i + 4 * kg]) = acc[i];
    if (kg == 0) {
      mg_m[wave][head] = m;
      mg_l[wave][head] = ls;
    }
  }
  __syncthreads();
  for (int x = tid; x < NREP * kDim; x += 256) {
    const int h = x >> 7, d = x & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mg_m[w][h]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (mg_m[w][h] == -INFINITY) continue;
      const float e = __builtin_amdgcn_exp2f(mg_m[w][h] - M);
      num += e * mbuf[w][h][d];
      den += e * mg_l[w][h];
    }
    float* dst = a.part + (static_cast<size_t>(b * a.Hq + g * NREP + h) * a.n_splits + split) * kPart;
    dst[d] = num;
    if (d == 0) {
      dst[128] = M * 0.69314718055994531f;  // back to natural-log units for the combine
      dst[129] = den;
    }
  }
}

template <bool QBF16>
void* pick(int rep) {
  switch (rep) {
    case 1: return reinterpret_cast<void*>(&splitk_bypass_kernel<1, QBF16>);
    case 2: return reinterpret_cast<void*>(&splitk_bypass_kernel<2, QBF16>);
    case 4: return reinterpret_cast<void*>(&splitk_bypass_kernel<4, QBF16>);
    case 8: return reinterpret_cast<void*>(&splitk_bypass_kernel<8, QBF16>);
  }
  return nullptr;
}

}  // namespace

tq_status launch_splitk_bypass(const tq_layer* L, const DecodePlan& plan, const void* q, tq_dtype q_dtype,
                               const void* pool, const int* block_table, int max_blocks_per_seq,
                               const int* seq_lens, float softmax_scale, float* part, void* stream) {
  if (L->lay.block_bytes != kPageBytes)
    return fail(TQ_ERR_UNSUPPORTED, "store layout does not match the bypass decode's page layout");
  if (plan.split_tokens <= 0 || plan.split_tokens > kMaxSplitTokens || plan.split_tokens % kPage)
    return fail(TQ_ERR_UNSUPPORTED, "bypass decode: split of %d tokens", plan.split_tokens);
  BypassArgs a;
  a.pool = static_cast<const unsigned char*>(pool);
  a.seq_lens = seq_lens;
  a.q = q;
  a.part = part;
  a.max_blocks = max_blocks_per_seq;
  a.Hq = plan.n_q_heads;
  a.Hkv = L->cfg.n_kv_heads;
  a.n_splits = plan.n_splits;
  a.split_tokens = plan.split_tokens;
  a.batch = plan.batch;
  a.work_list = plan.work_list ? 1 : 0;
  a.qscale = softmax_scale * 1.4426950408889634f;
  void* fn = (q_dtype == TQ_BF16) ? pick<true>(plan.rep) : pick<false>(plan.rep);
  if (!fn) return fail(TQ_ERR_UNSUPPORTED, "no bypass decode kernel for rep=%d", plan.rep);
  const int* btab = block_table;
  void* args[] = {&a, &btab};
  const dim3 grid(static_cast<unsigned>(plan.n_splits * L->cfg.n_kv_heads * plan.batch));
  hipError_t e = hipLaunchKernel(fn, grid, dim3(256), args, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TQ_ERR_HIP, "decode split-K launch: %s", hipGetErrorString(e));
  return TQ_OK;
}

}  // namespace tq
