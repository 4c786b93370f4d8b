// Split-K paged decode attention over the compressed store (gfx950).
//
// "turbo-attn 0.24.0", "How it works": since the head's rotation is orthogonal,
// attention of the rotated query over the rotated store equals the original
// attention; the decode reads the packed records and forms scores, softmax and
// the value sum in one kernel, never writing an expanded copy of the cache.
// "turbo-attn 0.24.0", "Configuration" (TKV_DECODE_SPLITS) and "tiny-turboquant
// 0.18.0", "Fused decode-attention path": the context is split across
// workgroups whose partials are merged by a second launch.
// "How 0xsero/turboquant works", "Key Storage and Attention Scoring": scores come
// from the compressed keys alone:
//   s_i = scale * (n_i / sqrt d) * (q'.c[idx_i] + sqrt(pi/2)/m * gamma_i * u.(2 z_i - 1)),
//   q' = R_g q, u = S_g q'  (QJL residual estimator).
//
// Launch 1 (prologue, compressed layers): q', u per (sequence, query head)
//   into the workspace.
// Launch 2 (split-K):  one workgroup per (split, KV head, sequence) serves all
//   query heads of its KV head so the KV is read once (the compressed mainloop
//   is in decode_mainloop.hip, the uncompressed one in decode_bypass.hip).
// Launch 3 (combine): merge the split partials with the running-max rescaling,
//   un-rotate o = R_g^T o', cast and store.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "tq_internal.hpp"

namespace tq {
namespace {

constexpr int kPart = kDim + 4;  // acc[128], m, l, pad, pad

// ---------------------------------------------------------------- prologue
// q' = R_g q and u = S_g q' = (S_g R_g) q: both are products of q itself with
// a fixed matrix, W = [R_g; P_g] (256 x 128, P_g = S_g R_g formed once per
// layer), so they run side by side on the matrix core with no dependency
// between them.  The outputs are written as the Q.K operand of the split-K
// mainloop (qa): q' and kappa*u split into float16 hi + lo pieces, placed as
// rows of the matrix-core A operand.  Dim i of a row sits in lane
// row + 16 (i / 32), K-step (i % 32) / 8, element i % 8.  Rows (R = query heads
// per KV head, h = head within the group):
//   R <= 4: one tile, rows part*R + h for parts q' hi, q' lo, ku hi, ku lo
//           (rows 4R..15 zero)
//   R == 8: tile 0 rows h / 8+h = q' hi / lo, tile 1 the same for kappa*u.
//
// Out = Q W^T on v_mfma_f32_16x16x32_f16: the 16 rows of a tile are 16 / R
// sequences x R query heads of KV head g; column tile t (16 of them) is
// output coordinates 16t..16t+15 of W.  Q and W are split into float16 hi + lo
// pieces (22 significant bits) and Q_hi W_hi + Q_hi W_lo + Q_lo W_hi is
// accumulated in float32 (each instruction sums its exact products and rounds
// once).  Workgroup (g, sequence group, z) is four independent waves, wave w
// taking column tile 4z + w: twelve matrix-core instructions, no LDS, no
// barrier.  W's pieces are stored per (head, tile, K-step, piece) in the
// lane order of the B operand, one 16-byte read per lane.
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool QBF16>
__global__ __launch_bounds__(256) void prologue_kernel(const void* q, const u32x4* __restrict__ opq,
                                                       unsigned short* qa, int B, int Hq, int rep, float kappa) {
  const int g = blockIdx.x, Hkv = gridDim.x;
  const int lane = threadIdx.x & 63;
  const int t = 4 * blockIdx.z + (threadIdx.x >> 6);  // column tile
  const int col = lane & 15, kg = lane >> 4;
  const int spg = 16 / rep;  // sequences per tile
  const int b0 = blockIdx.y * spg;
  // W pieces of this tile: [4 K-steps][hi, lo], issued first
  u32x4 wv[4][2];
  {
    const u32x4* src = opq + (static_cast<size_t>(g) * 16 + t) * 4 * 2 * 64 + lane;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      wv[s][0] = src[(2 * s) * 64];
      wv[s][1] = src[(2 * s + 1) * 64];
    }
  }
  // Q row m = lane % 16: sequence b0 + m / rep, head g*rep + m % rep; dims 32s + 8kg .. +7
  half8 qh[4], ql[4];
  {
    const int bq = b0 + col / rep;
    const bool ok = bq < B;
    const size_t row = static_cast<size_t>(ok ? bq : 0) * Hq + g * rep + col % rep;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8];
      if constexpr (QBF16) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const unsigned short*>(q) + row * 128 + 32 * s + 8 * kg);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = __uint_as_float(v[e] << 16);
          x[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
        }
      } else {
        const float* p = static_cast<const float*>(q) + row * 128 + 32 * s + 8 * kg;
        const floatx4 a = *reinterpret_cast<const floatx4*>(p);
        const floatx4 c = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = a[e];
          x[4 + e] = c[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = ok ? x[e] : 0.0f;
        const _Float16 hi = static_cast<_Float16>(v);
        qh[s][e] = hi;
        ql[s][e] = static_cast<_Float16>(v - static_cast<float>(hi));
      }
    }
  }
  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const half8 wh = __builtin_bit_cast(half8, wv[s][0]);
    const half8 wl = __builtin_bit_cast(half8, wv[s][1]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[s], wh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[s], wl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql[s], wh, acc, 0, 0, 0);
  }
  // lane (col, kg) holds rows 4kg + r of column 16t + col
  const bool is_u = t >= 8;
  const int d = 16 * (t & 7) + col;
  const int nset = rep == 8 ? 2 : 1;
  const int kgi = d >> 5, ks = (d >> 3) & 3, j = d & 7;
  auto put = [&](int b, int set, int row, _Float16 v) {
    const size_t at = ((((static_cast<size_t>(b) * Hkv + g) * nset + set) * 4 + ks) * 64 + row + 16 * kgi) * 8 + j;
    qa[at] = __builtin_bit_cast(unsigned short, v);
  };
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * kg + r;
    const int b = b0 + m / rep, h = m % rep;
    if (b >= B) continue;
    const float v = is_u ? kappa * acc[r] : acc[r];
    const _Float16 hi = static_cast<_Float16>(v);
    const _Float16 lo = static_cast<_Float16>(v - static_cast<float>(hi));
    if (rep == 8) {
      put(b, is_u ? 1 : 0, h, hi);
      put(b, is_u ? 1 : 0, 8 + h, lo);
    } else {
      put(b, 0, (is_u ? 2 * rep : 0) + h, hi);
      put(b, 0, (is_u ? 3 * rep : rep) + h, lo);
    }
  }
  // rows 4R..15 of a one-tile operand are zero (column tiles 0..7 cover the dims)
  if (rep < 4 && !is_u) {
    const int nz = 16 - 4 * rep;
    for (int x = kg; x < spg * nz; x += 4) {
      const int b = b0 + x / nz, row = 4 * rep + x % nz;
      if (b < B) put(b, 0, row, static_cast<_Float16>(0.0f));
    }
  }
}

// ---------------------------------------------------------------- combine
// o'[d] of one query head from its ns split partials p[s] = (acc[128], m, l):
// sum_s e^{m_s - M} acc_s[d] / sum_s e^{m_s - M} l_s.  Splits are taken 8 at a
// time with all of a group's reads issued before any is used (one memory round
// trip per group), merged with a running max.
struct Group8 {
  float m[8], l[8], a[8];
};
// Reads of splits s0 .. s0+7 (indices clamped to below `lim`; entries past the
// sequence's splits are read but never used).
// `stride` is the distance in floats between consecutive splits of p.
__device__ __forceinline__ void read_group(const float* p, int s0, int lim, int d, Group8& g, int stride = kPart) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const float* q = p + (s0 + u < lim ? s0 + u : s0) * stride;
    g.m[u] = q[128];
    g.l[u] = q[129];
    g.a[u] = q[d];
  }
}
__device__ __forceinline__ void merge_group(const Group8& g, int s0, int ns, float& M, float& num, float& den) {
  float mg = M;
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (s0 + u < ns) mg = fmaxf(mg, g.m[u]);
  const float f = (M == -INFINITY) ? 0.0f : __expf(M - mg);
  num *= f;
  den *= f;
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (s0 + u < ns) {
      const float e = __expf(g.m[u] - mg);
      num = fmaf(e, g.a[u], num);
      den = fmaf(e, g.l[u], den);
    }
  M = mg;
}
// `first` holds the reads of splits 0..7, issued before ns was known.  The
// rest are read four groups (32 splits) at a time, all reads of a round issued
// before any is merged: one memory round trip per 32 splits.
__device__ __forceinline__ float merge_partials(const float* p, int ns, int d, const Group8& first) {
  float M = -INFINITY, num = 0.0f, den = 0.0f;
  merge_group(first, 0, ns, M, num, den);
  for (int s0 = 8; s0 < ns; s0 += 32) {
    Group8 g[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s0 + 8 * u < ns) read_group(p, s0 + 8 * u, ns, d, g[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s0 + 8 * u < ns) merge_group(g[u], s0 + 8 * u, ns, M, num, den);
  }
  return num / den;
}


// One workgroup of 512 lanes per (KV head g, sequence b): merge each query
// head's split partials with the running-max rescaling, then o = R_g^T o'
// (compressed layers; lane (c, i) holds column i of rows 32c..32c+31 of R_g
// and the quarters are summed through LDS in a fixed order), cast and store.
template <bool OUT_BF16, bool BYPASS>
__global__ __launch_bounds__(512) void combine_kernel(const float* part, const int* seq_lens, const float* R,
                                                      void* out, int Hq, int rep, int n_splits,
                                                      int split_tokens) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, c = tid >> 7, i = tid & 127;
  const int n = rep * 128;
  const int bh0 = b * Hq + g * rep;
  // The first group of partials (at most two outputs per lane: rep <= 8) is
  // read before the sequence length, so that the two reads overlap.
  Group8 first[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int o = tid + 512 * k;
    if (o < n)
      read_group(part + static_cast<size_t>(bh0 + (o >> 7)) * n_splits * kPart, 0, n_splits, o & 127, first[k]);
  }
  const int T = seq_lens[b];
  // (a length above max_seq_len, a caller error, reads no partial past the workspace)
  const int ns = T > 0 ? min((T + split_tokens - 1) / split_tokens, n_splits) : 0;
  __shared__ float so[8][128], pr[4][8][128];
  float rr[32];
  if constexpr (!BYPASS) {
    const float* r = R + static_cast<size_t>(g) * 128 * 128 + (32 * c) * 128 + i;
#pragma unroll
    for (int u = 0; u < 32; ++u) rr[u] = r[u * 128];
  }
  auto store = [&](int h, int d, float o) {
    const size_t at = static_cast<size_t>(bh0 + h) * 128 + d;
    if constexpr (OUT_BF16) {
      const unsigned u = __float_as_uint(o);
      static_cast<unsigned short*>(out)[at] = static_cast<unsigned short>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    } else {
      static_cast<float*>(out)[at] = o;
    }
  };
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int o = tid + 512 * k;
    if (o < n) {
      const int h = o >> 7, d = o & 127;
      const float v =
          ns > 0 ? merge_partials(part + static_cast<size_t>(bh0 + h) * n_splits * kPart, ns, d, first[k]) : 0.0f;
      if constexpr (BYPASS) store(h, d, v);
      else so[h][d] = v;
    }
  }
  if constexpr (!BYPASS) {
    __syncthreads();
    for (int h = 0; h < rep; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int u = 0; u < 32; ++u) acc = fmaf(rr[u], so[h][32 * c + u], acc);
      pr[c][h][i] = acc;
    }
    __syncthreads();
    for (int o = tid; o < n; o += 512) {
      const int h = o >> 7, d = o & 127;
      store(h, d, (pr[0][h][d] + pr[1][h][d]) + (pr[2][h][d] + pr[3][h][d]));
    }
  }
}

// Small batches over many splits: one 512-lane workgroup per (KV head g,
// sequence b, query head h).  Quarter c of the lanes (lane (c, i) holds dim i)
// merges the head's splits c, c + 4, c + 8, ...: its first 16 splits are read
// before the sequence length and the rest 32 at a time, so up to 64 splits take
// one memory round trip.  The four quarters' running maxima and sums are merged
// in LDS, then o = R_g^T o' is formed as in combine_kernel (lane (c, i) holds a
// quarter of column i of R_g, the quarters summed in LDS in a fixed order).
template <bool OUT_BF16, bool BYPASS>
__global__ __launch_bounds__(512) void combine_head_kernel(const float* part, const int* seq_lens, const float* R,
                                                           void* out, int Hq, int rep, int n_splits,
                                                           int split_tokens) {
  const int g = blockIdx.x, b = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, c = tid >> 7, i = tid & 127;
  const int bh = b * Hq + g * rep + h;
  // quarter c's splits c + 4j: a slice of the head's partials with a 4-split stride
  const float* p = part + (static_cast<size_t>(bh) * n_splits + c) * kPart;
  const int stride = 4 * kPart;
  const int lim = n_splits > c ? (n_splits - c + 3) / 4 : 0;  // quarter c's splits in the workspace
  Group8 first[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (8 * k < lim) read_group(p, 8 * k, lim, i, first[k], stride);
  float rr[32];
  if constexpr (!BYPASS) {
    const float* r = R + static_cast<size_t>(g) * 128 * 128 + (32 * c) * 128 + i;
#pragma unroll
    for (int u = 0; u < 32; ++u) rr[u] = r[u * 128];
  }
  const int T = seq_lens[b];
  // (a length above max_seq_len, a caller error, reads no partial past the workspace)
  const int ns = T > 0 ? min((T + split_tokens - 1) / split_tokens, n_splits) : 0;
  const int nq = ns > c ? (ns - c + 3) / 4 : 0;  // quarter c's splits of this sequence (nq <= lim)
  float M = -INFINITY, num = 0.0f, den = 0.0f;
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (8 * k < nq) merge_group(first[k], 8 * k, nq, M, num, den);
  for (int s0 = 16; s0 < nq; s0 += 32) {
    Group8 gr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s0 + 8 * u < nq) read_group(p, s0 + 8 * u, nq, i, gr[u], stride);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s0 + 8 * u < nq) merge_group(gr[u], s0 + 8 * u, nq, M, num, den);
  }
  __shared__ float qm[4], qd[4], qn[4][128], so[128], pr[4][128];
  if (i == 0) {
    qm[c] = M;
    qd[c] = den;
  }
  qn[c][i] = num;
  __syncthreads();
  // every quarter forms o'[i] from the same LDS values; quarter 0 keeps it
  float o = 0.0f;
  const float Mx = fmaxf(fmaxf(qm[0], qm[1]), fmaxf(qm[2], qm[3]));
  if (Mx > -INFINITY) {
    float nn = 0.0f, dd = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float e = qm[k] == -INFINITY ? 0.0f : __expf(qm[k] - Mx);
      nn = fmaf(e, qn[k][i], nn);
      dd = fmaf(e, qd[k], dd);
    }
    o = nn / dd;
  }
  auto store = [&](float v) {
    const size_t at = static_cast<size_t>(bh) * 128 + i;
    if constexpr (OUT_BF16) {
      const unsigned u = __float_as_uint(v);
      static_cast<unsigned short*>(out)[at] = static_cast<unsigned short>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    } else {
      static_cast<float*>(out)[at] = v;
    }
  };
  if constexpr (BYPASS) {
    if (c == 0) store(o);
  } else {
    if (c == 0) so[i] = o;
    __syncthreads();
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < 32; ++u) acc = fmaf(rr[u], so[32 * c + u], acc);
    pr[c][i] = acc;
    __syncthreads();
    if (c == 0) store((pr[0][i] + pr[1][i]) + (pr[2][i] + pr[3][i]));
  }
}

}  // namespace

tq_status launch_decode(const tq_layer* L, const DecodePlan& plan, const void* q, tq_dtype q_dtype,
                        const void* pool, const int* block_table, int max_blocks_per_seq,
                        const int* seq_lens, float softmax_scale, void* out, tq_dtype out_dtype,
                        void* workspace, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bypass = L->cfg.bypass != 0;
  char* ws = static_cast<char*>(workspace);
  float* part = reinterpret_cast<float*>(ws + plan.ws_part);

  // 1. prologue (compressed layers; the bypass kernel reads q itself)
  if (!bypass && max_blocks_per_seq > 0) {
    void* fn = (q_dtype == TQ_BF16) ? reinterpret_cast<void*>(&prologue_kernel<true>)
                                    : reinterpret_cast<void*>(&prologue_kernel<false>);
    const u32x4* opq = reinterpret_cast<const u32x4*>(L->dOpQ);
    unsigned short* qa = reinterpret_cast<unsigned short*>(ws + plan.ws_qa);
    int B = plan.batch, Hq = plan.n_q_heads, rep = plan.rep;
    // sqrt(pi/2) / m, m = d; 0 for the key modes without QJL, whose split-K
    // kernels then see zero projection rows in the query operand
    float kappa = L->cfg.key_mode == TQ_KEY_QJL ? static_cast<float>(std::sqrt(M_PI / 2.0) / kDim) : 0.0f;
    void* args[] = {const_cast<void**>(&q), &opq, &qa, &B, &Hq, &rep, &kappa};
    const int spg = 16 / rep;
    ProfScope prof(kKPrologue, stream);
    hipError_t e = hipLaunchKernel(fn, dim3(L->cfg.n_kv_heads, (plan.batch + spg - 1) / spg, 4), dim3(256), args, 0, s);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "decode prologue launch: %s", hipGetErrorString(e));
  }
  // 2. split-K mainloop (a table with no blocks per row means every sequence is
  //    empty: the combine alone writes the zero output)
  if (max_blocks_per_seq > 0) {
    ProfScope prof(kKSplitK, stream);
    tq_status st = bypass ? launch_splitk_bypass(L, plan, q, q_dtype, pool, block_table, max_blocks_per_seq,
                                                 seq_lens, softmax_scale, part, stream)
                          : launch_splitk_tq(L, plan, pool, block_table, max_blocks_per_seq, seq_lens,
                                             softmax_scale, ws + plan.ws_qa, part, stream);
    if (st != TQ_OK) return st;
  }
  // 3. combine + un-rotation.  Many splits over few (sequence, query head)
  // rows: one workgroup per query head, the splits shared by four lane quarters;
  // otherwise one workgroup per (sequence, KV head).
  {
    const bool per_head =
        plan.n_splits > 8 && static_cast<long long>(plan.batch) * plan.n_q_heads <= 2LL * std::max(L->cu_count, 1);
    void* fn;
    if (per_head) {
      if (bypass) fn = (out_dtype == TQ_BF16) ? reinterpret_cast<void*>(&combine_head_kernel<true, true>)
                                              : reinterpret_cast<void*>(&combine_head_kernel<false, true>);
      else fn = (out_dtype == TQ_BF16) ? reinterpret_cast<void*>(&combine_head_kernel<true, false>)
                                       : reinterpret_cast<void*>(&combine_head_kernel<false, false>);
    } else {
      if (bypass) fn = (out_dtype == TQ_BF16) ? reinterpret_cast<void*>(&combine_kernel<true, true>)
                                              : reinterpret_cast<void*>(&combine_kernel<false, true>);
      else fn = (out_dtype == TQ_BF16) ? reinterpret_cast<void*>(&combine_kernel<true, false>)
                                       : reinterpret_cast<void*>(&combine_kernel<false, false>);
    }
    const float* R = L->dR;
    int Hq = plan.n_q_heads, rep = plan.rep, ns = plan.n_splits, st = plan.split_tokens;
    void* args[] = {&part, const_cast<int**>(&seq_lens), &R, &out, &Hq, &rep, &ns, &st};
    const dim3 grid = per_head ? dim3(L->cfg.n_kv_heads, plan.batch, plan.rep) : dim3(L->cfg.n_kv_heads, plan.batch);
    ProfScope prof(kKCombine, stream);
    hipError_t e = hipLaunchKernel(fn, grid, dim3(512), args, 0, s);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "decode combine launch: %s", hipGetErrorString(e));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TQ_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return TQ_OK;
}

// ------------------------------------------------ allocation-free decode
// The decode workspace of tq_decode_attn_noalloc: a fixed array in device
// memory, one per GPU the library runs on, held until the process ends.  Host
// code never uses the array's name as an address (in host code it is only a
// stand-in for the symbol): the device address comes from hipGetSymbolAddress,
// taken once per device with that device current and kept in g_scratch_ptr.
// Every call on a GPU uses that GPU's array, so calls that overlap on one GPU
// (on different streams) race; nothing in it needs clearing between calls (each
// launch writes what the next one reads: the prologue all query operands, each
// split its partials, and the combine reads only the splits that ran).
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

tq_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TQ_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(TQ_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TQ_OK;
}
}  // namespace

}  // namespace tq

extern "C" tq_status tq_decode_attn_noalloc(const tq_layer* L, const void* q, tq_dtype q_dtype, int batch,
                                            int n_q_heads, const void* pool, long long num_blocks,
                                            const int* block_table, int max_blocks_per_seq, const int* seq_lens,
                                            int max_seq_len, float softmax_scale, int num_splits, void* out,
                                            tq_dtype out_dtype, void* hip_stream) {
  using namespace tq;
  clear_error();
  DecodePlan p;
  float scale = 0.0f;
  tq_status st = prepare_decode(L, q, q_dtype, batch, n_q_heads, pool, num_blocks, block_table, max_blocks_per_seq,
                                seq_lens, max_seq_len, softmax_scale, num_splits, out, out_dtype, &p, &scale);
  if (st != TQ_OK || batch == 0) return st;
  if (p.ws_bytes > kScratchBytes)
    return fail(TQ_ERR_UNSUPPORTED,
                "decode workspace of %zu bytes exceeds the %zu-byte static scratch of tq_decode_attn_noalloc "
                "(use tq_decode_attn with a caller workspace)", p.ws_bytes, kScratchBytes);
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != TQ_OK) return st;
  return launch_decode(L, p, q, q_dtype, pool, block_table, max_blocks_per_seq, seq_lens, scale, out, out_dtype,
                       ws, hip_stream);
}
