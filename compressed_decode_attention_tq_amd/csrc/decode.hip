// Split-K paged decode attention over the compressed store (gfx950).
//
// "turbo-attn 0.24.0", "How it works": the query is rotated once by the head's
// rotation and attention runs in the rotated space; decode unpacks, dequantises
// and runs Q.K, online softmax and P.V in one pass with no decompress buffer.
// "turbo-attn 0.24.0", "Configuration" (TKV_DECODE_SPLITS) and "tiny-turboquant
// 0.18.0", "Fused decode-attention path": the context is split across
// workgroups whose partials are merged by a second launch.
// "How 0xsero/turboquant works", "Key Storage and Attention Scoring": scores come
// from the compressed keys alone:
//   s_i = scale * (n_i / sqrt d) * (q'.c[idx_i] + sqrt(pi/2)/m * gamma_i * u.(2 z_i - 1)),
//   q' = R_g q, u = S_g q'  (QJL residual estimator).
//
// Launch 1 (prologue): q', u per (sequence, query head) into the workspace.
// Launch 2 (split-K):  one workgroup per (split, KV head, sequence) serves all
//   query heads of its KV head so the compressed KV is read once.  Four waves
//   take 64-token chunks in turn; within a chunk a lane scores one token, then
//   the chunk's values are accumulated with lanes owning 2 coordinates each.
//   Online softmax keeps a running max/sum per head (wave reductions).
// Launch 3 (combine): merge the split partials with the running-max rescaling,
//   un-rotate o = R_g^T o', cast and store.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>

#include "tq_internal.hpp"

namespace tq {
namespace {

constexpr int kPart = kDim + 4;  // acc[128], m, l, pad, pad

struct DecodeArgs {
  const unsigned char* pool;
  const int* block_table;
  const int* seq_lens;
  const float* qu;  // [B*Hq][2][128]
  float* part;      // [B*Hq][n_splits][kPart]
  long long max_blocks;
  int Hq, Hkv, n_splits, split_tokens;
  float scale;
  unsigned block_bytes, off_kc, off_ks, off_kn, off_vc, off_vsz;
  float cent[16];
};

__device__ __forceinline__ float half_lo(unsigned w) { return __half2float(__ushort_as_half(static_cast<unsigned short>(w & 0xffffu))); }
__device__ __forceinline__ float half_hi(unsigned w) { return __half2float(__ushort_as_half(static_cast<unsigned short>(w >> 16))); }
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float wave_max(float x) {
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Code j (0..127) of a B-bit LSB-first bitstream held in 32-bit words.
template <int B>
__device__ __forceinline__ int code_at(const unsigned* w, int j) {
  const int bit = B * j;
  const int wi = bit >> 5, sh = bit & 31;
  unsigned x = w[wi] >> sh;
  if (sh + B > 32) x |= w[wi + 1] << (32 - sh);
  return static_cast<int>(x & ((1u << B) - 1u));
}

// ---------------------------------------------------------------- prologue
template <bool QBF16, bool BYPASS>
__global__ __launch_bounds__(128) void prologue_kernel(const void* q, const float* RT, const float* ST,
                                                       float* qu, int Hq, int rep) {
  const int bh = blockIdx.x;
  const int g = (bh % Hq) / rep;
  const int i = threadIdx.x;
  __shared__ float sq[128], sp[128];
  float x;
  if constexpr (QBF16) {
    x = __uint_as_float(static_cast<unsigned>(static_cast<const unsigned short*>(q)[bh * 128 + i]) << 16);
  } else {
    x = static_cast<const float*>(q)[bh * 128 + i];
  }
  if constexpr (BYPASS) {
    qu[bh * 256 + i] = x;
    qu[bh * 256 + 128 + i] = 0.0f;
    return;
  } else {
    sq[i] = x;
    __syncthreads();
    const float* rt = RT + static_cast<size_t>(g) * 128 * 128;
    const float* st = ST + static_cast<size_t>(g) * 128 * 128;
    float a = 0.0f;
    for (int j = 0; j < 128; ++j) a = fmaf(rt[j * 128 + i], sq[j], a);
    sp[i] = a;
    __syncthreads();
    float u = 0.0f;
    for (int j = 0; j < 128; ++j) u = fmaf(st[j * 128 + i], sp[j], u);
    qu[bh * 256 + i] = a;
    qu[bh * 256 + 128 + i] = u;
  }
}

// ----------------------------------------------------------------- split-K
// KB == 0 selects the uncompressed bf16 (bypass) page format.
template <int NREP, int KB, int VB>
__global__ __launch_bounds__(256) void splitk_kernel(DecodeArgs a) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int T = a.seq_lens[b];
  const int start = split * a.split_tokens;
  if (start >= T) return;
  const int end = min(T, start + a.split_tokens);

  __shared__ float qs[NREP][128];
  __shared__ float us[NREP][128];
  __shared__ float cb[16];
  __shared__ float wm[4][NREP], wl[4][NREP];
  __shared__ float wacc[4][NREP][128];

  const int h0 = g * NREP;
  for (int x = threadIdx.x; x < NREP * 128; x += 256) {
    const int r = x >> 7, d = x & 127;
    const float* src = a.qu + static_cast<size_t>(b * a.Hq + h0 + r) * 256;
    qs[r][d] = src[d];
    us[r][d] = src[128 + d];
  }
  if (threadIdx.x < 16) cb[threadIdx.x] = a.cent[threadIdx.x];
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float kappa = 0.0097916396f;  // sqrt(pi/2) / 128
  const float inv_sqrt_d = 0.08838834764831845f;
  float m[NREP], l[NREP], acc[NREP][2];
#pragma unroll
  for (int r = 0; r < NREP; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0f;
    acc[r][0] = acc[r][1] = 0.0f;
  }

  for (int c0 = start + wave * 64; c0 < end; c0 += 256) {
    const int tok = c0 + lane;
    const bool valid = tok < end;
    long long rbase = 0;
    int off = 0;
    float s[NREP];
    if (valid) {
      const int blk = a.block_table[b * a.max_blocks + (tok >> 4)];
      off = tok & 15;
      rbase = (static_cast<long long>(blk) * a.Hkv + g) * a.block_bytes;
      const unsigned char* rec = a.pool + rbase;
      if constexpr (KB == 0) {
        const unsigned* kw = reinterpret_cast<const unsigned*>(rec + off * 256);
        float A[NREP];
#pragma unroll
        for (int r = 0; r < NREP; ++r) A[r] = 0.0f;
#pragma unroll 8
        for (int d2 = 0; d2 < 64; ++d2) {
          const unsigned w = kw[d2];
          const float k0 = bf16_lo(w), k1 = bf16_hi(w);
#pragma unroll
          for (int r = 0; r < NREP; ++r) A[r] = fmaf(qs[r][2 * d2 + 1], k1, fmaf(qs[r][2 * d2], k0, A[r]));
        }
#pragma unroll
        for (int r = 0; r < NREP; ++r) s[r] = a.scale * A[r];
      } else {
        const unsigned* kc = reinterpret_cast<const unsigned*>(rec + a.off_kc + off * (16 * KB));
        const unsigned* ks = reinterpret_cast<const unsigned*>(rec + a.off_ks + off * 16);
        const unsigned kn = *reinterpret_cast<const unsigned*>(rec + a.off_kn + off * 4);
        unsigned w[4 * KB + 1];
#pragma unroll
        for (int x = 0; x < 4 * KB; ++x) w[x] = kc[x];
        w[4 * KB] = 0;
        unsigned sw[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) sw[x] = ks[x];
        float A[NREP], Bs[NREP];
#pragma unroll
        for (int r = 0; r < NREP; ++r) A[r] = Bs[r] = 0.0f;
#pragma unroll
        for (int d = 0; d < 128; ++d) {
          const float c = cb[code_at<KB>(w, d)];
          const bool bit = (sw[d >> 5] >> (d & 31)) & 1u;
#pragma unroll
          for (int r = 0; r < NREP; ++r) {
            A[r] = fmaf(qs[r][d], c, A[r]);
            Bs[r] += bit ? us[r][d] : -us[r][d];
          }
        }
        const float nn = half_lo(kn), gg = half_hi(kn);
#pragma unroll
        for (int r = 0; r < NREP; ++r) s[r] = a.scale * (nn * inv_sqrt_d) * (A[r] + kappa * gg * Bs[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < NREP; ++r) s[r] = -INFINITY;
    }

    // online softmax (lane 0 of the chunk is always a valid token)
#pragma unroll
    for (int r = 0; r < NREP; ++r) {
      const float mnew = fmaxf(m[r], wave_max(s[r]));
      const float alpha = (m[r] == -INFINITY) ? 0.0f : __expf(m[r] - mnew);
      const float p = valid ? __expf(s[r] - mnew) : 0.0f;
      l[r] = l[r] * alpha + wave_sum(p);
      acc[r][0] *= alpha;
      acc[r][1] *= alpha;
      m[r] = mnew;
      s[r] = p;
    }

    // values: lane owns coordinates 2*lane, 2*lane+1
    const int ntok = min(64, end - c0);
    for (int j = 0; j < ntok; ++j) {
      const long long rb = __shfl(rbase, j, 64);
      const int oj = __shfl(off, j, 64);
      const unsigned char* rec = a.pool + rb;
      float v0, v1;
      if constexpr (KB == 0) {
        const unsigned w = reinterpret_cast<const unsigned*>(rec + 4096 + oj * 256)[lane];
        v0 = bf16_lo(w);
        v1 = bf16_hi(w);
      } else {
        const unsigned char* vc = rec + a.off_vc + oj * (16 * VB);
        const int bit = VB * 2 * lane;
        unsigned two = vc[bit >> 3];
        if ((bit & 7) + 2 * VB > 8) two |= static_cast<unsigned>(vc[(bit >> 3) + 1]) << 8;
        two >>= (bit & 7);
        const float c0v = static_cast<float>(two & ((1u << VB) - 1u));
        const float c1v = static_cast<float>((two >> VB) & ((1u << VB) - 1u));
        const unsigned sz = reinterpret_cast<const unsigned*>(rec + a.off_vsz + oj * 16)[(2 * lane) >> 5];
        const float sc = half_lo(sz), ze = half_hi(sz);
        v0 = fmaf(sc, c0v, ze);
        v1 = fmaf(sc, c1v, ze);
      }
#pragma unroll
      for (int r = 0; r < NREP; ++r) {
        const float p = __shfl(s[r], j, 64);
        acc[r][0] = fmaf(p, v0, acc[r][0]);
        acc[r][1] = fmaf(p, v1, acc[r][1]);
      }
    }
  }

  // merge the four waves
#pragma unroll
  for (int r = 0; r < NREP; ++r) {
    if (lane == 0) {
      wm[wave][r] = m[r];
      wl[wave][r] = l[r];
    }
    wacc[wave][r][2 * lane] = acc[r][0];
    wacc[wave][r][2 * lane + 1] = acc[r][1];
  }
  __syncthreads();
  for (int x = threadIdx.x; x < NREP * 128; x += 256) {
    const int r = x >> 7, d = x & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][r]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (wm[w][r] == -INFINITY) continue;
      const float e = __expf(wm[w][r] - M);
      num += e * wacc[w][r][d];
      den += e * wl[w][r];
    }
    float* dst = a.part + (static_cast<size_t>(b * a.Hq + h0 + r) * a.n_splits + split) * kPart;
    dst[d] = num;
    if (d == 0) {
      dst[128] = M;
      dst[129] = den;
    }
  }
}

// ---------------------------------------------------------------- combine
template <bool OUT_BF16, bool BYPASS>
__global__ __launch_bounds__(128) void combine_kernel(const float* part, const int* seq_lens, const float* R,
                                                      void* out, int Hq, int rep, int n_splits,
                                                      int split_tokens) {
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int g = (bh % Hq) / rep;
  const int i = threadIdx.x;
  const int T = seq_lens[b];
  __shared__ float so[128];
  float o = 0.0f;
  if (T > 0) {
    const int ns = (T + split_tokens - 1) / split_tokens;
    const float* p = part + static_cast<size_t>(bh) * n_splits * kPart;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, p[s * kPart + 128]);
    float num = 0.0f, den = 0.0f;
    for (int s = 0; s < ns; ++s) {
      const float e = __expf(p[s * kPart + 128] - M);
      num += e * p[s * kPart + i];
      den += e * p[s * kPart + 129];
    }
    o = num / den;
    if constexpr (!BYPASS) {
      so[i] = o;
      __syncthreads();
      const float* r = R + static_cast<size_t>(g) * 128 * 128;
      float a = 0.0f;
      for (int j = 0; j < 128; ++j) a = fmaf(r[j * 128 + i], so[j], a);
      o = a;
    }
  }
  if constexpr (OUT_BF16) {
    const unsigned u = __float_as_uint(o);
    const unsigned r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    static_cast<unsigned short*>(out)[bh * 128 + i] = static_cast<unsigned short>(r);
  } else {
    static_cast<float*>(out)[bh * 128 + i] = o;
  }
}

template <int NREP, int KB>
void* pick_splitk_vb(int vb) {
  if constexpr (KB == 0) {
    return reinterpret_cast<void*>(&splitk_kernel<NREP, 0, 0>);
  } else {
    switch (vb) {
      case 2: return reinterpret_cast<void*>(&splitk_kernel<NREP, KB, 2>);
      case 3: return reinterpret_cast<void*>(&splitk_kernel<NREP, KB, 3>);
      case 4: return reinterpret_cast<void*>(&splitk_kernel<NREP, KB, 4>);
    }
  }
  return nullptr;
}

template <int NREP>
void* pick_splitk_kb(int kb, int vb) {
  switch (kb) {
    case 0: return pick_splitk_vb<NREP, 0>(vb);
    case 2: return pick_splitk_vb<NREP, 2>(vb);
    case 3: return pick_splitk_vb<NREP, 3>(vb);
    case 4: return pick_splitk_vb<NREP, 4>(vb);
  }
  return nullptr;
}

void* pick_splitk(int rep, int kb, int vb) {
  switch (rep) {
    case 1: return pick_splitk_kb<1>(kb, vb);
    case 2: return pick_splitk_kb<2>(kb, vb);
    case 4: return pick_splitk_kb<4>(kb, vb);
    case 8: return pick_splitk_kb<8>(kb, vb);
  }
  return nullptr;
}

}  // namespace

tq_status launch_decode(const tq_layer* L, const DecodePlan& plan, const void* q, tq_dtype q_dtype,
                        const void* pool, const int* block_table, int max_blocks_per_seq,
                        const int* seq_lens, float softmax_scale, void* out, tq_dtype out_dtype,
                        void* workspace, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bypass = L->cfg.bypass != 0;
  char* ws = static_cast<char*>(workspace);
  float* qu = reinterpret_cast<float*>(ws + plan.ws_qu);
  float* part = reinterpret_cast<float*>(ws + plan.ws_part);
  const int bh = plan.batch * plan.n_q_heads;

  // 1. prologue
  {
    void* fn;
    if (bypass) fn = (q_dtype == TQ_BF16) ? reinterpret_cast<void*>(&prologue_kernel<true, true>)
                                          : reinterpret_cast<void*>(&prologue_kernel<false, true>);
    else fn = (q_dtype == TQ_BF16) ? reinterpret_cast<void*>(&prologue_kernel<true, false>)
                                   : reinterpret_cast<void*>(&prologue_kernel<false, false>);
    const float* RT = L->dRT;
    const float* ST = L->dST;
    int Hq = plan.n_q_heads, rep = plan.rep;
    void* args[] = {const_cast<void**>(&q), &RT, &ST, &qu, &Hq, &rep};
    ProfScope prof(kKPrologue, stream);
    hipError_t e = hipLaunchKernel(fn, dim3(bh), dim3(128), args, 0, s);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "decode prologue launch: %s", hipGetErrorString(e));
  }
  // 2. split-K mainloop
  {
    DecodeArgs a;
    a.pool = static_cast<const unsigned char*>(pool);
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.qu = qu;
    a.part = part;
    a.max_blocks = max_blocks_per_seq;
    a.Hq = plan.n_q_heads;
    a.Hkv = L->cfg.n_kv_heads;
    a.n_splits = plan.n_splits;
    a.split_tokens = plan.split_tokens;
    a.scale = softmax_scale;
    a.block_bytes = static_cast<unsigned>(L->lay.block_bytes);
    a.off_kc = static_cast<unsigned>(L->lay.off_kc);
    a.off_ks = static_cast<unsigned>(L->lay.off_ks);
    a.off_kn = static_cast<unsigned>(L->lay.off_kn);
    a.off_vc = static_cast<unsigned>(L->lay.off_vc);
    a.off_vsz = static_cast<unsigned>(L->lay.off_vsz);
    for (int i = 0; i < 16; ++i) a.cent[i] = L->centroids[i];
    void* fn = pick_splitk(plan.rep, bypass ? 0 : L->cfg.k_bits, bypass ? 0 : L->cfg.v_bits);
    if (!fn) return fail(TQ_ERR_UNSUPPORTED, "no decode kernel for this variant");
    void* args[] = {&a};
    const dim3 grid(plan.n_splits, L->cfg.n_kv_heads, plan.batch);
    ProfScope prof(kKSplitK, stream);
    hipError_t e = hipLaunchKernel(fn, grid, dim3(256), args, 0, s);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "decode split-K launch: %s", hipGetErrorString(e));
  }
  // 3. combine + un-rotation
  {
    void* fn;
    if (bypass) fn = (out_dtype == TQ_BF16) ? reinterpret_cast<void*>(&combine_kernel<true, true>)
                                            : reinterpret_cast<void*>(&combine_kernel<false, true>);
    else fn = (out_dtype == TQ_BF16) ? reinterpret_cast<void*>(&combine_kernel<true, false>)
                                     : reinterpret_cast<void*>(&combine_kernel<false, false>);
    const float* R = L->dR;
    int Hq = plan.n_q_heads, rep = plan.rep, ns = plan.n_splits, st = plan.split_tokens;
    void* args[] = {&part, const_cast<int**>(&seq_lens), &R, &out, &Hq, &rep, &ns, &st};
    ProfScope prof(kKCombine, stream);
    hipError_t e = hipLaunchKernel(fn, dim3(bh), dim3(128), args, 0, s);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "decode combine launch: %s", hipGetErrorString(e));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TQ_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return TQ_OK;
}

}  // namespace tq
