// Fused K+V compression into the paged store (gfx950).
//
// Keys ("How 0xsero/turboquant works", "Compression Pipeline"; "turbo-attn
// 0.24.0", "How it works"; "5x Faster LLM Inference? ...", "Example 4:
// Kernel-Level Operations"):
//   n = ||k||, t = sqrt(d) R k / n, idx_j = #{i : beta_i < t_j},
//   rho = t - c[idx], gamma = ||rho||, z_j = [(S rho)_j >= 0];
//   stored: packed idx, packed z, fp16 n, fp16 gamma.
// Values ("How 0xsero/turboquant works", "Value Compression"; "tiny-turboquant
// 0.18.0", "Measured quality": groups of 32 with their own scale/zero):
//   v' = R v; per 32-wide group scale = fp16((max-min)/(2^b-1)), zero = fp16(min),
//   code = clamp(rint((v' - zero)/scale), 0, 2^b-1)  (0 when scale == 0).
// Values coded like the keys' codebook part ("5x Faster LLM Inference? ...",
// "What is TurboQuant-GPU?": 3-bit MSE values), with their own codebook:
//   nv = ||v||, t = sqrt(d) v' / nv, code = #{i : vbeta_i < t}; stored fp16 nv.
//
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "tq_internal.hpp"

namespace tq {
namespace {

struct CompressArgs {
  const void* k;
  const void* v;
  long long k_stride;
  long long v_stride;
  const long long* slots;
  unsigned char* pool;
  const float* RT;  // [H][128][128], RT[h][j][i] = R_h[i][j]
  const float* ST;  // [H][128][128], ST[h][j][i] = S_h[i][j]
  int H;
  int km;  // key mode: 0 QJL, 1 codebook only, 2 codebook only with norm-corrected magnitude
  int vm;  // value mode: 0 group scale/zero, 1 codebook codes and one fp16 norm
  unsigned block_bytes;
  unsigned off_kc, off_ks, off_kn, off_vc, off_vsz;
  float cent[16];
  float bnd[16];
  float vcent[16];  // value codebook (vm == 1)
  float vbnd[16];
};

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, long long idx) {
  if constexpr (BF16) {
    const unsigned short b = static_cast<const unsigned short*>(p)[idx];
    return __uint_as_float(static_cast<unsigned>(b) << 16);
  } else {
    return static_cast<const float*>(p)[idx];
  }
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
// Squared norms are summed in float64: a vector of tiny entries (say 2^-70) has a
// squared norm below the float32 normal range, where float32 keeps too few bits
// for the standardising factor sqrt(d) / n.
__device__ __forceinline__ double wave_sum_d(double x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Element index of the value code of (coordinate dim, in-page token t) in the
// page's Vc stream: lane block 16 (t / 8) + dim % 16, group 2 (dim / 16) + (t % 8) / 4
// of four codes, element t % 4.  The eight codes of (tile dim / 16, column,
// token half) form one contiguous run, which the decode loads as a whole.
__device__ __forceinline__ unsigned vcode_elem(int dim, int t) {
  const unsigned block = 16u * static_cast<unsigned>(t >> 3) + static_cast<unsigned>(dim & 15);
  const unsigned group = 2u * static_cast<unsigned>(dim >> 4) + static_cast<unsigned>((t & 7) >> 2);
  return (block * 16u + group) * 4u + static_cast<unsigned>(t & 3);
}

// 32-bit word w of the LSB-first bitstream of 128 b-bit codes.
template <int B>
__device__ __forceinline__ unsigned pack_word(const unsigned char* codes, int w) {
  unsigned word = 0;
  const int first = (32 * w) / B;
  const int last = (32 * w + 31) / B;
  for (int j = first; j <= last && j < 128; ++j) {
    const int shift = B * j - 32 * w;
    const unsigned c = codes[j];
    word |= (shift >= 0) ? (c << shift) : (c >> (-shift));
  }
  return word;
}

// One workgroup of 512 lanes per (token, KV head).  Lane (c, i) = (lane / 128,
// lane % 128) holds column i of rows 32c..32c+31 of R^T and S^T (loaded before
// anything else, so the loads overlap) and forms that quarter of each dot
// product; the quarters are summed through LDS in a fixed order.  Lanes 0..127
// then own coordinate i for the scalar work.
template <bool BF16, int KB, int VB>
__global__ __launch_bounds__(512) void compress_kernel(CompressArgs a) {
  const long long tok = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, c = tid >> 7, i = tid & 127;
  const long long slot = a.slots[tok];
  if (slot < 0) return;

  __shared__ float sk[128], sv[128], srho[128], red[4];
  __shared__ double rk2[2], rv2[2];
  __shared__ float pk[4][128], pv[4][128];
  __shared__ unsigned char ck[128];
  __shared__ unsigned sbits[4];
  __shared__ __half sgroup[8];

  float rt[32], st[32];
  {
    const float* r = a.RT + static_cast<size_t>(h) * 128 * 128 + (32 * c) * 128 + i;
    const float* s = a.ST + static_cast<size_t>(h) * 128 * 128 + (32 * c) * 128 + i;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      rt[u] = r[u * 128];
      st[u] = s[u * 128];
    }
  }
  float kx = 0.0f;
  if (c == 0) {
    kx = load_elem<BF16>(a.k, tok * a.k_stride + h * 128 + i);
    sk[i] = kx;
    const double w2 = wave_sum_d(static_cast<double>(kx) * kx);
    if ((i & 63) == 0) rk2[i >> 6] = w2;
  } else if (c == 1) {
    const float vx = load_elem<BF16>(a.v, tok * a.v_stride + h * 128 + i);
    sv[i] = vx;
    const double w2 = wave_sum_d(static_cast<double>(vx) * vx);  // ||v||^2 (codebook-coded values)
    if ((i & 63) == 0) rv2[i >> 6] = w2;
  }
  __syncthreads();
  {
    float ak = 0.0f, av = 0.0f;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      ak = fmaf(rt[u], sk[32 * c + u], ak);
      av = fmaf(rt[u], sv[32 * c + u], av);
    }
    pk[c][i] = ak;
    pv[c][i] = av;
  }
  __syncthreads();

  constexpr float top = static_cast<float>((1 << VB) - 1);
  float n = 0.0f, rv = 0.0f;
  int code = 0;
  __half s16, z16;
  if (c == 0) {
    const float rk = (pk[0][i] + pk[1][i]) + (pk[2][i] + pk[3][i]);
    rv = (pv[0][i] + pv[1][i]) + (pv[2][i] + pv[3][i]);
    // keys: standardise, quantise, residual
    n = static_cast<float>(sqrt(rk2[0] + rk2[1]));
    const float t = (n > 0.0f) ? rk * (sqrtf(128.0f) / n) : 0.0f;
    int idx = 0;
#pragma unroll
    for (int b = 0; b < (1 << KB) - 1; ++b) idx += (a.bnd[b] < t) ? 1 : 0;
    const float rho = t - a.cent[idx];
    ck[i] = static_cast<unsigned char>(idx);
    srho[i] = rho;
    // squared norm of the residual (QJL) or of the centroid vector (norm correction)
    const float gt = (a.km == 2) ? a.cent[idx] : rho;
    const float g2 = wave_sum(gt * gt);
    if ((i & 63) == 0) red[2 + (i >> 6)] = g2;
    if (a.vm == 1) {
      // values: standardise by the vector norm, then the value codebook
      const float nv = static_cast<float>(sqrt(rv2[0] + rv2[1]));
      const float tv = (nv > 0.0f) ? rv * (sqrtf(128.0f) / nv) : 0.0f;
#pragma unroll
      for (int b = 0; b < (1 << VB) - 1; ++b) code += (a.vbnd[b] < tv) ? 1 : 0;
      if (i == 0) sgroup[0] = __float2half_rn(nv);
    } else {
      // values: group min/max over 32 lanes
      float mn = rv, mx = rv;
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, off, 32));
        mx = fmaxf(mx, __shfl_xor(mx, off, 32));
      }
      s16 = __float2half_rn((mx - mn) / top);
      z16 = __float2half_rn(mn);
      const float s = __half2float(s16);
      const float z = __half2float(z16);
      if (s > 0.0f) code = static_cast<int>(fminf(fmaxf(rintf((rv - z) / s), 0.0f), top));
      if ((i & 31) == 0) {
        sgroup[(i >> 5) * 2] = s16;
        sgroup[(i >> 5) * 2 + 1] = z16;
      }
    }
  }
  __syncthreads();
  if (a.km == 0) {  // QJL residual signs (workgroup-uniform branch)
    {
      float ay = 0.0f;
#pragma unroll
      for (int u = 0; u < 32; ++u) ay = fmaf(st[u], srho[32 * c + u], ay);
      pk[c][i] = ay;
    }
    __syncthreads();
    if (c == 0) {
      const float y = (pk[0][i] + pk[1][i]) + (pk[2][i] + pk[3][i]);
      const unsigned long long bal = __ballot(y >= 0.0f);
      if ((i & 63) == 0) {
        sbits[(i >> 6) * 2] = static_cast<unsigned>(bal);
        sbits[(i >> 6) * 2 + 1] = static_cast<unsigned>(bal >> 32);
      }
    }
  } else if (tid < 4) {
    sbits[tid] = 0u;
  }
  __syncthreads();
  if (c != 0) return;  // lanes 0..127 store the record

  unsigned char* base = a.pool + (static_cast<size_t>(slot >> 4) * a.H + h) * a.block_bytes;
  const int off = static_cast<int>(slot & 15);
  // value code of coordinate i in the lane-blocked Vc stream (element
  // ((16 (off / 8) + i % 16) 16 + 2 (i / 16) + (off % 8) / 4) 4 + off % 4).
  // Neighbouring tokens of the page share these words, so the field is cleared
  // and set with atomics on disjoint bit masks.
  {
    unsigned* vw = reinterpret_cast<unsigned*>(base + a.off_vc);
    const unsigned bit = vcode_elem(i, off) * VB;
    const unsigned w = bit >> 5, sh = bit & 31;
    const unsigned mask = (1u << VB) - 1u;
    const unsigned cc = static_cast<unsigned>(code);
    atomicAnd(&vw[w], ~(mask << sh));
    atomicOr(&vw[w], cc << sh);
    if (sh + VB > 32) {
      atomicAnd(&vw[w + 1], ~(mask >> (32 - sh)));
      atomicOr(&vw[w + 1], cc >> (32 - sh));
    }
  }
  if (i < 4 * KB) {
    // word i of the 128-code key stream lies in 32-dim block i / KB
    const int blk = i / KB, wi = i % KB;
    reinterpret_cast<unsigned*>(base + a.off_kc + (blk * 16 + off) * (4 * KB))[wi] = pack_word<KB>(ck, i);
  } else if (a.km == 0 && i >= 64 && i < 68) {
    const int blk = i - 64;
    *reinterpret_cast<unsigned*>(base + a.off_ks + (blk * 16 + off) * 4) = sbits[blk];
  } else if (i == 68) {
    const float g2 = red[2] + red[3];
    // stored magnitude: n, or n sqrt(d) / ||c[idx]|| with norm correction; with
    // QJL the pair (n, gamma), without QJL the magnitude alone (no sign field)
    const __half hn = __float2half_rn(a.km == 2 ? n * sqrtf(128.0f) / sqrtf(g2) : n);
    if (a.km == 0) {
      const __half hg = __float2half_rn(sqrtf(g2));
      const unsigned w = static_cast<unsigned>(__half_as_ushort(hn)) |
                         (static_cast<unsigned>(__half_as_ushort(hg)) << 16);
      *reinterpret_cast<unsigned*>(base + a.off_kn + off * 4) = w;
    } else {
      *reinterpret_cast<unsigned short*>(base + a.off_kn + off * 2) = __half_as_ushort(hn);
    }
  } else if (a.vm == 1 && i == 72) {
    // the token's fp16 value norm (two bytes of its own)
    *reinterpret_cast<unsigned short*>(base + a.off_vsz + off * 2) = __half_as_ushort(sgroup[0]);
  } else if (a.vm == 0 && i >= 72 && i < 76) {
    const int g = i - 72;
    const unsigned w = static_cast<unsigned>(__half_as_ushort(sgroup[2 * g])) |
                       (static_cast<unsigned>(__half_as_ushort(sgroup[2 * g + 1])) << 16);
    reinterpret_cast<unsigned*>(base + a.off_vsz + off * 16)[g] = w;
  }
}

// Uncompressed (bf16) layers: copy one (token, head) of K and V into the page,
// keys as the token's row of K [16][128], values as the token's column of the
// dim-major V^T [128][16].
__global__ __launch_bounds__(64) void store_bypass_kernel(const unsigned short* k, const unsigned short* v,
                                                          long long k_stride, long long v_stride,
                                                          const long long* slots, unsigned char* pool,
                                                          int H, unsigned block_bytes) {
  const long long tok = blockIdx.x;
  const int h = blockIdx.y;
  const long long slot = slots[tok];
  if (slot < 0) return;
  const int i = threadIdx.x;  // 2 elements each
  unsigned char* base = pool + (static_cast<size_t>(slot >> 4) * H + h) * block_bytes;
  const int off = static_cast<int>(slot & 15);
  const unsigned* ks = reinterpret_cast<const unsigned*>(k + tok * k_stride + h * 128);
  const unsigned* vs = reinterpret_cast<const unsigned*>(v + tok * v_stride + h * 128);
  reinterpret_cast<unsigned*>(base + off * 256)[i] = ks[i];
  const unsigned w = vs[i];
  unsigned short* vt = reinterpret_cast<unsigned short*>(base + 4096) + off;
  vt[(2 * i) * 16] = static_cast<unsigned short>(w & 0xffffu);
  vt[(2 * i + 1) * 16] = static_cast<unsigned short>(w >> 16);
}

template <bool BF16, int KB>
void* pick_vb(int vb) {
  switch (vb) {
    case 2: return reinterpret_cast<void*>(&compress_kernel<BF16, KB, 2>);
    case 3: return reinterpret_cast<void*>(&compress_kernel<BF16, KB, 3>);
    case 4: return reinterpret_cast<void*>(&compress_kernel<BF16, KB, 4>);
  }
  return nullptr;
}

template <bool BF16>
void* pick(int kb, int vb) {
  switch (kb) {
    case 1: return pick_vb<BF16, 1>(vb);
    case 2: return pick_vb<BF16, 2>(vb);
    case 3: return pick_vb<BF16, 3>(vb);
    case 4: return pick_vb<BF16, 4>(vb);
  }
  return nullptr;
}

}  // namespace

tq_status launch_compress(const tq_layer* L, const void* k, const void* v, tq_dtype in_dtype,
                          long long n_tokens, long long k_stride, long long v_stride,
                          const long long* slots, void* pool, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  ProfScope prof(kKCompress, stream);
  if (!L->cfg.bypass && compress_mfma_applies(L, k, v, in_dtype, n_tokens, k_stride, v_stride)) {
    tq_status st = launch_compress_mfma(L, k, v, n_tokens, k_stride, v_stride, slots, pool, stream);
    if (st != TQ_OK) return st;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "compress launch: %s", hipGetErrorString(e));
    return TQ_OK;
  }
  if (L->cfg.bypass && ((k_stride | v_stride) & 1))
    return fail(TQ_ERR_UNSUPPORTED, "bypass compress needs even token strides");
  void* fn = nullptr;
  CompressArgs a;
  if (!L->cfg.bypass) {
    a.RT = L->dRT;
    a.ST = L->dST;
    a.H = L->cfg.n_kv_heads;
    a.block_bytes = static_cast<unsigned>(L->lay.block_bytes);
    a.km = static_cast<int>(L->cfg.key_mode);
    a.vm = L->cfg.value_mode == TQ_VAL_MSE ? 1 : 0;
    a.off_kc = static_cast<unsigned>(L->lay.off_kc);
    a.off_ks = static_cast<unsigned>(L->lay.off_ks);
    a.off_kn = static_cast<unsigned>(L->lay.off_kn);
    a.off_vc = static_cast<unsigned>(L->lay.off_vc);
    a.off_vsz = static_cast<unsigned>(L->lay.off_vsz);
    for (int i = 0; i < 16; ++i) {
      a.cent[i] = L->centroids[i];
      a.bnd[i] = L->boundaries[i];
      a.vcent[i] = L->v_centroids[i];
      a.vbnd[i] = L->v_boundaries[i];
    }
    fn = (in_dtype == TQ_BF16) ? pick<true>(L->cfg.k_bits, L->cfg.v_bits) : pick<false>(L->cfg.k_bits, L->cfg.v_bits);
    if (!fn) return fail(TQ_ERR_UNSUPPORTED, "no compress kernel for k_bits=%d v_bits=%d", L->cfg.k_bits, L->cfg.v_bits);
  }
  // One workgroup per (token, head) (512 lanes; 64 for bypass layers): launched
  // over token ranges of at most 2^22, so that no launch exceeds 2^31 work-items
  // in the token dimension.
  constexpr long long kRange = 1LL << 22;
  const size_t esz = in_dtype == TQ_BF16 ? 2 : 4;
  for (long long t0 = 0; t0 < n_tokens; t0 += kRange) {
    const long long n = n_tokens - t0 < kRange ? n_tokens - t0 : kRange;
    const dim3 grid(static_cast<unsigned>(n), static_cast<unsigned>(L->cfg.n_kv_heads));
    const void* kr = static_cast<const unsigned char*>(k) + static_cast<size_t>(t0) * k_stride * esz;
    const void* vr = static_cast<const unsigned char*>(v) + static_cast<size_t>(t0) * v_stride * esz;
    const long long* sr = slots + t0;
    if (L->cfg.bypass) {
      hipLaunchKernelGGL(store_bypass_kernel, grid, dim3(64), 0, s,
                         static_cast<const unsigned short*>(kr), static_cast<const unsigned short*>(vr),
                         k_stride, v_stride, sr, static_cast<unsigned char*>(pool),
                         L->cfg.n_kv_heads, static_cast<unsigned>(L->lay.block_bytes));
    } else {
      a.k = kr;
      a.v = vr;
      a.k_stride = k_stride;
      a.v_stride = v_stride;
      a.slots = sr;
      a.pool = static_cast<unsigned char*>(pool);
      void* args[] = {&a};
      hipError_t e = hipLaunchKernel(fn, grid, dim3(512), args, 0, s);
      if (e != hipSuccess) return fail(TQ_ERR_HIP, "compress launch: %s", hipGetErrorString(e));
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "compress launch: %s", hipGetErrorString(e));
  }
  return TQ_OK;
}

}  // namespace tq
