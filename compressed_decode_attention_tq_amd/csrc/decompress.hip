// Reconstruction of keys and values from the paged store, in the original basis
// ("turbo-attn 0.24.0", "How it works": a decompress path feeding an ordinary
// attention kernel; "tiny-turboquant 0.18.0", "Fused decode-attention path").
// For token i of KV head g:
//   khat_i = (n16_i / sqrt d) R_g^T (c[idx_i] + kappa gamma16_i S_g^T sigma_i)
//          = (n16_i / sqrt d) (c[idx_i]^T R_g + kappa gamma16_i sigma_i^T P_g)^T,  P_g = S_g R_g
//   vhat_i = R_g^T (zero16 + scale16 code_i)
// so that q . khat_i is the decode's score estimator before the softmax scale
// ("How 0xsero/turboquant works", "Key Storage and Attention Scoring").
//
// One workgroup of four waves per (16-token tile, KV head).  The tile's records
// are expanded once into LDS as float16 matrix-core A operands (16 tokens x 128
// dims): the codebook values (exact), the signs (+-1, exact) and the rotated
// values v' = zero + scale code split into hi + lo pieces.  Wave w then forms
// output dims 32w..32w+31 (two 16-wide column tiles) on v_mfma_f32_16x16x32_f16
// against R_g and P_g held as float16 hi + lo B operands (fp32-faithful sums).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>

#include "tq_internal.hpp"

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kARow = 136;  // float16 elements per LDS operand row (128 + pad)
constexpr int kMaxPage = 256 * 8 + 576;  // bytes of a K4/V4 page, the largest

struct DArgs {
  const unsigned char* pool;
  const long long* slots;
  void* kout;  // [n][H][128]
  void* vout;
  const u32x4* opd;  // [H][8 column tiles][4 K-steps][R hi, R lo, P hi, P lo][64 lanes] x 8 float16
  long long n_tokens;
  int H;
  unsigned block_bytes;
  unsigned off_kc, off_ks, off_kn, off_vc, off_vsz;
  float kappa;
  float cent[16];
  int vm;           // value mode: 0 group scale/zero, 1 codebook codes and one fp16 norm
  int qjl;          // 1: sign field and (n, gamma) pairs; 0: no sign field, Kn = [16] fp16 n
  float vcent[16];  // value codebook (vm == 1)
};

__device__ __forceinline__ floatx4 mfma(const half8& a, const half8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Eight consecutive outputs from LDS as one 16-byte (bf16, nearest even) or two
// 16-byte (fp32) stores.
template <bool BF16>
__device__ __forceinline__ void store8(void* out, size_t at, const float* src) {
  if constexpr (BF16) {
    u32x4 pk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned lo = __float_as_uint(src[2 * i]), hi = __float_as_uint(src[2 * i + 1]);
      pk[i] = ((lo + 0x7fffu + ((lo >> 16) & 1u)) >> 16) | (((hi + 0x7fffu + ((hi >> 16) & 1u)) >> 16) << 16);
    }
    *reinterpret_cast<u32x4*>(static_cast<unsigned short*>(out) + at) = pk;
  } else {
    float* o = static_cast<float*>(out) + at;
    *reinterpret_cast<floatx4*>(o) = *reinterpret_cast<const floatx4*>(src);
    *reinterpret_cast<floatx4*>(o + 4) = *reinterpret_cast<const floatx4*>(src + 4);
  }
}

template <bool BF16>
__device__ __forceinline__ void put(void* out, size_t at, float x) {
  if constexpr (BF16) {
    const unsigned u = __float_as_uint(x);
    static_cast<unsigned short*>(out)[at] = static_cast<unsigned short>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  } else {
    static_cast<float*>(out)[at] = x;
  }
}

// Expand dims d0..d0+7 of in-page token o (o = t for a whole-page tile) from
// `page` (global memory or an LDS copy) into the tile's A operands.
template <int KB, int VB, typename Row, typename Scal>
__device__ __forceinline__ void expand(const DArgs& a, const unsigned char* page, int t, int d0, int tid, Row ac, Row az,
                                       Row avh, Row avl, Scal sn, Scal sg, int o = -1) {
  if (o < 0) o = t;
  const int blk = d0 >> 5, e0 = d0 & 31;
  // key codes: 8 codes of KB bits at bit e0*KB of the token's 32-dim block record
  const unsigned char* kc = page + a.off_kc + (blk * 16 + o) * 4 * KB + (e0 / 8) * KB;
  unsigned x = 0;
#pragma unroll
  for (int b = 0; b < KB; ++b) x |= static_cast<unsigned>(kc[b]) << (8 * b);
  // sign bits of dims d0..d0+7 and (n, gamma); without QJL no signs and gamma 0
  const unsigned zb = a.qjl ? page[a.off_ks + (blk * 16 + o) * 4 + e0 / 8] : 0u;
  const unsigned kn = a.qjl ? *reinterpret_cast<const unsigned*>(page + a.off_kn + o * 4)
                            : *reinterpret_cast<const unsigned short*>(page + a.off_kn + o * 2);
  // value metadata: the group's scale and zero, or (codebook-coded values) the
  // token's norm / sqrt(d), read from a last field of 32 bytes per page
  float sc, zr;
  if (a.vm == 1) {
    const unsigned short vn = *reinterpret_cast<const unsigned short*>(page + a.off_vsz + o * 2);
    sc = __half2float(__ushort_as_half(vn)) * 0.08838834764831845f;
    zr = 0.0f;
  } else {
    const unsigned sz = *reinterpret_cast<const unsigned*>(page + a.off_vsz + o * 16 + (d0 >> 5) * 4);
    sc = __half2float(__ushort_as_half(static_cast<unsigned short>(sz & 0xffffu)));
    zr = __half2float(__ushort_as_half(static_cast<unsigned short>(sz >> 16)));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ac[t][d0 + i] = static_cast<_Float16>(a.cent[(x >> (KB * i)) & ((1u << KB) - 1u)]);
    az[t][d0 + i] = ((zb >> i) & 1u) ? static_cast<_Float16>(1.0f) : static_cast<_Float16>(-1.0f);
    // value code of (dim d0 + i, token o) in the lane-blocked stream
    const int j = d0 + i;
    const unsigned e = ((16u * (o >> 3) + (j & 15)) * 16u + 2u * (j >> 4) + ((o & 7) >> 2)) * 4u + (o & 3);
    const unsigned bit = e * VB;
    const unsigned char* vb = page + a.off_vc + (bit >> 3);
    const unsigned w = static_cast<unsigned>(vb[0]) | (static_cast<unsigned>(vb[1]) << 8);
    const unsigned code = (w >> (bit & 7)) & ((1u << VB) - 1u);
    const float v = (a.vm == 1) ? sc * a.vcent[code] : fmaf(sc, static_cast<float>(code), zr);
    const _Float16 h = static_cast<_Float16>(v);
    avh[t][d0 + i] = h;
    avl[t][d0 + i] = static_cast<_Float16>(v - static_cast<float>(h));
  }
  if ((tid & 15) == 0) {
    sn[t] = __half2float(__ushort_as_half(static_cast<unsigned short>(kn & 0xffffu))) * 0.08838834764831845f;
    sg[t] = a.kappa * __half2float(__ushort_as_half(static_cast<unsigned short>(kn >> 16)));
  }
}

template <int KB, int VB, bool OUT_BF16>
__global__ __launch_bounds__(256) void decompress_kernel(DArgs a) {
  const int g = blockIdx.y;
  const long long t0 = static_cast<long long>(blockIdx.x) * 16;
  const int tid = threadIdx.x;
  __shared__ __attribute__((aligned(16))) _Float16 ac[16][kARow];   // codebook values
  __shared__ __attribute__((aligned(16))) _Float16 az[16][kARow];   // signs +-1
  __shared__ __attribute__((aligned(16))) _Float16 avh[16][kARow];  // v' hi
  __shared__ __attribute__((aligned(16))) _Float16 avl[16][kARow];  // v' lo
  __shared__ float sn[16], sg[16];
  __shared__ __attribute__((aligned(16))) float stk[4][16][36], stv[4][16][36];  // per-wave output staging

  // ---- expand the records: thread (t, c) = (tid / 16, tid % 16) takes dims 8c..8c+7 of token t.
  // A tile that is one whole aligned page (16 consecutive slots from a multiple
  // of 16) is first copied into LDS with one 16-byte read per thread; other
  // tiles read each token's fields from its own page.
  __shared__ __attribute__((aligned(16))) unsigned char pg[kMaxPage];
  const int t = tid >> 4, d0 = 8 * (tid & 15);
  bool whole = t0 + 16 <= a.n_tokens;
  long long s0 = -1;
  if (whole) {
    s0 = a.slots[t0];
    whole = s0 >= 0 && (s0 & 15) == 0;
#pragma unroll
    for (int j = 1; j < 16; ++j) whole = whole && a.slots[t0 + j] == s0 + j;
  }
  if (whole) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.pool + (static_cast<size_t>(s0 >> 4) * a.H + g) * a.block_bytes);
    if (tid * 16 < static_cast<int>(a.block_bytes)) reinterpret_cast<u32x4*>(pg)[tid] = src[tid];
    __syncthreads();
    expand<KB, VB>(a, pg, t, d0, tid, ac, az, avh, avl, sn, sg);
  } else {
    const long long slot = (t0 + t < a.n_tokens) ? a.slots[t0 + t] : -1;
    if (slot >= 0) {
      expand<KB, VB>(a, a.pool + (static_cast<size_t>(slot >> 4) * a.H + g) * a.block_bytes + 0, t, d0, tid, ac, az,
                     avh, avl, sn, sg, static_cast<int>(slot & 15));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ac[t][d0 + i] = az[t][d0 + i] = avh[t][d0 + i] = avl[t][d0 + i] = static_cast<_Float16>(0.0f);
      }
      if ((tid & 15) == 0) sn[t] = sg[t] = 0.0f;
    }
  }
  __syncthreads();

  // ---- wave w: column tiles 2w, 2w + 1 (dims 32w .. 32w + 31)
  const int lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int nt = 2 * w + u;
    floatx4 k1 = {0.0f, 0.0f, 0.0f, 0.0f}, k2 = k1, vv = k1;
    const u32x4* op = a.opd + (static_cast<size_t>(g) * 8 + nt) * 4 * 4 * 64 + lane;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const half8 rh = __builtin_bit_cast(half8, op[(4 * s + 0) * 64]);
      const half8 rl = __builtin_bit_cast(half8, op[(4 * s + 1) * 64]);
      const half8 ph = __builtin_bit_cast(half8, op[(4 * s + 2) * 64]);
      const half8 pl = __builtin_bit_cast(half8, op[(4 * s + 3) * 64]);
      const int k0 = 32 * s + 8 * kg;
      const half8 xc = *reinterpret_cast<const half8*>(&ac[col][k0]);
      const half8 xz = *reinterpret_cast<const half8*>(&az[col][k0]);
      const half8 xh = *reinterpret_cast<const half8*>(&avh[col][k0]);
      const half8 xl = *reinterpret_cast<const half8*>(&avl[col][k0]);
      k1 = mfma(xc, rh, k1);
      k1 = mfma(xc, rl, k1);
      k2 = mfma(xz, ph, k2);
      k2 = mfma(xz, pl, k2);
      vv = mfma(xh, rh, vv);
      vv = mfma(xh, rl, vv);
      vv = mfma(xl, rh, vv);
    }
    // lane (col, kg) holds tokens 4kg + r of output dim 16 nt + col: into this
    // wave's staging tile (tokens x its 32 dims)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * kg + r;
      stk[w][t][16 * u + col] = sn[t] * fmaf(sg[t], k2[r], k1[r]);
      stv[w][t][16 * u + col] = vv[r];
    }
  }
  // lane (token l / 4, segment l % 4) stores 8 consecutive dims of K and of V
  // (the staging tile is this wave's own: its LDS writes and reads stay in order)
  {
    const int t = lane >> 2, c8 = 8 * (lane & 3);
    if (t0 + t < a.n_tokens) {
      const size_t at = (static_cast<size_t>(t0 + t) * a.H + g) * 128 + 32 * w + c8;
      store8<OUT_BF16>(a.kout, at, &stk[w][t][c8]);
      store8<OUT_BF16>(a.vout, at, &stv[w][t][c8]);
    }
  }
}

// Uncompressed (bypass) pages: K [16][128] token-major, V^T [128][16] dim-major (bf16).
template <bool OUT_BF16>
__global__ __launch_bounds__(128) void decompress_bypass_kernel(const unsigned char* pool, const long long* slots,
                                                                void* kout, void* vout, int H, unsigned block_bytes) {
  const long long tok = blockIdx.x;
  const int g = blockIdx.y, d = threadIdx.x;
  const long long slot = slots[tok];
  const size_t at = (static_cast<size_t>(tok) * H + g) * 128 + d;
  float kx = 0.0f, vx = 0.0f;
  if (slot >= 0) {
    const unsigned short* page = reinterpret_cast<const unsigned short*>(
        pool + (static_cast<size_t>(slot >> 4) * H + g) * block_bytes);
    const int o = static_cast<int>(slot & 15);
    kx = __uint_as_float(static_cast<unsigned>(page[o * 128 + d]) << 16);
    vx = __uint_as_float(static_cast<unsigned>(page[2048 + d * 16 + o]) << 16);
  }
  put<OUT_BF16>(kout, at, kx);
  put<OUT_BF16>(vout, at, vx);
}

template <int KB, bool BF>
void* pick_v(int vb) {
  switch (vb) {
    case 2: return reinterpret_cast<void*>(&decompress_kernel<KB, 2, BF>);
    case 3: return reinterpret_cast<void*>(&decompress_kernel<KB, 3, BF>);
    case 4: return reinterpret_cast<void*>(&decompress_kernel<KB, 4, BF>);
  }
  return nullptr;
}
template <bool BF>
void* pick_kv(int kb, int vb) {
  switch (kb) {
    case 1: return pick_v<1, BF>(vb);
    case 2: return pick_v<2, BF>(vb);
    case 3: return pick_v<3, BF>(vb);
    case 4: return pick_v<4, BF>(vb);
  }
  return nullptr;
}

}  // namespace

tq_status launch_decompress(const tq_layer* L, const void* pool, const long long* slots, long long n_tokens,
                            void* k_out, void* v_out, tq_dtype out_dtype, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = out_dtype == TQ_BF16;
  const int H = L->cfg.n_kv_heads;
  const size_t row_bytes = static_cast<size_t>(H) * kDim * (bf ? 2 : 4);  // output bytes per token
  // Launched over token ranges (multiples of 16) small enough that no launch
  // exceeds 2^31 work-items in the token dimension: 128 lanes per token for
  // bypass layers, 256 per 16-token tile otherwise.
  const long long range = L->cfg.bypass ? (1LL << 24) : (1LL << 27);
  void* fn = nullptr;
  DArgs a;
  if (L->cfg.bypass) {
    fn = bf ? reinterpret_cast<void*>(&decompress_bypass_kernel<true>)
            : reinterpret_cast<void*>(&decompress_bypass_kernel<false>);
  } else {
    a.pool = static_cast<const unsigned char*>(pool);
    a.opd = reinterpret_cast<const u32x4*>(L->dOpD);
    a.H = H;
    a.block_bytes = static_cast<unsigned>(L->lay.block_bytes);
    a.off_kc = static_cast<unsigned>(L->lay.off_kc);
    a.off_ks = static_cast<unsigned>(L->lay.off_ks);
    a.off_kn = static_cast<unsigned>(L->lay.off_kn);
    a.off_vc = static_cast<unsigned>(L->lay.off_vc);
    a.off_vsz = static_cast<unsigned>(L->lay.off_vsz);
    a.kappa = static_cast<float>(std::sqrt(M_PI / 2.0) / kDim);
    for (int i = 0; i < 16; ++i) {
      a.cent[i] = L->centroids[i];
      a.vcent[i] = L->v_centroids[i];
    }
    a.vm = L->cfg.value_mode == TQ_VAL_MSE ? 1 : 0;
    a.qjl = L->cfg.key_mode == TQ_KEY_QJL ? 1 : 0;
    fn = bf ? pick_kv<true>(L->cfg.k_bits, L->cfg.v_bits) : pick_kv<false>(L->cfg.k_bits, L->cfg.v_bits);
    if (!fn) return fail(TQ_ERR_UNSUPPORTED, "no decompress kernel for k_bits=%d v_bits=%d", L->cfg.k_bits,
                         L->cfg.v_bits);
  }
  for (long long t0 = 0; t0 < n_tokens; t0 += range) {
    const long long n = n_tokens - t0 < range ? n_tokens - t0 : range;
    const long long* sr = slots + t0;
    void* kr = static_cast<unsigned char*>(k_out) + static_cast<size_t>(t0) * row_bytes;
    void* vr = static_cast<unsigned char*>(v_out) + static_cast<size_t>(t0) * row_bytes;
    hipError_t e;
    if (L->cfg.bypass) {
      const unsigned char* p = static_cast<const unsigned char*>(pool);
      unsigned bb = static_cast<unsigned>(L->lay.block_bytes);
      int hh = H;
      void* args[] = {&p, &sr, &kr, &vr, &hh, &bb};
      e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(n), H), dim3(128), args, 0, s);
    } else {
      a.slots = sr;
      a.kout = kr;
      a.vout = vr;
      a.n_tokens = n;
      void* args[] = {&a};
      e = hipLaunchKernel(fn, dim3(static_cast<unsigned>((n + 15) / 16), H), dim3(256), args, 0, s);
    }
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "decompress launch: %s", hipGetErrorString(e));
  }
  return TQ_OK;
}

}  // namespace tq
