// Split-K mainloop of paged decode attention over the compressed store (gfx950).
//
// Scores ("How 0xsero/turboquant works", "Key Storage and Attention Scoring";
// "turbo-attn 0.24.0", "How it works": query rotated once, attention in the
// rotated space, one pass with no decompress buffer):
//   s_i = scale * (n_i / sqrt d) * (q'.c[idx_i] + sqrt(pi/2)/128 * gamma_i * u.(2 z_i - 1)).
// Values ("How 0xsero/turboquant works", "Value Compression"):
//   o' = sum_i p_i (zero_i + scale_i * code_i), per 32-wide group.
//
// Both contractions run on v_mfma_f32_16x16x32_f16 with float32 accumulation:
//  * Q.K: A = q' split into two float16 pieces (hi + lo, 22 significant bits)
//    and u in float16 (the QJL term is ~10% of a score); B = the float16 stored
//    codebook values c[idx] (exact) and the +-1 signs (exact), dequantised from
//    the packed codes through LDS lookup tables.  Rows = query heads of the GQA
//    group (head h at row 4(h%4) + h/4), columns = 16 tokens, K = 32 dims.
//  * P.V: A = the centred value codes, code - 2^(b-1), as float16 integers
//    (a bias exponent OR-ed onto the masked code bits, then one packed
//    subtract -- exact); B = w = p * scale split into two float16 pieces.  Rows = 16 coordinates,
//    columns = query heads, K = 32 tokens (two pages).  The per-group offset
//    sum_i p_i (zero_i + 2^(b-1) scale_i) is accumulated on the vector ALU.
//    Centring keeps both sums free of a large cancelling offset, which
//    matters because the matrix-core accumulate truncates.
// A wave takes a 32-token chunk (two 16-token pages) at a time; the four waves
// of a workgroup take chunks in turn and merge at the end.  Online softmax keeps
// a running max per head (16-lane row reductions), rescaling only when the max
// grows by more than kRescale (the factor is folded into the final merge).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>

#include "tq_internal.hpp"

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kPart = kDim + 4;
constexpr float kRescale = 3.0f;   // tolerated growth of the running max (natural log units)
constexpr float kKappa = 0.0097916396f;  // sqrt(pi/2) / 128
constexpr float kInvSqrtD = 0.08838834764831845f;

struct MainArgs {
  const unsigned char* pool;
  const int* block_table;
  const int* seq_lens;
  const float* qu;  // [B*Hq][2][128]: q' then u
  float* part;      // [B*Hq][n_splits][kPart]
  long long max_blocks;
  int Hq, Hkv, n_splits, split_tokens;
  float scale;
  unsigned block_bytes, off_kc, off_ks, off_kn, off_vc, off_vsz;
  float cent[16];
};

__device__ __forceinline__ floatx4 mfma(const half8& a, const half8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half8 as_h8(u32x4 v) { return __builtin_bit_cast(half8, v); }
__device__ __forceinline__ float h_lo(unsigned w) { return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(w & 0xffffu))); }
__device__ __forceinline__ float h_hi(unsigned w) { return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(w >> 16))); }
__device__ __forceinline__ unsigned h_bits(float x) { return __builtin_bit_cast(unsigned short, static_cast<_Float16>(x)); }

// Max over the 16 lanes of a row (lanes 16r..16r+15).
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, __shfl_xor(x, 1, 64));
  x = fmaxf(x, __shfl_xor(x, 2, 64));
  x = fmaxf(x, __shfl_xor(x, 4, 64));
  x = fmaxf(x, __shfl_xor(x, 8, 64));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  return x;
}

// Packed float16 pair of (a, b), round toward zero; the remainder is exact in float32.
__device__ __forceinline__ unsigned pk_rtz(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(a, b));
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// float16 exponent bits (both halves) whose mantissa step at bit p is 1: value 2^(10-p).
__device__ __forceinline__ unsigned bias_bits(int p) {
  const unsigned e = static_cast<unsigned>(25 - p) << 10;
  return e | (e << 16);
}
// float16 bits (both halves) of bias + 2^(VB-1): subtracting them from (bias + code)
// leaves the centred code, code - 2^(VB-1), exactly.
template <int VB>
__device__ __forceinline__ unsigned centre_bits(unsigned bias) {
  const float v = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(bias & 0xffffu))) +
                  static_cast<float>(1 << (VB - 1));
  const unsigned h = __builtin_bit_cast(unsigned short, static_cast<_Float16>(v));
  return h | (h << 16);
}
// Packed float16 subtract (both halves): exact for the small integers here.
__device__ __forceinline__ unsigned sub_bias(unsigned x, unsigned bias) {
  const half2v r = __builtin_bit_cast(half2v, x) - __builtin_bit_cast(half2v, bias);
  return __builtin_bit_cast(unsigned, r);
}

// B operand of the Q.K product for K-chunk kc: the float16 codebook values of
// the lane's 8 dims (32kg + 8kc .. +7), from the packed codes of those 32 dims.
template <int KB>
__device__ __forceinline__ half8 dequant_keys(const unsigned* kc, int chunk, const unsigned* lut) {
  u32x4 r;
  if constexpr (KB == 4) {
    const unsigned x = kc[chunk];  // 8 nibbles = dims 8*chunk .. +7
    r[0] = lut[x & 0xffu];
    r[1] = lut[(x >> 8) & 0xffu];
    r[2] = lut[(x >> 16) & 0xffu];
    r[3] = lut[x >> 24];
  } else if constexpr (KB == 2) {
    const unsigned x = kc[chunk >> 1] >> (16 * (chunk & 1));  // 16 bits = 8 dims
    const u32x2* l2 = reinterpret_cast<const u32x2*>(lut);
    const u32x2 a = l2[x & 0xffu];
    const u32x2 b = l2[(x >> 8) & 0xffu];
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  } else {  // KB == 3: 24 bits at bit 24*chunk of the lane's 96
    const int bit = 24 * chunk;
    const int w = bit >> 5, sh = bit & 31;
    const unsigned lo = kc[w];
    const unsigned hi = (w + 1 < 3) ? kc[w + 1] : 0u;
    const unsigned x = sh ? ((lo >> sh) | (hi << (32 - sh))) : lo;
    r[0] = lut[x & 63u];
    r[1] = lut[(x >> 6) & 63u];
    r[2] = lut[(x >> 12) & 63u];
    r[3] = lut[(x >> 18) & 63u];
  }
  return as_h8(r);
}

// Row of a P.V tile holds dim 32G + dim_in_group(row, a).
template <int VB>
__device__ __forceinline__ int v_dim(int row, int a) {
  if constexpr (VB == 2) return 4 * (row & 7) + 2 * a + (row >> 3);
  return 2 * row + a;
}
typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;
typedef __attribute__((address_space(3))) unsigned char lbyte;

// Byte layout of one (block, head) page; the host checks that it matches the
// store layout before launching.
template <int KB, int VB>
struct PageLayout {
  static constexpr int kc = 0;
  static constexpr int ks = 256 * KB;
  static constexpr int kn = ks + 256;
  static constexpr int vc = kn + 64;
  static constexpr int vsz = vc + 256 * VB;
  static constexpr int bytes = vsz + 256;
  static constexpr int copies = (bytes + 1023) / 1024;  // 64 lanes x 16 B per copy
  static constexpr int lds = 1024 * copies;
};

// s_waitcnt with vmcnt <= n (lgkmcnt and expcnt not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // The memory clobber keeps every LDS read of the staged page below the wait.
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Copy one page from global memory straight into LDS (no registers): each
// instruction moves 64 lanes x 16 B to dst + 16*lane; lanes past the page end
// re-read the page start and only fill the LDS padding.
template <int KB, int VB>
__device__ __forceinline__ void stage_page(const unsigned char* page, unsigned char* dst, int lane) {
  using PL = PageLayout<KB, VB>;
#pragma unroll
  for (int i = 0; i < PL::copies; ++i) {
    const int off = 1024 * i + 16 * lane;
    const unsigned char* src = page + (off < PL::bytes ? off : 0);
    // Issued as inline asm on purpose: the compiler's wait insertion treats an
    // LDS-DMA copy it can see as aliasing every later LDS read and drains the
    // vector-memory counter before the first one, which serialises the double
    // buffer.  Completion of these copies is awaited explicitly (wait_vmcnt).
    const unsigned m0 = __builtin_amdgcn_readfirstlane(
        (unsigned)(unsigned long)(lbyte*)(dst + 1024 * i));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 ::"v"(src), "s"(m0) : "memory", "m0");
  }
}

// The block table comes as its own read-only, non-aliased parameter so that the
// wave-uniform block-id reads become scalar loads (they must not wait on the
// vector-memory counter that tracks the page copies in flight).
template <int NREP, int KB, int VB>
__global__ __launch_bounds__(256) void splitk_mfma_kernel(MainArgs a, const int* __restrict__ btab) {
  using PL = PageLayout<KB, VB>;
  constexpr int HPL = NREP > 4 ? 2 : 1;           // heads per lane in the score layout
  constexpr int VC = 16 * VB;                      // value-code bytes per token
  constexpr int LUTC = (KB == 4) ? 256 : (KB == 2 ? 512 : 64);  // dwords
  constexpr float kMidCode = static_cast<float>(1 << (VB - 1));
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int T = a.seq_lens[b];
  const int start = split * a.split_tokens;
  if (start >= T) return;
  const int end = min(T, start + a.split_tokens);

  __shared__ unsigned lut_c[LUTC];
  __shared__ u32x4 lut_s[256];
  // per wave, two stages of two pages each (the chunk being processed and the next)
  __shared__ __attribute__((aligned(16))) unsigned char stg[4][2][2][PL::lds];
  __shared__ __attribute__((aligned(16))) unsigned short wl[4][4][2][NREP][32];  // P.V weights (fp16)
  __shared__ __attribute__((aligned(16))) unsigned zero16[4];
  __shared__ float mg_m[4][NREP], mg_l[4][NREP];
  __shared__ float mg_z[4][NREP][4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const long long tbl = static_cast<long long>(b) * a.max_blocks;
  auto page_ptr = [&](int blk) {
    return a.pool + (static_cast<long long>(blk) * a.Hkv + g) * a.block_bytes;
  };

  // first chunk of this wave: start its copy before the table/operand setup
  int c0 = start + wave * 32;
  int nb0 = 0, nb1 = 0;
  if (c0 < end) {
    const int b0 = btab[tbl + (c0 >> 4)];
    const int b1 = (c0 + 16 < end) ? btab[tbl + (c0 >> 4) + 1] : b0;
    stage_page<KB, VB>(page_ptr(b0), &stg[wave][0][0][0], lane);
    stage_page<KB, VB>(page_ptr(b1), &stg[wave][0][1][0], lane);
    const int cn = c0 + 128;
    if (cn < end) {
      nb0 = btab[tbl + (cn >> 4)];
      nb1 = (cn + 16 < end) ? btab[tbl + (cn >> 4) + 1] : nb0;
    }
  }

  // ---- tables
  {
    const int e = tid;  // 256 threads, 256 entries
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned lo = ((e >> (2 * i)) & 1) ? 0x3C00u : 0xBC00u;
      const unsigned hi = ((e >> (2 * i + 1)) & 1) ? 0x3C00u : 0xBC00u;
      w[i] = lo | (hi << 16);
    }
    lut_s[e] = w;
    if constexpr (KB == 4) {
      lut_c[e] = h_bits(a.cent[e & 15]) | (h_bits(a.cent[e >> 4]) << 16);
    } else if constexpr (KB == 2) {
      lut_c[2 * e] = h_bits(a.cent[e & 3]) | (h_bits(a.cent[(e >> 2) & 3]) << 16);
      lut_c[2 * e + 1] = h_bits(a.cent[(e >> 4) & 3]) | (h_bits(a.cent[e >> 6]) << 16);
    } else {
      if (e < 64) lut_c[e] = h_bits(a.cent[e & 7]) | (h_bits(a.cent[e >> 3]) << 16);
    }
    if (tid < 4) zero16[tid] = 0u;
  }

  // ---- Q.K A operands: row = l%16 -> head g4 + 4r (if any), dims 32kg + 8kc + j
  half8 qhi[4], qlo[4], qu16[4];
  {
    const int r = col & 3, g4 = col >> 2;
    const int h = g4 + 4 * r;
    const bool has = (h < NREP) && (NREP > 4 || r == 0);
    // unconditional vector loads from a valid row, then zero the rows without a head
    const float* src = a.qu + static_cast<size_t>(b * a.Hq + g * NREP + (has ? h : 0)) * 256 + 32 * kg;
    const float keep = has ? 1.0f : 0.0f;
    floatx4 qv[8], uv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qv[i] = reinterpret_cast<const floatx4*>(src)[i];
      uv[i] = reinterpret_cast<const floatx4*>(src + 128)[i];
    }
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float q = keep * qv[2 * kc + (j >> 2)][j & 3];
        const float u = keep * uv[2 * kc + (j >> 2)][j & 3];
        const _Float16 qh = static_cast<_Float16>(q);
        qhi[kc][j] = qh;
        qlo[kc][j] = static_cast<_Float16>(q - static_cast<float>(qh));
        qu16[kc][j] = static_cast<_Float16>(u);
      }
    }
  }
  __syncthreads();

  // ---- per-wave running state
  float m_used[HPL], lsum[HPL], zacc[HPL][4];
#pragma unroll
  for (int hs = 0; hs < HPL; ++hs) {
    m_used[hs] = -INFINITY;
    lsum[hs] = 0.0f;
#pragma unroll
    for (int G = 0; G < 4; ++G) zacc[hs][G] = 0.0f;
  }
  floatx4 accv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) accv[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  // Pipeline: while a chunk is processed from one LDS stage, the next chunk's
  // pages are already being copied into the other; block ids run one further.
  int stage = 0;
  for (; c0 < end; c0 += 128, stage ^= 1) {
    const int cn = c0 + 128;
    if (cn < end) {
      stage_page<KB, VB>(page_ptr(nb0), &stg[wave][stage ^ 1][0][0], lane);
      stage_page<KB, VB>(page_ptr(nb1), &stg[wave][stage ^ 1][1][0], lane);
      const int cnn = cn + 128;
      if (cnn < end) {
        nb0 = btab[tbl + (cnn >> 4)];
        nb1 = (cnn + 16 < end) ? btab[tbl + (cnn >> 4) + 1] : nb0;
      }
      wait_vmcnt<2 * PL::copies>();
    } else {
      wait_vmcnt<0>();
    }
    const unsigned char* pg[2] = {&stg[wave][stage][0][0], &stg[wave][stage][1][0]};

    // ---- scores: one 16-token tile per page
    float s[2][HPL];
    bool valid[2];
    unsigned vsz[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const unsigned* kp = reinterpret_cast<const unsigned*>(pg[t] + PL::kc + col * (16 * KB) + kg * (4 * KB));
      unsigned kcw[KB];
#pragma unroll
      for (int i = 0; i < KB; ++i) kcw[i] = kp[i];
      const unsigned ksw = *reinterpret_cast<const unsigned*>(pg[t] + PL::ks + col * 16 + kg * 4);
      floatx4 acca = {0.0f, 0.0f, 0.0f, 0.0f}, accb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const half8 bc = dequant_keys<KB>(kcw, kc, lut_c);
        const half8 bs = as_h8(lut_s[(ksw >> (8 * kc)) & 0xffu]);
        acca = mfma(qhi[kc], bc, acca);
        acca = mfma(qlo[kc], bc, acca);
        accb = mfma(qu16[kc], bs, accb);
      }
      // score layout: lane (token col, row group kg) holds head kg + 4*hs in slot hs
      const unsigned kn = *reinterpret_cast<const unsigned*>(pg[t] + PL::kn + col * 4);
      const u32x4 sz = *reinterpret_cast<const u32x4*>(pg[t] + PL::vsz + col * 16);
      vsz[t][0] = sz[0]; vsz[t][1] = sz[1]; vsz[t][2] = sz[2]; vsz[t][3] = sz[3];
      valid[t] = (c0 + 16 * t + col) < end;
      const float alpha = a.scale * kInvSqrtD * h_lo(kn);
      const float kgam = kKappa * h_hi(kn);
#pragma unroll
      for (int hs = 0; hs < HPL; ++hs) {
        const float v = alpha * (acca[hs] + kgam * accb[hs]);
        s[t][hs] = valid[t] ? v : -INFINITY;
      }
    }

    // ---- online softmax (running max per head, lazy rescale)
    float p[2][HPL];
    bool need_any = false;
    float cmax[HPL];
#pragma unroll
    for (int hs = 0; hs < HPL; ++hs) {
      cmax[hs] = row_max16(fmaxf(s[0][hs], s[1][hs]));
      need_any |= cmax[hs] > m_used[hs] + kRescale;
    }
    if (__builtin_amdgcn_ballot_w64(need_any) != 0ull) {
      float fac[HPL];
#pragma unroll
      for (int hs = 0; hs < HPL; ++hs) {
        const float mnew = (cmax[hs] > m_used[hs] + kRescale) ? cmax[hs] : m_used[hs];
        fac[hs] = (m_used[hs] == -INFINITY) ? 0.0f : __expf(m_used[hs] - mnew);
        m_used[hs] = mnew;
        lsum[hs] *= fac[hs];
#pragma unroll
        for (int G = 0; G < 4; ++G) zacc[hs][G] *= fac[hs];
      }
      // P.V accumulators: column = head; its factor lives in score-layout row group h%4
      float f0 = __shfl(fac[0], 16 * (col & 3), 64);
      float fc = f0;
      if constexpr (HPL == 2) {
        const float f1 = __shfl(fac[1], 16 * (col & 3), 64);
        fc = (col >= 4) ? f1 : f0;
      }
      if (col >= NREP) fc = 1.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) accv[i] *= fc;
    }
#pragma unroll
    for (int hs = 0; hs < HPL; ++hs) {
      p[0][hs] = __expf(s[0][hs] - m_used[hs]);
      p[1][hs] = __expf(s[1][hs] - m_used[hs]);
      lsum[hs] += p[0][hs] + p[1][hs];
    }

    // ---- P.V weights w = p * scale (two float16 pieces) -> LDS, zero term on the VALU
#pragma unroll
    for (int hs = 0; hs < HPL; ++hs) {
      const int h = kg + 4 * hs;
      if (h < NREP) {
#pragma unroll
        for (int G = 0; G < 4; ++G) {
          const float w0 = valid[0] ? p[0][hs] * h_lo(vsz[0][G]) : 0.0f;
          const float w1 = valid[1] ? p[1][hs] * h_lo(vsz[1][G]) : 0.0f;
          const float z0 = valid[0] ? p[0][hs] * h_hi(vsz[0][G]) : 0.0f;
          const float z1 = valid[1] ? p[1][hs] * h_hi(vsz[1][G]) : 0.0f;
          // value = (zero + mid*scale) + scale*(code - mid): the matrix cores take the
          // centred part, so neither sum carries a large cancelling offset
          zacc[hs][G] += z0 + z1 + kMidCode * (w0 + w1);
          const unsigned hi = pk_rtz(w0, w1);
          const unsigned lo = pk_rtz(w0 - h_lo(hi), w1 - h_hi(hi));
          *reinterpret_cast<unsigned*>(&wl[wave][G][0][h][2 * col]) = hi;
          *reinterpret_cast<unsigned*>(&wl[wave][G][1][h][2 * col]) = lo;
        }
      }
    }

    // ---- P.V on the matrix cores
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const u32x4* wsrc_hi = (col < NREP) ? reinterpret_cast<const u32x4*>(&wl[wave][G][0][col][8 * kg])
                                          : reinterpret_cast<const u32x4*>(zero16);
      const u32x4* wsrc_lo = (col < NREP) ? reinterpret_cast<const u32x4*>(&wl[wave][G][1][col][8 * kg])
                                          : reinterpret_cast<const u32x4*>(zero16);
      const half8 whi = as_h8(*wsrc_hi);
      const half8 wlo = as_h8(*wsrc_lo);
      u32x4 x0, x1;  // A operands of the group's two row tiles (codes as float16 integers)
      if constexpr (VB == 4 || VB == 2) {
        const int byte = (VB == 4) ? (16 * G + col) : (8 * G + (col & 7));
        // field of tile a at bit p of each 16-bit half; OR-ing the float16
        // exponent whose mantissa step at bit p is 1 gives (2^(10-p) + code),
        // exactly; the packed subtract then leaves the code.
        unsigned m0, m1, b0, b1;
        if constexpr (VB == 4) {
          m0 = 0x000F000Fu; b0 = 0x64006400u;   // bit 0: 1024 + code
          m1 = 0x00F000F0u; b1 = 0x54005400u;   // bit 4:   64 + code
        } else {
          const int f0 = col >> 3;
          m0 = 0x00030003u << (2 * f0);
          m1 = 0x00030003u << (2 * (2 + f0));
          b0 = bias_bits(2 * f0);
          b1 = bias_bits(2 * (2 + f0));
        }
        const unsigned c0s = centre_bits<VB>(b0), c1s = centre_bits<VB>(b1);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = 4 * kg + q;
          u16x2 pr;
          pr[0] = pg[0][PL::vc + t * VC + byte];
          pr[1] = pg[1][PL::vc + t * VC + byte];
          const unsigned xv = __builtin_bit_cast(unsigned, pr);
          x0[q] = sub_bias((xv & m0) | b0, c0s);
          x1[q] = sub_bias((xv & m1) | b1, c1s);
        }
      } else {  // VB == 3: dims (2 col, 2 col + 1) of group G = bits 6 col .. +5 of the group's 96
        const int bit = 6 * col;
        const int w = bit >> 5, sh = bit & 31;
        const int w2 = (sh > 26) ? w + 1 : w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = 4 * kg + q;
          const unsigned* g0 = reinterpret_cast<const unsigned*>(pg[0] + PL::vc + t * VC + 12 * G);
          const unsigned* g1 = reinterpret_cast<const unsigned*>(pg[1] + PL::vc + t * VC + 12 * G);
          const unsigned y0 = __builtin_amdgcn_alignbit(g0[w2], g0[w], sh);
          const unsigned y1 = __builtin_amdgcn_alignbit(g1[w2], g1[w], sh);
          x0[q] = sub_bias((y0 & 7u) | ((y1 & 7u) << 16) | 0x64006400u, centre_bits<VB>(0x64006400u));
          x1[q] = sub_bias(((y0 >> 3) & 7u) | (((y1 >> 3) & 7u) << 16) | 0x64006400u, centre_bits<VB>(0x64006400u));
        }
      }
      const half8 a0 = as_h8(x0), a1 = as_h8(x1);
      accv[2 * G] = mfma(a0, whi, accv[2 * G]);
      accv[2 * G] = mfma(a0, wlo, accv[2 * G]);
      accv[2 * G + 1] = mfma(a1, whi, accv[2 * G + 1]);
      accv[2 * G + 1] = mfma(a1, wlo, accv[2 * G + 1]);
    }
  }

  // ---- per-wave results -> LDS, then merge the four waves
#pragma unroll
  for (int hs = 0; hs < HPL; ++hs) {
    const int h = kg + 4 * hs;
    const float ls = row_sum16(lsum[hs]);
    float zs[4];
#pragma unroll
    for (int G = 0; G < 4; ++G) zs[G] = row_sum16(zacc[hs][G]);
    if (h < NREP && col == 0) {
      mg_m[wave][h] = m_used[hs];
      mg_l[wave][h] = ls;
#pragma unroll
      for (int G = 0; G < 4; ++G) mg_z[wave][h][G] = zs[G];
    }
  }
  __syncthreads();
  // reuse the weight area (each wave's slice is its own former weight slice):
  // acc [4 waves][NREP][128] floats
  static_assert(sizeof(wl) == 4 * NREP * 128 * sizeof(float), "merge area size");
  float* mbuf = reinterpret_cast<float*>(&wl[0][0][0][0][0]);
  if (col < NREP) {
    const int h = col;
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const float z = mg_z[wave][h][G];
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 4 * kg + r;
          const int d = 32 * G + v_dim<VB>(row, aa);
          mbuf[(wave * NREP + h) * 128 + d] = accv[2 * G + aa][r] + z;
        }
      }
    }
  }
  __syncthreads();
  for (int x = tid; x < NREP * 128; x += 256) {
    const int h = x >> 7, d = x & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mg_m[w][h]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (mg_m[w][h] == -INFINITY) continue;
      const float e = __expf(mg_m[w][h] - M);
      num += e * mbuf[(w * NREP + h) * 128 + d];
      den += e * mg_l[w][h];
    }
    float* dst = a.part + (static_cast<size_t>(b * a.Hq + g * NREP + h) * a.n_splits + split) * kPart;
    dst[d] = num;
    if (d == 0) {
      dst[128] = M;
      dst[129] = den;
    }
  }
}

template <int NREP, int KB>
void* pick_vb(int vb) {
  switch (vb) {
    case 2: return reinterpret_cast<void*>(&splitk_mfma_kernel<NREP, KB, 2>);
    case 3: return reinterpret_cast<void*>(&splitk_mfma_kernel<NREP, KB, 3>);
    case 4: return reinterpret_cast<void*>(&splitk_mfma_kernel<NREP, KB, 4>);
  }
  return nullptr;
}
template <int NREP>
void* pick_kb(int kb, int vb) {
  switch (kb) {
    case 2: return pick_vb<NREP, 2>(vb);
    case 3: return pick_vb<NREP, 3>(vb);
    case 4: return pick_vb<NREP, 4>(vb);
  }
  return nullptr;
}

}  // namespace

tq_status launch_splitk_tq(const tq_layer* L, const DecodePlan& plan, const void* pool, const int* block_table,
                           int max_blocks_per_seq, const int* seq_lens, float softmax_scale, const float* qu,
                           float* part, void* stream) {
  {
    const unsigned kb = L->cfg.k_bits, vb = L->cfg.v_bits;
    const tq::Layout& ly = L->lay;
    if (ly.off_kc != 0 || ly.off_ks != 256 * kb || ly.off_kn != 256 * kb + 256 || ly.off_vc != 256 * kb + 320 ||
        ly.off_vsz != 256 * (kb + vb) + 320 || ly.block_bytes != 256 * (kb + vb) + 576)
      return fail(TQ_ERR_UNSUPPORTED, "store layout does not match the decode kernels' page layout");
  }
  MainArgs a;
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
  void* fn = nullptr;
  switch (plan.rep) {
    case 1: fn = pick_kb<1>(L->cfg.k_bits, L->cfg.v_bits); break;
    case 2: fn = pick_kb<2>(L->cfg.k_bits, L->cfg.v_bits); break;
    case 4: fn = pick_kb<4>(L->cfg.k_bits, L->cfg.v_bits); break;
    case 8: fn = pick_kb<8>(L->cfg.k_bits, L->cfg.v_bits); break;
  }
  if (!fn) return fail(TQ_ERR_UNSUPPORTED, "no decode kernel for rep=%d k_bits=%d v_bits=%d", plan.rep,
                       L->cfg.k_bits, L->cfg.v_bits);
  const int* btab = block_table;
  void* args[] = {&a, &btab};
  const dim3 grid(plan.n_splits, L->cfg.n_kv_heads, plan.batch);
  hipError_t e = hipLaunchKernel(fn, grid, dim3(256), args, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TQ_ERR_HIP, "decode split-K launch: %s", hipGetErrorString(e));
  return TQ_OK;
}

}  // namespace tq
