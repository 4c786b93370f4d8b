// Fused K+V compression on the matrix cores (gfx950), bf16 inputs.
//
// Same computation as compress.hip ("How 0xsero/turboquant works", "Compression
// Pipeline" and "Value Compression"; "5x Faster LLM Inference? ...", "Example 4:
// Kernel-Level Operations": normalise -> rotate -> quantise -> pack in one pass):
//   keys:   n = ||k||, t = sqrt(d) R k / n, idx = #{beta < t}, rho = t - c[idx],
//           gamma = ||rho||, z = [S rho >= 0]
//   values: v' = R v; per 32-group scale16 = fp16((max-min)/(2^b-1)), zero16 = fp16(min),
//           code = clamp(rint((v' - zero16)/scale16), 0, 2^b-1)  (0 when scale16 == 0)
//
// The three 128x128 contractions (R k, R v, S rho) are v_mfma_f32_16x16x32_f16
// tiles: 16 output coordinates x 16 tokens x 32 inputs.  float16 operands carry
// float32 precision by splitting: R = R_hi + R_lo and S = S_hi + S_lo (22
// significant bits, prepared once per layer), rho = rho_hi + rho_lo; bf16 inputs
// are exact in float16 after a power-of-two scale per vector (the norm's
// exponent).  Products are exact, each instruction sums exactly and rounds once
// to nearest, so every contraction chains its split passes into one float32
// accumulator: R k = R_hi k + R_lo k, S rho = S_hi rho_hi + S_hi rho_lo + S_lo rho_hi.
//
// A workgroup is 8 waves and serves one KV head: wave w owns output rows
// 16w..16w+15 and keeps its R and S operands in registers for the whole launch.
// Tiles of 16 tokens stream through: their K and V rows are copied straight into
// LDS (double-buffered), scaled to float16 operands once, contracted, quantised,
// and the results assembled into a page image in LDS.  A tile that is one whole
// aligned page (16 consecutive slots from a multiple of 16) is stored with
// coalesced 16-byte writes; any other tile is scattered token by token, with the
// dimension-major value codes set by atomic clear/set of their bits.
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
typedef __attribute__((address_space(3))) unsigned char lbyte;

constexpr int kRow = 136;  // float16 elements per LDS operand row (128 + pad)
constexpr int kCodeRow = 132;  // bytes per LDS code row (128 + pad)

struct CArgs {
  const unsigned short* k;  // bf16 bits
  const unsigned short* v;
  long long k_stride, v_stride;  // elements per token
  unsigned char* pool;
  const u32x4* opa;  // R/S operands, see tq_layer::dOpA
  long long n_tokens;
  long long n_tiles;
  int H;
  unsigned block_bytes;
  float cent[16];
  float bnd[16];
};

__device__ __forceinline__ floatx4 mfma(const half8& a, const half8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half8 as_h8(u32x4 v) { return __builtin_bit_cast(half8, v); }

// Cross-row exchanges (gfx950): see the decode mainloop.
__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                                  false, false);
  a = __builtin_bit_cast(float, static_cast<unsigned>(r[0]));
  b = __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                                  false, false);
  a = __builtin_bit_cast(float, static_cast<unsigned>(r[0]));
  b = __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
}
// Sum / min / max over the four 16-lane rows (every lane gets the result for its column).
__device__ __forceinline__ float rows_sum(float x) {
  float a = x, b = x;
  swap32(a, b);
  float y = a + b, c = y, d = y;
  swap16(c, d);
  return c + d;
}
__device__ __forceinline__ float rows_min(float x) {
  float a = x, b = x;
  swap32(a, b);
  float y = fminf(a, b), c = y, d = y;
  swap16(c, d);
  return fminf(c, d);
}
__device__ __forceinline__ float rows_max(float x) {
  float a = x, b = x;
  swap32(a, b);
  float y = fmaxf(a, b), c = y, d = y;
  swap16(c, d);
  return fmaxf(c, d);
}
// Sum over the 32 lanes of each half-wave (lanes 32q..32q+31).
__device__ __forceinline__ float half_sum(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  x += __shfl_xor(x, 16, 64);
  return x;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// One 64-lane x 16 B copy from global memory into LDS at dst + 16*lane (inline
// asm so the compiler's waits do not drain on it; awaited with wait_vmcnt).
__device__ __forceinline__ void copy_to_lds(const void* src, void* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      static_cast<unsigned>(reinterpret_cast<unsigned long>((lbyte*)dst)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0)
               : "memory", "m0");
}

// Page image offsets (same format as the store).
template <int KB, int VB>
struct Page {
  static constexpr int kc = 0;
  static constexpr int ks = 256 * KB;
  static constexpr int kn = ks + 256;
  static constexpr int vc = kn + 64;
  static constexpr int vsz = vc + 256 * VB;
  static constexpr int bytes = vsz + 256;
};

// Slot ids come as their own read-only, non-aliased parameter: the reads are
// wave-uniform and become scalar loads, which do not wait on the tile copies.
template <int KB, int VB>
__global__ __launch_bounds__(512) void compress_mfma_kernel(CArgs a, const long long* __restrict__ slots) {
  using PG = Page<KB, VB>;
  constexpr int LEVELS = 1 << KB;
  constexpr float kTop = static_cast<float>((1 << VB) - 1);
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kg = lane >> 4;

  __shared__ __attribute__((aligned(16))) unsigned short kv_in[2][2][16][128];  // [stage][K,V][token][dim] bf16
  __shared__ __attribute__((aligned(16))) _Float16 opk[16][kRow];   // scaled float16 key operand
  __shared__ __attribute__((aligned(16))) _Float16 opv[16][kRow];   // scaled float16 value operand
  __shared__ __attribute__((aligned(16))) _Float16 orh[16][kRow];   // rho hi
  __shared__ __attribute__((aligned(16))) _Float16 orl[16][kRow];   // rho lo
  __shared__ __attribute__((aligned(16))) unsigned char kcode[16][kCodeRow];
  __shared__ __attribute__((aligned(16))) unsigned char zbit[16][kCodeRow];
  __shared__ __attribute__((aligned(16))) unsigned char vcode[16][kCodeRow];
  __shared__ __attribute__((aligned(16))) unsigned char img[PG::bytes];
  __shared__ float fk[16], fv[16], gpart[8][16], vmin[8][16], vmax[8][16];
  __shared__ unsigned short n16s[16];

  // ---- this wave's R and S operands (row tile w), kept for the whole launch
  half8 Rhi[4], Rlo[4], Shi[4], Slo[4];
  {
    const u32x4* op = a.opa + static_cast<size_t>(h * 8 + w) * 4 * 4 * 64 + lane;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      Rhi[s] = as_h8(op[(0 * 4 + s) * 64]);
      Rlo[s] = as_h8(op[(1 * 4 + s) * 64]);
      Shi[s] = as_h8(op[(2 * 4 + s) * 64]);
      Slo[s] = as_h8(op[(3 * 4 + s) * 64]);
    }
  }

  // Consume the operands once here so the compiler's wait for these loads is not
  // placed inside the tile loop, where it would also cover the tile copies.
#pragma unroll
  for (int s = 0; s < 4; ++s) asm volatile("" ::"v"(Rhi[s]), "v"(Rlo[s]), "v"(Shi[s]), "v"(Slo[s]));

  // K/V rows of a tile into LDS: waves 0-3 copy K tokens 4w..4w+3, waves 4-7 the
  // V tokens; lane covers 16 B of a 256 B row.  Tokens past the end re-read token 0.
  auto stage_tile = [&](long long tile, int st) {
    const int kv = w >> 2;
    const int tok = 4 * (w & 3) + (lane >> 4);
    long long n = tile * 16 + tok;
    if (n >= a.n_tokens) n = 0;
    const unsigned short* base = kv ? a.v : a.k;
    const long long stride = kv ? a.v_stride : a.k_stride;
    const unsigned short* src = base + n * stride + static_cast<long long>(h) * 128 + (lane & 15) * 8;
    copy_to_lds(src, &kv_in[st][kv][4 * (w & 3)][0]);
  };

  long long tile = blockIdx.x;
  int st = 0;
  if (tile < a.n_tiles) stage_tile(tile, 0);
  for (; tile < a.n_tiles; tile += gridDim.x, st ^= 1) {
    const long long next = tile + gridDim.x;
    if (next < a.n_tiles) {
      stage_tile(next, st ^ 1);
      wait_vmcnt<1>();
    } else {
      wait_vmcnt<0>();
    }
    // ---- slots of this tile (scalar), whole-page test
    long long sl[16];
    bool full = true;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      sl[j] = (tile * 16 + j < a.n_tokens) ? slots[tile * 16 + j] : -1;
      full = full && sl[j] == sl[0] + j;
    }
    full = full && sl[0] >= 0 && (sl[0] & 15) == 0;
    __syncthreads();  // tile rows in LDS (every wave waited on its copy)

    // ---- A: norms, power-of-two scales, float16 operands (thread: token tid/32, dims 4p..4p+3)
    {
      const int tk = tid >> 5, p = tid & 31;
      const u32x2 kr = *reinterpret_cast<const u32x2*>(&kv_in[st][0][tk][4 * p]);
      const u32x2 vr = *reinterpret_cast<const u32x2*>(&kv_in[st][1][tk][4 * p]);
      float kx[4], vx[4];
      kx[0] = __uint_as_float(kr[0] << 16); kx[1] = __uint_as_float(kr[0] & 0xffff0000u);
      kx[2] = __uint_as_float(kr[1] << 16); kx[3] = __uint_as_float(kr[1] & 0xffff0000u);
      vx[0] = __uint_as_float(vr[0] << 16); vx[1] = __uint_as_float(vr[0] & 0xffff0000u);
      vx[2] = __uint_as_float(vr[1] << 16); vx[3] = __uint_as_float(vr[1] & 0xffff0000u);
      float k2 = 0.0f, v2 = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        k2 = fmaf(kx[i], kx[i], k2);
        v2 = fmaf(vx[i], vx[i], v2);
      }
      k2 = half_sum(k2);
      v2 = half_sum(v2);
      const float n = sqrtf(k2), nv = sqrtf(v2);
      // scale 2^-e with n in [2^e, 2^(e+1)): every scaled entry lies in (-2, 2)
      const int ek = (n > 0.0f) ? ilogbf(n) : 0;
      const int ev = (nv > 0.0f) ? ilogbf(nv) : 0;
      const float sk = ldexpf(1.0f, -ek), sv = ldexpf(1.0f, -ev);
      typedef _Float16 half4 __attribute__((ext_vector_type(4)));
      half4 hk, hv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hk[i] = static_cast<_Float16>(kx[i] * sk);
        hv[i] = static_cast<_Float16>(vx[i] * sv);
      }
      *reinterpret_cast<half4*>(&opk[tk][4 * p]) = hk;
      *reinterpret_cast<half4*>(&opv[tk][4 * p]) = hv;
      if (p == 0) {
        // t = sqrt(d) R k / n = sqrt(d) 2^e / n * (R k_scaled); zero norm -> t = 0
        fk[tk] = (n > 0.0f) ? ldexpf(sqrtf(128.0f) / n, ek) : 0.0f;
        fv[tk] = ldexpf(1.0f, ev);
        n16s[tk] = __half_as_ushort(__float2half_rn(n));
      }
    }
    __syncthreads();

    // ---- B: t = R k, codes, residual; v' = R v and its group extremes (row tile w)
    float vp[4];
    {
      floatx4 T = {0.0f, 0.0f, 0.0f, 0.0f};
      half8 kb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) kb[s] = *reinterpret_cast<const half8*>(&opk[col][32 * s + 8 * kg]);
#pragma unroll
      for (int s = 0; s < 4; ++s) T = mfma(Rhi[s], kb[s], T);
#pragma unroll
      for (int s = 0; s < 4; ++s) T = mfma(Rlo[s], kb[s], T);
      const float f = fk[col];
      float rho[4], g2 = 0.0f;
      unsigned codes = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float t = T[r] * f;
        int idx = 0;
#pragma unroll
        for (int i = 0; i < LEVELS - 1; ++i) idx += (a.bnd[i] < t) ? 1 : 0;
        float c = a.cent[0];
#pragma unroll
        for (int i = 1; i < LEVELS; ++i) c = (idx == i) ? a.cent[i] : c;
        rho[r] = t - c;
        g2 = fmaf(rho[r], rho[r], g2);
        codes |= static_cast<unsigned>(idx) << (8 * r);
      }
      g2 = rows_sum(g2);
      if (kg == 0) gpart[w][col] = g2;
      typedef _Float16 half4 __attribute__((ext_vector_type(4)));
      half4 rh, rl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rh[r] = static_cast<_Float16>(rho[r]);
        rl[r] = static_cast<_Float16>(rho[r] - static_cast<float>(rh[r]));
      }
      const int d0 = 16 * w + 4 * kg;
      *reinterpret_cast<half4*>(&orh[col][d0]) = rh;
      *reinterpret_cast<half4*>(&orl[col][d0]) = rl;
      *reinterpret_cast<unsigned*>(&kcode[col][d0]) = codes;

      floatx4 V = {0.0f, 0.0f, 0.0f, 0.0f};
      half8 vb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) vb[s] = *reinterpret_cast<const half8*>(&opv[col][32 * s + 8 * kg]);
#pragma unroll
      for (int s = 0; s < 4; ++s) V = mfma(Rhi[s], vb[s], V);
#pragma unroll
      for (int s = 0; s < 4; ++s) V = mfma(Rlo[s], vb[s], V);
      const float g = fv[col];
      float mn = INFINITY, mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vp[r] = V[r] * g;
        mn = fminf(mn, vp[r]);
        mx = fmaxf(mx, vp[r]);
      }
      mn = rows_min(mn);
      mx = rows_max(mx);
      if (kg == 0) {
        vmin[w][col] = mn;
        vmax[w][col] = mx;
      }
    }
    __syncthreads();

    // ---- C: y = S rho -> signs; value codes; per-token metadata into the page image
    {
      floatx4 Y = {0.0f, 0.0f, 0.0f, 0.0f};
      half8 rh[4], rl[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        rh[s] = *reinterpret_cast<const half8*>(&orh[col][32 * s + 8 * kg]);
        rl[s] = *reinterpret_cast<const half8*>(&orl[col][32 * s + 8 * kg]);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) Y = mfma(Shi[s], rh[s], Y);
#pragma unroll
      for (int s = 0; s < 4; ++s) Y = mfma(Shi[s], rl[s], Y);
#pragma unroll
      for (int s = 0; s < 4; ++s) Y = mfma(Slo[s], rh[s], Y);
      unsigned zb = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) zb |= (Y[r] >= 0.0f ? 1u : 0u) << (8 * r);
      const int d0 = 16 * w + 4 * kg;
      *reinterpret_cast<unsigned*>(&zbit[col][d0]) = zb;

      const int G = w >> 1;
      const float mn = fminf(vmin[2 * G][col], vmin[2 * G + 1][col]);
      const float mx = fmaxf(vmax[2 * G][col], vmax[2 * G + 1][col]);
      const __half s16 = __float2half_rn((mx - mn) / kTop);
      const __half z16 = __float2half_rn(mn);
      const float sc = __half2float(s16), zr = __half2float(z16);
      unsigned vc = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int code = 0;
        if (sc > 0.0f) code = static_cast<int>(fminf(fmaxf(rintf((vp[r] - zr) / sc), 0.0f), kTop));
        vc |= static_cast<unsigned>(code) << (8 * r);
      }
      *reinterpret_cast<unsigned*>(&vcode[col][d0]) = vc;
      if ((w & 1) == 0 && kg == 0)
        *reinterpret_cast<unsigned*>(&img[PG::vsz + col * 16 + G * 4]) =
            static_cast<unsigned>(__half_as_ushort(s16)) | (static_cast<unsigned>(__half_as_ushort(z16)) << 16);
      if (w == 7 && kg == 0) {
        float g2 = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) g2 += gpart[i][col];
        const unsigned short g16 = __half_as_ushort(__float2half_rn(sqrtf(g2)));
        *reinterpret_cast<unsigned*>(&img[PG::kn + col * 4]) =
            static_cast<unsigned>(n16s[col]) | (static_cast<unsigned>(g16) << 16);
      }
    }
    __syncthreads();

    // ---- D: pack codes and signs into the page image
    if (tid < 64) {
      // key codes: token t, 32-dim block b -> 4*KB bytes of LSB-first b-bit codes
      const int t = tid & 15, b = tid >> 4;
      unsigned wd[KB];
#pragma unroll
      for (int i = 0; i < KB; ++i) wd[i] = 0u;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const unsigned x = *reinterpret_cast<const unsigned*>(&kcode[t][32 * b + 4 * q]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * q + r, bit = KB * e;
          const unsigned c = (x >> (8 * r)) & 0xffu;
          wd[bit >> 5] |= c << (bit & 31);
          if ((bit & 31) + KB > 32) wd[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
        }
      }
      unsigned* dst = reinterpret_cast<unsigned*>(&img[PG::kc + (b * 16 + t) * 4 * KB]);
#pragma unroll
      for (int i = 0; i < KB; ++i) dst[i] = wd[i];
    } else if (tid < 128) {
      // sign bits: token t, block b -> one word
      const int t = tid & 15, b = (tid >> 4) & 3;
      unsigned wd = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const unsigned x = *reinterpret_cast<const unsigned*>(&zbit[t][32 * b + 4 * q]);
        wd |= ((x & 1u) | ((x >> 7) & 2u) | ((x >> 14) & 4u) | ((x >> 21) & 8u)) << (4 * q);
      }
      *reinterpret_cast<unsigned*>(&img[PG::ks + (b * 16 + t) * 4]) = wd;
    } else if (tid < 256) {
      // value codes: dimension row d = 16 tokens x VB bits
      const int d = tid - 128;
      unsigned long long row = 0;
#pragma unroll
      for (int t = 0; t < 16; ++t) row |= static_cast<unsigned long long>(vcode[t][d]) << (VB * t);
      unsigned char* dst = &img[PG::vc + d * 2 * VB];
      if constexpr (VB == 2) {
        *reinterpret_cast<unsigned*>(dst) = static_cast<unsigned>(row);
      } else if constexpr (VB == 4) {
        *reinterpret_cast<unsigned long long*>(dst) = row;
      } else {
        unsigned short* d16 = reinterpret_cast<unsigned short*>(dst);
        d16[0] = static_cast<unsigned short>(row);
        d16[1] = static_cast<unsigned short>(row >> 16);
        d16[2] = static_cast<unsigned short>(row >> 32);
      }
    }
    __syncthreads();

    // ---- E: store
    if (full) {
      unsigned char* page = a.pool + (static_cast<size_t>(sl[0] >> 4) * a.H + h) * a.block_bytes;
      for (int o = 16 * tid; o < PG::bytes; o += 16 * 512)
        *reinterpret_cast<u32x4*>(page + o) = *reinterpret_cast<const u32x4*>(&img[o]);
    } else {
      // token by token: fixed-size fields copied, value-code bits set atomically
#pragma unroll 1
      for (int t = 0; t < 16; ++t) {
        const long long s = sl[t];
        if (s < 0) continue;
        unsigned char* page = a.pool + (static_cast<size_t>(s >> 4) * a.H + h) * a.block_bytes;
        const int o = static_cast<int>(s & 15);
        const int f = tid;  // word of the token's record
        if (f < 4 * KB) {  // key codes: block f / KB, word f % KB
          const int b = f / KB, i = f % KB;
          reinterpret_cast<unsigned*>(page + PG::kc + (b * 16 + o) * 4 * KB)[i] =
              reinterpret_cast<const unsigned*>(&img[PG::kc + (b * 16 + t) * 4 * KB])[i];
        } else if (f < 4 * KB + 4) {
          const int b = f - 4 * KB;
          *reinterpret_cast<unsigned*>(page + PG::ks + (b * 16 + o) * 4) =
              *reinterpret_cast<const unsigned*>(&img[PG::ks + (b * 16 + t) * 4]);
        } else if (f == 4 * KB + 4) {
          *reinterpret_cast<unsigned*>(page + PG::kn + o * 4) = *reinterpret_cast<const unsigned*>(&img[PG::kn + t * 4]);
        } else if (f < 4 * KB + 9) {
          const int G = f - (4 * KB + 5);
          reinterpret_cast<unsigned*>(page + PG::vsz + o * 16)[G] =
              reinterpret_cast<const unsigned*>(&img[PG::vsz + t * 16])[G];
        } else if (f >= 128 && f < 256) {
          const int d = f - 128;
          unsigned* vw = reinterpret_cast<unsigned*>(page + PG::vc);
          const unsigned c = vcode[t][d];
          const unsigned bit = static_cast<unsigned>(16 * d + o) * VB;
          const unsigned wi = bit >> 5, sh = bit & 31, mask = (1u << VB) - 1u;
          atomicAnd(&vw[wi], ~(mask << sh));
          atomicOr(&vw[wi], c << sh);
          if (sh + VB > 32) {
            atomicAnd(&vw[wi + 1], ~(mask >> (32 - sh)));
            atomicOr(&vw[wi + 1], c >> (32 - sh));
          }
        }
      }
    }
    __syncthreads();  // the next tile rewrites slots, codes and the image
  }
}

template <int KB>
void* pick_v(int vb) {
  switch (vb) {
    case 2: return reinterpret_cast<void*>(&compress_mfma_kernel<KB, 2>);
    case 3: return reinterpret_cast<void*>(&compress_mfma_kernel<KB, 3>);
    case 4: return reinterpret_cast<void*>(&compress_mfma_kernel<KB, 4>);
  }
  return nullptr;
}
void* pick_kv(int kb, int vb) {
  switch (kb) {
    case 2: return pick_v<2>(vb);
    case 3: return pick_v<3>(vb);
    case 4: return pick_v<4>(vb);
  }
  return nullptr;
}

}  // namespace

bool compress_mfma_applies(const tq_layer* L, const void* k, const void* v, tq_dtype in_dtype, long long n_tokens,
                           long long k_stride, long long v_stride) {
  if (L->cfg.bypass || in_dtype != TQ_BF16 || !L->dOpA) return false;
  if (n_tokens < 64) return false;  // a handful of appended tokens: the per-token kernel is quicker
  // 16-byte aligned rows for the direct-to-LDS copies
  if ((k_stride % 8) || (v_stride % 8)) return false;
  if ((reinterpret_cast<unsigned long>(k) | reinterpret_cast<unsigned long>(v)) & 15) return false;
  return true;
}

tq_status launch_compress_mfma(const tq_layer* L, const void* k, const void* v, long long n_tokens,
                               long long k_stride, long long v_stride, const long long* slots, void* pool,
                               void* stream) {
  CArgs a;
  a.k = static_cast<const unsigned short*>(k);
  a.v = static_cast<const unsigned short*>(v);
  a.k_stride = k_stride;
  a.v_stride = v_stride;
  a.pool = static_cast<unsigned char*>(pool);
  a.opa = reinterpret_cast<const u32x4*>(L->dOpA);
  a.n_tokens = n_tokens;
  a.n_tiles = (n_tokens + 15) / 16;
  a.H = L->cfg.n_kv_heads;
  a.block_bytes = static_cast<unsigned>(L->lay.block_bytes);
  for (int i = 0; i < 16; ++i) {
    a.cent[i] = L->centroids[i];
    a.bnd[i] = L->boundaries[i];
  }
  void* fn = pick_kv(L->cfg.k_bits, L->cfg.v_bits);
  if (!fn) return fail(TQ_ERR_UNSUPPORTED, "no compress kernel for k_bits=%d v_bits=%d", L->cfg.k_bits, L->cfg.v_bits);
  // one resident workgroup per CU per head share, each looping over its tiles
  const int cus = L->cu_count > 0 ? L->cu_count : 256;
  long long gx = (static_cast<long long>(cus) * 2 + a.H - 1) / a.H;
  if (gx > a.n_tiles) gx = a.n_tiles;
  if (gx < 1) gx = 1;
  const long long* sp = slots;
  void* args[] = {&a, &sp};
  hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(a.H)), dim3(512), args, 0,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TQ_ERR_HIP, "compress launch: %s", hipGetErrorString(e));
  return TQ_OK;
}

}  // namespace tq
