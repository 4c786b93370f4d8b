// Split-K mainloop of paged decode attention over the compressed store (gfx950).
//
// Scores ("How 0xsero/turboquant works", "Key Storage and Attention Scoring";
// "turbo-attn 0.24.0", "How it works": the query is rotated once and the packed
// records are read directly, with no expanded copy of the cache):
//   s_i = scale * (n_i / sqrt d) * (q'.c[idx_i] + sqrt(pi/2)/128 * gamma_i * u.(2 z_i - 1)).
// Values ("How 0xsero/turboquant works", "Value Compression"):
//   o' = sum_i p_i (zero_i + scale_i * code_i), per 32-wide group;
// or, for values coded like the keys' codebook part ("5x Faster LLM
// Inference? ...", "What is TurboQuant-GPU?": MSE-coded values),
//   o' = sum_i p_i (nv_i / sqrt d) cv[code_i].
//
// Both contractions run on v_mfma_f32_16x16x32_f16 with float32 accumulation.
//
// Q.K: A = the query operand prepared by the prologue: q' and kappa*u, each
// split into two float16 pieces (hi + lo, 22 significant bits), stacked as
// rows of the 16-row tile (4 query heads: rows 0-3 q' hi, 4-7 q' lo, 8-11
// kappa u hi, 12-15 kappa u lo; 8 heads use two tiles, q' and kappa u).
// B = 16 tokens x 32 dims: the float16 stored codebook values c[idx] (exact)
// in four K-steps, then the +-1 signs (exact) in four more, dequantised from
// the packed codes through LDS lookup tables.  The code steps and the sign
// steps accumulate separately; the rows are folded into one score per
// (token, head) with cross-lane swaps, gamma applied to the sign part.
//
// P.V: A = 16 coordinates x 32 token slots: the centred value codes
// code - 2^(b-1) as float16 integers (a bias exponent OR-ed onto the masked
// code bits, then one packed subtract -- exact).  B = 32 token slots x 16
// columns: w = p * scale in two float16 pieces, hi in columns 0..R-1 and lo in
// columns R..2R-1 (R query heads), so one instruction takes both.  The
// per-group offset sum_i p_i (zero_i + 2^(b-1) scale_i) is accumulated on the
// vector ALU.  Centring keeps both sums free of a large cancelling offset (each
// accumulate rounds at the accumulator's magnitude, so a 1024-biased code would
// bury the signal).  MSE-coded values: A = the float16 value-codebook entries of
// the codes (exact; two codes per lookup in a replicated LDS table), B = the
// weights p * nv16 / sqrt(d) in two float16 pieces, the same for every group;
// no offset term.
//
// A wave takes a 32-token chunk (two 16-token pages) at a time; the four waves
// of a workgroup take chunks in turn and merge at the end.  While a chunk is
// processed from registers, the next chunk's page fields are loaded straight
// from global memory into a second register set (a two-chunk ring).  Online
// softmax keeps a running max per head, rescaling only when it grows by more
// than kRescale.  Registers and the lookup tables below are sized so that three
// workgroups share a CU.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "split_items.hpp"
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x3 __attribute__((ext_vector_type(3)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kPart = kDim + 4;
constexpr float kRescale = 3.0f;  // tolerated growth of the running max (natural log units)
constexpr float kInvSqrtD = 0.08838834764831845f;

struct MainArgs {
  const unsigned char* pool;
  const int* seq_lens;
  const u32x4* qa;  // prologue output: [B*Hkv][sets][4 K-steps][64 lanes] x 8 float16
  float* part;      // [B*Hq][n_splits][kPart]
  long long max_blocks;
  int Hq, Hkv, n_splits, split_tokens;
  int batch, work_list;  // item order of the grid (split_items.hpp)
  float scale;
  unsigned block_bytes;
  float cent[16];
  float vcent[16];  // value codebook (MSE-coded values)
};

__device__ __forceinline__ floatx4 mfma(const half8& a, const half8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half8 as_h8(u32x4 v) { return __builtin_bit_cast(half8, v); }
__device__ __forceinline__ float h_lo(unsigned w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(w & 0xffffu)));
}
__device__ __forceinline__ float h_hi(unsigned w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(w >> 16)));
}
__device__ __forceinline__ unsigned h_bits(float x) {
  return __builtin_bit_cast(unsigned short, static_cast<_Float16>(x));
}

// Max / sum over the 16 lanes of a row (lanes 16r..16r+15); every lane gets it.
// One DPP-sourced VALU op per step; each step is preceded by the two wait
// states a DPP read of a just-written VGPR needs.
#define TQ_ROW_STEP(op, ctrl) \
  asm volatile("s_nop 1\n\t" op " %0, %1, %1 " ctrl " row_mask:0xf bank_mask:0xf" : "=v"(x) : "v"(x))
__device__ __forceinline__ float row_max16(float x) {
  TQ_ROW_STEP("v_max_f32_dpp", "quad_perm:[1,0,3,2]");
  TQ_ROW_STEP("v_max_f32_dpp", "quad_perm:[2,3,0,1]");
  TQ_ROW_STEP("v_max_f32_dpp", "row_ror:4");
  TQ_ROW_STEP("v_max_f32_dpp", "row_ror:8");
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  TQ_ROW_STEP("v_add_f32_dpp", "quad_perm:[1,0,3,2]");
  TQ_ROW_STEP("v_add_f32_dpp", "quad_perm:[2,3,0,1]");
  TQ_ROW_STEP("v_add_f32_dpp", "row_ror:4");
  TQ_ROW_STEP("v_add_f32_dpp", "row_ror:8");
  return x;
}
// x + (x of the lane NREP columns further along the 16-lane row).
template <int NREP>
__device__ __forceinline__ float add_from_col(float x) {
  float r;
  if constexpr (NREP == 8)
    asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(x));
  else if constexpr (NREP == 4)
    asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_ror:12 row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(x));
  else if constexpr (NREP == 2)
    asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_ror:14 row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(x));
  else
    asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_ror:15 row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(x));
  return r;
}
#undef TQ_ROW_STEP

// Cross-row exchanges (gfx950).  swap32(a, b): lanes 32..63 of a trade places
// with lanes 0..31 of b.  swap16(a, b): odd 16-lane rows of a trade places with
// the even rows of b.
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

// (x & m) | b and (a << 16) | b in one instruction each (VOP3 takes at most one
// scalar or literal operand on gfx950, so the constants are kept in VGPRs).
__device__ __forceinline__ unsigned and_or(unsigned x, unsigned m, unsigned b) {
  unsigned r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(b));
  return r;
}
__device__ __forceinline__ unsigned hi16_or(unsigned a, unsigned b) {
  unsigned r;
  asm("v_lshl_or_b32 %0, %1, 16, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Packed float16 subtract (both halves): exact for the small integers here.
__device__ __forceinline__ unsigned sub_h2(unsigned x, unsigned y) {
  const half2v r = __builtin_bit_cast(half2v, x) - __builtin_bit_cast(half2v, y);
  return __builtin_bit_cast(unsigned, r);
}

// Lookup tables in LDS, several copies of each so that the random
// code-indexed reads of a wave spread over the banks.  A key entry maps one
// byte of packed codes to float16 codebook values (KB 4: two codes -> two
// values, 4 bytes; KB 2: four codes -> four values, 8 bytes; KB 1: eight codes
// -> eight values, 16 bytes; KB 3: 6 bits of two codes -> two values, 4 bytes,
// entries 0..63 only); a sign entry maps a byte of 8 sign bits to eight float16
// +-1 (16 bytes).  The tables are sized so that three workgroups share a CU:
//   KB 1, 2, 4: 64 bytes of key copies per entry (4 of 16 bytes, 8 of 8, 16
//   of 4) and 4 sign copies of 16 bytes, each table 256 entries at a 64-byte
//   stride (16 KB each);
//   KB 3: 32 key copies of 4 bytes for entries 0..63 at a 128-byte stride
//   (8 KB), then 8 sign copies at a 128-byte stride (32 KB).
// A lookup address is one byte permute, which puts the code byte in bits
// 8..15 and the lane's copy offset, given scaled up by the stride's shift, in
// bits 0..7, then a shift right (by 2 for the 64-byte tables, by 1 for the
// 3-bit sign table; the 3-bit key address is formed from its 6-bit field
// directly).  Without QJL there is no sign table; MSE-coded values add the
// value-codebook table beside these.  Every variant at up to four query heads
// per KV head stays within a third of the CU's LDS.
template <int KB>
struct KeyLut {
  static constexpr int copy_bytes = KB == 1 ? 16 : KB == 2 ? 8 : 4;
};
template <int KB, bool MSEV, bool QJL>
struct LutShape {
  static constexpr int mode = KB == 3 ? 1 : 2;
  static constexpr int key_stride = mode == 1 ? 128 : 64;
  static constexpr int key_shift = mode == 2 ? 2 : 0;  // permute >> key_shift (1, 2, 4 bits)
  static constexpr int key_copies = mode == 2 ? 64 / KeyLut<KB>::copy_bytes : 32;
  static constexpr int sign_copies = mode == 2 ? 4 : 8;
  static constexpr int sign_shift = mode == 1 ? 1 : 2;
  static constexpr int sign_base = mode == 1 ? 64 * 128 : 256 * 64;
  static constexpr int sign_stride = mode == 1 ? 128 : 64;
  static constexpr int bytes = sign_base + (QJL ? 256 * sign_stride : 0);
};

// LDS address of entry `byte k of x` for a lane whose copy offset is `off`
// (< 256): one v_perm_b32 puts off in byte 0 and the code byte in byte 1.
template <int K>
__device__ __forceinline__ unsigned lut_addr(unsigned x, unsigned off) {
  return __builtin_amdgcn_perm(x, off, 0x0C0C0000u | ((4u + K) << 8));
}

// B operand of the Q.K product for K-step s: the float16 codebook values of the
// lane's 8 dims (32kg + 8s .. +7), from the packed codes of its 32-dim block.
// lut: the table's LDS base; koff: the lane's key copy offset.
template <int KB, int MODE>
__device__ __forceinline__ half8 dequant_keys(const unsigned* kc, int s, const unsigned char* lut, unsigned koff) {
  u32x4 r;
  if constexpr (KB == 1) {
    // byte s of the block's 32 one-bit codes = dims 8s .. 8s+7: one 16-byte entry
    constexpr int sh = MODE == 2 ? 2 : 0;
    return as_h8(*reinterpret_cast<const u32x4*>(lut + (((s == 0)   ? lut_addr<0>(kc[0], koff)
                                                          : (s == 1) ? lut_addr<1>(kc[0], koff)
                                                          : (s == 2) ? lut_addr<2>(kc[0], koff)
                                                                     : lut_addr<3>(kc[0], koff)) >> sh)));
  } else if constexpr (KB == 4) {
    const unsigned x = kc[s];  // 8 nibbles
    constexpr int sh = MODE == 2 ? 2 : 0;
    r[0] = *reinterpret_cast<const unsigned*>(lut + (lut_addr<0>(x, koff) >> sh));
    r[1] = *reinterpret_cast<const unsigned*>(lut + (lut_addr<1>(x, koff) >> sh));
    r[2] = *reinterpret_cast<const unsigned*>(lut + (lut_addr<2>(x, koff) >> sh));
    r[3] = *reinterpret_cast<const unsigned*>(lut + (lut_addr<3>(x, koff) >> sh));
  } else if constexpr (KB == 2) {
    const unsigned x = kc[s >> 1];  // bytes 2(s%2), 2(s%2)+1 = 8 dims
    constexpr int sh = MODE == 2 ? 2 : 0;
    const u32x2 a = *reinterpret_cast<const u32x2*>(lut + (((s & 1) ? lut_addr<2>(x, koff) : lut_addr<0>(x, koff)) >> sh));
    const u32x2 b = *reinterpret_cast<const u32x2*>(lut + (((s & 1) ? lut_addr<3>(x, koff) : lut_addr<1>(x, koff)) >> sh));
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  } else {  // KB == 3: 24 bits at bit 24 s of the block's 96
    const int bit = 24 * s;
    const int w = bit >> 5, sh = bit & 31;
    const unsigned x = (w + 1 < 3) ? __builtin_amdgcn_alignbit(kc[w + 1], kc[w], sh) : (kc[w] >> sh);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      r[q] = *reinterpret_cast<const unsigned*>(lut + ((((x >> (6 * q)) & 63u) << (MODE == 1 ? 7 : 8)) | koff));
  }
  return as_h8(r);
}

// float16 bits (both halves) whose exponent makes mantissa bit p weigh 1:
// OR-ed onto a code field masked at bits p.., the value is 2^(10-p) + code.
constexpr unsigned bias_bits(int p) { return static_cast<unsigned>(25 - p) * 0x04000400u; }
// float16 bits (both halves) of 2^(10-p) + 2^(VB-1): subtracting them leaves the
// centred code exactly.
constexpr unsigned centre_bits(int p, int vb) {
  return (static_cast<unsigned>(25 - p) * 0x0400u + ((1u << (vb - 1)) << p)) * 0x10001u;
}

// A operand of the P.V product for tile i (coordinates 16i .. 16i+15): the
// lane's run of 8 codes of coordinate 16i + col (tokens 8(kg%2) .. +7 of page
// kg/2, token 8(kg%2) + k at bit VB k of the run).  Element pair cc of the
// operand is (token cc, token 4 + cc): the run's two 4-code groups go to the
// two float16 halves, each code becomes a centred float16 integer exactly.
// The lane's run of 8 codes for tile i with tokens 0..3 in the low 16 bits and
// tokens 4..7 in the high 16 bits (field k of each half at bit VB k).
template <int VB>
__device__ __forceinline__ unsigned value_run(const unsigned* vc, int i) {
  if constexpr (VB == 4) {
    return vc[i];
  } else if constexpr (VB == 2) {
    // bytes 2(i%2), 2(i%2)+1 of the dword -> bytes 0 and 2 (zeros between)
    return __builtin_amdgcn_perm(vc[i >> 1], vc[i >> 1], (i & 1) ? 0x0C030C02u : 0x0C010C00u);
  } else {  // VB == 3: 24 bits at bit 24 i of the lane's 192
    const int bit = 24 * i, w = bit >> 5, sh = bit & 31;
    const unsigned f = (sh <= 8) ? (vc[w] >> sh) : __builtin_amdgcn_alignbit(vc[w + 1], vc[w], sh);
    return hi16_or((f >> 12) & 0xfffu, f & 0xfffu);
  }
}

template <int VB>
__device__ __forceinline__ half8 value_operand(const unsigned* vc, int i) {
  const unsigned x = value_run<VB>(vc, i);
  // Field cc sits at bit VB*cc of each half.  Fields that end inside the
  // float16 mantissa (bits 0..9) are used in place with a matching exponent;
  // the others are shifted down by 8 first.
  constexpr unsigned m = (1u << VB) - 1u;
  u32x4 r;
  const unsigned x8 = x >> 8;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const int p = VB * cc;
    const bool fits = p + VB <= 10;
    const int q = fits ? p : p - 8;
    const unsigned src = fits ? x : x8;
    const unsigned mask = (m << q) * 0x10001u;
    r[cc] = sub_h2(and_or(src, mask, bias_bits(q)), centre_bits(q, VB));
  }
  return as_h8(r);
}

// Value-codebook table of MSE-coded values: entry code_a | code_b << VB holds the
// float16 pair (cv[code_a], cv[code_b]), in `copies` adjacent copies so that the
// code-indexed reads of a wave spread over the LDS banks (2, 4 or 8 KB).
template <int VB>
struct ValLut {
  static constexpr int entries = 1 << (2 * VB);
  static constexpr int copies = VB == 2 ? 32 : VB == 3 ? 16 : 8;
  static constexpr int words = entries * copies;
};

// A operand of the P.V product for tile i with MSE-coded values: element pair cc
// = (token cc, token cc + 4) of the run, both codebook values from one lookup.
template <int VB>
__device__ __forceinline__ half8 value_operand_mse(const unsigned* vc, int i, const unsigned* vlut, unsigned vcopy) {
  const unsigned x = value_run<VB>(vc, i);
  constexpr unsigned m = (1u << VB) - 1u;
  u32x4 r;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const unsigned idx = ((x >> (VB * cc)) & m) | (((x >> (16 + VB * cc)) & m) << VB);
    r[cc] = vlut[idx * ValLut<VB>::copies + vcopy];
  }
  return as_h8(r);
}

// P.V operand slot of (page pg, in-page token t): the inverse of value_operand's
// element order (slot 8kg + j holds page kg/2, token 8(kg%2) + j/2 + 4(j%2)).
__device__ __forceinline__ int pv_slot(int pg, int t) {
  return 16 * pg + 8 * (t >> 3) + 2 * (t & 3) + ((t >> 2) & 1);
}

// Byte layout of one (block, head) page; the host checks that it matches the
// store layout before launching.
// MSEV: the last field is Vn [16] fp16 (the values' norms) instead of the
// groups' scale and zero.  !QJL (key modes without residual signs): no sign
// field, Kn [16] fp16 holds the magnitude alone.
template <int KB, int VB, bool MSEV, bool QJL>
struct PageLayout {
  static constexpr int kc = 0;
  static constexpr int ks = 256 * KB;
  static constexpr int kn = ks + (QJL ? 256 : 0);
  static constexpr int vc = kn + (QJL ? 64 : 32);
  static constexpr int vsz = vc + 256 * VB;
  static constexpr int bytes = vsz + (MSEV ? 32 : 256);
};

// Dword-aligned vector types for the global loads.
typedef unsigned u32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef unsigned u32x3a __attribute__((ext_vector_type(3), aligned(4)));
typedef unsigned u32x2a __attribute__((ext_vector_type(2), aligned(4)));

// One lane's share of one 32-token chunk (pages 0 and 1), loaded from the pool
// straight into registers: every field is stored so that this share is one
// contiguous read per field.
template <int KB, int VB, bool MSEV>
struct Chunk {
  unsigned kc[2][KB];   // key codes of 32-dim block kg of token col
  unsigned ks[2];       // their sign bits
  unsigned kn[2];       // float16 n, gamma of token col
  u32x4 sz[2];          // float16 scale, zero of token col's 4 groups (group-coded values)
  unsigned vn[2];       // float16 value norm of token col (MSE-coded values)
  unsigned vc[2 * VB];  // value-code runs of lane block 16(kg%2) + col of page kg/2
};

// The lane's byte offsets of its fields inside a page (loop-invariant).
struct LaneOffsets {
  unsigned kc, ks, kn, sz, vc;
};
template <int KB, int VB, bool MSEV, bool QJL>
__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
  using PL = PageLayout<KB, VB, MSEV, QJL>;
  const unsigned col = lane & 15, kg = lane >> 4;
  return LaneOffsets{PL::kc + static_cast<unsigned>(lane) * (4 * KB), PL::ks + 4u * lane,
                     PL::kn + (QJL ? 4u : 2u) * col,
                     PL::vsz + (MSEV ? 2u : 16u) * col, PL::vc + (16u * (kg & 1u) + col) * (8 * VB)};
}

// Loads of one lane: a page base common to the wave plus a 32-bit lane offset.
template <int KB, int VB, bool MSEV, bool QJL>
__device__ __forceinline__ void load_chunk(Chunk<KB, VB, MSEV>& c, const unsigned char* p0, const unsigned char* p1,
                                           const LaneOffsets& o, bool second_page_values) {
  const unsigned char* pg[2] = {p0, p1};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const unsigned char* kp = pg[t] + o.kc;
    if constexpr (KB == 4) {
      const u32x4a v = *reinterpret_cast<const u32x4a*>(kp);
      c.kc[t][0] = v[0]; c.kc[t][1] = v[1]; c.kc[t][2] = v[2]; c.kc[t][3] = v[3];
    } else if constexpr (KB == 3) {
      const u32x3a v = *reinterpret_cast<const u32x3a*>(kp);
      c.kc[t][0] = v[0]; c.kc[t][1] = v[1]; c.kc[t][2] = v[2];
    } else if constexpr (KB == 1) {
      c.kc[t][0] = *reinterpret_cast<const unsigned*>(kp);
    } else {
      const u32x2a v = *reinterpret_cast<const u32x2a*>(kp);
      c.kc[t][0] = v[0]; c.kc[t][1] = v[1];
    }
    if constexpr (QJL) {
      c.ks[t] = *reinterpret_cast<const unsigned*>(pg[t] + o.ks);
      c.kn[t] = *reinterpret_cast<const unsigned*>(pg[t] + o.kn);
    } else {  // the magnitude alone, in the low half (gamma taken as 0)
      c.kn[t] = *reinterpret_cast<const unsigned short*>(pg[t] + o.kn);
    }
    if constexpr (MSEV)
      c.vn[t] = *reinterpret_cast<const unsigned short*>(pg[t] + o.sz);
    else
      c.sz[t] = *reinterpret_cast<const u32x4*>(pg[t] + o.sz);
  }
  const unsigned char* vp = (second_page_values ? p1 : p0) + o.vc;
  if constexpr (VB == 4) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(vp);
    const u32x4 b = *reinterpret_cast<const u32x4*>(vp + 16);
    c.vc[0] = a[0]; c.vc[1] = a[1]; c.vc[2] = a[2]; c.vc[3] = a[3];
    c.vc[4] = b[0]; c.vc[5] = b[1]; c.vc[6] = b[2]; c.vc[7] = b[3];
  } else if constexpr (VB == 2) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(vp);
    c.vc[0] = a[0]; c.vc[1] = a[1]; c.vc[2] = a[2]; c.vc[3] = a[3];
  } else {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const u32x2a a = *reinterpret_cast<const u32x2a*>(vp + 8 * u);
      c.vc[2 * u] = a[0];
      c.vc[2 * u + 1] = a[1];
    }
  }
}

// Query heads of the group held by a lane of the score layout: lane (token
// col, row group kg) holds head head(kg, hs) in slot hs.
template <int NREP>
struct ScoreMap {
  static constexpr int HPL = NREP == 8 ? 2 : 1;  // heads per lane
  static __device__ __forceinline__ int head(int kg, int hs) {
    if constexpr (NREP == 8) return 4 * (kg & 1) + 2 * (kg >> 1) + hs;
    if constexpr (NREP == 4 || NREP == 2) return kg;
    return 0;
  }
  static __device__ __forceinline__ bool active(int kg) {
    if constexpr (NREP >= 4) return true;
    if constexpr (NREP == 2) return kg < 2;
    return kg == 0;
  }
  // row group holding head h, and its slot
  static __device__ __forceinline__ int kg_of(int h) {
    if constexpr (NREP == 8) return ((h >> 2) & 1) | (((h >> 1) & 1) << 1);
    if constexpr (NREP == 4 || NREP == 2) return h;
    return 0;
  }
  static __device__ __forceinline__ int hs_of(int h) {
    if constexpr (NREP == 8) return h & 1;
    return 0;
  }
};

// Fold the Q.K accumulators of one 16-token tile into scores (before the
// per-token factor alpha): acc1 = code steps, acc2 = sign steps, g = gamma.
// Without QJL (acc2 unused) the prologue has written zero projection rows, so
// the rows that would hold kappa u contribute nothing to acc1 and need no mask.
template <int NREP, bool QJL>
__device__ __forceinline__ void fold_scores(const floatx4& acc1, const floatx4& acc2, float g, int kg,
                                            float (&out)[ScoreMap<NREP>::HPL]) {
  if constexpr (!QJL) {
    if constexpr (NREP == 8) {
      float x0 = acc1[0], x1 = acc1[1], x2 = acc1[2], x3 = acc1[3];
      swap32(x0, x2);
      swap32(x1, x3);
      out[0] = x0 + x2;
      out[1] = x1 + x3;
    } else if constexpr (NREP == 4) {
      float x0 = acc1[0], x1 = acc1[1], x2 = acc1[2], x3 = acc1[3];
      swap32(x0, x2);
      swap32(x1, x3);
      float y0 = x0 + x2, y1 = x1 + x3;
      swap16(y0, y1);
      out[0] = y0 + y1;
    } else if constexpr (NREP == 2) {
      float x0 = acc1[0] + acc1[2], x1 = acc1[1] + acc1[3];
      swap16(x0, x1);
      out[0] = x0 + x1;
    } else {
      out[0] = acc1[0] + acc1[1];
    }
  } else if constexpr (NREP == 8) {
    // tile 1 (q') rows 0-7 hi, 8-15 lo; tile 2 (kappa u) the same; row group kg
    // holds rows 4kg..4kg+3 -> hi/lo halves are lanes l and l+32
    float x0 = fmaf(g, acc2[0], acc1[0]), x1 = fmaf(g, acc2[1], acc1[1]);
    float x2 = fmaf(g, acc2[2], acc1[2]), x3 = fmaf(g, acc2[3], acc1[3]);
    swap32(x0, x2);
    swap32(x1, x3);
    out[0] = x0 + x2;
    out[1] = x1 + x3;
  } else if constexpr (NREP == 4) {
    // row group kg: 0 q' hi, 1 q' lo, 2 kappa u hi, 3 kappa u lo; slot r = head
    const bool sgn = kg >= 2;
    float x0 = sgn ? g * acc2[0] : acc1[0], x1 = sgn ? g * acc2[1] : acc1[1];
    float x2 = sgn ? g * acc2[2] : acc1[2], x3 = sgn ? g * acc2[3] : acc1[3];
    swap32(x0, x2);
    swap32(x1, x3);
    float y0 = x0 + x2, y1 = x1 + x3;
    swap16(y0, y1);
    out[0] = y0 + y1;
  } else if constexpr (NREP == 2) {
    // rows 0-1 q' hi, 2-3 q' lo (row group 0), 4-5 kappa u hi, 6-7 lo (group 1)
    float x0 = (kg == 1) ? g * (acc2[0] + acc2[2]) : acc1[0] + acc1[2];
    float x1 = (kg == 1) ? g * (acc2[1] + acc2[3]) : acc1[1] + acc1[3];
    swap16(x0, x1);
    out[0] = x0 + x1;
  } else {
    // rows 0 q' hi, 1 q' lo, 2 kappa u hi, 3 kappa u lo (row group 0)
    out[0] = (acc1[0] + acc1[1]) + g * (acc2[2] + acc2[3]);
  }
}


// Chunks held per wave: the pages of the next kRing - 1 chunks are being read
// while one is processed (two measured faster than three: fewer registers,
// same streaming rate).
constexpr int kRing = 2;

// The block table comes as its own read-only, non-aliased parameter.
// MSEV: values coded like the keys' codebook part (norm + value codebook).
template <int NREP, int KB, int VB, bool MSEV, bool QJL>
__global__ __launch_bounds__(256) void splitk_mfma_kernel(MainArgs a, const int* __restrict__ btab) {
  using SM = ScoreMap<NREP>;
  using KL = KeyLut<KB>;
  using VL = ValLut<VB>;
  constexpr int HPL = SM::HPL;
  constexpr int NSET = NREP == 8 ? 2 : 1;
  constexpr int WC = 2 * NREP;  // used P.V columns (hi, lo per head)
  constexpr float kMidCode = static_cast<float>(1 << (VB - 1));
  const SplitItem item = split_item(a.seq_lens, a.batch, a.Hkv, a.split_tokens, a.n_splits, a.work_list != 0);
  if (item.b < 0) return;  // past the work list (the whole workgroup)
  const int split = item.split, g = item.g, b = item.b;
  const int start = split * a.split_tokens;

  using LT = LutShape<KB, MSEV, QJL>;
  __shared__ __attribute__((aligned(16))) unsigned char lut[LT::bytes > 2048 * NREP ? LT::bytes : 2048 * NREP];
  __shared__ __attribute__((aligned(16))) unsigned short wl[4][MSEV ? 1 : 4][WC][32];  // P.V weights (float16)
  __shared__ unsigned vlut[MSEV ? VL::words : 1];  // value-codebook pairs (MSE-coded values)
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

  // Block ids of this wave's pages, one per lane: lane 2j + p holds page p of
  // the wave's chunk j (chunk j = tokens start + 32 (wave + 4j) .. +31; at most
  // 32 chunks per wave).  They and the query operand (prepared by the prologue)
  // are read before the sequence length is known, so that the three reads
  // overlap instead of forming a chain.  Table entries past the context (the
  // index clamped to the row) are read but never dereferenced: a page id is
  // used only for a chunk whose first token lies inside the context, and a
  // second page only when its first token does too, so padding entries of a
  // row may hold anything (-1 included).
  // (The host launches no split kernel for a table of zero blocks per row.)
  int ids;
  {
    const int tok = start + 32 * (wave + 4 * (lane >> 1)) + 16 * (lane & 1);
    const long long pg = static_cast<long long>(tok >> 4);
    ids = btab[tbl + (pg < a.max_blocks ? pg : a.max_blocks - 1)];
  }
  half8 qa[NSET][4];
  {
    const u32x4* src = a.qa + static_cast<size_t>(b * a.Hkv + g) * NSET * 4 * 64 + lane;
#pragma unroll
    for (int st = 0; st < NSET; ++st)
#pragma unroll
      for (int s = 0; s < 4; ++s) qa[st][s] = as_h8(src[(st * 4 + s) * 64]);
  }
  const int T = a.seq_lens[b];
  if (start >= T) {
    // the reads above stay ahead of this test (their results are not needed here)
    asm volatile("" ::"v"(ids));
#pragma unroll
    for (int st = 0; st < NSET; ++st)
#pragma unroll
      for (int s = 0; s < 4; ++s) asm volatile("" ::"v"(qa[st][s]));
    return;
  }
  const int end = min(T, start + a.split_tokens);
  const LaneOffsets lofs = lane_offsets<KB, VB, MSEV, QJL>(lane);
  const int span = end - start - 32 * wave;
  const int nch = span > 0 ? (span + 127) / 128 : 0;  // chunks of this wave
  auto load = [&](Chunk<KB, VB, MSEV>& c, int j) {
    const int c0 = start + 32 * (wave + 4 * j);
    // A wave with no chunk in the context (its first chunk starts at or past
    // the end) still issues the ring's loads, from block 0 (the pool holds at
    // least one block), so that no table entry past the context is used.
    const int b0 = nch > 0 ? __builtin_amdgcn_readlane(ids, 2 * j) : 0;
    const int b1 = (nch > 0 && c0 + 16 < end) ? __builtin_amdgcn_readlane(ids, 2 * j + 1) : b0;
    load_chunk<KB, VB, MSEV, QJL>(c, page_ptr(b0), page_ptr(b1), lofs, kg >= 2);
  };
  // Every step loads one chunk (past the wave's last chunk, the last one again:
  // a few cached re-reads) so that the number of loads in flight is the same on
  // every path, and each wait leaves the younger chunks' loads outstanding.
  const int jmax = nch > 0 ? nch - 1 : 0;
  Chunk<KB, VB, MSEV> ring[kRing];
#pragma unroll
  for (int r = 0; r < kRing; ++r) load(ring[r], r < jmax ? r : jmax);

  // ---- tables (lane copies); the codebook is staged in LDS from scalar
  //      registers so that no vector load joins the chunk loads in flight
  __shared__ unsigned short cent_h[16], vcent_h[16];
  if (tid == 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) cent_h[e] = static_cast<unsigned short>(h_bits(a.cent[e]));
    if constexpr (MSEV) {
#pragma unroll
      for (int e = 0; e < 16; ++e) vcent_h[e] = static_cast<unsigned short>(h_bits(a.vcent[e]));
    }
  }
  __syncthreads();
  if constexpr (MSEV) {
    constexpr unsigned m = (1u << VB) - 1u;
    for (int x = tid; x < VL::words; x += 256) {
      const unsigned e = static_cast<unsigned>(x / VL::copies);
      vlut[x] = vcent_h[e & m] | (static_cast<unsigned>(vcent_h[e >> VB]) << 16);
    }
  }
  {
    // lane tid fills entry tid of both tables, all copies (16-byte stores)
    const int e = tid;
    u32x4 kv = {0u, 0u, 0u, 0u};
    if constexpr (KB == 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        kv[q] = cent_h[(e >> (2 * q)) & 1] | (static_cast<unsigned>(cent_h[(e >> (2 * q + 1)) & 1]) << 16);
    } else if constexpr (KB == 4) {
      const unsigned v = cent_h[e & 15] | (static_cast<unsigned>(cent_h[e >> 4]) << 16);
      kv = u32x4{v, v, v, v};
    } else if constexpr (KB == 2) {
      const unsigned v0 = cent_h[e & 3] | (static_cast<unsigned>(cent_h[(e >> 2) & 3]) << 16);
      const unsigned v1 = cent_h[(e >> 4) & 3] | (static_cast<unsigned>(cent_h[e >> 6]) << 16);
      kv = u32x4{v0, v1, v0, v1};
    } else {
      const unsigned v = cent_h[e & 7] | (static_cast<unsigned>(cent_h[(e >> 3) & 7]) << 16);
      kv = u32x4{v, v, v, v};
    }
    u32x4 sv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const unsigned lo = ((e >> (2 * q)) & 1) ? 0x3C00u : 0xBC00u;
      const unsigned hi = ((e >> (2 * q + 1)) & 1) ? 0x3C00u : 0xBC00u;
      sv[q] = lo | (hi << 16);
    }
    constexpr int kq = LT::key_copies * KL::copy_bytes / 16;  // 16-byte stores per key entry
    constexpr int sq = LT::sign_copies;                       // (16 bytes per sign copy)
    if (e < (LT::mode == 1 ? 64 : 256)) {
      u32x4* ent = reinterpret_cast<u32x4*>(&lut[e * LT::key_stride]);
#pragma unroll
      for (int q = 0; q < kq; ++q) ent[q] = kv;  // key copies
    }
    if constexpr (QJL) {
      u32x4* ent = reinterpret_cast<u32x4*>(&lut[LT::sign_base + e * LT::sign_stride]);
#pragma unroll
      for (int q = 0; q < sq; ++q) ent[q] = sv;  // sign copies
    }
    if (tid < 4) zero16[tid] = 0u;
  }
  __syncthreads();
  const unsigned koff = static_cast<unsigned>((lane % LT::key_copies) * KL::copy_bytes) << LT::key_shift;
  const unsigned soff = static_cast<unsigned>((lane % LT::sign_copies) * 16) << LT::sign_shift;

  // ---- per-wave running state (score layout: slot hs = head SM::head(kg, hs))
  const bool active = SM::active(kg);
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
  const float sc = a.scale * kInvSqrtD;
  const int slot0 = pv_slot(0, col);

  const unsigned vcopy = static_cast<unsigned>(lane % VL::copies);
  // tail (std::true_type or std::false_type): whether the chunk may reach past
  // the split's end.  Only a wave's last chunk can, so the others are compiled
  // without the end-of-context selects (fewer instructions and registers).
  auto process = [&](const Chunk<KB, VB, MSEV>& c, int c0, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
    // ---- scores: one 16-token tile per page
    float s[2][HPL];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      floatx4 acc1 = {0.0f, 0.0f, 0.0f, 0.0f}, acc2 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        acc1 = mfma(qa[0][st], dequant_keys<KB, LT::mode>(c.kc[t], st, lut, koff), acc1);
        if constexpr (QJL) {
          const unsigned sp = (st == 0) ? lut_addr<0>(c.ks[t], soff)
                            : (st == 1) ? lut_addr<1>(c.ks[t], soff)
                            : (st == 2) ? lut_addr<2>(c.ks[t], soff) : lut_addr<3>(c.ks[t], soff);
          const unsigned sa = LT::sign_base + (sp >> LT::sign_shift);
          acc2 = mfma(qa[NSET - 1][st], as_h8(*reinterpret_cast<const u32x4*>(lut + sa)), acc2);
        }
      }
      const bool valid = TAIL ? (active && (c0 + 16 * t + col) < end) : active;
      float f[HPL];
      fold_scores<NREP, QJL>(acc1, acc2, h_hi(c.kn[t]), kg, f);
      const float alpha = sc * h_lo(c.kn[t]);
#pragma unroll
      for (int hs = 0; hs < HPL; ++hs) s[t][hs] = valid ? alpha * f[hs] : -INFINITY;
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
      // P.V column col holds head col % NREP (hi, then lo); its factor lives in
      // row group kg_of(head), slot hs_of(head)
      const int hc = col % NREP;
      const int srcl = 16 * SM::kg_of(hc);
      float fc = __shfl(fac[0], srcl, 64);
      if constexpr (HPL == 2) {
        const float f1 = __shfl(fac[1], srcl, 64);
        fc = SM::hs_of(hc) ? f1 : fc;
      }
      if (col >= WC) fc = 1.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) accv[i] *= fc;
    }
#pragma unroll
    for (int hs = 0; hs < HPL; ++hs) {
      p[0][hs] = __expf(s[0][hs] - m_used[hs]);
      p[1][hs] = __expf(s[1][hs] - m_used[hs]);
      lsum[hs] += p[0][hs] + p[1][hs];
    }

    // ---- P.V weights w = p * scale in two float16 pieces -> LDS (slots
    //      pv_slot(page, col)); offset term p (zero + mid scale) on the VALU.
    //      Past the context end (slots never written may hold any bits) the
    //      scale and zero are taken as 0, so that p = 0 gives exact zeros.
    if constexpr (MSEV) {
      // w = p * nv16 / sqrt(d), the same for every group (no offset term); a
      // never-written slot past the context end gets the norm 0
      float nv[2] = {h_lo(c.vn[0]) * kInvSqrtD, h_lo(c.vn[1]) * kInvSqrtD};
      if (TAIL && c0 + 32 > end) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
          if (c0 + 16 * t + col >= end) nv[t] = 0.0f;
      }
      if (active) {
#pragma unroll
        for (int hs = 0; hs < HPL; ++hs) {
          const int h = SM::head(kg, hs);
          const float w0 = p[0][hs] * nv[0], w1 = p[1][hs] * nv[1];
          const _Float16 hi0 = static_cast<_Float16>(w0), hi1 = static_cast<_Float16>(w1);
          const _Float16 lo0 = static_cast<_Float16>(fmaf(p[0][hs], nv[0], -static_cast<float>(hi0)));
          const _Float16 lo1 = static_cast<_Float16>(fmaf(p[1][hs], nv[1], -static_cast<float>(hi1)));
          unsigned short* wh = &wl[wave][0][h][0];
          unsigned short* wo = &wl[wave][0][NREP + h][0];
          wh[slot0] = __builtin_bit_cast(unsigned short, hi0);
          wh[slot0 + 16] = __builtin_bit_cast(unsigned short, hi1);
          wo[slot0] = __builtin_bit_cast(unsigned short, lo0);
          wo[slot0 + 16] = __builtin_bit_cast(unsigned short, lo1);
        }
      }
      const u32x4* wsrc = (col < WC) ? reinterpret_cast<const u32x4*>(&wl[wave][0][col][8 * kg])
                                     : reinterpret_cast<const u32x4*>(zero16);
      const half8 w = as_h8(*wsrc);
#pragma unroll
      for (int i = 0; i < 8; ++i) accv[i] = mfma(value_operand_mse<VB>(c.vc, i, vlut, vcopy), w, accv[i]);
      return;
    }
    u32x4 sz[2] = {c.sz[0], c.sz[1]};
    if (TAIL && c0 + 32 > end) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
        if (c0 + 16 * t + col >= end) sz[t] = u32x4{0u, 0u, 0u, 0u};
    }
    if (active) {
#pragma unroll
      for (int hs = 0; hs < HPL; ++hs) {
        const int h = SM::head(kg, hs);
#pragma unroll
        for (int G = 0; G < 4; ++G) {
          const _Float16 s0 = __builtin_bit_cast(_Float16, static_cast<unsigned short>(sz[0][G] & 0xffffu));
          const _Float16 s1 = __builtin_bit_cast(_Float16, static_cast<unsigned short>(sz[1][G] & 0xffffu));
          const _Float16 z0 = __builtin_bit_cast(_Float16, static_cast<unsigned short>(sz[0][G] >> 16));
          const _Float16 z1 = __builtin_bit_cast(_Float16, static_cast<unsigned short>(sz[1][G] >> 16));
          const float w0 = p[0][hs] * static_cast<float>(s0);
          const float w1 = p[1][hs] * static_cast<float>(s1);
          const _Float16 hi0 = static_cast<_Float16>(w0), hi1 = static_cast<_Float16>(w1);
          const _Float16 lo0 = static_cast<_Float16>(fmaf(p[0][hs], static_cast<float>(s0), -static_cast<float>(hi0)));
          const _Float16 lo1 = static_cast<_Float16>(fmaf(p[1][hs], static_cast<float>(s1), -static_cast<float>(hi1)));
          zacc[hs][G] = fmaf(p[0][hs], fmaf(kMidCode, static_cast<float>(s0), static_cast<float>(z0)), zacc[hs][G]);
          zacc[hs][G] = fmaf(p[1][hs], fmaf(kMidCode, static_cast<float>(s1), static_cast<float>(z1)), zacc[hs][G]);
          unsigned short* wh = &wl[wave][G][h][0];
          unsigned short* wo = &wl[wave][G][NREP + h][0];
          wh[slot0] = __builtin_bit_cast(unsigned short, hi0);
          wh[slot0 + 16] = __builtin_bit_cast(unsigned short, hi1);
          wo[slot0] = __builtin_bit_cast(unsigned short, lo0);
          wo[slot0 + 16] = __builtin_bit_cast(unsigned short, lo1);
        }
      }
    }

    // ---- P.V on the matrix cores: tile i = coordinates 16i .. 16i+15 (group i/2)
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const u32x4* wsrc = (col < WC) ? reinterpret_cast<const u32x4*>(&wl[wave][G][col][8 * kg])
                                     : reinterpret_cast<const u32x4*>(zero16);
      const half8 w = as_h8(*wsrc);
      accv[2 * G] = mfma(value_operand<VB>(c.vc, 2 * G), w, accv[2 * G]);
      accv[2 * G + 1] = mfma(value_operand<VB>(c.vc, 2 * G + 1), w, accv[2 * G + 1]);
    }
  };

  // Whole rounds of kRing chunks that do not hold the wave's last chunk (every
  // step processes one and loads one), then the last 1..kRing chunks, already
  // in flight, with the end-of-context masking.
  int j0 = 0;
  for (; j0 + kRing < nch; j0 += kRing) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      const int j = j0 + r;
      process(ring[r], start + 32 * (wave + 4 * j), std::false_type{});
      load(ring[r], j + kRing < jmax ? j + kRing : jmax);
    }
  }
#pragma unroll
  for (int r = 0; r < kRing; ++r)
    if (j0 + r < nch) process(ring[r], start + 32 * (wave + 4 * (j0 + r)), std::true_type{});

  // ---- per-wave results -> LDS, then merge the four waves
#pragma unroll
  for (int hs = 0; hs < HPL; ++hs) {
    const int h = SM::head(kg, hs);
    const float ls = row_sum16(lsum[hs]);
    float zs[4];
#pragma unroll
    for (int G = 0; G < 4; ++G) zs[G] = row_sum16(zacc[hs][G]);
    if (active && col == 0) {
      mg_m[wave][h] = m_used[hs];
      mg_l[wave][h] = ls;
#pragma unroll
      for (int G = 0; G < 4; ++G) mg_z[wave][h][G] = zs[G];
    }
  }
  // P.V accumulators: lane (col, kg) holds coordinate 16i + 4kg + r of column
  // col; add the lo column (col + NREP) onto the hi column
  // (row rotate by 16 - NREP: lane c of a 16-lane row reads lane c + NREP)
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) accv[i][r] = add_from_col<NREP>(accv[i][r]);
  __syncthreads();  // every wave is past its loop: the tables' space is free
  float* mbuf = reinterpret_cast<float*>(&lut[0]);  // [4 waves][NREP][128]
  static_assert(sizeof(lut) >= 4 * NREP * 128 * sizeof(float), "merge area size");
  if (col < NREP) {
    const int h = col;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float z = mg_z[wave][h][i >> 1];
#pragma unroll
      for (int r = 0; r < 4; ++r) mbuf[(wave * NREP + h) * 128 + 16 * i + 4 * kg + r] = accv[i][r] + z;
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

template <int NREP, int KB, bool MSEV, bool QJL>
void* pick_vb(int vb) {
  switch (vb) {
    case 2: return reinterpret_cast<void*>(&splitk_mfma_kernel<NREP, KB, 2, MSEV, QJL>);
    case 3: return reinterpret_cast<void*>(&splitk_mfma_kernel<NREP, KB, 3, MSEV, QJL>);
    case 4: return reinterpret_cast<void*>(&splitk_mfma_kernel<NREP, KB, 4, MSEV, QJL>);
  }
  return nullptr;
}
template <int NREP, bool MSEV, bool QJL>
void* pick_kb(int kb, int vb) {
  switch (kb) {
    case 1: return pick_vb<NREP, 1, MSEV, QJL>(vb);
    case 2: return pick_vb<NREP, 2, MSEV, QJL>(vb);
    case 3: return pick_vb<NREP, 3, MSEV, QJL>(vb);
    case 4: return pick_vb<NREP, 4, MSEV, QJL>(vb);
  }
  return nullptr;
}
template <int NREP>
void* pick_mode(bool msev, bool qjl, int kb, int vb) {
  return msev ? (qjl ? pick_kb<NREP, true, true>(kb, vb) : pick_kb<NREP, true, false>(kb, vb))
              : (qjl ? pick_kb<NREP, false, true>(kb, vb) : pick_kb<NREP, false, false>(kb, vb));
}

}  // namespace

tq_status launch_splitk_tq(const tq_layer* L, const DecodePlan& plan, const void* pool, const int* block_table,
                           int max_blocks_per_seq, const int* seq_lens, float softmax_scale, const void* qa,
                           float* part, void* stream) {
  {
    const unsigned kb = L->cfg.k_bits, vb = L->cfg.v_bits;
    const unsigned last = L->cfg.value_mode == TQ_VAL_MSE ? 32 : 256;
    const unsigned key_meta = L->cfg.key_mode == TQ_KEY_QJL ? 320 : 32;  // Ks + Kn, or Kn alone
    const unsigned kn = L->cfg.key_mode == TQ_KEY_QJL ? 256 * kb + 256 : 256 * kb;
    const tq::Layout& ly = L->lay;
    if (ly.off_kc != 0 || ly.off_ks != 256 * kb || ly.off_kn != kn || ly.off_vc != 256 * kb + key_meta ||
        ly.off_vsz != 256 * (kb + vb) + key_meta || ly.block_bytes != 256 * (kb + vb) + key_meta + last)
      return fail(TQ_ERR_UNSUPPORTED, "store layout does not match the decode kernels' page layout");
  }
  MainArgs a;
  a.pool = static_cast<const unsigned char*>(pool);
  a.seq_lens = seq_lens;
  a.qa = static_cast<const u32x4*>(qa);
  a.part = part;
  a.max_blocks = max_blocks_per_seq;
  a.Hq = plan.n_q_heads;
  a.Hkv = L->cfg.n_kv_heads;
  a.n_splits = plan.n_splits;
  a.split_tokens = plan.split_tokens;
  a.batch = plan.batch;
  a.work_list = plan.work_list ? 1 : 0;
  a.scale = softmax_scale;
  a.block_bytes = static_cast<unsigned>(L->lay.block_bytes);
  for (int i = 0; i < 16; ++i) {
    a.cent[i] = L->centroids[i];
    a.vcent[i] = L->v_centroids[i];
  }
  const bool msev = L->cfg.value_mode == TQ_VAL_MSE, qjl = L->cfg.key_mode == TQ_KEY_QJL;
  void* fn = nullptr;
  switch (plan.rep) {
    case 1: fn = pick_mode<1>(msev, qjl, L->cfg.k_bits, L->cfg.v_bits); break;
    case 2: fn = pick_mode<2>(msev, qjl, L->cfg.k_bits, L->cfg.v_bits); break;
    case 4: fn = pick_mode<4>(msev, qjl, L->cfg.k_bits, L->cfg.v_bits); break;
    case 8: fn = pick_mode<8>(msev, qjl, L->cfg.k_bits, L->cfg.v_bits); break;
  }
  if (!fn) return fail(TQ_ERR_UNSUPPORTED, "no decode kernel for rep=%d k_bits=%d v_bits=%d", plan.rep,
                       L->cfg.k_bits, L->cfg.v_bits);
  const int* btab = block_table;
  void* args[] = {&a, &btab};
  const dim3 grid(static_cast<unsigned>(plan.n_splits * L->cfg.n_kv_heads * plan.batch));
  hipError_t e = hipLaunchKernel(fn, grid, dim3(256), args, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TQ_ERR_HIP, "decode split-K launch: %s", hipGetErrorString(e));
  return TQ_OK;
}

}  // namespace tq
