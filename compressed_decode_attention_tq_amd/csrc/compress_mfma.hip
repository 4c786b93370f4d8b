// Fused K+V compression on the matrix cores (gfx950), bf16 inputs.
//
// Same computation as compress.hip ("How 0xsero/turboquant works", "Compression
// Pipeline" and "Value Compression"; "5x Faster LLM Inference? ...", "Example 4:
// Kernel-Level Operations": normalise -> rotate -> quantise -> pack in one pass):
//   keys:   n = ||k||, t = sqrt(d) R k / n, idx = #{beta < t}, rho = t - c[idx],
//           gamma = ||rho||, z = [S rho >= 0]
//   values: v' = R v; per 32-group scale16 = fp16((max-min)/(2^b-1)), zero16 = fp16(min),
//           code = clamp(rint((v' - zero16)/scale16), 0, 2^b-1)  (0 when scale16 == 0);
//           or, coded like the keys' codebook part ("5x Faster LLM Inference? ...",
//           "What is TurboQuant-GPU?": MSE-coded values), nv = ||v||,
//           code = #{beta_v < sqrt(d) v' / nv} with the value codebook, Vn = fp16(nv)
//
// The three 128x128 contractions are 16x16x32 matrix-core tiles (16 output
// coordinates x 16 tokens x 32 inputs).  The matrix core forms exact products,
// sums them exactly and rounds once to nearest per instruction, so split
// operands give float32-faithful results chained in one accumulator:
//  * R k and R v on the bf16 MFMA: the bf16 inputs are the B operand as they
//    are, R is three bf16 pieces (hi + mid + lo = R exactly);
//  * S rho on the float16 MFMA: S and rho as float16 hi + lo pieces (22 bits),
//    S rho = S_hi rho_hi + S_hi rho_lo + S_lo rho_hi.
//
// A workgroup is 8 waves and serves one KV head: wave w owns output rows
// 16w..16w+15 and keeps its R operands (and S_lo) in registers, S_hi in LDS, for
// the whole launch.  Tiles of 16 tokens stream through: their K and V rows are
// copied straight into a ring of LDS slots several tiles ahead (each row rotated
// by its token index so that the lanes reading one 32-dim slice hit distinct
// banks), contracted, quantised, and the packed fields written into a page
// image in LDS.  A tile that is one whole
// aligned page (16 consecutive slots from a multiple of 16) is stored with
// coalesced 16-byte writes; any other tile is scattered token by token, with the
// lane-blocked value codes set by atomic clear/set of their bits.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>

#include "f16_pieces.hpp"
#include "lds_copy.hpp"
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRow = 136;      // float16 elements per LDS operand row (128 + pad)

struct CArgs {
  const unsigned short* k;  // bf16 bits
  const unsigned short* v;
  long long k_stride, v_stride;  // elements per token
  unsigned char* pool;
  const u32x4* opa;  // R/S operands, see tq_layer::dOpA
  long long n_tokens;
  long long n_tiles;
  int H;
  int km;  // key mode: 0 QJL, 1 codebook only, 2 codebook only with norm-corrected magnitude
  float rscale;  // Hadamard layers: |R_ij| (the A operand holds the +-1 pattern)
  unsigned block_bytes;
  float cent[16];
  float bnd[16];
  float vcent[16];  // value codebook (MSE-coded values)
  float vbnd[16];
};

__device__ __forceinline__ floatx4 mfma_h(const half8& a, const half8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_b(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Cross-row exchanges (gfx950): swap32(a, b) trades lanes 32..63 of a with
// lanes 0..31 of b; swap16(a, b) trades the odd 16-lane rows of a with the even
// rows of b.
__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                                  false, false);
  a = __builtin_bit_cast(float, static_cast<unsigned>(r[0]));
  b = __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
}
__device__ __forceinline__ void swap16u(unsigned& a, unsigned& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = static_cast<unsigned>(r[0]);
  b = static_cast<unsigned>(r[1]);
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  unsigned x = __builtin_bit_cast(unsigned, a), y = __builtin_bit_cast(unsigned, b);
  swap16u(x, y);
  a = __builtin_bit_cast(float, x);
  b = __builtin_bit_cast(float, y);
}
// Sum / min / max over the four 16-lane rows (every lane gets its column's result).
__device__ __forceinline__ float rows_sum(float x) {
  float a = x, b = x;
  swap32(a, b);
  float y = a + b, c = y, d = y;
  swap16(c, d);
  return c + d;
}
// The combining min / max are plain instructions: the operands are ordinary
// values already, so no quieting of signalling NaNs is wanted around them.
__device__ __forceinline__ float min_raw(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float rows_min(float x) {
  float a = x, b = x;
  swap32(a, b);
  float y = min_raw(a, b), c = y, d = y;
  swap16(c, d);
  return min_raw(c, d);
}
__device__ __forceinline__ float rows_max(float x) {
  float a = x, b = x;
  swap32(a, b);
  float y = max_raw(a, b), c = y, d = y;
  swap16(c, d);
  return max_raw(c, d);
}


// Page image offsets (same format as the store; MSEV: the last field is Vn
// [16] fp16 instead of the groups' scale and zero; without QJL there is no sign
// field and Kn holds the magnitude alone, [16] fp16).
template <int KB, int VB, bool MSEV, bool QJL>
struct Page {
  static constexpr int kc = 0;
  static constexpr int ks = 256 * KB;
  static constexpr int kn = ks + (QJL ? 256 : 0);
  static constexpr int vc = kn + (QJL ? 64 : 32);
  static constexpr int vsz = vc + 256 * VB;
  static constexpr int bytes = vsz + (MSEV ? 32 : 256);
};

// Code of t in a symmetric codebook of 2 HALF levels: idx = #{beta < t}, ties to
// the lower cell.  For t <= 0 the count of positive boundaries uses the next
// float above |t|, so a boundary equal to |t| counts as "not below".  *cp = the
// chosen centroid's magnitude.
template <int HALF>
__device__ __forceinline__ int sym_code(float t, const float* cent, const float* bnd, float* cp) {
  const float m = fabsf(t);
  const float mq = (t > 0.0f) ? m : __uint_as_float(__float_as_uint(m) + 1u);
  int cnt = 0;
  float c = cent[HALF];
#pragma unroll
  for (int j = 0; j < HALF - 1; ++j) {
    const bool above = bnd[HALF + j] < mq;
    cnt += above ? 1 : 0;
    c = above ? cent[HALF + j + 1] : c;
  }
  *cp = c;
  return (t > 0.0f) ? HALF + cnt : HALF - 1 - cnt;
}

// sqrt(d) / n from n^2 (0 for a zero vector): the reciprocal square root where
// n^2 is a normal float, the quotient of roots for a subnormal n^2.
__device__ __forceinline__ float std_factor(float n2) {
  return (n2 >= 1.17549435e-38f) ? sqrtf(128.0f) * __builtin_amdgcn_rsqf(n2)
                                 : (n2 > 0.0f ? sqrtf(128.0f) / sqrtf(n2) : 0.0f);
}

// Bits of word p (0 .. 2 VB - 1) of a value-code run (the 64 codes of one
// coordinate column and half page: code 8 i + k at bits VB (8 i + k), k the
// offset within the half) that hold the codes of offsets k >= m.  The pattern
// repeats every 8 VB bits and a run starts on a word boundary.
template <int VB>
__device__ __forceinline__ unsigned vc_upper_mask(int p, int m) {
  constexpr int G = 8 * VB;
  const unsigned long long per = ((1ull << G) - 1ull) & ~((1ull << (VB * m)) - 1ull);
  unsigned long long q = 0;
#pragma unroll
  for (int i = 0; i < 64; i += G) q |= per << i;
  return static_cast<unsigned>(q >> ((32 * p) % G));
}

// Wait until at most n of this wave's vector-memory operations are outstanding,
// for n rounded down to one of the counts the tile loop can ask for with a
// ring of P tiles and two operations per fetched tile (3P - 2 in steady state,
// 2 (P - 1), ..., 2, 0 otherwise); wave-uniform n.  Loads and stores retire in
// issue order on this counter, so "at most n left" means every operation issued
// before the last n has completed.
template <int P>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  static_assert(P == 3, "wait levels are spelled out for a ring of three tiles");
  if (n >= 7)
    wait_vmcnt<7>();
  else if (n >= 4)
    wait_vmcnt<4>();
  else if (n >= 2)
    wait_vmcnt<2>();
  else
    wait_vmcnt<0>();
}

// Slot ids come as their own read-only, non-aliased parameter: the reads are
// wave-uniform and become scalar loads, which do not wait on the tile copies.
//
// The K/V rows and slots of P tiles are in flight at once (a ring of P LDS
// slots): HBM latency is covered by P tiles of work instead of one.  Every wave
// issues exactly two copies per tile it fetches (its share of the rows, then
// two of the tile's slots) and, for a whole-page tile, exactly one 16-byte page
// store, so the wait for tile k counts the operations issued after that tile's
// copies: 3P - 2 in steady state (the 2 (P - 1) copies of later tiles and the P
// page stores in between).  When a store was split or scattered, or a copy
// skipped, within that window, the wait counts only the copies known to follow,
// which is never more than what is outstanding.
//
// Page offsets: MFMA column c of a tile is page offset c.  A tile whose first
// token sits at offset r of its page is read rotated: column c takes the tile's
// input token (c - r) mod 16 (the rows stay in input order in LDS).  So a tile
// of 16 consecutive slots from offset 0 is one page image, and a tile whose
// first 16 - r tokens end one page and whose last r tokens start another (a
// sequence of a prefill batch that began at any token) is one image of two
// page parts, offsets r..15 for the first page and 0..r-1 for the second.
//
// HAD: the layer's rotation is a randomised Hadamard matrix, all entries
// +-rscale: R k = rscale (sign pattern) k, one exact bf16 pass instead of three.
// QJL: keys get the residual signs and gamma (key mode 0); otherwise the key
// mode (1 or 2: plain or norm-corrected magnitude) comes from a.km.
// MSEV: values coded like the keys' codebook part (value norm + value codebook).
template <int KB, int VB, int P, bool HAD, bool QJL, bool MSEV>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, QJL ? 4 : 8))) void compress_mfma_kernel(CArgs a, const long long* __restrict__ slots) {
  using PG = Page<KB, VB, MSEV, QJL>;
  constexpr int HALF = 1 << (KB - 1);  // codebook levels per sign
  constexpr float kTop = static_cast<float>((1 << VB) - 1);
  constexpr int kChunks = PG::bytes / 16;  // 16-byte chunks of a page (at most 164 = 8 waves x 21 lanes)
  static_assert(PG::bytes % 16 == 0 && kChunks <= 8 * 64, "page store mapping");
  static_assert(P >= 1 && 2 * P - 1 <= 15, "copy ring depth");
  const int h = blockIdx.y;
  const int lane0 = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);

  __shared__ __attribute__((aligned(16))) unsigned short kv_in[P][2][16][128];  // [slot][K,V][token][dim] bf16
  __shared__ __attribute__((aligned(16))) _Float16 orh[16][kRow];  // rho hi
  __shared__ __attribute__((aligned(16))) _Float16 orl[16][kRow];  // rho lo
  __shared__ __attribute__((aligned(16))) unsigned char img[PG::bytes];
  __shared__ float gpart[8][16], vmin[8][16], vmax[8][16];
  __shared__ __attribute__((aligned(16))) u32x4 s_hi[8][4][64];  // S_hi operands per wave and K-step
  __shared__ __attribute__((aligned(16))) long long sring[P][16];  // slots of the tiles in the ring

  // ---- this wave's R and S operands (row tile w), kept for the whole launch
  bf16x8 R0[4], R1[HAD ? 1 : 4], R2[HAD ? 1 : 4];
  half8 S1[4];
  {
    const u32x4* op = a.opa + static_cast<size_t>(h * 8 + w) * kOpSets * 4 * 64 + lane0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      R0[s] = __builtin_bit_cast(bf16x8, op[(0 * 4 + s) * 64]);
      if constexpr (!HAD) {
        R1[s] = __builtin_bit_cast(bf16x8, op[(1 * 4 + s) * 64]);
        R2[s] = __builtin_bit_cast(bf16x8, op[(2 * 4 + s) * 64]);
      }
      if constexpr (QJL) {  // the projection operands serve the residual signs only
        s_hi[w][s][lane0] = op[(3 * 4 + s) * 64];
        S1[s] = __builtin_bit_cast(half8, op[(4 * 4 + s) * 64]);
      }
    }
  }
  // Consume the operands here so that the compiler's wait for these loads is
  // not placed inside the tile loop, where it would also drain the copy ring.
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    asm volatile("" ::"v"(R0[s]));
    if constexpr (QJL) asm volatile("" ::"v"(S1[s]));
    if constexpr (!HAD) asm volatile("" ::"v"(R1[s]), "v"(R2[s]));
  }
  wait_vmcnt<0>();

  // K/V rows of one tile into ring slot `slot`: waves 0-3 copy K tokens 4w..4w+3,
  // waves 4-7 the V tokens.  Lane c of token row t fetches 16-byte chunk
  // (c - t) mod 16 of the row, so LDS position p of row t holds chunk
  // (p - t) mod 16.  Tokens past the end re-read token 0.
  auto stage = [&](long long tile, int slot, int lane) {
    const int kv = w >> 2;
    const int t = 4 * (w & 3) + (lane >> 4);
    const int q = ((lane & 15) - t) & 15;
    const unsigned short* base = kv ? a.v : a.k;
    const long long stride = kv ? a.v_stride : a.k_stride;
    void* dst = &kv_in[slot][kv][4 * (w & 3)][0];
    if (tile * 16 + 16 <= a.n_tokens) {
      // whole tile: the tile's first row (wave-uniform) plus a 32-bit lane offset
      const unsigned short* row0 = base + tile * 16 * stride + static_cast<long long>(h) * 128;
      copy_to_lds(row0 + (static_cast<unsigned>(t) * static_cast<unsigned>(stride) + static_cast<unsigned>(q) * 8u), dst);
    } else {
      long long n = tile * 16 + t;
      if (n >= a.n_tokens) n = 0;
      copy_to_lds(base + n * stride + static_cast<long long>(h) * 128 + q * 8, dst);
    }
    // slots 2w, 2w + 1 of the tile (one lane, 16 bytes); past the end, the last
    // two slots of the input (at least 64 tokens) stand in and are not used
    if (lane == 0) {
      long long i = tile * 16 + 2 * w;
      if (i + 2 > a.n_tokens) i = a.n_tokens - 2;
      copy_to_lds(slots + i, &sring[slot][2 * w]);
    }
  };

  const long long first = blockIdx.x, step = gridDim.x;
  // tiles of this workgroup (fewer than 2^31: the grid has at least one workgroup per CU and head)
  const int mine = first < a.n_tiles ? static_cast<int>((a.n_tiles - 1 - first) / step + 1) : 0;
  const int pro = mine < P ? mine : P;
  for (int j = 0; j < pro; ++j) stage(first + j * step, j, lane0);
  if constexpr (KB == 1 || KB == 3) {  // key-code words are OR-ed into; each tile's store clears them again
    for (int i = static_cast<int>(threadIdx.x); i < PG::ks / 4; i += 512) reinterpret_cast<unsigned*>(img)[i] = 0u;
  }
  unsigned clean = 0;  // bit i: iteration k-1-i issued two copies and one page store
  int slot = 0;  // k mod P
  for (int k = 0; k < mine; ++k, slot = (slot == P - 1) ? 0 : slot + 1) {
    const long long tile = first + static_cast<long long>(k) * step;
    // Lane-dependent addresses are recomputed in every iteration from an opaque
    // copy of the lane index: kept live across the loop they would not fit in
    // the 128 registers that let two workgroups share a CU.
    int lane = lane0;
    asm volatile("" : "+v"(lane));
    const int tid = 64 * w + lane;
    const int col = lane & 15, kg = lane >> 4;
    int after;  // operations known to be issued after this tile's copies
    if (k < P) {
      after = 2 * (pro - 1 - k);
    } else if ((clean & ((1u << P) - 1)) == (1u << P) - 1) {
      after = 3 * P - 2;
    } else {
      const int last = (k - 1 < mine - 1 - P) ? k - 1 : mine - 1 - P;
      after = 2 * (last - (k - P + 1) + 1);
    }
    wait_vmcnt_upto<P>(after);
    __syncthreads();  // tile rows and slots in LDS (every wave waited on its copies)
    // ---- the tile's slots (lane j < 16: input token j) and its store mode:
    // whole page (r = 0, 16 consecutive slots), two page parts (16 - r
    // consecutive slots from offset r, then r from offset 0 of a page), or
    // token by token
    const long long n0 = tile * 16;
    const long long sj = (n0 + (lane & 15) < a.n_tokens) ? sring[slot][lane & 15] : -1;
    const long long sA = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(sj)) |
                         (static_cast<long long>(__builtin_amdgcn_readfirstlane(static_cast<unsigned>(sj >> 32))) << 32);
    const int rot = sA >= 0 ? static_cast<int>(sA & 15) : 0;  // page offset of the tile's first token
    const int na = 16 - rot;  // tokens of the first part
    const long long sB = rot > 0 ? (static_cast<long long>(__builtin_amdgcn_readlane(static_cast<unsigned>(sj), na)) |
                                  (static_cast<long long>(__builtin_amdgcn_readlane(static_cast<unsigned>(sj >> 32), na)) << 32))
                               : sA;
    int mode;  // 1 whole page, 2 two page parts, 0 token by token
    {
      const int jj = lane & 15;
      const long long want = jj < na ? sA + jj : sB + (jj - na);
      const bool ok = sA >= 0 && sB >= 0 && (sB & 15) == (rot > 0 ? 0 : sA & 15) && sj == want;
      const bool all = (__builtin_amdgcn_ballot_w64(ok) & 0xffffull) == 0xffffull;
      mode = all ? (rot == 0 ? 1 : 2) : 0;
    }
    const bool full = mode == 1;

    // ---- B1: T = R k, V = R v (row tile w, 16 tokens), and every wave's own
    // ||k||^2: the Gram product of the tile's key rows with themselves, whose
    // diagonal is the squared norms (bf16 products are exact and each
    // instruction rounds its 32-term sum once).  The K/V operands are read one
    // K-step at a time (8 registers live, not 32); the key chunk a lane holds
    // is both the A row (token col) and the B column (token col) of the step.
    floatx4 T = {0.0f, 0.0f, 0.0f, 0.0f}, V = {0.0f, 0.0f, 0.0f, 0.0f}, NK = {0.0f, 0.0f, 0.0f, 0.0f};
    floatx4 NV = {0.0f, 0.0f, 0.0f, 0.0f};  // MSE-coded values: the values' Gram product
    const int row = (col - rot) & 15;  // input token of column (page offset) col
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int pos = (4 * s + kg + row) & 15;  // chunk 4s + kg of that token
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&kv_in[slot][0][row][8 * pos]);
      const bf16x8 vb = *reinterpret_cast<const bf16x8*>(&kv_in[slot][1][row][8 * pos]);
      T = mfma_b(R0[s], kb, T);
      V = mfma_b(R0[s], vb, V);
      NK = mfma_b(kb, kb, NK);
      if constexpr (MSEV) NV = mfma_b(vb, vb, NV);
      if constexpr (!HAD) {
        T = mfma_b(R1[s], kb, T);
        V = mfma_b(R1[s], vb, V);
        T = mfma_b(R2[s], kb, T);
        V = mfma_b(R2[s], vb, V);
      }
    }
    if constexpr (HAD) {
#pragma unroll
      for (int r = 0; r < 4; ++r) V[r] *= a.rscale;  // v' = rscale (sign pattern) v
    }
    // Gram entry (col, col) sits in lane col + 16 (col / 4), element col % 4.
    // The standardising factor sqrt(d)/n comes from the reciprocal square root
    // (within an ulp or so, like the quotient of rounded roots); the stored
    // norm n16 is taken from the correctly rounded root by the wave storing it.
    float f, k2, v2 = 0.0f;
    {
      const int e = col & 3;
      const float d01 = (e & 1) ? NK[1] : NK[0];
      const float d23 = (e & 1) ? NK[3] : NK[2];
      k2 = __shfl((e & 2) ? d23 : d01, col + 16 * (col >> 2), 64);
      f = std_factor(k2);  // zero norm: t = 0
      if constexpr (HAD) f *= a.rscale;  // t = (sqrt(d) / n) rscale (sign pattern) k
      if constexpr (MSEV) {
        const float e01 = (e & 1) ? NV[1] : NV[0];
        const float e23 = (e & 1) ? NV[3] : NV[2];
        v2 = __shfl((e & 2) ? e23 : e01, col + 16 * (col >> 2), 64);
      }
    }
    // A squared norm below 2^-100 (every entry below 2^-50) has too few float32
    // bits for the standardising factor, or none (products below the smallest
    // subnormal): rare, so recomputed here from the tile rows scaled by 2^100
    // (exact), with sqrt(d)/n = sqrt(d) 2^100 / ||2^100 x||.  Such a vector's
    // stored norm rounds to float16 0.
    float fv = MSEV ? std_factor(v2) : 0.0f;
    if (__builtin_amdgcn_ballot_w64(k2 < 0x1p-100f || (MSEV && v2 < 0x1p-100f)) != 0ull) {
      float sk2 = 0.0f, sv2 = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int pos = (4 * s + kg + row) & 15;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xk = __uint_as_float(static_cast<unsigned>(kv_in[slot][0][row][8 * pos + e]) << 16) * 0x1p100f;
          const float xv = __uint_as_float(static_cast<unsigned>(kv_in[slot][1][row][8 * pos + e]) << 16) * 0x1p100f;
          sk2 = fmaf(xk, xk, sk2);
          sv2 = fmaf(xv, xv, sv2);
        }
      }
      sk2 = rows_sum(sk2);
      sv2 = rows_sum(sv2);
      if (k2 < 0x1p-100f) {
        f = sk2 > 0.0f ? sqrtf(128.0f) * 0x1p100f * __builtin_amdgcn_rsqf(sk2) : 0.0f;
        if constexpr (HAD) f *= a.rscale;
        k2 = 0.0f;
      }
      if (MSEV && v2 < 0x1p-100f) {
        fv = sv2 > 0.0f ? sqrtf(128.0f) * 0x1p100f * __builtin_amdgcn_rsqf(sv2) : 0.0f;
        v2 = 0.0f;
      }
    }

    // ---- B2: t, codes, residual (rho -> LDS), key codes -> image; value extremes
    float vp[4];
    {
      float rho[4], g2 = 0.0f;
      unsigned codes = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float t = T[r] * f;
        float cp;
        const int idx = sym_code<HALF>(t, a.cent, a.bnd, &cp);
        rho[r] = t - ((t > 0.0f) ? cp : -cp);
        // squared norm of the residual (QJL) or of the centroid vector (norm correction)
        const float gt = QJL ? rho[r] : (a.km == 2 ? cp : 0.0f);
        g2 = fmaf(gt, gt, g2);
        codes |= static_cast<unsigned>(idx) << (KB * r);
      }
      g2 = rows_sum(g2);
      if (kg == 0) gpart[w][col] = g2;
      // the stored magnitude n (not the norm-corrected one, which needs the
      // residual sums of every wave): wave 3, which reaches the next barrier
      // early (its SIMD's matrix core served it first in B1)
      if (w == 3 && kg == 0 && (QJL || a.km != 2))
        *reinterpret_cast<unsigned short*>(&img[PG::kn + col * (QJL ? 4 : 2)]) =
            __half_as_ushort(__float2half_rn(sqrtf(k2)));
      // rho as float16 hi (RNE) and lo = float16(rho - hi), two coordinates per word
      u32x2 rh, rl;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        rh[r] = pack_f16(rho[2 * r], rho[2 * r + 1]);
        rl[r] = residual_pair(rho[2 * r], rho[2 * r + 1], rh[r]);
      }
      const int d0 = 16 * w + 4 * kg;
      if constexpr (QJL) {  // the residual feeds the QJL projection only
        *reinterpret_cast<u32x2*>(&orh[col][d0]) = rh;
        *reinterpret_cast<u32x2*>(&orl[col][d0]) = rl;
      }
      // key codes of dims d0..d0+3 = elements e0..e0+3 of block w/2 (4 KB bits)
      const int b = w >> 1, e0 = 16 * (w & 1) + 4 * kg;
      unsigned char* rec = &img[PG::kc + (b * 16 + col) * 4 * KB];
      if constexpr (KB == 2) {
        rec[e0 / 4] = static_cast<unsigned char>(codes);
      } else if constexpr (KB == 4) {
        *reinterpret_cast<unsigned short*>(rec + e0 / 2) = static_cast<unsigned short>(codes);
      } else {  // 1 or 3 bits: the four codes' field may share a word with other lanes' (or straddle two)
        const int bit = KB * e0, wi = bit >> 5, sh = bit & 31;
        unsigned* rw = reinterpret_cast<unsigned*>(rec);
        atomicOr(&rw[wi], codes << sh);
        if (sh + 4 * KB > 32) atomicOr(&rw[wi + 1], codes >> (32 - sh));
      }

#pragma unroll
      for (int r = 0; r < 4; ++r) vp[r] = V[r];
      if constexpr (!MSEV) {
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
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
    }
    __syncthreads();  // rho, norms and extremes in LDS; every wave is past B1, so
                      // ring slot `slot` may be refilled
    const bool fetch = k + P < mine;
    if (fetch) stage(first + static_cast<long long>(k + P) * step, slot, lane);

    // ---- C: y = S rho -> sign bits; value codes; per-token metadata
    {
      const int G = w >> 1;
      // sign nibble of dims d0..d0+3 (bit r = dim d0 + r); two row groups make a
      // byte (zero bits without QJL)
      unsigned nib = 0;
      if constexpr (QJL) {
        floatx4 Y = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const half8 sh = __builtin_bit_cast(half8, s_hi[w][s][lane]);
          const half8 rh = *reinterpret_cast<const half8*>(&orh[col][32 * s + 8 * kg]);
          const half8 rl = *reinterpret_cast<const half8*>(&orl[col][32 * s + 8 * kg]);
          Y = mfma_h(sh, rh, Y);
          Y = mfma_h(sh, rl, Y);
          Y = mfma_h(S1[s], rh, Y);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) nib |= (Y[r] >= 0.0f ? 1u : 0u) << r;
      }
      if constexpr (QJL) {
        unsigned ea = nib, eb = nib;
        swap16u(ea, eb);  // even row groups: ea = own, eb = the next group's nibble
        if ((kg & 1) == 0)
          img[PG::ks + ((w >> 1) * 16 + col) * 4 + 2 * (w & 1) + (kg >> 1)] = static_cast<unsigned char>(ea | (eb << 4));
      }

      unsigned x0, x1, x2, x3;
      __half s16, z16;
      if constexpr (MSEV) {
        // t = sqrt(d) v' / ||v|| against the value codebook (ties to the lower cell)
        const unsigned sh = VB * (col & 7);
        float cpv;
        x0 = static_cast<unsigned>(sym_code<(1 << (VB - 1))>(vp[0] * fv, a.vcent, a.vbnd, &cpv)) << sh;
        x1 = static_cast<unsigned>(sym_code<(1 << (VB - 1))>(vp[1] * fv, a.vcent, a.vbnd, &cpv)) << sh;
        x2 = static_cast<unsigned>(sym_code<(1 << (VB - 1))>(vp[2] * fv, a.vcent, a.vbnd, &cpv)) << sh;
        x3 = static_cast<unsigned>(sym_code<(1 << (VB - 1))>(vp[3] * fv, a.vcent, a.vbnd, &cpv)) << sh;
      } else {
      const float mn = fminf(vmin[2 * G][col], vmin[2 * G + 1][col]);
      const float mx = fmaxf(vmax[2 * G][col], vmax[2 * G + 1][col]);
      // (mx - mn) / kTop as the correctly rounded float32 quotient: product by
      // the rounded reciprocal, then one residual step (exact residual by fma)
      const float span = mx - mn;
      const float q0s = span * (1.0f / kTop);
      s16 = __float2half_rn(fmaf(fmaf(-q0s, kTop, span), 1.0f / kTop, q0s));
      z16 = __float2half_rn(mn);
      const float sc = __half2float(s16), zr = __half2float(z16);
      // reciprocal of the scale with one correction step
      const float inv0 = __builtin_amdgcn_rcpf(sc);
      const float inv = fmaf(fmaf(-sc, inv0, 1.0f), inv0, inv0);
      const float invz = (sc > 0.0f) ? inv : 0.0f;  // a zero scale gives code 0
      {
        // quotient to a couple of float32 ulps: a code can move only within
        // ~1e-7 relative of a rounding midpoint
        const unsigned sh = VB * (col & 7);
        x0 = static_cast<unsigned>(__builtin_amdgcn_fmed3f(rintf((vp[0] - zr) * invz), 0.0f, kTop)) << sh;
        x1 = static_cast<unsigned>(__builtin_amdgcn_fmed3f(rintf((vp[1] - zr) * invz), 0.0f, kTop)) << sh;
        x2 = static_cast<unsigned>(__builtin_amdgcn_fmed3f(rintf((vp[2] - zr) * invz), 0.0f, kTop)) << sh;
        x3 = static_cast<unsigned>(__builtin_amdgcn_fmed3f(rintf((vp[3] - zr) * invz), 0.0f, kTop)) << sh;
      }
      }
      // Value codes into the image's Vc field, in lane blocks: the run of
      // block (h, c, i) holds tokens 8h..8h+7 of coordinate 16i + c (token
      // 8h + j at bit VB j), VB bytes at (16h + c) 8VB + VB i.  This wave holds
      // coordinates 16w + 4kg + r of token col (x_r, already at bit VB (col % 8)),
      // i.e. block i = w: each run is an OR over the 8 lanes of a half row
      // (lane ^ 1, lane ^ 2, then the mirrored lane of the half row), and lane
      // j < 4 of the half row stores run r = j.  One DPP instruction per step;
      // the four runs interleave, so each step reads a result written three
      // instructions before (the first one after the required two wait states).
      asm volatile(
          "s_nop 1\n\t"
          "v_or_b32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_or_b32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_or_b32_dpp %2, %2, %2 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_or_b32_dpp %3, %3, %3 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_or_b32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
          "v_or_b32_dpp %1, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
          "v_or_b32_dpp %2, %2, %2 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
          "v_or_b32_dpp %3, %3, %3 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
          "v_or_b32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
          "v_or_b32_dpp %1, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
          "v_or_b32_dpp %2, %2, %2 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
          "v_or_b32_dpp %3, %3, %3 row_half_mirror row_mask:0xf bank_mask:0xf"
          : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3));
      {
        const int j = col & 7;
        if (j < 4) {
          const unsigned x = (j & 2) ? ((j & 1) ? x3 : x2) : ((j & 1) ? x1 : x0);
          unsigned char* dst = &img[PG::vc + (16 * (col >> 3) + 4 * kg + j) * 8 * VB + VB * w];
          if constexpr (VB == 4) {
            *reinterpret_cast<unsigned*>(dst) = x;
          } else if constexpr (VB == 2) {
            *reinterpret_cast<unsigned short*>(dst) = static_cast<unsigned short>(x);
          } else {
            dst[0] = static_cast<unsigned char>(x);
            dst[1] = static_cast<unsigned char>(x >> 8);
            dst[2] = static_cast<unsigned char>(x >> 16);
          }
        }
      }
      if constexpr (MSEV) {
        if (w == 6 && kg == 0)
          *reinterpret_cast<unsigned short*>(&img[PG::vsz + col * 2]) = __half_as_ushort(__float2half_rn(sqrtf(v2)));
      } else if ((w & 1) == 0 && kg == 0) {
        *reinterpret_cast<unsigned*>(&img[PG::vsz + col * 16 + G * 4]) =
            static_cast<unsigned>(__half_as_ushort(s16)) | (static_cast<unsigned>(__half_as_ushort(z16)) << 16);
      }
      if (w == 1 && kg == 0 && (QJL || a.km == 2)) {
        float g2 = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) g2 += gpart[i][col];
        // with QJL gamma beside n; without QJL and with norm correction the
        // magnitude n sqrt(d) / ||c[idx]|| (the plain n was written in B2)
        if constexpr (QJL) {
          *reinterpret_cast<unsigned short*>(&img[PG::kn + col * 4 + 2]) = __half_as_ushort(__float2half_rn(sqrtf(g2)));
        } else {
          *reinterpret_cast<unsigned short*>(&img[PG::kn + col * 2]) =
              __half_as_ushort(__float2half_rn(sqrtf(k2) * sqrtf(128.0f) / sqrtf(g2)));
        }
      }
    }
    __syncthreads();  // the page image is complete

    // ---- E: store
    if (full) {
      // one 16-byte store per wave: chunk w + 8 * lane (lane 0 is always in range)
      unsigned char* page = a.pool + (static_cast<size_t>(sA >> 4) * a.H + h) * a.block_bytes;
      const int c = w + 8 * lane;
      if (c < kChunks) {
        *reinterpret_cast<u32x4*>(page + 16 * c) = *reinterpret_cast<const u32x4*>(&img[16 * c]);
        if constexpr (KB == 1 || KB == 3) {  // key-code words are OR-ed into: clear what this lane read
          if (c < PG::ks / 16) *reinterpret_cast<u32x4*>(&img[16 * c]) = u32x4{0u, 0u, 0u, 0u};
        }
      }
    } else if (mode == 2) {
      // two page parts: offsets r..15 of the image to page A, 0..r-1 to page B.
      // Per-token fields move in units of 4 bytes (2 for the 16-bit magnitude
      // and norm fields), each unit one offset's; a value-code word holds the
      // codes of eight offsets, so a word with offsets of both parts is merged
      // into both pages with atomic clear / set of its bits (the neighbouring
      // tiles write the other bits of those pages' words the same way).
      unsigned char* pa = a.pool + (static_cast<size_t>(sA >> 4) * a.H + h) * a.block_bytes;
      unsigned char* pb = a.pool + (static_cast<size_t>(sB >> 4) * a.H + h) * a.block_bytes;
      constexpr int nKc = 64 * KB;        // word (16 b + o) KB + i
      constexpr int nKs = QJL ? 64 : 0;   // word 16 b + o
      constexpr int nKn = 16;             // unit o (4 bytes with QJL, else 2)
      constexpr int nVz = MSEV ? 16 : 64; // unit o (2 bytes), or word 4 o + G
      for (int u = tid; u < nKc + nKs + nKn + nVz; u += 512) {
        if (u < nKc) {
          const int o = (u / KB) & 15;
          *reinterpret_cast<unsigned*>((o >= rot ? pa : pb) + PG::kc + 4 * u) =
              *reinterpret_cast<const unsigned*>(&img[PG::kc + 4 * u]);
        } else if (u < nKc + nKs) {
          const int v = u - nKc, o = v & 15;
          *reinterpret_cast<unsigned*>((o >= rot ? pa : pb) + PG::ks + 4 * v) =
              *reinterpret_cast<const unsigned*>(&img[PG::ks + 4 * v]);
        } else if (u < nKc + nKs + nKn) {
          const int o = u - nKc - nKs;
          if constexpr (QJL)
            *reinterpret_cast<unsigned*>((o >= rot ? pa : pb) + PG::kn + 4 * o) =
                *reinterpret_cast<const unsigned*>(&img[PG::kn + 4 * o]);
          else
            *reinterpret_cast<unsigned short*>((o >= rot ? pa : pb) + PG::kn + 2 * o) =
                *reinterpret_cast<const unsigned short*>(&img[PG::kn + 2 * o]);
        } else {
          const int v = u - nKc - nKs - nKn;
          if constexpr (MSEV)
            *reinterpret_cast<unsigned short*>((v >= rot ? pa : pb) + PG::vsz + 2 * v) =
                *reinterpret_cast<const unsigned short*>(&img[PG::vsz + 2 * v]);
          else
            *reinterpret_cast<unsigned*>(((v >> 2) >= rot ? pa : pb) + PG::vsz + 4 * v) =
                *reinterpret_cast<const unsigned*>(&img[PG::vsz + 4 * v]);
        }
      }
      // value-code words: word u holds offsets 8 hh .. 8 hh + 7, hh = u / (32 VB)
      for (int u = tid; u < 64 * VB; u += 512) {
        const unsigned x = *reinterpret_cast<const unsigned*>(&img[PG::vc + 4 * u]);
        const int hh = u / (32 * VB), rs = rot >> 3;
        const unsigned ma = hh > rs ? ~0u : (hh < rs ? 0u : vc_upper_mask<VB>(u % (2 * VB), rot & 7));
        unsigned* wa = reinterpret_cast<unsigned*>(pa + PG::vc) + u;
        unsigned* wb = reinterpret_cast<unsigned*>(pb + PG::vc) + u;
        if (ma == ~0u) {
          *wa = x;
        } else if (ma == 0u) {
          *wb = x;
        } else {
          atomicAnd(wa, ~ma);
          atomicOr(wa, x & ma);
          atomicAnd(wb, ma);
          atomicOr(wb, x & ~ma);
        }
      }
      if constexpr (KB == 1 || KB == 3) {  // clear the key-code words read above
        for (int u = tid; u < nKc; u += 512) reinterpret_cast<unsigned*>(&img[PG::kc])[u] = 0u;
      }
    } else {
      // token by token: fixed-size fields copied, value-code bits set atomically;
      // image offset t holds the tile's input token (t - rot) mod 16
#pragma unroll 1
      for (int t = 0; t < 16; ++t) {
        const int j = (t - rot) & 15;
        // (the ring slot of this tile's slots is being refilled by now: read again)
        const long long s = n0 + j < a.n_tokens ? slots[n0 + j] : -1;
        if (s < 0) continue;
        unsigned char* page = a.pool + (static_cast<size_t>(s >> 4) * a.H + h) * a.block_bytes;
        const int o = static_cast<int>(s & 15);
        const int f = tid;  // word of the token's record
        if (f < 4 * KB) {  // key codes: block f / KB, word f % KB
          const int b = f / KB, i = f % KB;
          reinterpret_cast<unsigned*>(page + PG::kc + (b * 16 + o) * 4 * KB)[i] =
              reinterpret_cast<const unsigned*>(&img[PG::kc + (b * 16 + t) * 4 * KB])[i];
        } else if (f < 4 * KB + 4) {  // sign words (none without QJL)
          if constexpr (QJL) {
            const int b = f - 4 * KB;
            *reinterpret_cast<unsigned*>(page + PG::ks + (b * 16 + o) * 4) =
                *reinterpret_cast<const unsigned*>(&img[PG::ks + (b * 16 + t) * 4]);
          }
        } else if (f == 4 * KB + 4) {
          if constexpr (QJL)
            *reinterpret_cast<unsigned*>(page + PG::kn + o * 4) = *reinterpret_cast<const unsigned*>(&img[PG::kn + t * 4]);
          else
            *reinterpret_cast<unsigned short*>(page + PG::kn + o * 2) =
                *reinterpret_cast<const unsigned short*>(&img[PG::kn + t * 2]);
        } else if (f < 4 * KB + 9) {  // value metadata: word G of the token's record
          const int G = f - (4 * KB + 5);
          if constexpr (MSEV) {
            if (G == 0)
              *reinterpret_cast<unsigned short*>(page + PG::vsz + o * 2) =
                  *reinterpret_cast<const unsigned short*>(&img[PG::vsz + t * 2]);
          } else {
            reinterpret_cast<unsigned*>(page + PG::vsz + o * 16)[G] =
                reinterpret_cast<const unsigned*>(&img[PG::vsz + t * 16])[G];
          }
        } else if (f >= 128 && f < 256) {
          const int d = f - 128;
          unsigned* vw = reinterpret_cast<unsigned*>(page + PG::vc);
          // token t's code of coordinate d, read from its run in the image
          const unsigned et = ((16u * (t >> 3) + (d & 15)) * 16u + 2u * (d >> 4) + ((t & 7) >> 2)) * 4u + (t & 3);
          const unsigned bt = et * VB;
          const unsigned xb = img[PG::vc + (bt >> 3)] | (static_cast<unsigned>(img[PG::vc + (bt >> 3) + 1]) << 8);
          const unsigned c = (xb >> (bt & 7)) & ((1u << VB) - 1u);
          // lane-blocked Vc stream: block 16 (o / 8) + d % 16, group 2 (d / 16) + (o % 8) / 4
          const unsigned elem = ((16u * (o >> 3) + (d & 15)) * 16u + 2u * (d >> 4) + ((o & 7) >> 2)) * 4u + (o & 3);
          const unsigned bit = elem * VB;
          const unsigned wi = bit >> 5, sh = bit & 31, mask = (1u << VB) - 1u;
          atomicAnd(&vw[wi], ~(mask << sh));
          atomicOr(&vw[wi], c << sh);
          if (sh + VB > 32) {
            atomicAnd(&vw[wi + 1], ~(mask >> (32 - sh)));
            atomicOr(&vw[wi + 1], c >> (32 - sh));
          }
        }
      }
      if constexpr (KB == 1 || KB == 3) {  // clear the key-code words this thread read
        if (tid < 4 * KB) {
#pragma unroll 1
          for (int t = 0; t < 16; ++t)
            reinterpret_cast<unsigned*>(&img[PG::kc + ((tid / KB) * 16 + t) * 4 * KB])[tid % KB] = 0u;
        }
      }
    }
    clean = (clean << 1) | ((fetch && full) ? 1u : 0u);
    // (the next tile writes LDS only after its first barrier, which every wave
    //  reaches after this store's image reads)
  }
  wait_vmcnt<0>();
}

constexpr int kRing = 3;  // tiles in flight per workgroup
template <int KB, bool HAD, bool QJL, bool MSEV>
void* pick_v(int vb) {
  switch (vb) {
    case 2: return reinterpret_cast<void*>(&compress_mfma_kernel<KB, 2, kRing, HAD, QJL, MSEV>);
    case 3: return reinterpret_cast<void*>(&compress_mfma_kernel<KB, 3, kRing, HAD, QJL, MSEV>);
    case 4: return reinterpret_cast<void*>(&compress_mfma_kernel<KB, 4, kRing, HAD, QJL, MSEV>);
  }
  return nullptr;
}
template <bool HAD, bool QJL, bool MSEV>
void* pick_kv(int kb, int vb) {
  switch (kb) {
    case 1: return pick_v<1, HAD, QJL, MSEV>(vb);
    case 2: return pick_v<2, HAD, QJL, MSEV>(vb);
    case 3: return pick_v<3, HAD, QJL, MSEV>(vb);
    case 4: return pick_v<4, HAD, QJL, MSEV>(vb);
  }
  return nullptr;
}
template <bool MSEV>
void* pick_rot(bool had, bool qjl, int kb, int vb) {
  return had ? (qjl ? pick_kv<true, true, MSEV>(kb, vb) : pick_kv<true, false, MSEV>(kb, vb))
             : (qjl ? pick_kv<false, true, MSEV>(kb, vb) : pick_kv<false, false, MSEV>(kb, vb));
}

}  // namespace

bool compress_mfma_applies(const tq_layer* L, const void* k, const void* v, tq_dtype in_dtype, long long n_tokens,
                           long long k_stride, long long v_stride) {
  if (L->cfg.bypass || in_dtype != TQ_BF16 || !L->dOpA) return false;
  if (n_tokens < 64) return false;  // a handful of appended tokens: the per-token kernel is quicker
  // 16-byte aligned rows for the direct-to-LDS copies
  if ((k_stride % 8) || (v_stride % 8)) return false;
  // a tile's row offsets (15 strides) are 32-bit
  if (k_stride > (1LL << 26) || v_stride > (1LL << 26) || k_stride < 0 || v_stride < 0) return false;
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
  a.km = static_cast<int>(L->cfg.key_mode);
  a.rscale = L->r_scale;
  a.block_bytes = static_cast<unsigned>(L->lay.block_bytes);
  for (int i = 0; i < 16; ++i) {
    a.cent[i] = L->centroids[i];
    a.bnd[i] = L->boundaries[i];
    a.vcent[i] = L->v_centroids[i];
    a.vbnd[i] = L->v_boundaries[i];
  }
  const bool had = L->cfg.rotation == TQ_ROT_HADAMARD, qjl = L->cfg.key_mode == TQ_KEY_QJL;
  void* fn = L->cfg.value_mode == TQ_VAL_MSE ? pick_rot<true>(had, qjl, L->cfg.k_bits, L->cfg.v_bits)
                                             : pick_rot<false>(had, qjl, L->cfg.k_bits, L->cfg.v_bits);
  if (!fn) return fail(TQ_ERR_UNSUPPORTED, "no compress kernel for k_bits=%d v_bits=%d", L->cfg.k_bits, L->cfg.v_bits);
  // Workgroups loop over their tiles: as many as fit on the chip at once over all
  // heads (resident workgroups per CU from the kernel's register and LDS use).
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 512, 0) != hipSuccess || per_cu < 1) per_cu = 1;
  const int cus = L->cu_count > 0 ? L->cu_count : 256;
  long long gx = (static_cast<long long>(cus) * per_cu + a.H - 1) / a.H;
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
