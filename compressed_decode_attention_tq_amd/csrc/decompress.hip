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

#include "f16_pieces.hpp"
#include "lds_copy.hpp"
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
      // (one packed conversion, nearest even)
      const bf16x2 b = {static_cast<__bf16>(src[2 * i]), static_cast<__bf16>(src[2 * i + 1])};
      pk[i] = __builtin_bit_cast(unsigned, b);
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
  float vx[8];
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
    vx[i] = (a.vm == 1) ? sc * a.vcent[code] : fmaf(sc, static_cast<float>(code), zr);
  }
  // v' as float16 hi + lo of the float32 value (pieces against the same hi)
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const unsigned hh = pack_f16(vx[i], vx[i + 1]);
    const unsigned ll = residual_pair(vx[i], vx[i + 1], hh);
    *reinterpret_cast<unsigned*>(&avh[t][d0 + i]) = hh;
    *reinterpret_cast<unsigned*>(&avl[t][d0 + i]) = ll;
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

// Loads of T at byte address p, typed by address space: an LDS page image
// (ds_read) or a page in global memory, so that the common path is never a
// FLAT access (whose waits would also cover the in-flight copies).
template <typename T>
__device__ __forceinline__ T ld(const lds_byte* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
template <typename T>
__device__ __forceinline__ T ld(const unsigned char* p) {
  return *reinterpret_cast<const T*>(p);
}

// ---------------------------------------------------------------- persistent
// Inputs of 64+ tokens: one workgroup of sixteen waves per KV head and a share
// of its 16-token tiles, in two roles that work on consecutive tiles at once.
// Waves 8..15 copy and expand: each tile's 16 slots are copied into an LDS ring
// four tiles ahead and its page two tiles ahead (the page address comes from
// the slots, by then in LDS for two iterations), and tile k is expanded into
// one of two A-operand buffers.  Waves 0..7 contract: wave w forms output dims
// 16w..16w+15 of tile k-1 from the other buffer, with that column tile's B
// operands (R hi, lo and, with QJL, P hi, lo: 64 VGPRs) held in registers for
// the whole launch, and stores them.  One workgroup barrier per tile hands the
// buffers over.  Every copying wave issues exactly one slot copy and one page
// copy per tile, so its wait for tile k's page (and tile k+2's slots, issued
// before it) is a counted one; the contracting waves never wait on memory in
// the loop.
// A tile that is not one whole aligned page reads its records from global
// memory in the expansion (the page copied for it is not used).
constexpr int kPageChunks = kMaxPage / 16 + 4;  // page ring slot, with room for the per-wave rounding

// Field offsets of a compressed page as a function of the variant: Kc [16
// tokens x 4 blocks] of 4 KB bytes, Ks (QJL) 4 bytes each, Kn (n, gamma) or
// n, Vc lane-blocked VB-bit codes, then per-group scale/zero or one norm.
// The ring kernel takes them as constants (every field read is then a fixed
// offset from one per-lane address); its launcher checks them against the
// layer's layout.
struct PageFields {
  unsigned kc, ks, kn, vc, vsz, bytes;
};
__host__ __device__ constexpr PageFields page_fields(int kb, int vb, bool qjl, bool msev) {
  PageFields f{};
  f.kc = 0;
  f.ks = f.kc + 16u * (kDim * kb / 8);
  f.kn = f.ks + (qjl ? 16u * (kDim / 8) : 0u);
  f.vc = f.kn + 16u * (qjl ? 4u : 2u);
  f.vsz = f.vc + 16u * (kDim * vb / 8);
  f.bytes = f.vsz + 16u * (msev ? 2u : 4u * (kDim / kGroup));
  return f;
}

template <int KB, int VB, bool OUT_BF16, bool QJL, bool MSEV>
__global__ __launch_bounds__(1024) void decompress_ring_kernel(DArgs a) {
  const int g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool mma = wave < 8;  // contracting role (else copying and expanding)
  const int w = wave & 7;
  const int col = lane & 15, kg = lane >> 4;

  // Two buffers of a tile's A operands (key codebook values, value operands
  // and, with QJL, signs +-1; the value operands are the group codes as
  // float16 integers, or with MSE-coded values the value codebook entries: all
  // exact in float16), of its Kn words and of its value metadata (the
  // per-group scale/zero words, or the value norms of MSE-coded values); each
  // kind is one array, so an access is one per-lane address plus a constant
  // offset, which keeps the loop's live registers few.
  constexpr int NA = QJL ? 3 : 2;
  __shared__ __attribute__((aligned(16))) _Float16 aop[2][NA][16][kARow];
  __shared__ __attribute__((aligned(16))) unsigned char knb[2][64];
  __shared__ __attribute__((aligned(16))) unsigned char vnb[2][MSEV ? 32 : 4];
  __shared__ __attribute__((aligned(16))) unsigned szb[2][MSEV ? 1 : 16][4];  // [token][group]
  // Two buffers of a tile's outputs: the K and V rows of its 16 tokens (bf16
  // pairs or fp32 values per word; the 4-word row padding puts the rows a
  // half wave writes at once on distinct banks).  The contracting waves write
  // one after a tile's products and store it, as whole rows, in the next
  // iteration.
  constexpr int kSRow = OUT_BF16 ? 68 : 132;
  __shared__ __attribute__((aligned(16))) unsigned stage[2][2][16][kSRow];
  __shared__ __attribute__((aligned(16))) u32x4 pring[3][kPageChunks];
  __shared__ __attribute__((aligned(16))) long long sring[8][16];
  __shared__ _Float16 cent_h[16];   // key codebook (float16 values: exact)
  __shared__ _Float16 vcent_h[16];  // value codebook (float16 values: exact)

  // ---- contracting waves: B operands of column tile w
  half8 RH[4], RL[4], PH[QJL ? 4 : 1], PL[QJL ? 4 : 1];
  if (mma) {
    const u32x4* op = a.opd + (static_cast<size_t>(g) * 8 + w) * 4 * 4 * 64 + lane;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      RH[s] = __builtin_bit_cast(half8, op[(4 * s + 0) * 64]);
      RL[s] = __builtin_bit_cast(half8, op[(4 * s + 1) * 64]);
      if constexpr (QJL) {
        PH[s] = __builtin_bit_cast(half8, op[(4 * s + 2) * 64]);
        PL[s] = __builtin_bit_cast(half8, op[(4 * s + 3) * 64]);
      }
    }
    // Consume the operands here, so that the compiler's wait for their loads
    // is not placed at their first use inside the tile loop.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      asm volatile("" ::"v"(RH[s]), "v"(RL[s]));
      if constexpr (QJL) asm volatile("" ::"v"(PH[s]), "v"(PL[s]));
    }
    wait_vmcnt<0>();
  }
  if (tid < 16) {
    cent_h[tid] = static_cast<_Float16>(a.cent[tid]);
    vcent_h[tid] = static_cast<_Float16>(a.vcent[tid]);
  }

  const long long n_tiles = (a.n_tokens + 15) / 16;
  const long long first = blockIdx.x, step = gridDim.x;
  const int mine = first < n_tiles ? static_cast<int>((n_tiles - 1 - first) / step + 1) : 0;
  if (mine == 0) return;  // the whole workgroup (uniform)
  auto tile_of = [&](int j) { return first + static_cast<long long>(j < mine ? j : mine - 1) * step; };
  constexpr PageFields F = page_fields(KB, VB, QJL, MSEV);
  constexpr int nch = static_cast<int>(F.bytes / 16);
  constexpr int per = (nch + 7) / 8;  // page chunks per copying wave

  // (copying waves) slots 2w, 2w+1 of tile j (one lane; near the input's end
  // the last two slots of the input are copied instead, so the ragged last
  // tile's entry is not read by position)
  auto copy_slots = [&](int j) {
    if (lane == 0) {
      long long i = tile_of(j) * 16 + 2 * w;
      if (i + 2 > a.n_tokens) i = a.n_tokens - 2;
      copy_to_lds(a.slots + i, &sring[j & 7][2 * w]);
    }
  };
  // slot of token lane % 16 of tile j from the ring (-1 past the input's end)
  auto ring_slot = [&](int j) {
    const long long n0 = tile_of(j) * 16;
    return n0 + (lane & 15) < a.n_tokens ? sring[j & 7][lane & 15] : -1LL;
  };
  // the tile's first slot and whether its slots are one whole aligned page,
  // from ring_slot's value in every lane (wave-uniform results)
  auto page_of = [&](long long sj, long long* s0) {
    const long long f = static_cast<long long>(__builtin_amdgcn_readfirstlane(static_cast<unsigned>(sj))) |
                        (static_cast<long long>(__builtin_amdgcn_readfirstlane(static_cast<unsigned>(sj >> 32))) << 32);
    *s0 = f;
    const bool ok = f >= 0 && (f & 15) == 0 && sj == f + (lane & 15);
    return (__builtin_amdgcn_ballot_w64(ok) & 0xffffull) == 0xffffull;
  };
  // (copying waves) page of tile j, first slot s0, into ring slot j % 3, each
  // wave its share of chunks; a tile that is not a whole page copies the page
  // of its first slot, or block 0
  auto copy_page = [&](int j, long long s0) {
    const long long blk = s0 >= 0 ? (s0 >> 4) : 0;
    const unsigned char* src = a.pool + (static_cast<size_t>(blk) * a.H + g) * F.bytes;
    if (lane < per) {
      const int c = w * per + lane;
      copy_to_lds(src + 16 * (c < nch ? c : 0), &pring[j % 3][w * per]);
    }
  };

  // ---- prologue: slots of tiles 0..3, then pages of tiles 0, 1.  The first
  // slot and whole-page flag of a tile are found once, when its page copy is
  // issued two iterations ahead, and carried to its expansion in scalar
  // registers (s0c, wholec: tile k; s0n, wholen: tile k+1).
  long long s0c = 0, s0n = 0;
  bool wholec = false, wholen = false;
  if (!mma) {
    for (int j = 0; j < 4; ++j) copy_slots(j);
    wait_vmcnt<0>();
  }
  __syncthreads();
  if (!mma) {
    wholec = page_of(ring_slot(0), &s0c);
    copy_page(0, s0c);
    wholen = page_of(ring_slot(1), &s0n);
    copy_page(1, s0n);
  }

  // expansion: copying-wave thread u takes token t, dims d0..d0+3.  With 4-bit
  // values, copying wave e = u / 64 takes tokens 8 (e % 2) + l % 8 and quads
  // e / 2 + 4 (l / 8) of its lanes l, so all its dims have one residue modulo
  // 16 and its reads of the value codes (lane-blocked runs) fall on distinct
  // LDS banks or share a word; with 2- and 3-bit values (fewer such conflicts)
  // 32 consecutive lanes take one token, so each token's A-operand row is
  // written as 256 contiguous bytes.
  const int u = tid & 511;
  const int t = VB == 4 ? 8 * ((u >> 6) & 1) + (u & 7) : u >> 5;
  const int d0 = VB == 4 ? 4 * ((u >> 7) + 4 * ((u >> 3) & 7)) : 4 * (u & 31);
  // The two roles run loops of their own with one workgroup barrier per
  // iteration each (mine + 2 of them), so the copying loop does not hold the
  // contracting waves' 64 registers of B operands.  At the barrier of
  // iteration k: tile k's page and tile k+2's slots are in LDS, tile k-1's A
  // operands expanded, and tile k-2's products formed (its buffer is free) and
  // staged.
  if (!mma) {
#pragma unroll 1
    for (int k = 0; k <= mine + 1; ++k) {
      // operations issued after tile k's page copy: the page copy of tile 1
      // (k = 0); the slot copy of tile k+3 and the page copy of k+1
      if (k < mine) {
        if (k == 0)
          wait_vmcnt<1>();
        else
          wait_vmcnt<2>();
      }
      __syncthreads();
      if (k >= mine) continue;

      // ---- expand tile k: thread (t, d0) -> A operands of token t, dims d0..d0+3
      auto& ac = aop[k & 1][0];
      auto& avh = aop[k & 1][1];
      auto& az = aop[k & 1][NA - 1];  // (QJL only)
      const long long n0 = tile_of(k) * 16;
      const bool whole = wholec;
      // The expansion of token t's dims d0..d0+3 from its record at in-page
      // offset o in two parts: fetch only issues the loads of the record's
      // fields (so that other work can be placed while they are in flight),
      // emit decodes them, looks the codes up and writes the A operands.
      struct Raw {
        unsigned k0, k1, z, sz, v0[4], v1[4];
      };
      // value codes: element ((16 (o / 8) + jd % 16) 16 + 2 (jd / 16) + (o % 8) / 4) 4 + o % 4
      // of the Vc field; dims d0 + i step the element by 64, so the byte by 8 VB
      // and the bit position within it stays (one byte for VB = 2, 4; two for 3)
      auto vel = [&](int o) {
        return ((16u * (o >> 3) + (d0 & 15)) * 16u + 2u * (d0 >> 4) + ((o & 7) >> 2)) * 4u + (o & 3);
      };
      auto fetch = [&](auto page, int o) {
        Raw r{};
        const int blk = d0 >> 5, e0 = d0 & 31;
        // key codes of dims d0..d0+3: 4 KB bits at bit e0 KB of the block record
        // (one byte for KB <= 2, an aligned halfword for KB = 4, two bytes for 3)
        const auto kc = page + F.kc + (blk * 16 + o) * 4 * KB + ((e0 * KB) >> 3);
        if constexpr (KB == 4) {
          r.k0 = ld<unsigned short>(kc);
        } else {
          r.k0 = ld<unsigned char>(kc);
          if constexpr (KB == 3) r.k1 = ld<unsigned char>(kc + 1);
        }
        if constexpr (QJL) r.z = ld<unsigned char>(page + F.ks + (blk * 16 + o) * 4 + (e0 >> 3));
        // (MSE-coded values: the token's norm is applied after the products)
        if constexpr (!MSEV) r.sz = ld<unsigned>(page + F.vsz + o * 16 + blk * 4);
        const auto vb = page + F.vc + ((vel(o) * VB) >> 3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          r.v0[i] = ld<unsigned char>(vb + 8 * VB * i);
          if constexpr (VB == 3) r.v1[i] = ld<unsigned char>(vb + 8 * VB * i + 1);
        }
        return r;
      };
      auto emit = [&](const Raw& r, int o) {
        const int e0 = d0 & 31;
        unsigned kx;
        if constexpr (KB == 4)
          kx = r.k0;
        else if constexpr (KB == 3)
          kx = (r.k0 | (r.k1 << 8)) >> ((e0 * KB) & 7);
        else
          kx = r.k0 >> ((e0 * KB) & 7);
        const unsigned zb = QJL ? r.z >> (e0 & 7) : 0u;
        const unsigned vsh = (vel(o) * VB) & 7;
        _Float16 hc[4], hz[4], hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hc[i] = cent_h[(kx >> (KB * i)) & ((1u << KB) - 1u)];
          hz[i] = ((zb >> i) & 1u) ? static_cast<_Float16>(1.0f) : static_cast<_Float16>(-1.0f);
          const unsigned vw = VB == 3 ? (r.v0[i] | (r.v1[i] << 8)) : r.v0[i];
          const unsigned code = (vw >> vsh) & ((1u << VB) - 1u);
          hv[i] = MSEV ? vcent_h[code] : static_cast<_Float16>(static_cast<float>(code));
        }
        *reinterpret_cast<half4*>(&ac[t][d0]) = half4{hc[0], hc[1], hc[2], hc[3]};
        if constexpr (QJL) *reinterpret_cast<half4*>(&az[t][d0]) = half4{hz[0], hz[1], hz[2], hz[3]};
        *reinterpret_cast<half4*>(&avh[t][d0]) = half4{hv[0], hv[1], hv[2], hv[3]};
        // (group values: the group's scale/zero word, by the thread of its first dims)
        if constexpr (!MSEV)
          if (e0 == 0) szb[k & 1][t][d0 >> 5] = r.sz;
      };
      constexpr int kn_bytes = QJL ? 4 : 2;  // Kn bytes per token
      // copies of tile k+4's slots and tile k+2's page
      long long s02;
      bool whole2;
      __builtin_amdgcn_sched_barrier(0);
      if (whole) {
        // The page image in the ring (LDS reads).  Tile k+2's slots are read
        // with its fields, so that the two LDS round trips overlap, and that
        // tile's copies are issued before the codebook lookups.
        const lds_byte* pg = (const lds_byte*)(&pring[k % 3][0]);
        const long long sj2 = ring_slot(k + 2);
        const Raw r = fetch(pg, t);
        __builtin_amdgcn_sched_barrier(0);
        whole2 = page_of(sj2, &s02);
        copy_slots(k + 4);
        copy_page(k + 2, s02);
        __builtin_amdgcn_sched_barrier(0);
        emit(r, t);
        // its Kn words as they are
        if (u < 4 * kn_bytes) *reinterpret_cast<unsigned*>(&knb[k & 1][4 * u]) = ld<unsigned>(pg + F.kn + 4 * u);
        if constexpr (MSEV)
          if (u >= 32 && u < 40)
            *reinterpret_cast<unsigned*>(&vnb[k & 1][4 * (u - 32)]) = ld<unsigned>(pg + F.vsz + 4 * (u - 32));
      } else {
        whole2 = page_of(ring_slot(k + 2), &s02);
        copy_slots(k + 4);
        copy_page(k + 2, s02);
        __builtin_amdgcn_sched_barrier(0);
        // (the ragged last tile's ring entry holds shifted slots near the input's end)
        const long long slot =
            n0 + t < a.n_tokens ? (n0 + 16 <= a.n_tokens ? sring[k & 7][t] : a.slots[n0 + t]) : -1;
        if (slot >= 0) {
          const unsigned char* pg = a.pool + (static_cast<size_t>(slot >> 4) * a.H + g) * F.bytes;
          const int o = static_cast<int>(slot & 15);
          emit(fetch(pg, o), o);
          if (d0 == 0) {  // (one thread per token)
            if constexpr (QJL)
              *reinterpret_cast<unsigned*>(&knb[k & 1][4 * t]) = ld<unsigned>(pg + F.kn + 4 * o);
            else
              *reinterpret_cast<unsigned short*>(&knb[k & 1][2 * t]) = ld<unsigned short>(pg + F.kn + 2 * o);
            if constexpr (MSEV)
              *reinterpret_cast<unsigned short*>(&vnb[k & 1][2 * t]) = ld<unsigned short>(pg + F.vsz + 2 * o);
          }
        } else {
          const half4 z4 = {static_cast<_Float16>(0.0f), static_cast<_Float16>(0.0f), static_cast<_Float16>(0.0f),
                            static_cast<_Float16>(0.0f)};
          *reinterpret_cast<half4*>(&ac[t][d0]) = z4;
          if constexpr (QJL) *reinterpret_cast<half4*>(&az[t][d0]) = z4;
          *reinterpret_cast<half4*>(&avh[t][d0]) = z4;
          if constexpr (!MSEV)
            if ((d0 & 31) == 0) szb[k & 1][t][d0 >> 5] = 0u;
          if (d0 == 0) {
            if constexpr (QJL)
              *reinterpret_cast<unsigned*>(&knb[k & 1][4 * t]) = 0u;
            else
              *reinterpret_cast<unsigned short*>(&knb[k & 1][2 * t]) = 0;
            if constexpr (MSEV) *reinterpret_cast<unsigned short*>(&vnb[k & 1][2 * t]) = 0;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      wholec = wholen;
      s0c = s0n;
      wholen = whole2;
      s0n = s02;
    }
  } else {
    // Group values: the column sums of R over each K-step's 32 rows (one value
    // group), rows of ones times R hi + lo, for the groups' zero terms.
    float csum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (!MSEV) {
      const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        floatx4 c = {0.0f, 0.0f, 0.0f, 0.0f};
        c = mfma(ones, RH[s], c);
        c = mfma(ones, RL[s], c);
        csum[s] = c[0];
      }
    }
#pragma unroll 1
    for (int k = 0; k <= mine + 1; ++k) {
      __syncthreads();
      if (k == 0) continue;

      // ---- store tile k-2 from its staging: wave w, rows 4w..4w+3 of the 32
      // (K rows of tokens 0..15, then V rows), 16 lanes a row, 16 contiguous
      // bytes each (two 16-byte pieces for fp32), as non-temporal stores: the
      // output is written once and not read back by this launch (layer store
      // 189 against 195 us with ordinary stores)
      if (k >= 2) {
        const int ridx = 4 * w + (lane >> 4), kv = ridx >> 4, tt = ridx & 15, c = lane & 15;
        const unsigned* row = &stage[k & 1][kv][tt][0];
        const long long n = tile_of(k - 2) * 16 + tt;
        if (n < a.n_tokens) {
          void* out = kv ? a.vout : a.kout;
          const size_t at = (static_cast<size_t>(n) * a.H + g) * 128;
          if constexpr (OUT_BF16) {
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(row + 4 * c),
                                        reinterpret_cast<u32x4*>(static_cast<unsigned short*>(out) + at + 8 * c));
          } else {
            float* o = static_cast<float*>(out) + at;
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(row + 4 * c), reinterpret_cast<u32x4*>(o + 4 * c));
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(row + 64 + 4 * c),
                                        reinterpret_cast<u32x4*>(o + 64 + 4 * c));
          }
        }
      }
      if (k > mine) continue;

      // ---- contract tile k-1: wave w, output dims 16w + col of tokens 4kg + r
      const int b = (k - 1) & 1;
      floatx4 k1 = {0.0f, 0.0f, 0.0f, 0.0f}, k2 = k1, vv = k1;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c0 = 32 * s + 8 * kg;
        const half8 xc = *reinterpret_cast<const half8*>(&aop[b][0][col][c0]);
        const half8 xh = *reinterpret_cast<const half8*>(&aop[b][1][col][c0]);
        // Group values: K-step s spans one group, v' = zero + scale code on it,
        // so its share of V is scale (codes . R) + zero (column sum of R); the
        // codes' products go first, so that they are done when the group's
        // scale and zero are applied after the key products.
        floatx4 vs = {0.0f, 0.0f, 0.0f, 0.0f};
        unsigned sz[4];
        if constexpr (!MSEV) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sz[r] = szb[b][4 * kg + r][s];
          vs = mfma(xh, RH[s], vs);
          vs = mfma(xh, RL[s], vs);
        }
        k1 = mfma(xc, RH[s], k1);
        k1 = mfma(xc, RL[s], k1);
        // (the fences keep each read next to its products: with all of a K-step's
        // reads issued at once the copying waves' LDS round trips took longer,
        // and the launch with them; layer store 189 against 207 us)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (QJL) {
          const half8 xz = *reinterpret_cast<const half8*>(&aop[b][NA - 1][col][c0]);
          k2 = mfma(xz, PH[s], k2);
          k2 = mfma(xz, PL[s], k2);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MSEV) {
          vv = mfma(xh, RH[s], vv);
          vv = mfma(xh, RL[s], vv);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sc = __half2float(__ushort_as_half(static_cast<unsigned short>(sz[r] & 0xffffu)));
            const float zr = __half2float(__ushort_as_half(static_cast<unsigned short>(sz[r] >> 16)));
            vv[r] = fmaf(sc, vs[r], fmaf(zr, csum[s], vv[r]));
          }
        }
        // one K-step's A operands live at a time (next to the 64 registers of B
        // operands): the scheduler may not hoist the next step's reads above here
        __builtin_amdgcn_sched_barrier(0);
      }
      // ---- stage tile k-1: lane (col, kg) holds rows 4kg..4kg+3 of output dim
      // 16w + col; K = n (x1 + kappa gamma x2), n and gamma as float16
      float kx[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = 4 * kg + r;
        if constexpr (QJL) {
          const unsigned kn = *reinterpret_cast<const unsigned*>(&knb[b][4 * tt]);
          const float sn = __half2float(__ushort_as_half(static_cast<unsigned short>(kn & 0xffffu))) *
                           0.08838834764831845f;
          const float sg = a.kappa * __half2float(__ushort_as_half(static_cast<unsigned short>(kn >> 16)));
          kx[r] = sn * fmaf(sg, k2[r], k1[r]);
        } else {
          const unsigned short kn = *reinterpret_cast<const unsigned short*>(&knb[b][2 * tt]);
          kx[r] = __half2float(__ushort_as_half(kn)) * 0.08838834764831845f * k1[r];
        }
        // MSE-coded values: V = (nv / sqrt(d)) (codebook values . R), nv as float16
        if constexpr (MSEV) {
          const unsigned short vn = *reinterpret_cast<const unsigned short*>(&vnb[b][2 * tt]);
          vv[r] *= __half2float(__ushort_as_half(vn)) * 0.08838834764831845f;
        }
      }
      const int dc = 16 * w + col;
      auto& st = stage[b];
      if constexpr (OUT_BF16) {
        // two adjacent dims per word: of a lane pair (col, col ^ 1) the even lane
        // writes rows 4kg, 4kg+1 and the odd lane rows 4kg+2, 4kg+3, each with
        // the partner's values taken across the pair
        const bool odd = col & 1;
        const int r0 = 4 * kg + (odd ? 2 : 0);
        auto put_pairs = [&](int kv, float x0, float x1, float x2, float x3) {
          const bf16x2 p01 = {static_cast<__bf16>(x0), static_cast<__bf16>(x1)};
          const bf16x2 p23 = {static_cast<__bf16>(x2), static_cast<__bf16>(x3)};
          const unsigned b01 = __builtin_bit_cast(unsigned, p01), b23 = __builtin_bit_cast(unsigned, p23);
          const unsigned send = odd ? b01 : b23;
          // quad_perm [1, 0, 3, 2]: the word of lane col ^ 1
          const unsigned recv =
              static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(send), 0xB1, 0xF, 0xF, false));
          const unsigned keep = odd ? b23 : b01;
          // even lane: (own, partner) of rows r0, r0+1; odd lane: (partner, own)
          const unsigned lo = odd ? recv : keep, hi = odd ? keep : recv;
          st[kv][r0][dc >> 1] = (lo & 0xffffu) | (hi << 16);
          st[kv][r0 + 1][dc >> 1] = (lo >> 16) | (hi & 0xffff0000u);
        };
        put_pairs(0, kx[0], kx[1], kx[2], kx[3]);
        put_pairs(1, vv[0], vv[1], vv[2], vv[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          st[0][4 * kg + r][dc] = __float_as_uint(kx[r]);
          st[1][4 * kg + r][dc] = __float_as_uint(vv[r]);
        }
      }
    }
  }
  wait_vmcnt<0>();
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
template <int KB, bool BF, bool QJL, bool MSEV>
void* pick_ring_v(int vb) {
  switch (vb) {
    case 2: return reinterpret_cast<void*>(&decompress_ring_kernel<KB, 2, BF, QJL, MSEV>);
    case 3: return reinterpret_cast<void*>(&decompress_ring_kernel<KB, 3, BF, QJL, MSEV>);
    case 4: return reinterpret_cast<void*>(&decompress_ring_kernel<KB, 4, BF, QJL, MSEV>);
  }
  return nullptr;
}
template <bool BF, bool QJL, bool MSEV>
void* pick_ring_kv(int kb, int vb) {
  switch (kb) {
    case 1: return pick_ring_v<1, BF, QJL, MSEV>(vb);
    case 2: return pick_ring_v<2, BF, QJL, MSEV>(vb);
    case 3: return pick_ring_v<3, BF, QJL, MSEV>(vb);
    case 4: return pick_ring_v<4, BF, QJL, MSEV>(vb);
  }
  return nullptr;
}
void* pick_ring(bool bf, bool qjl, bool msev, int kb, int vb) {
  if (bf) {
    if (qjl) return msev ? pick_ring_kv<true, true, true>(kb, vb) : pick_ring_kv<true, true, false>(kb, vb);
    return msev ? pick_ring_kv<true, false, true>(kb, vb) : pick_ring_kv<true, false, false>(kb, vb);
  }
  if (qjl) return msev ? pick_ring_kv<false, true, true>(kb, vb) : pick_ring_kv<false, true, false>(kb, vb);
  return msev ? pick_ring_kv<false, false, true>(kb, vb) : pick_ring_kv<false, false, false>(kb, vb);
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
    if (n_tokens >= 64) {
      // persistent ring kernel: as many workgroups over all heads as fit on the
      // chip at once, each looping over its head's tiles
      void* rf = pick_ring(bf, a.qjl != 0, a.vm == 1, L->cfg.k_bits, L->cfg.v_bits);
      const PageFields f = page_fields(L->cfg.k_bits, L->cfg.v_bits, a.qjl != 0, a.vm == 1);
      if (f.kc != L->lay.off_kc || f.ks != L->lay.off_ks || f.kn != L->lay.off_kn || f.vc != L->lay.off_vc ||
          f.vsz != L->lay.off_vsz || f.bytes != L->lay.block_bytes)
        return fail(TQ_ERR_UNSUPPORTED, "decompress: page layout does not match the kernel's field offsets");
      if (!rf) return fail(TQ_ERR_UNSUPPORTED, "no decompress kernel for k_bits=%d v_bits=%d", L->cfg.k_bits,
                           L->cfg.v_bits);
      int per_cu = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, rf, 1024, 0) != hipSuccess || per_cu < 1) per_cu = 1;
      const int cus = L->cu_count > 0 ? L->cu_count : 256;
      const long long n_tiles = (n_tokens + 15) / 16;
      long long gx = (static_cast<long long>(cus) * per_cu + H - 1) / H;
      if (gx > n_tiles) gx = n_tiles;
      if (gx < 1) gx = 1;
      a.slots = slots;
      a.kout = k_out;
      a.vout = v_out;
      a.n_tokens = n_tokens;
      void* args[] = {&a};
      hipError_t e = hipLaunchKernel(rf, dim3(static_cast<unsigned>(gx), H), dim3(1024), args, 0, s);
      if (e != hipSuccess) return fail(TQ_ERR_HIP, "decompress launch: %s", hipGetErrorString(e));
      return TQ_OK;
    }
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
