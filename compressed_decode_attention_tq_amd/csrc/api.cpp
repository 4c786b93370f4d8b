// C ABI of libtq: argument validation, layer state, store layout and decode
// planning.  Kernels live in compress.hip and decode.hip.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "tq_internal.hpp"

namespace tq {

namespace {
thread_local std::string g_error;
}

tq_status fail(tq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

void clear_error() { g_error.clear(); }

tq_status validate_config(const tq_layer_config* cfg) {
  if (!cfg) return fail(TQ_ERR_INVALID_ARGUMENT, "null layer config");
  if (cfg->head_dim != kDim)
    return fail(TQ_ERR_UNSUPPORTED, "head_dim %d not supported (only %d)", cfg->head_dim, kDim);
  if (cfg->n_kv_heads < 1) return fail(TQ_ERR_INVALID_ARGUMENT, "n_kv_heads must be >= 1");
  if (cfg->block_size != kPage)
    return fail(TQ_ERR_UNSUPPORTED, "block_size %d not supported (only %d)", cfg->block_size, kPage);
  if (cfg->layer < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "layer index must be >= 0");
  if (cfg->bypass) return TQ_OK;
  if (cfg->k_bits < 1 || cfg->k_bits > 4)
    return fail(TQ_ERR_UNSUPPORTED, "k_bits %d not supported (1..4)", cfg->k_bits);
  if (cfg->v_bits < 2 || cfg->v_bits > 4)
    return fail(TQ_ERR_UNSUPPORTED, "v_bits %d not supported (2..4)", cfg->v_bits);
  if (cfg->v_group != kGroup)
    return fail(TQ_ERR_UNSUPPORTED, "v_group %d not supported (only %d)", cfg->v_group, kGroup);
  if (cfg->dist != TQ_DIST_GAUSSIAN && cfg->dist != TQ_DIST_SPHERE)
    return fail(TQ_ERR_INVALID_ARGUMENT, "unknown codebook density %d", static_cast<int>(cfg->dist));
  if (cfg->key_mode != TQ_KEY_QJL && cfg->key_mode != TQ_KEY_MSE && cfg->key_mode != TQ_KEY_MSE_NC)
    return fail(TQ_ERR_INVALID_ARGUMENT, "unknown key mode %d", static_cast<int>(cfg->key_mode));
  if (cfg->rotation != TQ_ROT_HAAR && cfg->rotation != TQ_ROT_HADAMARD)
    return fail(TQ_ERR_INVALID_ARGUMENT, "unknown rotation family %d", static_cast<int>(cfg->rotation));
  if (cfg->value_mode != TQ_VAL_GROUP && cfg->value_mode != TQ_VAL_MSE)
    return fail(TQ_ERR_INVALID_ARGUMENT, "unknown value mode %d", static_cast<int>(cfg->value_mode));
  return TQ_OK;
}

tq_status make_layout(const tq_layer_config* cfg, Layout* out) {
  tq_status st = validate_config(cfg);
  if (st != TQ_OK) return st;
  Layout l;
  if (cfg->bypass) {
    l.bypass = true;
    l.off_kc = 0;                              // K [16][128] bf16
    l.off_vc = static_cast<size_t>(kPage) * kDim * 2;   // V [16][128] bf16
    l.block_bytes = 2 * l.off_vc;
    *out = l;
    return TQ_OK;
  }
  l.k_bits = cfg->k_bits;
  l.v_bits = cfg->v_bits;
  l.kc_bytes = kDim * cfg->k_bits / 8;
  // key modes without QJL: no sign field and no gamma, the magnitude alone
  const bool qjl = cfg->key_mode == TQ_KEY_QJL;
  l.ks_bytes = qjl ? kDim / 8 : 0;
  l.kn_bytes = qjl ? 4 : 2;
  l.vc_bytes = kDim * cfg->v_bits / 8;
  // last field: per-group fp16 scale/zero, or one fp16 norm with MSE values
  l.vsz_bytes = cfg->value_mode == TQ_VAL_MSE ? 2 : 4 * (kDim / kGroup);
  size_t o = 0;
  l.off_kc = o; o += static_cast<size_t>(kPage) * l.kc_bytes;
  l.off_ks = o; o += static_cast<size_t>(kPage) * l.ks_bytes;
  l.off_kn = o; o += static_cast<size_t>(kPage) * l.kn_bytes;
  l.off_vc = o; o += static_cast<size_t>(kPage) * l.vc_bytes;
  l.off_vsz = o; o += static_cast<size_t>(kPage) * l.vsz_bytes;
  l.block_bytes = o;
  *out = l;
  return TQ_OK;
}

namespace {

// Stored codebook of `bits` bits: Lloyd-Max centroids rounded to float16 (the
// decode kernels' MFMA operand type), boundaries at the exact midpoints of the
// stored centroids, both as float32 values.
tq_status stored_codebook(int bits, tq_dist dist, float* cent, float* bnd) {
  double c[256], b[255];
  tq_status st = lloyd_max(bits, dist, kDim, c, b, nullptr);
  if (st != TQ_OK) return st;
  const int L = 1 << bits;
  double c16[256];
  for (int i = 0; i < L; ++i) c16[i] = static_cast<double>(static_cast<_Float16>(c[i]));
  for (int i = 0; i < L; ++i) cent[i] = static_cast<float>(c16[i]);
  for (int i = 0; i + 1 < L; ++i) bnd[i] = static_cast<float>(0.5 * (c16[i] + c16[i + 1]));
  return TQ_OK;
}

// Host state of one layer: R, S (float32, [H][d][d]) and the float32 codebook.
tq_status build_state(const tq_layer_config* cfg, std::vector<float>* R, std::vector<float>* S,
                      float* cent, float* bnd, int* levels) {
  const int d = kDim, H = cfg->n_kv_heads;
  if (R) R->resize(static_cast<size_t>(H) * d * d);
  if (S) S->resize(static_cast<size_t>(H) * d * d);
  std::vector<double> tmp(static_cast<size_t>(d) * d);
  for (int h = 0; h < H; ++h) {
    if (R) {
      if (!cfg->bypass && cfg->rotation == TQ_ROT_HADAMARD)
        hadamard_rotation(cfg->seed, cfg->layer, h, d, tmp.data());
      else
        haar_rotation(cfg->seed, cfg->layer, h, d, tmp.data());
      for (size_t i = 0; i < tmp.size(); ++i) (*R)[h * tmp.size() + i] = static_cast<float>(tmp[i]);
    }
    if (S) {
      gaussians(cfg->seed, static_cast<uint64_t>(cfg->layer), static_cast<uint64_t>(h),
                kTagProjection, tmp.size(), tmp.data());
      for (size_t i = 0; i < tmp.size(); ++i) (*S)[h * tmp.size() + i] = static_cast<float>(tmp[i]);
    }
  }
  *levels = 0;
  if (!cfg->bypass) {
    tq_status st = stored_codebook(cfg->k_bits, cfg->dist, cent, bnd);
    if (st != TQ_OK) return st;
    *levels = 1 << cfg->k_bits;
  }
  return TQ_OK;
}

tq_status hip_fail(hipError_t e, const char* what) {
  return fail(TQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int env_splits() {
  const char* s = std::getenv("TQ_DECODE_SPLITS");
  if (!s || !*s) return 0;
  const int v = std::atoi(s);
  return v > 0 ? v : 0;
}

// TQ_DECODE_WORK_LIST: "0" plain item order, "1" work list, unset or other: automatic.
int env_work_list() {
  const char* s = std::getenv("TQ_DECODE_WORK_LIST");
  if (!s || (s[0] != '0' && s[0] != '1') || s[1] != 0) return -1;
  return s[0] - '0';
}

}  // namespace

tq_status plan_decode(const tq_layer* L, int batch, int n_q_heads, int max_seq_len, int num_splits,
                      DecodePlan* plan) {
  DecodePlan p;
  p.batch = batch;
  p.n_q_heads = n_q_heads;
  p.rep = n_q_heads / L->cfg.n_kv_heads;
  const int ctx = max_seq_len > 0 ? max_seq_len : 1;
  const int ctx64 = (ctx + 63) / 64 * 64;
  int splits = num_splits > 0 ? num_splits : env_splits();
  int split_tokens;
  if (splits > 0) {
    split_tokens = ((ctx + splits - 1) / splits + 63) / 64 * 64;
    if (split_tokens > kMaxSplitTokens) split_tokens = kMaxSplitTokens;  // the mainloop's per-wave chunk limit
  } else {
    // Automatic: about two workgroups per CU over (batch x kv_heads x splits),
    // each split 256..4096 tokens (whole 64-token chunks).  Three fit per CU,
    // but measured, splitting further costs more in partials and start-ups
    // than the third workgroup gains.
    const long long pairs = static_cast<long long>(batch) * L->cfg.n_kv_heads;
    const long long target = 2LL * (L->cu_count > 0 ? L->cu_count : 256);
    const long long want = pairs > 0 ? (target + pairs - 1) / pairs : 1;
    long long t = (ctx + want - 1) / want;
    t = (t + 63) / 64 * 64;
    if (t < 256) t = 256;
    if (t > kMaxSplitTokens) t = kMaxSplitTokens;
    if (t > ctx64) t = ctx64;
    split_tokens = static_cast<int>(t);
  }
  p.split_tokens = split_tokens;
  p.n_splits = (ctx + split_tokens - 1) / split_tokens;
  const long long items = static_cast<long long>(batch) * L->cfg.n_kv_heads * p.n_splits;
  if (items > 0x7fffffffLL)
    return fail(TQ_ERR_UNSUPPORTED, "decode grid of %lld workgroups (batch x kv_heads x splits) exceeds 2^31 - 1",
                items);
  // The work list pays one dependent read of seq_lens per workgroup; it is used
  // where the grid is more than about one round of workgroups (two per CU),
  // so that dispatch order and the last round matter.
  const int wl = env_work_list();
  p.work_list = wl >= 0 ? wl == 1 : items > 2LL * (L->cu_count > 0 ? L->cu_count : 256);
  const size_t bh = static_cast<size_t>(batch) * n_q_heads;
  auto align = [](size_t x) { return (x + 255) / 256 * 256; };
  p.ws_part = 0;
  p.ws_qa = p.ws_part + align(bh * static_cast<size_t>(p.n_splits) * (kDim + 4) * sizeof(float));
  // Q.K operand: per (sequence, KV head) 1 or 2 tiles x 4 K-steps x 64 lanes x 8 float16
  const size_t sets = p.rep == 8 ? 2 : 1;
  p.ws_bytes = p.ws_qa + align(static_cast<size_t>(batch) * L->cfg.n_kv_heads * sets * 4 * 64 * 8 * 2);
  if (p.ws_bytes == 0) p.ws_bytes = 256;
  *plan = p;
  return TQ_OK;
}

tq_status prepare_decode(const tq_layer* L, const void* q, tq_dtype q_dtype, int batch, int n_q_heads,
                         const void* pool, long long num_blocks, const int* block_table, int max_blocks_per_seq,
                         const int* seq_lens, int max_seq_len, float softmax_scale, int num_splits, void* out,
                         tq_dtype out_dtype, DecodePlan* plan, float* scale) {
  if (!L) return fail(TQ_ERR_INVALID_ARGUMENT, "null layer");
  if (batch < 0 || n_q_heads <= 0 || max_seq_len < 0 || num_splits < 0 || max_blocks_per_seq < 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "negative size");
  if (n_q_heads % L->cfg.n_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "n_q_heads %d not a multiple of n_kv_heads %d", n_q_heads,
                L->cfg.n_kv_heads);
  const int rep = n_q_heads / L->cfg.n_kv_heads;
  if (rep != 1 && rep != 2 && rep != 4 && rep != 8)
    return fail(TQ_ERR_UNSUPPORTED, "query heads per KV head = %d not supported (1, 2, 4, 8)", rep);
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16)
    return fail(TQ_ERR_UNSUPPORTED, "query dtype %d not supported (F32, BF16)", static_cast<int>(q_dtype));
  if (out_dtype != TQ_F32 && out_dtype != TQ_BF16)
    return fail(TQ_ERR_UNSUPPORTED, "output dtype %d not supported (F32, BF16)", static_cast<int>(out_dtype));
  if (static_cast<long long>(max_blocks_per_seq) * kPage < max_seq_len)
    return fail(TQ_ERR_INVALID_ARGUMENT, "max_blocks_per_seq*16 = %lld < max_seq_len %d",
                static_cast<long long>(max_blocks_per_seq) * kPage, max_seq_len);
  if (!(softmax_scale >= 0.0f) || std::isinf(softmax_scale))
    return fail(TQ_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
  if (batch == 0) return TQ_OK;
  if (!q || !pool || !block_table || !seq_lens || !out) return fail(TQ_ERR_INVALID_ARGUMENT, "null device pointer");
  if (num_blocks <= 0) return fail(TQ_ERR_INVALID_ARGUMENT, "num_blocks must be > 0");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0) return fail(TQ_ERR_INVALID_ARGUMENT, "q must be 16-byte aligned");
  tq_status st = plan_decode(L, batch, n_q_heads, max_seq_len, num_splits, plan);
  if (st != TQ_OK) return st;
  *scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt(static_cast<float>(kDim));
  return TQ_OK;
}

tq_status check_slots(const long long* slots, long long n, long long num_blocks) {
  for (long long i = 0; i < n; ++i)
    if (slots[i] >= num_blocks * kPage)
      return fail(TQ_ERR_INVALID_ARGUMENT, "slot_mapping[%lld] = %lld is past the pool (%lld blocks of %d)", i,
                  slots[i], num_blocks, kPage);
  return TQ_OK;
}

tq_status check_decode_tables(const int* seq_lens, const int* block_table, int batch, int max_blocks,
                              int max_seq_len, long long num_blocks) {
  for (int b = 0; b < batch; ++b) {
    const int T = seq_lens[b];
    if (T < 0 || T > max_seq_len || static_cast<long long>(T) > static_cast<long long>(max_blocks) * kPage)
      return fail(TQ_ERR_INVALID_ARGUMENT, "seq_lens[%d] = %d outside [0, min(max_seq_len %d, 16*max_blocks %d)]",
                  b, T, max_seq_len, max_blocks);
    const int pages = (T + kPage - 1) / kPage;
    for (int j = 0; j < pages; ++j) {
      const int id = block_table[static_cast<size_t>(b) * max_blocks + j];
      if (id < 0 || id >= num_blocks)
        return fail(TQ_ERR_INVALID_ARGUMENT, "block_table[%d][%d] = %d outside [0, %lld)", b, j, id, num_blocks);
    }
  }
  return TQ_OK;
}

bool debug_checks() {
  const char* e = std::getenv("TQ_DEBUG_CHECKS");  // read per call: a few hundred ns at most
  return e && *e && std::strcmp(e, "0") != 0;
}

namespace {

// Copies `bytes` of device memory to `host` on `stream` and waits for it.
tq_status fetch(void* host, const void* dev, size_t bytes, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(host, dev, bytes, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "debug check copy");
}

tq_status debug_check_slots(const long long* slots, long long n, long long num_blocks, void* stream) {
  std::vector<long long> h(static_cast<size_t>(n));
  tq_status st = fetch(h.data(), slots, h.size() * sizeof(long long), stream);
  return st != TQ_OK ? st : check_slots(h.data(), n, num_blocks);
}

}  // namespace

}  // namespace tq

using namespace tq;

extern "C" {

const char* tq_last_error(void) { return g_error.c_str(); }

int tq_abi_version(void) { return TQ_ABI_VERSION; }

tq_status tq_codebook_build(int bits, tq_dist dist, int dim, double* centroids, double* boundaries,
                            double* mse) {
  clear_error();
  if (bits < 1 || bits > 8) return fail(TQ_ERR_INVALID_ARGUMENT, "codebook bits must be 1..8, got %d", bits);
  if (!centroids || (bits > 0 && !boundaries)) return fail(TQ_ERR_INVALID_ARGUMENT, "null codebook output");
  double c[256], b[255];
  tq_status st = lloyd_max(bits, dist, dim, c, b, mse);
  if (st != TQ_OK) return st;
  const int L = 1 << bits;
  std::memcpy(centroids, c, sizeof(double) * L);
  std::memcpy(boundaries, b, sizeof(double) * (L - 1));
  return TQ_OK;
}

tq_status tq_store_layout(const tq_layer_config* cfg, size_t* block_bytes, size_t* field_offsets) {
  clear_error();
  if (!block_bytes) return fail(TQ_ERR_INVALID_ARGUMENT, "null block_bytes");
  Layout l;
  tq_status st = make_layout(cfg, &l);
  if (st != TQ_OK) return st;
  *block_bytes = l.block_bytes;
  if (field_offsets) {
    if (l.bypass) {
      field_offsets[0] = l.off_kc; field_offsets[1] = l.off_vc;
      field_offsets[2] = field_offsets[3] = field_offsets[4] = 0;
    } else {
      field_offsets[0] = l.off_kc; field_offsets[1] = l.off_ks; field_offsets[2] = l.off_kn;
      field_offsets[3] = l.off_vc; field_offsets[4] = l.off_vsz;
    }
  }
  return TQ_OK;
}

tq_status tq_layer_state_host(const tq_layer_config* cfg, float* R, float* S, float* centroids,
                              float* boundaries) {
  clear_error();
  tq_status st = validate_config(cfg);
  if (st != TQ_OK) return st;
  std::vector<float> r, s;
  float c[256], b[256];
  int levels = 0;
  st = build_state(cfg, R ? &r : nullptr, S ? &s : nullptr, c, b, &levels);
  if (st != TQ_OK) return st;
  if (R) std::memcpy(R, r.data(), r.size() * sizeof(float));
  if (S) std::memcpy(S, s.data(), s.size() * sizeof(float));
  if (centroids && levels) std::memcpy(centroids, c, levels * sizeof(float));
  if (boundaries && levels) std::memcpy(boundaries, b, (levels - 1) * sizeof(float));
  return TQ_OK;
}

tq_status tq_layer_create(const tq_layer_config* cfg, void* hip_stream, tq_layer** out) {
  clear_error();
  if (!out) return fail(TQ_ERR_INVALID_ARGUMENT, "null output pointer");
  *out = nullptr;
  tq_layer* L = new tq_layer();
  tq_status st = make_layout(cfg, &L->lay);
  if (st != TQ_OK) { delete L; return st; }
  L->cfg = *cfg;
  std::vector<float> R, S;
  st = build_state(cfg, &R, cfg->bypass ? nullptr : &S, L->centroids, L->boundaries, &L->levels);
  if (st != TQ_OK) { delete L; return st; }
  if (!cfg->bypass && cfg->value_mode == TQ_VAL_MSE) {
    st = stored_codebook(cfg->v_bits, cfg->dist, L->v_centroids, L->v_boundaries);
    if (st != TQ_OK) { delete L; return st; }
  }
  hipError_t e = hipGetDevice(&L->device);
  if (e != hipSuccess) { delete L; return hip_fail(e, "hipGetDevice"); }
  e = hipDeviceGetAttribute(&L->cu_count, hipDeviceAttributeMultiprocessorCount, L->device);
  if (e != hipSuccess) { delete L; return hip_fail(e, "hipDeviceGetAttribute"); }
  if (!cfg->bypass) {
    const int d = kDim, H = cfg->n_kv_heads;
    const size_t n = static_cast<size_t>(H) * d * d;
    std::vector<float> RT(n), ST(n);
    for (int h = 0; h < H; ++h)
      for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
          RT[(static_cast<size_t>(h) * d + j) * d + i] = R[(static_cast<size_t>(h) * d + i) * d + j];
          ST[(static_cast<size_t>(h) * d + j) * d + i] = S[(static_cast<size_t>(h) * d + i) * d + j];
        }
    float** bufs[3] = {&L->dR, &L->dRT, &L->dST};
    const std::vector<float>* src[3] = {&R, &RT, &ST};
    for (int i = 0; i < 3; ++i) {
      e = hipMalloc(reinterpret_cast<void**>(bufs[i]), n * sizeof(float));
      if (e != hipSuccess) {
        tq_layer_destroy(L);
        return fail(TQ_ERR_OUT_OF_MEMORY, "hipMalloc of layer state failed: %s", hipGetErrorString(e));
      }
      e = hipMemcpyAsync(*bufs[i], src[i]->data(), n * sizeof(float), hipMemcpyHostToDevice,
                         static_cast<hipStream_t>(hip_stream));
      if (e != hipSuccess) { tq_layer_destroy(L); return hip_fail(e, "hipMemcpyAsync"); }
    }
    // Matrix-core A operands for the compressor: R as three bf16 pieces
    // (hi + mid + lo = R exactly) and S as two float16 pieces (22 bits), in the
    // order the compressor loads per wave.
    auto bf16_rne = [](float x) -> unsigned short {
      const unsigned u = __builtin_bit_cast(unsigned, x);
      return static_cast<unsigned short>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    };
    auto bf16_val = [](unsigned short b) { return __builtin_bit_cast(float, static_cast<unsigned>(b) << 16); };
    if (cfg->rotation == TQ_ROT_HADAMARD) L->r_scale = std::fabs(R[0]);
    const size_t nop = static_cast<size_t>(H) * 8 * kOpSets * 4 * 64 * 8;
    std::vector<unsigned short> opa(nop);
    for (int h = 0; h < H; ++h)
      for (int w = 0; w < 8; ++w)
        for (int ks = 0; ks < 4; ++ks)
          for (int l = 0; l < 64; ++l)
            for (int j = 0; j < 8; ++j) {
              const int row = 16 * w + l % 16, col = 32 * ks + 8 * (l / 16) + j;
              const float r = R[(static_cast<size_t>(h) * d + row) * d + col];
              const float sv = S[(static_cast<size_t>(h) * d + row) * d + col];
              // Hadamard: the exact sign pattern (bf16 +-1), the magnitude applied after
              const bool had = cfg->rotation == TQ_ROT_HADAMARD;
              const unsigned short r0 = had ? bf16_rne(r < 0.0f ? -1.0f : 1.0f) : bf16_rne(r);
              const unsigned short r1 = had ? 0 : bf16_rne(r - bf16_val(r0));
              const unsigned short r2 = had ? 0 : bf16_rne(r - bf16_val(r0) - bf16_val(r1));
              const _Float16 s0 = static_cast<_Float16>(sv);
              const _Float16 s1 = static_cast<_Float16>(sv - static_cast<float>(s0));
              const unsigned short v[kOpSets] = {r0, r1, r2, __builtin_bit_cast(unsigned short, s0),
                                                 __builtin_bit_cast(unsigned short, s1)};
              for (int set = 0; set < kOpSets; ++set) {
                const size_t at = (((((static_cast<size_t>(h) * 8 + w) * kOpSets + set) * 4 + ks) * 64 + l) * 8) + j;
                opa[at] = v[set];
              }
            }
    e = hipMalloc(reinterpret_cast<void**>(&L->dOpA), nop * sizeof(unsigned short));
    if (e != hipSuccess) {
      tq_layer_destroy(L);
      return fail(TQ_ERR_OUT_OF_MEMORY, "hipMalloc of layer state failed: %s", hipGetErrorString(e));
    }
    e = hipMemcpyAsync(L->dOpA, opa.data(), nop * sizeof(unsigned short), hipMemcpyHostToDevice,
                       static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) { tq_layer_destroy(L); return hip_fail(e, "hipMemcpyAsync"); }
    // Matrix-core B operands for the decode prologue: W = [R; P] with P = S R
    // (the exact product of the stored float32 R and S, formed in float64), so
    // that q' = R q and u = S q' = P q are independent products of q.  Each entry
    // is split into float16 hi + lo pieces.
    const size_t nq = static_cast<size_t>(H) * 16 * 4 * 2 * 64 * 8;
    std::vector<unsigned short> opq(nq);
    // Decompress B operands: R[k][n] and P[k][n] (P = S R) as float16 hi + lo.
    const size_t nd = static_cast<size_t>(H) * 8 * 4 * 4 * 64 * 8;
    std::vector<unsigned short> opd(nd);
    {
      std::vector<double> W(static_cast<size_t>(2 * d) * d);
      for (int h = 0; h < H; ++h) {
        const float* Rh = R.data() + static_cast<size_t>(h) * d * d;
        const float* Sh = S.data() + static_cast<size_t>(h) * d * d;
        for (int i = 0; i < d; ++i)
          for (int j = 0; j < d; ++j) {
            W[static_cast<size_t>(i) * d + j] = Rh[i * d + j];
            double acc = 0.0;
            for (int k = 0; k < d; ++k) acc += static_cast<double>(Sh[i * d + k]) * static_cast<double>(Rh[k * d + j]);
            W[static_cast<size_t>(d + i) * d + j] = acc;
          }
        for (int t = 0; t < 16; ++t)
          for (int ks = 0; ks < 4; ++ks)
            for (int l = 0; l < 64; ++l)
              for (int j = 0; j < 8; ++j) {
                const double w = W[static_cast<size_t>(16 * t + l % 16) * d + 32 * ks + 8 * (l / 16) + j];
                const _Float16 hi = static_cast<_Float16>(w);
                const _Float16 lo = static_cast<_Float16>(w - static_cast<double>(hi));
                const size_t at = ((((static_cast<size_t>(h) * 16 + t) * 4 + ks) * 2) * 64 + l) * 8 + j;
                opq[at] = __builtin_bit_cast(unsigned short, hi);
                opq[at + 64 * 8] = __builtin_bit_cast(unsigned short, lo);
              }
        for (int t = 0; t < 8; ++t)
          for (int ks = 0; ks < 4; ++ks)
            for (int l = 0; l < 64; ++l)
              for (int j = 0; j < 8; ++j) {
                const int k = 32 * ks + 8 * (l / 16) + j, n = 16 * t + l % 16;
                const double mv[2] = {W[static_cast<size_t>(k) * d + n], W[static_cast<size_t>(d + k) * d + n]};
                for (int m = 0; m < 2; ++m) {
                  const _Float16 hi = static_cast<_Float16>(mv[m]);
                  const _Float16 lo = static_cast<_Float16>(mv[m] - static_cast<double>(hi));
                  const size_t at = ((((static_cast<size_t>(h) * 8 + t) * 4 + ks) * 4 + 2 * m) * 64 + l) * 8 + j;
                  opd[at] = __builtin_bit_cast(unsigned short, hi);
                  opd[at + 64 * 8] = __builtin_bit_cast(unsigned short, lo);
                }
              }
      }
    }
    e = hipMalloc(reinterpret_cast<void**>(&L->dOpD), nd * sizeof(unsigned short));
    if (e != hipSuccess) {
      tq_layer_destroy(L);
      return fail(TQ_ERR_OUT_OF_MEMORY, "hipMalloc of layer state failed: %s", hipGetErrorString(e));
    }
    e = hipMemcpyAsync(L->dOpD, opd.data(), nd * sizeof(unsigned short), hipMemcpyHostToDevice,
                       static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) { tq_layer_destroy(L); return hip_fail(e, "hipMemcpyAsync"); }
    e = hipMalloc(reinterpret_cast<void**>(&L->dOpQ), nq * sizeof(unsigned short));
    if (e != hipSuccess) {
      tq_layer_destroy(L);
      return fail(TQ_ERR_OUT_OF_MEMORY, "hipMalloc of layer state failed: %s", hipGetErrorString(e));
    }
    e = hipMemcpyAsync(L->dOpQ, opq.data(), nq * sizeof(unsigned short), hipMemcpyHostToDevice,
                       static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) { tq_layer_destroy(L); return hip_fail(e, "hipMemcpyAsync"); }
    e = hipStreamSynchronize(static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) { tq_layer_destroy(L); return hip_fail(e, "hipStreamSynchronize"); }
  }
  *out = L;
  return TQ_OK;
}

tq_status tq_layer_destroy(tq_layer* L) {
  clear_error();
  if (!L) return TQ_OK;
  hipError_t e1 = L->dR ? hipFree(L->dR) : hipSuccess;
  hipError_t e2 = L->dRT ? hipFree(L->dRT) : hipSuccess;
  hipError_t e3 = L->dST ? hipFree(L->dST) : hipSuccess;
  hipError_t e4 = L->dOpA ? hipFree(L->dOpA) : hipSuccess;
  hipError_t e5 = L->dOpQ ? hipFree(L->dOpQ) : hipSuccess;
  hipError_t e6 = L->dOpD ? hipFree(L->dOpD) : hipSuccess;
  delete L;
  if (e1 != hipSuccess) return hip_fail(e1, "hipFree");
  if (e2 != hipSuccess) return hip_fail(e2, "hipFree");
  if (e3 != hipSuccess) return hip_fail(e3, "hipFree");
  if (e4 != hipSuccess) return hip_fail(e4, "hipFree");
  if (e5 != hipSuccess) return hip_fail(e5, "hipFree");
  if (e6 != hipSuccess) return hip_fail(e6, "hipFree");
  return TQ_OK;
}

tq_status tq_layer_export(const tq_layer* L, float* R, float* S, float* centroids, float* boundaries,
                          float* v_centroids, float* v_boundaries, void* hip_stream) {
  clear_error();
  if (!L) return fail(TQ_ERR_INVALID_ARGUMENT, "null layer");
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const int d = kDim, H = L->cfg.n_kv_heads;
  const size_t n = static_cast<size_t>(H) * d * d;
  std::vector<float> st;
  if (!L->cfg.bypass) {
    if (R) {
      hipError_t e = hipMemcpyAsync(R, L->dR, n * sizeof(float), hipMemcpyDeviceToHost, s);
      if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    }
    if (S) {
      st.resize(n);
      hipError_t e = hipMemcpyAsync(st.data(), L->dST, n * sizeof(float), hipMemcpyDeviceToHost, s);
      if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    }
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    if (S)
      for (int h = 0; h < H; ++h)
        for (int i = 0; i < d; ++i)
          for (int j = 0; j < d; ++j)
            S[(static_cast<size_t>(h) * d + i) * d + j] = st[(static_cast<size_t>(h) * d + j) * d + i];
  }
  if (L->levels) {
    if (centroids) std::memcpy(centroids, L->centroids, L->levels * sizeof(float));
    if (boundaries) std::memcpy(boundaries, L->boundaries, (L->levels - 1) * sizeof(float));
  }
  if (!L->cfg.bypass && L->cfg.value_mode == TQ_VAL_MSE) {
    const int lv = 1 << L->cfg.v_bits;
    if (v_centroids) std::memcpy(v_centroids, L->v_centroids, lv * sizeof(float));
    if (v_boundaries) std::memcpy(v_boundaries, L->v_boundaries, (lv - 1) * sizeof(float));
  }
  return TQ_OK;
}

tq_status tq_layer_export_operands(const tq_layer* L, tq_operands which, void* host_out, size_t capacity,
                                   size_t* bytes, void* hip_stream) {
  clear_error();
  if (!L || !bytes) return fail(TQ_ERR_INVALID_ARGUMENT, "null argument");
  if (L->cfg.bypass) return fail(TQ_ERR_UNSUPPORTED, "bypass layers hold no matrix-core operands");
  const size_t H = static_cast<size_t>(L->cfg.n_kv_heads);
  const unsigned short* src = nullptr;
  size_t count = 0;
  switch (which) {
    case TQ_OPERANDS_COMPRESS: src = L->dOpA; count = H * 8 * kOpSets * 4 * 64 * 8; break;
    case TQ_OPERANDS_PROLOGUE: src = L->dOpQ; count = H * 16 * 4 * 2 * 64 * 8; break;
    case TQ_OPERANDS_DECOMPRESS: src = L->dOpD; count = H * 8 * 4 * 4 * 64 * 8; break;
    default: return fail(TQ_ERR_INVALID_ARGUMENT, "unknown operand buffer %d", static_cast<int>(which));
  }
  *bytes = count * sizeof(unsigned short);
  if (!host_out) return TQ_OK;
  if (capacity < *bytes) return fail(TQ_ERR_INVALID_ARGUMENT, "capacity %zu < %zu bytes", capacity, *bytes);
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  hipError_t e = hipMemcpyAsync(host_out, src, *bytes, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  return TQ_OK;
}

tq_status tq_compress_kv(const tq_layer* L, const void* k, const void* v, tq_dtype in_dtype,
                         long long n_tokens, long long k_token_stride, long long v_token_stride,
                         const long long* slot_mapping, void* pool, long long num_blocks,
                         void* hip_stream) {
  clear_error();
  if (!L) return fail(TQ_ERR_INVALID_ARGUMENT, "null layer");
  if (n_tokens < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "n_tokens must be >= 0");
  if (num_blocks <= 0) return fail(TQ_ERR_INVALID_ARGUMENT, "num_blocks must be > 0");
  const long long row = static_cast<long long>(L->cfg.n_kv_heads) * kDim;
  if (k_token_stride < row || v_token_stride < row)
    return fail(TQ_ERR_INVALID_ARGUMENT, "token strides must be >= n_kv_heads*128 (got %lld, %lld)",
                k_token_stride, v_token_stride);
  if (in_dtype != TQ_F32 && in_dtype != TQ_BF16)
    return fail(TQ_ERR_UNSUPPORTED, "compress input dtype %d not supported (F32, BF16)", static_cast<int>(in_dtype));
  if (L->cfg.bypass && in_dtype != TQ_BF16)
    return fail(TQ_ERR_UNSUPPORTED, "bypass layers store bf16: input dtype must be BF16");
  if (n_tokens == 0) return TQ_OK;
  if (!k || !v || !slot_mapping || !pool) return fail(TQ_ERR_INVALID_ARGUMENT, "null device pointer");
  if (n_tokens > (1LL << 31) - 1) return fail(TQ_ERR_UNSUPPORTED, "n_tokens too large for one launch");
  if (debug_checks()) {
    tq_status st = debug_check_slots(slot_mapping, n_tokens, num_blocks, hip_stream);
    if (st != TQ_OK) return st;
  }
  return launch_compress(L, k, v, in_dtype, n_tokens, k_token_stride, v_token_stride, slot_mapping,
                         pool, hip_stream);
}

tq_status tq_decompress_kv(const tq_layer* L, const void* pool, long long num_blocks, const long long* slot_mapping,
                           long long n_tokens, void* k_out, void* v_out, tq_dtype out_dtype, void* hip_stream) {
  clear_error();
  if (!L) return fail(TQ_ERR_INVALID_ARGUMENT, "null layer");
  if (n_tokens < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "n_tokens must be >= 0");
  if (num_blocks <= 0) return fail(TQ_ERR_INVALID_ARGUMENT, "num_blocks must be > 0");
  if (out_dtype != TQ_F32 && out_dtype != TQ_BF16)
    return fail(TQ_ERR_UNSUPPORTED, "decompress output dtype %d not supported (F32, BF16)", static_cast<int>(out_dtype));
  if (n_tokens == 0) return TQ_OK;
  if (!pool || !slot_mapping || !k_out || !v_out) return fail(TQ_ERR_INVALID_ARGUMENT, "null device pointer");
  if (n_tokens > (1LL << 31) - 1) return fail(TQ_ERR_UNSUPPORTED, "n_tokens too large for one launch");
  if (debug_checks()) {
    tq_status st = debug_check_slots(slot_mapping, n_tokens, num_blocks, hip_stream);
    if (st != TQ_OK) return st;
  }
  return launch_decompress(L, pool, slot_mapping, n_tokens, k_out, v_out, out_dtype, hip_stream);
}

tq_status tq_decode_workspace_size(const tq_layer* L, int batch, int n_q_heads, int max_seq_len,
                                   int num_splits, size_t* bytes) {
  clear_error();
  if (!L || !bytes) return fail(TQ_ERR_INVALID_ARGUMENT, "null argument");
  if (batch < 0 || n_q_heads <= 0 || max_seq_len < 0 || num_splits < 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "negative size");
  DecodePlan p;
  tq_status st = plan_decode(L, batch, n_q_heads, max_seq_len, num_splits, &p);
  if (st != TQ_OK) return st;
  *bytes = p.ws_bytes;
  return TQ_OK;
}

tq_status tq_decode_attn(const tq_layer* L, const void* q, tq_dtype q_dtype, int batch,
                         int n_q_heads, const void* pool, long long num_blocks,
                         const int* block_table, int max_blocks_per_seq, const int* seq_lens,
                         int max_seq_len, float softmax_scale, int num_splits, void* out,
                         tq_dtype out_dtype, void* workspace, size_t workspace_bytes,
                         void* hip_stream) {
  clear_error();
  DecodePlan p;
  float scale = 0.0f;
  tq_status st = prepare_decode(L, q, q_dtype, batch, n_q_heads, pool, num_blocks, block_table, max_blocks_per_seq,
                                seq_lens, max_seq_len, softmax_scale, num_splits, out, out_dtype, &p, &scale);
  if (st != TQ_OK || batch == 0) return st;
  if (!workspace) return fail(TQ_ERR_INVALID_ARGUMENT, "null device pointer");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < p.ws_bytes)
    return fail(TQ_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu bytes", workspace_bytes, p.ws_bytes);
  if (debug_checks()) {
    std::vector<int> hl(static_cast<size_t>(batch)), ht(static_cast<size_t>(batch) * max_blocks_per_seq);
    st = fetch(hl.data(), seq_lens, hl.size() * sizeof(int), hip_stream);
    if (st == TQ_OK && !ht.empty()) st = fetch(ht.data(), block_table, ht.size() * sizeof(int), hip_stream);
    if (st == TQ_OK) st = check_decode_tables(hl.data(), ht.data(), batch, max_blocks_per_seq, max_seq_len, num_blocks);
    if (st != TQ_OK) return st;
  }
  return launch_decode(L, p, q, q_dtype, pool, block_table, max_blocks_per_seq, seq_lens, scale, out,
                       out_dtype, workspace, hip_stream);
}

}  // extern "C"
