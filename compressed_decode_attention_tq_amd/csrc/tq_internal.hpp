// Internal declarations shared by the host code and the kernel launchers of libtq.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "tq.h"

namespace tq {

constexpr int kOpSets = 5;  // compressor operand sets per row tile
constexpr int kDim = 128;     // head_dim supported by the kernels
constexpr int kPage = 16;     // tokens per block
constexpr int kGroup = 32;    // value group width
// Longest context span of one split-K workgroup: its four waves take 32-token
// chunks in turn, at most 32 each (one block id per lane of a 64-lane wave).
constexpr int kMaxSplitTokens = 4096;

// ---------------------------------------------------------------- errors
tq_status fail(tq_status st, const char* fmt, ...);
void clear_error();

// ------------------------------------------------------------ random state
uint64_t mix64(uint64_t z);
uint64_t stream_key(uint64_t seed, uint64_t layer, uint64_t head, uint64_t tag);
void gaussians(uint64_t seed, uint64_t layer, uint64_t head, uint64_t tag, size_t count,
               double* out);
constexpr uint64_t kTagRotation = 1;
constexpr uint64_t kTagProjection = 2;
constexpr uint64_t kTagSigns = 3;

// Haar rotation (row-major d x d, float64) for (seed, layer, head).
void haar_rotation(uint64_t seed, int layer, int head, int d, double* out);
// Randomised Hadamard rotation H D / sqrt(d) (row-major d x d, float64), d a power of two.
void hadamard_rotation(uint64_t seed, int layer, int head, int d, double* out);

// Lloyd-Max codebook; returns TQ_OK or an error status.
tq_status lloyd_max(int bits, tq_dist dist, int dim, double* centroids, double* boundaries,
                    double* mse);

// ---------------------------------------------------------------- layout
struct Layout {
  bool bypass = false;
  int k_bits = 0, v_bits = 0;
  int kc_bytes = 0, ks_bytes = 0, kn_bytes = 0, vc_bytes = 0, vsz_bytes = 0;  // per token
  size_t off_kc = 0, off_ks = 0, off_kn = 0, off_vc = 0, off_vsz = 0;         // per block
  size_t block_bytes = 0;
};
tq_status make_layout(const tq_layer_config* cfg, Layout* out);
tq_status validate_config(const tq_layer_config* cfg);

// ------------------------------------------------------- debug checks
// Host-side validation of index arrays (the TQ_DEBUG_CHECKS=1 option copies
// them from the device first).  Return TQ_OK or TQ_ERR_INVALID_ARGUMENT.
tq_status check_slots(const long long* slots, long long n, long long num_blocks);
tq_status check_decode_tables(const int* seq_lens, const int* block_table, int batch, int max_blocks,
                              int max_seq_len, long long num_blocks);
bool debug_checks();

// ------------------------------------------------------------- profiling
enum KernelId { kKCompress = 0, kKPrologue = 1, kKSplitK = 2, kKCombine = 3, kKCount = 4 };
// Brackets one launch with HIP events when timing of `id` is enabled.
class ProfScope {
 public:
  ProfScope(int id, void* stream);
  ~ProfScope();

 private:
  int slot_ = -1;
  void* stream_;
};

}  // namespace tq

// ------------------------------------------------------------------ layer
struct tq_layer {
  tq_layer_config cfg;
  tq::Layout lay;
  int device = 0;
  int cu_count = 0;
  // Device state (float32).  R and S row-major [H][128][128]; RT = R^T per head.
  float* dR = nullptr;
  float* dRT = nullptr;
  float* dST = nullptr;
  // Matrix-core A operands of R and S for the compressor (16-bit patterns):
  // [H][8 row tiles][kOpSets: R bf16 hi, mid, lo; S fp16 hi, lo][4 K-steps][64 lanes][8],
  // lane l of (tile w, step s) holding M[16w + l%16][32s + 8(l/16) .. +7].
  unsigned short* dOpA = nullptr;
  // Hadamard layers: the compressor's A operands hold the exact +-1 pattern of R
  // (piece 0; pieces 1 and 2 zero) and the products are scaled by r_scale = |R_ij|.
  float r_scale = 1.0f;
  // Matrix-core B operands of W = [R; S R] (256 x 128) for the decode prologue
  // (float16 bits): [H][16 column tiles][4 K-steps][hi, lo][64 lanes][8], lane l
  // of (tile t, step s) holding W[16t + l%16][32s + 8(l/16) .. +7].
  unsigned short* dOpQ = nullptr;
  // Matrix-core B operands of R and P = S R for the decompress kernel (float16 bits):
  // [H][8 column tiles][4 K-steps][R hi, R lo, P hi, P lo][64 lanes][8], lane l of
  // (tile t, step s) holding M[32s + 8(l/16) .. +7][16t + l%16].
  unsigned short* dOpD = nullptr;
  float centroids[16] = {0};
  float boundaries[16] = {0};
  int levels = 0;
  // value codebook (layers with MSE-coded values): v_bits-bit, same density
  float v_centroids[16] = {0};
  float v_boundaries[16] = {0};
};

namespace tq {

// Kernel launchers (defined in the .hip files).  Arguments already validated.
tq_status launch_compress(const tq_layer* L, const void* k, const void* v, tq_dtype in_dtype,
                          long long n_tokens, long long k_stride, long long v_stride,
                          const long long* slots, void* pool, void* stream);
// Matrix-core compressor (bf16 inputs, 64+ tokens, 16-byte aligned rows).
bool compress_mfma_applies(const tq_layer* L, const void* k, const void* v, tq_dtype in_dtype, long long n_tokens,
                           long long k_stride, long long v_stride);
tq_status launch_compress_mfma(const tq_layer* L, const void* k, const void* v, long long n_tokens,
                               long long k_stride, long long v_stride, const long long* slots, void* pool,
                               void* stream);

struct DecodePlan {
  int batch = 0, n_q_heads = 0, rep = 0;
  int split_tokens = 0;   // tokens per split (multiple of 64)
  int n_splits = 0;       // splits per sequence
  bool work_list = false; // split-K item order: work list of live items (else plain order)
  size_t ws_part = 0;     // byte offset of split partials
  size_t ws_qa = 0;       // byte offset of the Q.K matrix-core operand (compressed layers)
  size_t ws_bytes = 0;    // total
};
tq_status plan_decode(const tq_layer* L, int batch, int n_q_heads, int max_seq_len,
                      int num_splits, DecodePlan* plan);
// Argument checks shared by the decode entry points (everything but the
// workspace); on TQ_OK with batch > 0, *plan and *scale are set.
tq_status prepare_decode(const tq_layer* L, const void* q, tq_dtype q_dtype, int batch, int n_q_heads,
                         const void* pool, long long num_blocks, const int* block_table, int max_blocks_per_seq,
                         const int* seq_lens, int max_seq_len, float softmax_scale, int num_splits, void* out,
                         tq_dtype out_dtype, DecodePlan* plan, float* scale);
tq_status launch_splitk_tq(const tq_layer* L, const DecodePlan& plan, const void* pool, const int* block_table,
                           int max_blocks_per_seq, const int* seq_lens, float softmax_scale, const void* qa,
                           float* part, void* stream);
// Uncompressed (bypass) layers: reads q directly (no prologue launch).
tq_status launch_splitk_bypass(const tq_layer* L, const DecodePlan& plan, const void* q, tq_dtype q_dtype,
                               const void* pool, const int* block_table, int max_blocks_per_seq,
                               const int* seq_lens, float softmax_scale, float* part, void* stream);
tq_status launch_decompress(const tq_layer* L, const void* pool, const long long* slots, long long n_tokens,
                            void* k_out, void* v_out, tq_dtype out_dtype, void* stream);
tq_status launch_decode(const tq_layer* L, const DecodePlan& plan, const void* q, tq_dtype q_dtype,
                        const void* pool, const int* block_table, int max_blocks_per_seq,
                        const int* seq_lens, float softmax_scale, void* out, tq_dtype out_dtype,
                        void* workspace, void* stream);

}  // namespace tq
