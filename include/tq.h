/*
 * tq.h -- C ABI of libtq, TurboQuant-style compressed KV cache for MI355X (gfx950).
 *
 * Two operations, both hand-written HIP kernels for gfx950:
 *
 *  1. tq_compress_kv: fused compression of key/value head vectors into a paged
 *     store.  Keys: norm, random orthogonal rotation, Lloyd-Max scalar codebook,
 *     1-bit QJL sign of the residual.  Values: the same rotation, then group
 *     scale/zero low-bit quantisation.  All payloads bit-packed.
 *       - "How 0xsero/turboquant works", sections "Compression Pipeline" and
 *         "Value Compression".
 *       - "5x Faster LLM Inference? This KV Cache Hack Changes Everything",
 *         "Example 4: Kernel-Level Operations" (normalise, rotate, Lloyd-Max
 *         quantise, pack; one fused launch for K and V).
 *       - "turbo-attn 0.24.0" (PyPI), "How it works" (rotate, store the
 *         magnitude, quantise to a shared codebook).
 *
 *  2. tq_decode_attn: split-K paged decode attention that scores queries against
 *     the compressed keys and accumulates the compressed values, dequantising
 *     inside the loop (no expanded float cache).
 *       - "turbo-attn 0.24.0", "How it works" (query rotated once, attention in
 *         the rotated space, one fused unpack/dequant/QK/online-softmax/PV pass)
 *         and "Configuration" (TKV_DECODE_SPLITS: split count autotuned or forced;
 *         TKV_NO_JIT: a missing variant is a hard error).
 *       - "How 0xsero/turboquant works", "Key Storage and Attention Scoring".
 *       - "tiny-turboquant 0.18.0", "Fused decode-attention path" (a partials
 *         launch, then a combine launch).
 *
 * Conventions
 *   - Every function returns tq_status; TQ_OK == 0.  On any other status a
 *     thread-local message is available from tq_last_error().  Nothing is ever
 *     silently degraded: an unsupported variant is TQ_ERR_UNSUPPORTED.
 *   - "device pointer" means memory on the current HIP device (hipMalloc,
 *     torch CUDA tensors); "host pointer" means ordinary CPU memory.
 *   - The caller owns every buffer passed in.  The library owns only tq_layer
 *     objects (rotation, projection and codebook state on the device).
 *   - Host-visible arguments are validated synchronously.  Kernels are enqueued
 *     asynchronously on the caller's stream (hipStream_t passed as void*, NULL =
 *     the null stream); a launch failure is reported as TQ_ERR_HIP.  The compress
 *     and decode entry points never allocate and never synchronise.
 *   - Contents of device buffers (slot ids, block ids, sequence lengths) are the
 *     caller's contract; they are not range-checked on the device.  Debug
 *     option: while the environment variable TQ_DEBUG_CHECKS is set (to
 *     anything but "0"; read at every call), tq_compress_kv and
 *     tq_decompress_kv copy slot_mapping, and tq_decode_attn copies seq_lens and
 *     the used block-table entries, to host memory (synchronising the stream)
 *     and return TQ_ERR_INVALID_ARGUMENT before any launch if a slot is past the
 *     pool, a length is outside [0, min(max_seq_len, 16*max_blocks_per_seq)] or
 *     a block id of a used page is outside [0, num_blocks).  Off by default: it
 *     allocates host memory and synchronises, which the hot path never does.
 *   - Supported: head_dim = 128, block_size = 16, v_group = 32,
 *     k_bits in {1,2,3,4}, v_bits in {2,3,4}, query heads per KV head in {1,2,4,8}.
 *
 * Store format (one pool per layer; exported by tq_store_layout)
 *   pool = uint8[num_blocks][n_kv_heads][block_bytes], 16 tokens per block,
 *   slot = block * 16 + offset.  Inside one (block, head) region ("page"),
 *   five fields.  Bit packing is LSB-first: element i of a b-bit stream
 *   occupies stream bits [b*i, b*i + b), stream bit k being bit k%8 of byte k/8.
 *     Kc  [4][16][4*k_bits]  key codebook indices: for 32-dim block j and token
 *                            t, the k_bits stream of dims 32j .. 32j+31
 *     Ks  [4][16][4]         QJL sign bits (1 <=> (S rho)_j >= 0), same blocking
 *     Kn  [16][2] fp16       ||k|| then gamma = ||rho||   ([16] fp16 ||k||, and no
 *                            Ks field, in the key modes without QJL)
 *     Vc  [32][64] v_bits    value codes in 32 lane blocks: for dim = 16i + c
 *                            and token t = 8h + k, block 16h + c, group
 *                            2i + k/4 of four codes, element k % 4 (one stream
 *                            in the order block, group, element)
 *     Vsz [16][4][2] fp16    per 32-wide group: scale then zero
 *   Every field is laid out so that one lane of the decode's 64-lane wave
 *   loads its share of a page with one contiguous read: key fields are blocked
 *   so that a 32-dim slice of one token is contiguous, and the value codes of
 *   8 tokens of one coordinate (one matrix-core operand row) are one run of
 *   8*v_bits bits, the 8 runs of a lane block adjacent.  A single token
 *   appended to a page therefore shares Vc bytes with its neighbours.
 *   Bypass (uncompressed) layers: region = K [16][128] bf16 (token-major), then
 *   V^T [128][16] bf16 (dim-major: the 16 tokens' values of one dim together).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 6

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, inconsistent sizes     */
  TQ_ERR_UNSUPPORTED = 2,      /* a shape / bit width / dtype the library has no kernel for */
  TQ_ERR_OUT_OF_MEMORY = 3,    /* device allocation in tq_layer_create failed         */
  TQ_ERR_HIP = 4,              /* a HIP runtime call or kernel launch failed           */
  TQ_ERR_NOT_CONVERGED = 5     /* Lloyd-Max iteration hit its iteration cap           */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

/* Density the key codebook is optimal for, in units of the standardised rotated
 * coordinate t = sqrt(d) (R k)_j / ||k||:
 *   TQ_DIST_GAUSSIAN: N(0,1)   ("5x Faster LLM Inference? ...", "What is TurboQuant-GPU?":
 *                               rotated coordinates are approximately Gaussian)
 *   TQ_DIST_SPHERE:   the exact marginal sqrt(d) u_j of u uniform on S^{d-1}
 *                     ("tiny-turboquant 0.18.0", "The algorithm in three lines":
 *                      the Beta-distribution codebook of the original method). */
typedef enum { TQ_DIST_GAUSSIAN = 0, TQ_DIST_SPHERE = 1 } tq_dist;

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* tq_last_error(void);

/* Returns TQ_ABI_VERSION of the built library. */
int tq_abi_version(void);

/* Lloyd-Max codebook ("How 0xsero/turboquant works", "Compression Pipeline":
 * Lloyd-Max codebooks precomputed per dimension and bit width).  Host only,
 * float64, no device needed.
 *   bits        1..8 (levels L = 2^bits)
 *   dist, dim   density (dim used by TQ_DIST_SPHERE; must be >= 3 there)
 *   centroids   host out [L], ascending
 *   boundaries  host out [L-1], boundaries[i] = (centroids[i] + centroids[i+1]) / 2
 *   mse         host out, nullable: expected squared error per coordinate
 * Iterates Lloyd's conditions from the quantile midpoints to max|delta c| < 1e-14,
 * at most 200,000 times; the 8-bit N(0,1) codebook does not reach that tolerance
 * within the cap and returns TQ_ERR_NOT_CONVERGED (the kernels use 1..4 bits). */
tq_status tq_codebook_build(int bits, tq_dist dist, int dim, double* centroids,
                            double* boundaries, double* mse);

/* Key estimator of a compressed layer.
 *   TQ_KEY_QJL     codebook codes plus the 1-bit QJL residual signs and the
 *                  residual norm gamma ("How 0xsero/turboquant works",
 *                  "Compression Pipeline" and "Key Storage and Attention Scoring").
 *   TQ_KEY_MSE     codebook codes and the vector norm only: no residual signs
 *                  (stored as zero bits) and gamma stored as 0, so the score
 *                  is the plain inner product with the codebook reconstruction
 *                  ("turbo-attn 0.24.0", "How it works": normalise, store one
 *                  magnitude, quantise each rotated coordinate to a shared codebook).
 *   TQ_KEY_MSE_NC  as TQ_KEY_MSE, with the stored magnitude norm-corrected to
 *                  n * sqrt(d) / ||c[idx]||, so that the reconstruction
 *                  (n16 / sqrt d) R^T c[idx] has the key's own norm ("turbo-attn
 *                  0.24.0", "Configuration", TKV_K_NC: norm-correction of K reads).
 * The two modes without QJL use a compact page: no sign field (Ks has 0 bytes,
 * its offset is Kn's) and Kn [16] fp16 holds the magnitude alone (18 bytes less
 * per token-head; 146 instead of 164 at K4/V4); the decode then runs no sign
 * products. */
typedef enum { TQ_KEY_QJL = 0, TQ_KEY_MSE = 1, TQ_KEY_MSE_NC = 2 } tq_key_mode;

/* Rotation family of a compressed layer (per KV head g).
 *   TQ_ROT_HAAR      dense Haar-random orthogonal R_g (default; QR of a Gaussian
 *                    matrix from the tag-1 stream, Mezzadri's sign fix).
 *   TQ_ROT_HADAMARD  randomised Hadamard R_g = H D / sqrt(d): H the Sylvester
 *                    Hadamard matrix (H[i][j] = (-1)^popcount(i & j)), D a diagonal
 *                    of random signs (+1 when the top bit of the tag-3 SplitMix64
 *                    output is 0) ("turbo-attn 0.24.0", "How it works": the KV rotation
 *                    is a fast Walsh-Hadamard transform).  Every entry
 *                    is +-1/sqrt(d), so the compressor's rotations take one
 *                    matrix-core pass on the exact +-1 pattern instead of three. */
typedef enum { TQ_ROT_HAAR = 0, TQ_ROT_HADAMARD = 1 } tq_rotation;

/* Value coding of a compressed layer.
 *   TQ_VAL_GROUP  v' = R_g v quantised per 32-wide group with its own fp16
 *                 scale and zero ("How 0xsero/turboquant works", "Value
 *                 Compression"); last page field Vsz [16][4][2] fp16.
 *   TQ_VAL_MSE    values coded like the keys' codebook part ("5x Faster LLM
 *                 Inference? ...", "What is TurboQuant-GPU?": 3-bit MSE values;
 *                 "Example 4": normalise -> rotate -> Lloyd-Max quantise -> pack):
 *                 nv = ||v||, t = sqrt(d) R_g v / nv, codes = v_bits-bit indices
 *                 into the stored Lloyd-Max codebook of the same density (float16
 *                 centroids, midpoint boundaries), value (nv16 / sqrt d) c[code];
 *                 the Vc stream keeps its order and the last field is Vn [16]
 *                 fp16 (K2 + QJL / V3: 102 bytes per token-head, 1632 per page).
 *                 tq_compress_kv writes such layers (with the per-token
 *                 compressor) and tq_decompress_kv reads them; tq_decode_attn
 *                 returns TQ_ERR_UNSUPPORTED for them. */
typedef enum { TQ_VAL_GROUP = 0, TQ_VAL_MSE = 1 } tq_value_mode;

typedef struct {
  int head_dim;             /* d; must be 128                                   */
  int n_kv_heads;           /* KV heads of the layer, >= 1                      */
  int k_bits;               /* key codebook bits, 1..4 (QJL adds 1 bit/coord)   */
  int v_bits;               /* value code bits, 2..4                            */
  int v_group;              /* value group width; must be 32                    */
  int block_size;           /* tokens per page; must be 16                      */
  int layer;                /* layer index, part of the random-state key        */
  tq_dist dist;             /* key codebook density                             */
  unsigned long long seed;  /* random-state seed                                */
  int bypass;               /* 1: uncompressed bf16 layer (bits/dist ignored)   */
  tq_key_mode key_mode;     /* key estimator (compressed layers)                */
  tq_rotation rotation;     /* rotation family (compressed layers)              */
  tq_value_mode value_mode; /* value coding (compressed layers)                 */
} tq_layer_config;

/* Opaque per-layer state.  Holds, on the device, for every KV head g:
 *   R_g  d x d random orthogonal rotation of the chosen family (float32), and
 *   S_g  d x d i.i.d. N(0,1) QJL projection (float32),
 * both drawn from SplitMix64 + Box-Muller streams keyed by (seed, layer, g, tag)
 * ("5x Faster LLM Inference? ...", "Example 1": a rotation precomputed and fixed
 * per head), plus the key codebook: Lloyd-Max centroids rounded to float16 and
 * the exact midpoints between them as decision boundaries.  Read-only after create;
 * may be used from several streams at once. */
typedef struct tq_layer tq_layer;

/* The state a layer would hold, computed on the host only (no device needed).
 *   R, S        host out [n_kv_heads][128][128] float32, row-major (nullable)
 *   centroids   host out [2^k_bits] float32 (nullable): float16-rounded Lloyd-Max centroids
 *   boundaries  host out [2^k_bits - 1] float32 (nullable): midpoints of the centroids */
tq_status tq_layer_state_host(const tq_layer_config* cfg, float* R, float* S, float* centroids,
                              float* boundaries);

/* Build the state on the host and upload it to the current device.  Allocates
 * device memory (owned by the layer until tq_layer_destroy) and synchronises
 * `hip_stream` once.  *out receives the new layer. */
tq_status tq_layer_create(const tq_layer_config* cfg, void* hip_stream, tq_layer** out);

/* Frees the layer's device memory.  NULL is accepted.  The caller must ensure no
 * kernel using the layer is still running. */
tq_status tq_layer_destroy(tq_layer* layer);

/* The state a created layer actually holds, copied back from the device (the
 * rotation/projection state and the codebooks of "How 0xsero/turboquant works",
 * "Compression Pipeline"):
 *   R, S          host out [n_kv_heads][128][128] float32, row-major (nullable):
 *                 the device copies of R_g and S_g the kernels read (S is held
 *                 transposed on the device and returned untransposed; a bypass
 *                 layer holds neither and leaves them untouched)
 *   centroids     host out [2^k_bits] float32 (nullable): the stored key codebook
 *   boundaries    host out [2^k_bits - 1] float32 (nullable)
 *   v_centroids   host out [2^v_bits] float32 (nullable): the stored value
 *                 codebook of a TQ_VAL_MSE layer (untouched otherwise)
 *   v_boundaries  host out [2^v_bits - 1] float32 (nullable)
 * Device-to-host copies on hip_stream, then one synchronisation of it; nothing is
 * allocated on the device.  Errors: TQ_ERR_INVALID_ARGUMENT for a null layer,
 * TQ_ERR_HIP if a copy fails. */
tq_status tq_layer_export(const tq_layer* layer, float* R, float* S, float* centroids, float* boundaries,
                          float* v_centroids, float* v_boundaries, void* hip_stream);

/* The matrix-core operand buffers a created layer derived from R and S, copied
 * back byte for byte (test and inspection aid):
 *   which = TQ_OPERANDS_COMPRESS    R as three bf16 pieces and S as two float16
 *           pieces, [H][8 row tiles][5 pieces][4 K-steps][64 lanes][8] uint16;
 *           lane l of (tile w, step s) holds M[16w + l%16][32s + 8(l/16) + j]
 *           (Hadamard layers: piece 0 the exact +-1 sign pattern of R, pieces
 *           1 and 2 zero)
 *         = TQ_OPERANDS_PROLOGUE    W = [R; S R] (the float64 product of the
 *           stored float32 matrices) as float16 hi + lo,
 *           [H][16 column tiles][4 K-steps][hi, lo][64 lanes][8] uint16; lane l
 *           of (tile t, step s) holds W[16t + l%16][32s + 8(l/16) + j]
 *         = TQ_OPERANDS_DECOMPRESS  R and P = S R as float16 hi + lo,
 *           [H][8 column tiles][4 K-steps][R hi, R lo, P hi, P lo][64 lanes][8]
 *           uint16; lane l of (tile t, step s) holds M[32s + 8(l/16) + j][16t + l%16]
 *   host_out   host out, nullable (then only *bytes is set)
 *   capacity   bytes available at host_out
 *   bytes      host out: the buffer's size
 * TQ_ERR_INVALID_ARGUMENT if capacity < the size (host_out non-null) or `which`
 * is unknown, TQ_ERR_UNSUPPORTED for a bypass layer (no operands), TQ_ERR_HIP if
 * the copy fails.  Synchronises hip_stream once. */
typedef enum { TQ_OPERANDS_COMPRESS = 0, TQ_OPERANDS_PROLOGUE = 1, TQ_OPERANDS_DECOMPRESS = 2 } tq_operands;
tq_status tq_layer_export_operands(const tq_layer* layer, tq_operands which, void* host_out, size_t capacity,
                                   size_t* bytes, void* hip_stream);

/* Byte layout of one (block, head) region of the pool.
 *   block_bytes    host out
 *   field_offsets  host out [5] (Kc, Ks, Kn, Vc, Vsz); for bypass layers
 *                  [K, V, 0, 0, 0]; nullable */
tq_status tq_store_layout(const tq_layer_config* cfg, size_t* block_bytes, size_t* field_offsets);

/* Fused K+V compression into the paged pool.
 *   k, v             device [n_tokens][n_kv_heads][128] of in_dtype (F32 or BF16);
 *                    token t of head g at k + t*k_token_stride + g*128 (elements)
 *   slot_mapping     device int64 [n_tokens]; slot < 0 skips the token
 *   pool             device uint8 [num_blocks][n_kv_heads][block_bytes]
 * Requires 0 <= slot < num_blocks*16 for every non-negative slot (not checked on
 * the device).  Tokens with equal slots race.  Bypass layers copy bf16 K/V (in_dtype
 * must be BF16 there). */
tq_status tq_compress_kv(const tq_layer* layer, const void* k, const void* v, tq_dtype in_dtype,
                         long long n_tokens, long long k_token_stride, long long v_token_stride,
                         const long long* slot_mapping, void* pool, long long num_blocks,
                         void* hip_stream);

/* Keys and values of n_tokens tokens reconstructed from the store, in the original
 * (un-rotated) basis ("turbo-attn 0.24.0", "How it works": a decompress path for
 * attention kernels that cannot read the codec; "tiny-turboquant 0.18.0", "Fused
 * decode-attention path"):
 *   khat = (n16 / sqrt d) R_g^T (c[idx] + sqrt(pi/2)/128 * gamma16 * S_g^T (2 z - 1))
 *   vhat = R_g^T (zero16 + scale16 * code)
 * so that softmax_scale * (q . khat) is the score tq_decode_attn forms for the
 * token (the QJL term is 0 in the key modes without QJL).  Bypass layers return
 * their stored bf16 values.
 *   pool          device pool written by tq_compress_kv (num_blocks blocks)
 *   slot_mapping  device int64 [n_tokens]: slot of each token; < 0 gives zero rows
 *   k_out, v_out  device [n_tokens][n_kv_heads][128] of out_dtype (F32, or BF16
 *                 rounded to nearest even); caller-owned
 * One launch on hip_stream; nothing is allocated.  Slots must be < 16*num_blocks
 * (the caller's contract, not checked on the device). */
tq_status tq_decompress_kv(const tq_layer* layer, const void* pool, long long num_blocks,
                           const long long* slot_mapping, long long n_tokens, void* k_out, void* v_out,
                           tq_dtype out_dtype, void* hip_stream);

/* Bytes of device workspace tq_decode_attn needs for this shape (num_splits as
 * passed to tq_decode_attn, 0 = automatic). */
tq_status tq_decode_workspace_size(const tq_layer* layer, int batch, int n_q_heads,
                                   int max_seq_len, int num_splits, size_t* bytes);

/* Paged decode attention over the compressed store, output in the original
 * (un-rotated) basis:
 *   out[b][h][:] = sum_i p_i * vhat_i over tokens i < seq_lens[b] of sequence b,
 *   p = softmax(s), s_i = softmax_scale * (||k_i||16 / sqrt d) *
 *       (q'.c[idx_i] + sqrt(pi/2)/128 * gamma_i * (S_g q').(2 z_i - 1)),  q' = R_g q,
 *   vhat_i = R_g^T (zero + scale * code_i),  g = h / (n_q_heads / n_kv_heads).
 * Arguments:
 *   q            device [batch][n_q_heads][128] of q_dtype (F32 or BF16), 16-byte
 *                aligned (rows are read with 16-byte loads)
 *   pool         device pool written by tq_compress_kv
 *   block_table  device int32 [batch][max_blocks_per_seq]: logical block j of
 *                sequence b -> physical block id in [0, num_blocks)
 *   seq_lens     device int32 [batch], 0 <= seq_lens[b] <= min(max_seq_len,
 *                16*max_blocks_per_seq); 0 gives a zero output row
 *   max_seq_len  host bound on seq_lens, used to plan the split-K grid
 *   softmax_scale  0 selects 1/sqrt(128)
 *   num_splits   0 = automatic (from max_seq_len, batch, heads and the CU count);
 *                otherwise the number of context splits per sequence, raised
 *                where needed so that no split spans more than 4096 tokens.
 *                The environment variable TQ_DECODE_SPLITS overrides 0.
 *                The split-K grid is batch x n_kv_heads x splits workgroups;
 *                when it is more than one round of resident workgroups, they
 *                take the live (sequence, split, head) items as a work list
 *                built on the device from seq_lens (whole splits first, heads
 *                spread over the XCDs), so that ragged batches keep every XCD
 *                busy.  TQ_DECODE_WORK_LIST=0 or 1 forces the plain item order
 *                or the work list (the output is the same bit for bit).
 *   out          device [batch][n_q_heads][128] of out_dtype (F32 or BF16, RNE)
 *   workspace    device scratch of at least tq_decode_workspace_size() bytes,
 *                256-byte aligned; contents need not be initialised
 * Three launches on hip_stream: query prologue, split-K mainloop, combine +
 * un-rotation epilogue. */
tq_status tq_decode_attn(const tq_layer* layer, const void* q, tq_dtype q_dtype, int batch,
                         int n_q_heads, const void* pool, long long num_blocks,
                         const int* block_table, int max_blocks_per_seq, const int* seq_lens,
                         int max_seq_len, float softmax_scale, int num_splits, void* out,
                         tq_dtype out_dtype, void* workspace, size_t workspace_bytes,
                         void* hip_stream);

/* tq_decode_attn without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, kernels and result as tq_decode_attn;
 * the workspace is instead a fixed 16 MiB array in device memory, one per GPU
 * the library runs on, held until the process ends.  It allocates nothing and
 * synchronises nothing (the first call on a device looks up that device's array
 * address once).  Returns TQ_ERR_UNSUPPORTED, before any launch, when the shape
 * needs a larger workspace than 16 MiB (tq_decode_workspace_size tells; e.g.
 * batch 64 x 32 query heads x 8 splits needs 8.9 MB).  All calls on one GPU share
 * its array: calls that overlap on one GPU (different streams) race, so they
 * must be ordered by the caller.  TQ_DEBUG_CHECKS is not honoured here (it
 * would allocate host memory). */
tq_status tq_decode_attn_noalloc(const tq_layer* layer, const void* q, tq_dtype q_dtype, int batch,
                                 int n_q_heads, const void* pool, long long num_blocks,
                                 const int* block_table, int max_blocks_per_seq, const int* seq_lens,
                                 int max_seq_len, float softmax_scale, int num_splits, void* out,
                                 tq_dtype out_dtype, void* hip_stream);

/* Kernel timing, a profiling aid (off by default).
 * Kernel ids: 0 = compress, 1 = decode prologue, 2 = decode split-K mainloop,
 * 3 = decode combine/epilogue.
 * tq_profile_enable(mask): while bit i of mask is set, every launch of kernel i
 *   is bracketed by two HIP events recorded on the caller's stream (mask 0 turns
 *   timing off).  Not thread-safe; meant for benchmarks.
 * tq_profile_read(kernel, total_ms, launches): waits for the recorded events and
 *   returns the summed kernel time (host out, milliseconds) and the number of
 *   timed launches (host out) since the last reset.
 * tq_profile_reset(): forgets all records (events are recycled, not freed). */
tq_status tq_profile_enable(unsigned mask);
tq_status tq_profile_read(int kernel, double* total_ms, long long* launches);
tq_status tq_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
