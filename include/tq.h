/*
 * tq.h — C ABI of the TurboQuant hot path on AMD Instinct MI355X (gfx950).
 *
 * TurboQuant compresses each key/value vector of an LLM KV cache online:
 * keep its norm, rotate it by a fixed random orthogonal matrix, quantize every
 * rotated coordinate to the nearest of 2^b Lloyd-Max centroids and store the
 * index; the inner-product ("prod") variant spends one of the b bits on a
 * 1-bit QJL sketch of the residual. Decode attention scores a full-precision
 * query against the packed keys, applies softmax and averages the packed
 * values.
 *
 * Pages that define the operations (cited by title and section):
 *   [DG]  "The Distortion Guarantee — How Good Is This?" (igniting.github.io
 *         turboquant slides, section 9)
 *   [B31] "I Spent 31 Hours On The Math Behind Turboquant So You Dont Have To"
 *         (onlylabs.fyi, Baseten)
 *   [OM]  "TurboQuant của Google: nén KV cache 6 lần, hay một paper cũ 9 tháng
 *         được PR lại?" (omelet.tech)
 *   [WY]  "内存厂商的噩梦来了：谷歌一篇论文如何让 KV Cache 内存占用缩小六倍"
 *         (wuyi.wiki)
 *
 * Conventions for every entry point:
 *   - All functions are extern "C" and return an int status: 0 (TQ_OK) or a
 *     negative tq_status. No C++ exception crosses the ABI.
 *   - Argument checks are synchronous: on any error nothing is launched and
 *     no output is written.
 *   - Pointers named "device" must point to HIP device memory (or memory the
 *     GPU can address); "host" pointers to host memory. The caller owns every
 *     buffer; the library never allocates or frees memory and keeps no global
 *     mutable state (apart from the fixed scratch of tq_attn_decode_noalloc
 *     and its per-device address), so calls on different streams may run
 *     concurrently as long as they do not write the same buffers.
 *   - `stream` is a hipStream_t (NULL = the default stream). Launches are
 *     asynchronous on it; a launch failure returns TQ_ERR_HIP, and faults
 *     during execution surface at the caller's next synchronization.
 *   - Head dimension d must be 128 for the GPU entry points.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum tq_status {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1,  /* null pointer, bad size, inconsistent shapes        */
  TQ_ERR_UNSUPPORTED = -2,  /* d != 128, bits outside 1..4, unknown variant/dtype  */
  TQ_ERR_HIP = -3,          /* a HIP launch or runtime call failed                */
  TQ_ERR_WORKSPACE = -4,    /* workspace / prepared buffer too small or misaligned */
  TQ_ERR_NO_CONVERGE = -5   /* Lloyd-Max iteration did not converge               */
};

enum tq_variant { TQ_MSE = 0, TQ_PROD = 1 };
enum tq_rotation { TQ_ROT_DENSE = 0, TQ_ROT_HADAMARD = 1 };
enum tq_split { TQ_SPLIT_NONE = 0, TQ_SPLIT_OUTLIER32 = 1 };
enum tq_dtype { TQ_F32 = 0, TQ_BF16 = 1 };

/* Head dimension supported by the GPU kernels. */
#define TQ_HEAD_DIM 128

/*
 * tq_codebook — Lloyd-Max scalar quantizer for one rotated coordinate (host).
 *
 * Defined by [OM] section "Lloyd-Max quantizer: chia bucket đúng chỗ",
 * eq. C(f,b): 2^bits centroids minimising Σ_i ∫_{cell i} (x - c_i)² f(x) dx,
 * for the density of one coordinate of a uniformly random unit vector in R^d,
 * f(x) = C (1-x²)^((d-3)/2) on [-1,1] ([OM] section "Trick đầu tiên: xoay
 * ngẫu nhiên trước khi nén", eq. f(x)).
 *
 *   d          dimension, 2 <= d <= 65536 (any d; the GPU kernels need 128)
 *   bits       0..8 (0 gives the single centroid 0, used by prod at b = 1)
 *   centroids  host out, double[2^bits], ascending, exactly antisymmetric
 *              (c[K-1-i] == -c[i])
 *   boundaries host out, double[2^bits - 1] (may be NULL when bits == 0),
 *              boundaries[i] = (c[i] + c[i+1]) / 2; the middle one is 0.0
 *   mse_unit   host out or NULL: d × the per-coordinate distortion, i.e. the
 *              expected ‖u - ũ‖² of a unit vector ([DG] "The Upper Bound")
 * Errors: TQ_ERR_INVALID_ARG (null outputs, d < 2), TQ_ERR_UNSUPPORTED
 * (bits > 8 or d > 65536), TQ_ERR_NO_CONVERGE.
 */
int tq_codebook(int d, int bits, double* centroids, double* boundaries, double* mse_unit);

/*
 * One quantizer instance (one per role: keys or values of a layer).
 * Every pointer is device memory owned by the caller; the library reads them.
 *   d          128
 *   bits       total bits per coordinate, 1..4
 *   variant    TQ_MSE: bits-bit Lloyd-Max codes
 *              TQ_PROD: (bits-1)-bit Lloyd-Max codes + 1-bit QJL sketch of
 *              the residual ([OM] QJL section; [WY] section 4.3)
 *   rot        float[d][d] row-major, the orthogonal Π; the rotated vector is
 *              y = Π·u ([OM] "Trick đầu tiên…")
 *   proj       float[d][d] row-major Gaussian S of the QJL sketch (PROD), else NULL
 *   centroids  float[2^bm] from tq_codebook(d, bm) rounded to float, bm = bits
 *              (MSE) or bits-1 (PROD); must be antisymmetric like the output
 *              of tq_codebook
 *   boundaries float[2^bm - 1], the midpoints (NULL allowed when bm == 0)
 *   prep       device buffer of tq_prep_bytes() bytes, 256-byte aligned,
 *              filled by tq_prepare() from the fields above before the
 *              quantizer is used by tq_encode / tq_attn_decode
 *   rotation   TQ_ROT_DENSE (0): rot is any orthogonal matrix (the Haar-random
 *              Π of [OM] "Trick đầu tiên…"); its fp16 hi/lo split enters the
 *              matrix cores.
 *              TQ_ROT_HADAMARD (1): rot is the randomized Walsh–Hadamard
 *              rotation Π = H·diag(s)/√d (H the Sylvester Hadamard matrix,
 *              s ∈ {±1}^d), the faster matrix alternative (WHT) that [WY]
 *              section 4.3 names after its code listing. Only the signs of rot's
 *              entries enter the matrix cores (H·diag(s), exact in fp16) and
 *              1/√d is applied in fp32; rot itself must hold that matrix
 *              (the decode merge reads it as given).
 *   split      TQ_SPLIT_NONE (0), or TQ_SPLIT_OUTLIER32 (1): the outlier-channel
 *              split of [OM] section "Thực nghiệm: 3.5 bit…" — 32 outlier
 *              channels at bits+1 bits and the other 96 at `bits` bits, as two
 *              independent TurboQuant instances (own norm, rotation and
 *              codebook each). Requires bits 2 or 3 ("2.5-bit" and
 *              "3.5-bit") and rotation TQ_ROT_DENSE. With TQ_MSE both groups
 *              are mse instances (Lloyd-Max widths bm + 1 and bm, bm = bits);
 *              with TQ_PROD both are prod instances (the outlier group at
 *              bits+1: `bits` of Lloyd-Max plus a 1-bit sketch with its own
 *              32×32 S_o; the regular group at bits: bits-1 of Lloyd-Max plus
 *              a sketch with a 96×96 S_r; own γ each), bm = bits - 1. Then:
 *                rot        unused (NULL allowed)
 *                rot_o      device float[32][32] row-major, the outlier
 *                           group's orthogonal Π_o
 *                rot_r      device float[96][96] row-major, the regular
 *                           group's orthogonal Π_r
 *                channels_o host int32[32]: the outlier channels, distinct,
 *                           in [0, 128), in the order of Π_o's columns; the
 *                           regular channels are the other 96 in increasing
 *                           order, the order of Π_r's columns. Read (and
 *                           checked) by tq_prepare only.
 *                proj       unused (NULL allowed)
 *                proj_o, proj_r  TQ_PROD: device float[32][32] and
 *                           float[96][96] row-major, the groups' Gaussian
 *                           sketch matrices S_o and S_r (NULL for TQ_MSE)
 *                centroids  the regular group's codebook, tq_codebook(96, bm)
 *                boundaries its midpoints
 *                centroids_o, boundaries_o  the outlier group's codebook,
 *                           tq_codebook(32, bm+1), float[2^(bm+1)] and
 *                           float[2^(bm+1) - 1]
 *              tq_prepare combines Π_o, Π_r, S_o, S_r and the channel list
 *              into the library's own operands in `prep`; afterwards only
 *              `prep` and the codebooks are read.
 *              Unsplit quantizers leave centroids_o, boundaries_o, rot_o,
 *              rot_r, channels_o, proj_o and proj_r NULL.
 */
typedef struct tq_quantizer {
  int d;
  int bits;
  int variant;
  const float* rot;
  const float* proj;
  const float* centroids;
  const float* boundaries;
  void* prep;
  int rotation;
  int split;
  const float* centroids_o;
  const float* boundaries_o;
  const float* rot_o;
  const float* rot_r;
  const int32_t* channels_o;
  const float* proj_o;
  const float* proj_r;
} tq_quantizer;

/*
 * Packed vectors, vector-major; caller-owned device memory.
 *   codes   uint8[n][d*bm/8]: code j of a vector occupies bits [j·bm, j·bm+bm)
 *           of that vector's byte string, least significant bit first (byte k
 *           holds stream bits 8k..8k+7); every 32 codes fill bm whole 32-bit
 *           words. NULL allowed when bm == 0.
 *   norms   float[n], ‖x‖ kept unquantized (the qwik-news HN thread: one
 *           scalar per vector, stored as is)
 *   qjl     uint8[n][d/8] (PROD, else NULL): bit j = 1 iff (S·r)_j >= 0, same
 *           LSB-first order
 *   gammas  float[n] (PROD, else NULL): ‖r‖, the residual norm the QJL
 *           estimator scales by
 * Split quantizers (TQ_SPLIT_OUTLIER32, b = bm: bits for TQ_MSE, bits-1 for
 * TQ_PROD):
 *   codes   uint8[n][16·b + 4]: the 128 codes in position order, position p
 *           with width b+1 when p mod 8 < 2 (outlier coordinate k sits at the
 *           k-th such position) and b otherwise (regular coordinate k at the
 *           k-th other position), one after another, each least significant
 *           bit first; every 8 positions take 8b + 2 bits
 *   norms   float[n][2]: ‖x_o‖ and ‖x_r‖ of the outlier and regular channels
 *   qjl     TQ_PROD: uint8[n][16], bit p the sign bit of the sketch value at
 *           position p (outlier sketch coordinate k at the k-th position with
 *           p mod 8 < 2, regular k at the k-th other one)
 *   gammas  TQ_PROD: float[n][2], γ_o and γ_r
 * Buffers must be 16-byte aligned.
 */
typedef struct tq_packed {
  uint8_t* codes;
  float* norms;
  uint8_t* qjl;
  float* gammas;
} tq_packed;

/* Size in bytes of the prepared-operand buffer of one quantizer. */
size_t tq_prep_bytes(void);

/*
 * tq_prepare — derive the GPU operands of a quantizer into q->prep.
 * Splits Π (and S·Πᵀ for PROD) into the matrix-core operand layout the
 * encoder uses; for a split quantizer it first assembles Π from Π_o, Π_r and
 * the outlier channels. Run once per quantizer (after its rot/proj/centroids
 * are written), on `stream`; later calls on the same stream see the result.
 * Errors: TQ_ERR_INVALID_ARG (null q/fields, prep misaligned, outlier
 * channels not 32 distinct values in [0, 128)), TQ_ERR_UNSUPPORTED (d, bits,
 * variant, rotation), TQ_ERR_HIP.
 */
int tq_prepare(const tq_quantizer* q, void* stream);

/*
 * tq_encode — TurboQuant encode of n vectors ([DG] "rotate, quantize, done";
 * [OM] sections "Trick đầu tiên…" and "Lloyd-Max quantizer…" for MSE; [OM]
 * QJL section and [WY] section 4.3 for PROD).
 *   norm n = ‖x‖; u = x/n (u = 0 when n = 0); y = Π·u;
 *   idx_j = #{i : boundaries[i] < y_j} (the nearest centroid, ties to the
 *   lower index); PROD adds r = u - Πᵀc[idx], γ = ‖r‖, bits sign(S·r).
 *   q         prepared quantizer
 *   x         device, n rows of d values, dtype x_dtype (TQ_F32 or TQ_BF16),
 *             row i at x + i*x_row_stride elements; rows 16-byte aligned
 *   n         number of vectors, >= 0 (0 is a no-op)
 *   x_row_stride  elements between rows, >= d, multiple of 8
 *   out       device outputs (see tq_packed)
 *   out_slot  device int64[n] or NULL: row i is stored at slot out_slot[i] of
 *             `out` (NULL: at slot i). This appends new tokens into a cache
 *             laid out as in tq_attn_decode. Slots must be >= 0, inside the
 *             caller's buffers and distinct; they are not checked.
 * Rows must hold finite values: the outputs of a row with a NaN or an
 * infinity are unspecified (and may differ between calls of different n).
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP.
 */
int tq_encode(const tq_quantizer* q, const void* x, int x_dtype, int64_t n,
              int64_t x_row_stride, const tq_packed* out, const int64_t* out_slot,
              void* stream);

/*
 * tq_attn_decode_workspace — bytes of device workspace tq_attn_decode needs
 * for this shape (a pure function of its arguments). Returns 0 for invalid
 * shapes.
 */
size_t tq_attn_decode_workspace(int B, int Hq, int Hkv, int64_t max_ctx);

/*
 * tq_attn_decode — one decode step of attention over a packed KV cache.
 * For every batch b and query head h, with KV head kv = h / (Hq/Hkv):
 *   out[b][h] = Σ_t softmax_t(scale·⟨q[b][h], k̃_t⟩) · ṽ_t
 * over t < ctx_lens[b] ([B31] section "KV Cache: The problem":
 * softmax(Q·Kᵀ/√d)·V; the query stays full precision, the "asymmetric
 * estimator" of [WY] section 4.2), where k̃, ṽ are the dequantized vectors:
 *   MSE:  x̃ = n Πᵀ c[idx]
 *   PROD: x̃ = n (Πᵀ c[idx] + √(π/2)/d · γ · Sᵀ s),  s_j = ±1 from the sketch.
 *   kq, vq     prepared quantizers of keys and values (vq must be TQ_MSE)
 *   query      device float[B][Hq][d]
 *   ctx_lens   device int32[B] or NULL (all max_ctx); values are clamped to
 *              [0, max_ctx]; a batch with length 0 gets an all-zero output
 *   max_ctx    tokens allocated per (b, kv head), >= 1
 *   k_cache, v_cache  packed caches: vector index ((b*Hkv + kv)*max_ctx + t)
 *   scale      softmax scale, usually 1/√d
 *   out        device float[B][Hq][d]
 *   workspace  device, >= tq_attn_decode_workspace(B, Hq, Hkv, max_ctx)
 *              bytes, 256-byte aligned; contents need not be initialised
 * Errors: TQ_ERR_INVALID_ARG (null pointers, B/Hq/Hkv < 1, Hq % Hkv != 0,
 * max_ctx < 1), TQ_ERR_UNSUPPORTED (d, bits, value quantizer not MSE),
 * TQ_ERR_WORKSPACE, TQ_ERR_HIP.
 */
int tq_attn_decode(const tq_quantizer* kq, const tq_quantizer* vq, const float* query,
                   int B, int Hq, int Hkv, const int32_t* ctx_lens, int64_t max_ctx,
                   const tq_packed* k_cache, const tq_packed* v_cache, float scale,
                   float* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * tq_attn_decode_phase — one of the three launches tq_attn_decode makes, for
 * callers that schedule or time them separately (same arguments, same checks):
 *   phase 1: query operands (Π_K·q and S·q per query head) into the workspace
 *   phase 2: split attention over the packed cache → per-split partials
 *   phase 3: combine the splits and rotate back into `out`
 * Running phases 1, 2, 3 in order on one stream equals tq_attn_decode. Phase
 * 2 reads what phase 1 wrote and phase 3 what phase 2 wrote, in `workspace`.
 * Errors: as tq_attn_decode, plus TQ_ERR_INVALID_ARG for another phase value.
 */
int tq_attn_decode_phase(int phase, const tq_quantizer* kq, const tq_quantizer* vq,
                         const float* query, int B, int Hq, int Hkv, const int32_t* ctx_lens,
                         int64_t max_ctx, const tq_packed* k_cache, const tq_packed* v_cache,
                         float scale, float* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * tq_decode_step — one online decode step: append the new key and value of
 * every (batch, KV head) to the packed caches, then decode attention over
 * the caches including them. Each token is compressed as it arrives and
 * attention reads the compressed cache ([WY] section 5, KV-cache
 * compression online; [B31] section "KV Cache: The problem").
 *   k_new, v_new  device rows of d values, dtype x_dtype (TQ_F32 or
 *                 TQ_BF16): row b*Hkv + kv (kv < Hkv) at x_row_stride*row
 *                 elements, 16-byte aligned; x_row_stride >= d, multiple of 8
 *   ctx_lens      device int32[B] or NULL (all max_ctx): the lengths AFTER
 *                 the append. The new rows of batch b are encoded exactly as
 *                 tq_encode encodes them and written to token slot
 *                 ctx_lens[b] - 1; a batch whose length is outside
 *                 [1, max_ctx] gets no write.
 *   other arguments as tq_attn_decode (same workspace size).
 * The result equals tq_encode of the new rows into those slots followed by
 * tq_attn_decode, bit for bit, for rows of finite values; the appends and the query operands share one
 * launch, so the step takes three launches instead of five. With split
 * quantizers (TQ_SPLIT_OUTLIER32, both) the appends run the split encoder,
 * and the query operands and the two appends are three launches of phase 1.
 * Errors: as tq_attn_decode and tq_encode (TQ_ERR_INVALID_ARG for null or
 * misaligned rows or a bad stride, TQ_ERR_UNSUPPORTED for another dtype).
 */
int tq_decode_step(const tq_quantizer* kq, const tq_quantizer* vq, const void* k_new,
                   const void* v_new, int x_dtype, int64_t x_row_stride, const float* query,
                   int B, int Hq, int Hkv, const int32_t* ctx_lens, int64_t max_ctx,
                   const tq_packed* k_cache, const tq_packed* v_cache, float scale, float* out,
                   void* workspace, size_t ws_bytes, void* stream);

/*
 * tq_decode_step_phase — one of tq_decode_step's three launches (same
 * arguments and checks): phase 1 appends the new rows and forms the query
 * operands, phases 2 and 3 are those of tq_attn_decode_phase. Running 1, 2, 3
 * in order on one stream equals tq_decode_step.
 * Errors: as tq_decode_step, plus TQ_ERR_INVALID_ARG for another phase value.
 */
int tq_decode_step_phase(int phase, const tq_quantizer* kq, const tq_quantizer* vq,
                         const void* k_new, const void* v_new, int x_dtype, int64_t x_row_stride,
                         const float* query, int B, int Hq, int Hkv, const int32_t* ctx_lens,
                         int64_t max_ctx, const tq_packed* k_cache, const tq_packed* v_cache,
                         float scale, float* out, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of the fixed device scratch tq_attn_decode_noalloc uses as its
 * workspace (16 MiB: enough for tq_attn_decode_workspace() of batch 64 x 8 KV
 * heads x 32 query heads at 16K tokens, or batch 4 x 8 x 64 at 128K). */
#define TQ_STATIC_SCRATCH_BYTES (16u << 20)

/*
 * tq_attn_decode_noalloc — tq_attn_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the same arguments without the workspace, the
 * same kernels and the same result bit for bit. Its workspace is a fixed
 * array of TQ_STATIC_SCRATCH_BYTES in the library's code object; each GPU
 * the library runs on holds its own copy until the process ends (its device
 * address is looked up on the first call on that GPU). The call allocates
 * nothing and frees nothing. Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (on different streams, or from different
 * host threads onto streams that are not ordered) race and give undefined
 * results; calls on one stream are ordered and safe. The array keeps the
 * last call's contents; nothing in it needs to start at zero.
 * Errors: as tq_attn_decode; TQ_ERR_WORKSPACE when the shape needs more
 * than TQ_STATIC_SCRATCH_BYTES (tq_attn_decode_workspace(B, Hq, Hkv,
 * max_ctx) > TQ_STATIC_SCRATCH_BYTES); TQ_ERR_HIP when no device is current
 * or the array's address cannot be found; TQ_ERR_UNSUPPORTED on a device
 * index of 64 or more.
 */
int tq_attn_decode_noalloc(const tq_quantizer* kq, const tq_quantizer* vq, const float* query,
                           int B, int Hq, int Hkv, const int32_t* ctx_lens, int64_t max_ctx,
                           const tq_packed* k_cache, const tq_packed* v_cache, float scale,
                           float* out, void* stream);

/*
 * tq_search_workspace — bytes of device workspace tq_search needs for these
 * sizes (a pure function of its arguments); 0 for invalid sizes.
 */
size_t tq_search_workspace(int nq, int64_t n, int k);

/*
 * tq_search — inner-product top-k over a packed database ([WY] section 6.4:
 * nearest-neighbour search by inner product over TurboQuant-encoded vectors,
 * scored by recall 1@k). For each query q_i, the k database vectors x_j
 * (j < n) with the largest estimated inner product ⟨q_i, x̃_j⟩, x̃ the
 * dequantized vector of tq_attn_decode's formulas (PROD: the unbiased
 * estimator), best first; equal scores are ordered by the lower index.
 *   q          prepared quantizer of the database (either variant, 1..4 bits)
 *   query      device float[nq][d], 16-byte aligned
 *   nq         number of queries, >= 1
 *   db         packed database, vector j in slot j (see tq_packed)
 *   n          database size, 1 <= n <= 2^26
 *   k          1 <= k <= min(32, n)
 *   scores     device float[nq][k]: the estimated inner products
 *   index      device int64[nq][k]: the vectors' slots
 *   workspace  device, >= tq_search_workspace(nq, n, k) bytes, 256-byte
 *              aligned; contents need not be initialised
 * Three launches on `stream`: the query operands, the scan (each workgroup
 * keeps its best k per query), and the merge over workgroups.
 * Errors: TQ_ERR_INVALID_ARG (null or misaligned pointers, nq < 1, k < 1,
 * k > n), TQ_ERR_UNSUPPORTED (k > 32, n > 2^26, d, bits, variant),
 * TQ_ERR_WORKSPACE, TQ_ERR_HIP.
 */
int tq_search(const tq_quantizer* q, const float* query, int nq, const tq_packed* db, int64_t n, int k,
              float* scores, int64_t* index, void* workspace, size_t ws_bytes, void* stream);

/*
 * Vectors longer than d = 128 (chunked search)
 * [WY] section 6.4 searches vectors of 200 (GloVe) and 1536 coordinates. A
 * vector of D coordinates is read here as C = ceil(D/128) chunks of 128
 * (coordinates D..128C-1 are zero), each chunk quantized on its own by the
 * same 128-coordinate quantizer (its own norm, and for PROD its own sketch and
 * γ). The estimated inner product of a query with a vector is the sum of the
 * chunks' estimates, Σ_c ⟨q_c, x̃_c⟩; zero padding leaves every exact inner
 * product unchanged. Packed chunked vectors are chunk-major: chunk c of
 * vector v is in slot c·n + v of the tq_packed buffers (n vectors), so that
 * every chunk's vectors form one ordinary packed database.
 */

/*
 * tq_encode_chunked — encode n vectors of `chunks` chunks each.
 *   x         device, row i (vector i) at x + i*x_row_stride elements, holding
 *             chunks·128 values (zero beyond the vector's own length); rows
 *             16-byte aligned; dtype TQ_F32 or TQ_BF16
 *   chunks    1 <= chunks <= 64
 *   x_row_stride  >= chunks·128, multiple of 8
 *   out       chunk-major packed output with room for chunks·n slots
 * One encoder launch per chunk on `stream`; same per-row definition and
 * errors as tq_encode.
 */
int tq_encode_chunked(const tq_quantizer* q, const void* x, int x_dtype, int64_t n, int chunks,
                      int64_t x_row_stride, const tq_packed* out, void* stream);

/*
 * tq_search_chunked_workspace — bytes of device workspace tq_search_chunked
 * needs (a pure function of its arguments); 0 for invalid sizes. For
 * chunks > 1 it includes a float buffer of 8·ceil(nq/8)·n running scores.
 */
size_t tq_search_chunked_workspace(int nq, int64_t n, int k, int chunks);

/*
 * tq_search_chunked — tq_search over chunked vectors: for each query q_i
 * (device float[nq][chunks·128], zero beyond the vectors' length, 16-byte
 * aligned), the k vectors with the largest Σ_c ⟨q_{i,c}, x̃_{j,c}⟩, best first,
 * equal scores ordered by the lower index. db is chunk-major (see above);
 * 1 <= chunks <= 64; the other arguments as in tq_search. Launches on
 * `stream`: per chunk, the query operands and a scan (chunks before the last
 * store running scores in the workspace, the last adds them and keeps
 * candidates), then the merge. chunks = 1 is tq_search.
 * Errors: as tq_search; chunks < 1 is TQ_ERR_INVALID_ARG, chunks > 64
 * TQ_ERR_UNSUPPORTED.
 */
int tq_search_chunked(const tq_quantizer* q, const float* query, int nq, int chunks, const tq_packed* db,
                      int64_t n, int k, float* scores, int64_t* index, void* workspace, size_t ws_bytes,
                      void* stream);

/*
 * tq_read_probe — a measurement aid, not a step of the codec: one plain
 * coalesced read of `bytes` of device memory with the 16-byte non-temporal
 * loads the decode kernels stream the packed cache with. Timed on a buffer
 * far larger than the last-level cache, its rate is the part's practical
 * read ceiling, beside which the decode rate is reported.
 *   buf      device, 16-byte aligned, read only
 *   bytes    > 0, a multiple of 16
 *   xor_out  device uint32: the XOR of the buffer's little-endian 32-bit
 *            words is XORed into it (set it to 0 first to read the XOR)
 * One launch on `stream`. Errors: TQ_ERR_INVALID_ARG (null or misaligned
 * pointers, bytes 0 or not a multiple of 16), TQ_ERR_HIP.
 */
int tq_read_probe(const void* buf, size_t bytes, uint32_t* xor_out, void* stream);

/* Human-readable text of a status code (static storage). */
const char* tq_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H_ */
