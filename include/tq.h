/*
 * tq.h -- C ABI of the TurboQuant-style online vector quantizer for AMD MI355X (gfx950).
 *
 * The method (TurboQuant technical overview, intelliparadigm.com; TurboQuant
 * deep dive, blog.hotdry.top): every vector is split into its L2 norm and a
 * unit direction; the direction is rotated by a seeded randomized Hadamard
 * transform (three rounds of a +-1 diagonal followed by a normalized
 * Walsh-Hadamard transform); every rotated coordinate is quantized with a
 * (b-1)-bit Lloyd-Max codebook solved for the Beta((D-1)/2, (D-1)/2) law of a
 * rotated coordinate; the residual gets a 1-bit QJL sign sketch under a
 * seeded Gaussian matrix.  A full-precision query is rotated the same way and
 * scored against the packed codes with an unbiased inner-product estimate.
 * Around that path: top-k selection (fused with scoring or on a score
 * matrix), the exact re-rank of a candidate set, TurboQuant-MSE plans (their
 * records dequantized, or scored by the quantized distance n <Pi y, c[idx]>),
 * decode attention over quantized values, and the KV-cache
 * policy layer (outlier channels by variance, appending one record per head).
 *
 * Conventions for every call:
 *   - Status is returned, never thrown; nothing aborts or prints.
 *   - "device" pointers are HIP device memory of the current device; "host"
 *     pointers are ordinary CPU memory.  The caller owns every buffer it passes.
 *   - `stream` is a hipStream_t (NULL = the default stream).  tq_encode,
 *     tq_encode_scatter, tq_score, tq_score_topk, tq_topk, tq_dequantize,
 *     tq_attend, tq_rerank, tq_calibrate_outliers and tq_qjl only enqueue work
 *     on it and return; their outputs are valid once the stream reaches that
 *     point.  A launch failure is reported as TQ_EDEVICE.
 *   - A plan is immutable after creation and may be used from several streams
 *     and threads at once.  Destroying a plan while work that uses it is still
 *     queued is undefined.
 *   - Workspaces: tq_score, tq_score_topk and tq_attend take their short-lived
 *     workspace (at most 256 MiB; larger ones are allocated per call) from a
 *     buffer kept per (device, stream), which the next such call on the same
 *     stream reuses: the stream orders the two calls' kernels, so no call
 *     allocates once the buffer is large enough.  The buffer grows by a
 *     stream-ordered free and allocation (hipFreeAsync / hipMallocAsync) and
 *     is held until the process ends.  A stream that is being captured into a
 *     graph gets a per-call allocation instead.  A stream handle that is
 *     destroyed while such a call's work is still queued must not be reused for
 *     a new stream until that work has finished.
 *
 * Code layout (the "record" of one vector; little-endian 32-bit words):
 *   For a sub-plan with rotated length D (a power of two, 32..2048) and R
 *   index bits, the record is, for each chunk g = 0 .. D/32-1:
 *       R words: bit t of word m = bit m of the index of coordinate 32g+t
 *       1 word:  bit t = QJL sign bit of projection row 32g+t (1 = non-negative)
 *   followed by float32 norm ||x|| and float32 residual norm gamma.
 *   Size: 4*(R+1)*D/32 + 8 bytes.  With an outlier mask the record of a vector
 *   is the regular sub-plan's record followed by the outlier sub-plan's
 *   record.  Records of consecutive vectors are contiguous.
 *   A TurboQuant-MSE plan (tq_plan_create_mse: all b bits on the Lloyd-Max
 *   codebook, R = b, no QJL stage) stores per chunk only the R index words,
 *   then float32 norm: 4*R*D/32 + 4 bytes.
 */
#ifndef TQ_H
#define TQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tq_status {
  TQ_OK = 0,
  TQ_EINVAL = -1,       /* invalid argument (null, size, alignment, range) */
  TQ_ENOMEM = -2,       /* host or device allocation failed */
  TQ_EDEVICE = -3,      /* no usable HIP device, or a HIP call/launch failed */
  TQ_EUNSUPPORTED = -4  /* valid request this build does not implement */
} tq_status;

typedef enum tq_dtype { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

typedef struct tq_plan tq_plan;

typedef enum tq_mode { TQ_MODE_INNER_PRODUCT = 0, TQ_MODE_MSE = 1 } tq_mode;

typedef struct tq_subplan_desc {
  int32_t d;              /* input channels of this sub-plan */
  int32_t D;              /* rotated length: max(32, next power of two >= d) */
  int32_t R;              /* index bits per coordinate (b - 1; b for an MSE plan) */
  int32_t k;              /* QJL rows (= D: one sign bit per rotated coordinate; 0 for MSE) */
  int32_t record_offset;  /* byte offset of this sub-plan's record in a vector's record */
  int32_t record_bytes;   /* 4*(R+1)*D/32 + 8 (MSE: 4*R*D/32 + 4) */
} tq_subplan_desc;

typedef struct tq_plan_desc {
  int32_t d;              /* channels of an input vector */
  int32_t n_subplans;     /* 1, or 2 with an outlier mask (0 = regular, 1 = outlier) */
  int32_t record_bytes;   /* bytes per encoded vector */
  int32_t mode;           /* tq_mode */
  int32_t n_heads;        /* channel lists per sub-plan: 1, or the heads of a layer plan */
  tq_subplan_desc sub[2];
} tq_plan_desc;

/* Human-readable name of a status code (static string). */
const char* tq_status_string(tq_status status);

/*
 * Create a plan: solve the Lloyd-Max codebook(s) on the host, draw the
 * rotation signs and the QJL matrix from `seed`, and upload them to the
 * current device.
 *   d            input dimension, 1 <= d <= 2048
 *   bits         b, total bits per coordinate for the regular channels, 2..5
 *                (b-1 Lloyd-Max bits + 1 QJL bit; TurboQuant overview §1.2.3)
 *   seed         64-bit seed of all plan randomness (overview §2.1.2)
 *   outlier_mask host array of d bytes (nonzero = outlier channel) or NULL;
 *                copied.  Outlier channels form a second, independent
 *                sub-plan with its own rotation and QJL matrix (overview
 *                §4.1.1 outlier channels); the mask must select 1..d-1 channels.
 *   outlier_bits b of the outlier sub-plan, 2..5 (ignored when the mask is NULL)
 *   out          receives the plan
 * Errors: TQ_EINVAL (range, null `out`), TQ_ENOMEM, TQ_EDEVICE (no device,
 * upload failure).  On error *out is set to NULL.
 */
tq_status tq_plan_create(int d, int bits, uint64_t seed, const uint8_t* outlier_mask,
                         int outlier_bits, tq_plan** out);

/*
 * Layer plan for the key cache of several heads (overview §4.1.1: analyse the
 * heads, keep about a quarter of each head's channels as outliers at a higher
 * bit-width).  Every head shares the plan's codebooks, rotations and QJL
 * matrices (the split plan of tq_plan_create with the same d, bits, seed and
 * outlier_bits), but gathers its regular and outlier channels by its own mask,
 * so one launch serves all heads of a layer.  Group g of tq_encode_groups,
 * tq_score, tq_score_noalloc and tq_score_topk uses head g % n_heads (e.g.
 * groups ordered [sequence][head]); vector i of tq_encode_scatter uses head
 * i % n_heads.  The result for head h equals what a plan made by
 * tq_plan_create(d, bits, seed, outlier_masks + h*d, outlier_bits) gives.
 *   outlier_masks  host [n_heads][d] bytes (nonzero = outlier), copied; every
 *                  head selects the same number of channels, 1..d-1
 *   2 <= d <= 128, 1 <= n_heads <= 1024, bits and outlier_bits 2..5.
 * tq_encode (use tq_encode_groups), tq_dequantize, tq_attend and tq_qjl do not
 * take layer plans (TQ_EINVAL / TQ_EUNSUPPORTED).
 * Errors: TQ_EINVAL (range, null, unequal outlier counts), TQ_ENOMEM, TQ_EDEVICE.
 */
tq_status tq_plan_create_heads(int d, int bits, uint64_t seed, int n_heads,
                               const uint8_t* outlier_masks, int outlier_bits, tq_plan** out);

/*
 * Create a TurboQuant-MSE plan (overview §1.2.1-1.2.2: rotation and a Lloyd-Max
 * quantizer on every coordinate; §4.1.1 recommends 3-bit MSE for most
 * attention heads, §4.2.1 MSE codes with the norm kept for the vectors of an
 * index): all b bits go to the codebook and there is no QJL matrix.  The
 * rotation is the one an inner-product plan with the same seed uses.
 *   d     input dimension, 1 <= d <= 2048
 *   bits  b = R, 1..4
 * tq_encode writes its records (layout above) and tq_dequantize reconstructs
 * them; tq_score, tq_score_noalloc and tq_score_topk score them (n <Pi y,
 * c[idx]>, see tq_score); tq_qjl returns TQ_EUNSUPPORTED for it.
 * Errors: TQ_EINVAL, TQ_ENOMEM, TQ_EDEVICE.  On error *out is set to NULL.
 */
tq_status tq_plan_create_mse(int d, int bits, uint64_t seed, tq_plan** out);

/* Release a plan's host and device tables.  NULL is accepted. */
void tq_plan_destroy(tq_plan* plan);

/* Describe a plan (sizes and record layout) into *desc (host memory). */
tq_status tq_plan_info(const tq_plan* plan, tq_plan_desc* desc);

/*
 * Encode n vectors (norm split, rotation, Lloyd-Max indices, residual norm,
 * QJL signs: overview §1.2, §2.1, §2.3; one fused launch for D <= 512).
 *   x      device, n rows of d elements of type dt, row i at x + i*ldx elements;
 *          4-byte aligned (bf16) / 4-byte aligned (f32)
 *   ldx    row stride in elements, ldx >= d
 *   codes  device, n * record_bytes bytes, 16-byte aligned; written entirely
 * For sub-plans with D >= 1024 the signs are computed by a second launch over
 * batches of up to 32768 vectors, whose residuals are kept in a stream-ordered
 * temporary of 4*D bytes per vector of the batch (hipMallocAsync / hipFreeAsync
 * on `stream`); an allocation failure is reported as TQ_ENOMEM or TQ_EDEVICE.
 * Errors: TQ_EINVAL (null with n > 0, n < 0, ldx < d, misalignment),
 * TQ_EDEVICE.  n = 0 is a no-op.
 */
tq_status tq_encode(const tq_plan* plan, const void* x, tq_dtype dt, int64_t n, int64_t ldx,
                    void* codes, void* stream);

/*
 * tq_encode of n_groups groups of n_per_group rows: rows g*n_per_group ..
 * +n_per_group-1 of x (row stride ldx) are group g, and their records are
 * records g*n_per_group .. of `codes`.  With a layer plan (tq_plan_create_heads)
 * group g gathers the channels of head g % n_heads; all groups and heads are
 * encoded by one launch per sub-plan.  With an ordinary plan it equals tq_encode
 * of n_groups*n_per_group rows.  1 <= n_groups <= 65535 when n_per_group > 0.
 * Errors: as tq_encode; TQ_EUNSUPPORTED for a layer plan with D > 128.
 */
tq_status tq_encode_groups(const tq_plan* plan, const void* x, tq_dtype dt, int64_t n_groups,
                           int64_t n_per_group, int64_t ldx, void* codes, void* stream);

/*
 * Score queries against encoded vectors with the unbiased estimate
 *   est = n_x * ( <y', c[idx]> + gamma * sqrt(pi/2)/k * sum_j (S y')_j (2 beta_j - 1) ),
 *   y' = the plan's rotation applied to the zero-padded query
 * (overview §1.2.3 and §4.2.2; deep dive §3: full-precision query against
 * low-precision data); summed over sub-plans when there is an outlier mask.
 * Queries and codes are grouped (grouped-query attention: query head h reads
 * key head h / nq_per_group):
 *   q       device, n_groups*nq_per_group rows of d elements (dtype dt), row
 *           stride ldq elements; rows g*nq_per_group .. +nq_per_group-1 are group g
 *   codes   device, n_groups * n records; group g's records start at record g*n
 *   scores  device float32 [n_groups*nq_per_group][n], row-major, written entirely
 * Raw inner-product estimates: no 1/sqrt(d), no softmax.  With a layer plan
 * (tq_plan_create_heads), n_groups must be a multiple of n_heads and group g
 * uses head g % n_heads.
 * Uses a workspace of n_groups*nq_per_group*(6*D) floats per sub-plan (the
 * per-stream buffer above).
 * A TurboQuant-MSE plan gives est = n <Pi pad(y), c[idx]>: the overview's
 * quantized distance (§4.2.2; the query stays full precision) with the norm
 * kept apart as §4.2.1 stores it.  It is not unbiased: over random rotations
 * its mean is <x, y> (1 - D E[(T - Q(T))^2]).  For D >= 256 it runs on the
 * decoded fp16 key tiles of the many-query scorer whatever the query count.
 * Errors: TQ_EINVAL (null, negative sizes, ldq < d, misalignment), TQ_ENOMEM,
 * TQ_EDEVICE.  Empty sizes are a no-op.
 */
tq_status tq_score(const tq_plan* plan, const void* q, tq_dtype dt, int64_t nq_per_group,
                   int64_t n_groups, int64_t ldq, const void* codes, int64_t n, float* scores,
                   void* stream);

/*
 * tq_score without any allocation, for callers that cannot allocate: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results and errors are those of tq_score (identical scores from the
 * same kernels), except that the query workspace is a fixed 16 MiB device array
 * inside the library (one per device, kept until the process ends) instead of a
 * stream-ordered temporary; no hipMalloc, hipFree or allocating routine is called.
 * A request whose workspace exceeds 16 MiB returns TQ_EINVAL before any launch.
 * For plans with every D <= 128 the workspace is about
 *   n_groups * ceil(nq_per_group/4) * (2^(R-1) + 1) * 2 KiB per sub-plan
 * (R index bits), e.g. 128 groups of 4 queries at 3 bits use 0.78 MiB; longer
 * vectors also keep y', S y' and the shares of its sum per query (8 D +
 * 4 ceil(D/128) bytes each, plus the images of the scorer).  Every call on a
 * device shares that device's array: calls that overlap on one device (different
 * streams, or host threads) race and must be ordered by the caller.
 */
tq_status tq_score_noalloc(const tq_plan* plan, const void* q, tq_dtype dt, int64_t nq_per_group,
                           int64_t n_groups, int64_t ldq, const void* codes, int64_t n,
                           float* scores, void* stream);

/*
 * Top-k per row of a score matrix (the first, quantized stage of two-stage
 * retrieval: overview §4.2.2): for each of nq rows of `scores` (device
 * float32 [nq][n]) the k largest values, ordered by (-value, index).
 *   ids   device int64 [nq][k], vals device float32 [nq][k]
 * Errors: TQ_EINVAL (null, k < 1, k > 64, k > n, n >= 2^31), TQ_EDEVICE.
 * NaN scores are not supported.
 */
tq_status tq_topk(const float* scores, int64_t nq, int64_t n, int k, int64_t* ids, float* vals,
                  void* stream);

/*
 * Score and select in one call (overview §4.2.2: the quantized first stage of
 * two-stage retrieval): for each query row, the k largest estimates of
 * tq_score against its group's n records, ordered by (-value, index), with
 * the same values tq_score would write.  Arguments as in tq_score, plus
 *   ids   device int64 [n_groups*nq_per_group][k]: record index within the group
 *   vals  device float32 [n_groups*nq_per_group][k]
 * For a single sub-plan with D > 128, D a multiple of 128 and at least 8
 * queries per group, the score matrix is never stored: the scorer keeps each
 * query's running best k in on-chip memory and a second launch merges the
 * per-workgroup lists (8*k bytes per query and workgroup slice, about 16384
 * workgroups).  Other shapes score into 4*n bytes per query row and select from
 * it.  Both live in the per-stream workspace above.
 * Errors: TQ_EINVAL (as tq_score; k < 1, k > 64, k > n, n >= 2^31),
 * TQ_ENOMEM, TQ_EDEVICE.  NaN estimates are not supported.
 */
tq_status tq_score_topk(const tq_plan* plan, const void* q, tq_dtype dt, int64_t nq_per_group,
                        int64_t n_groups, int64_t ldq, const void* codes, int64_t n, int k,
                        int64_t* ids, float* vals, void* stream);

/*
 * Reconstruct n vectors from their records (overview §4.1.2: dequantize in
 * one batch before the attention step): xhat = n_x * (Pi^T c[idx])[:d], the
 * centroids of the stored cells taken back through the rotation (Pi is
 * orthogonal, so its inverse is its transpose) and scaled by the stored norm.
 * For an inner-product plan this is the reconstruction of its (b-1)-bit first
 * stage (the sign sketch is not inverted); with an outlier mask each sub-plan
 * writes its own channels.
 *   codes  device, n records, 16-byte aligned
 *   x      device, n rows of d elements of type dt, row i at x + i*ldx
 *          elements; element-aligned; written entirely
 * Errors: TQ_EINVAL (null with n > 0, n < 0, ldx < d, misalignment),
 * TQ_EDEVICE.  n = 0 is a no-op.
 */
tq_status tq_dequantize(const tq_plan* plan, const void* codes, int64_t n, void* x, tq_dtype dt,
                        int64_t ldx, void* stream);

/*
 * Decode attention over quantized values (overview §4.1.2: the cache is
 * dequantized for the attention step): for query row r of group g,
 *   out[r] = sum_j softmax(scale * logits[r])_j * vhat_j,
 * with vhat_j the reconstruction (as tq_dequantize) of group g's record j.
 * The weighted centroids are summed in the rotated domain and the rotation is
 * undone once per row, so no value vector is reconstructed on its own.
 *   vplan   the values' plan (MSE or inner-product; one sub-plan)
 *   logits  device float32 [n_groups*nq_per_group][n], e.g. from tq_score;
 *           finite, or -inf for a masked token (weight 0).  A row needs at
 *           least one finite logit: a row masked everywhere has no softmax and
 *           its output is NaN.  NaN and +inf logits are not supported.
 *   vcodes  device, n_groups * n records of vplan (group g from record g*n)
 *   out     device, n_groups*nq_per_group rows of d elements (dt), stride ldo
 * Uses a workspace of (D + 2) floats per row and 1024-token chunk (the
 * per-stream buffer above).  Limits: n >= 1, n_groups <= 65535, nq_per_group <= 262140,
 * nq_per_group * n_groups < 2^31, ceil(n / 1024) * nq_per_group * n_groups
 * <= 2^33, scale finite.  nq_per_group = 0 or n_groups = 0 is a no-op.
 * Errors: TQ_EINVAL (range, null, ldo < d, misalignment: logits 4-byte,
 * vcodes 16-byte, out element-aligned), TQ_ENOMEM, TQ_EDEVICE;
 * TQ_EUNSUPPORTED for a plan with an outlier mask or more than 4 index bits
 * per coordinate (an MSE plan of 1..4 bits, an inner-product plan of 2..5).
 */
tq_status tq_attend(const tq_plan* vplan, const float* logits, int64_t nq_per_group,
                    int64_t n_groups, int64_t n, float scale, const void* vcodes, void* out,
                    tq_dtype dt, int64_t ldo, void* stream);

/*
 * Outlier channels of a head by variance (overview §4.1.1: about a quarter of
 * a head's channels are kept at a higher bit width; the outliers here are the
 * channels of largest variance over a calibration sample).  For every channel,
 * the population variance over the n sample rows in fp64 (two passes: the
 * mean, then the mean squared deviation, each summed in a fixed order); then
 * mask[c] = 1 for the n_out channels first in the order (-variance, channel),
 * 0 for the rest.  The mask, copied to the host, is the outlier_mask of
 * tq_plan_create.
 *   x     device, n rows of d elements (dt), row stride ldx elements; finite
 *   var   device double [d]; mask device uint8 [d]
 * Uses a stream-ordered temporary of at most 32 MiB.
 * Limits: n >= 1, 1 <= d <= 65536, 0 <= n_out <= d.
 * Errors: TQ_EINVAL (range, null, ldx < d, misalignment), TQ_ENOMEM,
 * TQ_EDEVICE.
 */
tq_status tq_calibrate_outliers(const void* x, tq_dtype dt, int64_t n, int64_t ldx, int d,
                                int n_out, double* var, uint8_t* mask, void* stream);

/*
 * Streaming append (overview §4.1.2: the cache grows by one record per head
 * and decode step): encode n vectors as tq_encode does and write record i to
 * row index[i] of a cache of cache_rows records, e.g. row g * capacity + t for
 * token t of group g.  Rows outside [0, cache_rows) are skipped; the other
 * rows of the cache are left as they are; with repeated rows, which record
 * lands there is unspecified.
 *   cache  device, cache_rows * record_bytes bytes, 16-byte aligned
 *   index  device int64 [n]
 * For plans whose sub-plans all have D <= 128 the records are written straight
 * to their rows (one launch per sub-plan, no temporary); longer vectors pass
 * through a stream-ordered temporary of n * record_bytes.  With a layer plan,
 * vector i uses head i % n_heads (n <= 65535).
 * Errors: TQ_EINVAL (null with n > 0, n < 0, ldx < d, misalignment),
 * TQ_ENOMEM, TQ_EDEVICE.  n = 0 is a no-op.
 */
tq_status tq_encode_scatter(const tq_plan* plan, const void* x, tq_dtype dt, int64_t n, int64_t ldx,
                            void* cache, int64_t cache_rows, const int64_t* index, void* stream);

/*
 * Second stage of two-stage retrieval (overview §4.2.2: the quantized first
 * stage screens a top-K, the second refines on the candidates): for each of nq
 * queries, the exact inner products with the full-precision vectors of its kc
 * candidates (fp32 accumulation), and the k best ordered by (-value, id).  No
 * plan is involved.
 *   q     device, nq rows of d elements (qdt), row stride ldq elements
 *   x     device, n rows of d elements (xdt), row stride ldx elements
 *   cand  device int64 [nq][kc]: candidate row ids (e.g. from tq_score_topk);
 *         ids outside [0, n) are skipped and repeated ids count once
 *   ids   device int64 [nq][k], vals device float32 [nq][k]; slots past the
 *         valid candidates get id -1 and value -inf
 * Limits: 1 <= d <= 8192, 1 <= k <= kc <= 256.
 * Errors: TQ_EINVAL (range, null, misalignment), TQ_EDEVICE.
 */
tq_status tq_rerank(const void* q, tq_dtype qdt, int64_t nq, int64_t ldq, const void* x,
                    tq_dtype xdt, int64_t n, int64_t ldx, int d, const int64_t* cand, int kc, int k,
                    int64_t* ids, float* vals, void* stream);

/*
 * The QJL stage alone (overview §2.3.2): beta_j = [ (S r)_j >= 0 ] for n
 * residual vectors r already in the rotated domain of sub-plan `subplan`.
 *   r     device float32 [n][D]
 *   beta  device uint32 [n][D/32]; bit t of word g = beta of row 32g+t
 * The same kernel code as the sign stage fused inside tq_encode.
 * Errors: TQ_EINVAL, TQ_EDEVICE.
 */
tq_status tq_qjl(const tq_plan* plan, int subplan, const float* r, int64_t n, uint32_t* beta,
                 void* stream);

/* ---- Host building blocks of a plan (no device needed) ---------------------------------- */

/*
 * Lloyd-Max codebook for one rotated coordinate in D dimensions with R bits
 * (overview §1.2.2, §2.2): 2^R ascending levels and 2^R - 1 thresholds (host
 * double arrays).  Density proportional to (1 - t^2)^((D-3)/2) on [-1, 1].
 * 3 <= D <= 65536, 1 <= R <= 8.  Errors: TQ_EINVAL.
 */
tq_status tq_codebook(int D, int R, double* levels, double* thresholds);

/*
 * The three +-1 rotation diagonals of sub-plan `subset` (0 regular, 1 outlier)
 * for `seed`: signs[r*D + i] in {+1, -1} (host int8 [3][D]).  32 <= D <= 65536,
 * D a power of two.  Errors: TQ_EINVAL.
 */
tq_status tq_rotation_signs(uint64_t seed, int subset, int D, int8_t* signs);

/*
 * The QJL matrix S (k x D) of sub-plan `subset`: bfloat16 bit patterns,
 * S[j*D + i] = bf16 round-to-nearest-even of a fp64 Box-Muller normal
 * (host uint16 [k][D]).  1 <= k, D <= 65536.  Errors: TQ_EINVAL.
 */
tq_status tq_qjl_matrix(uint64_t seed, int subset, int k, int D, uint16_t* S_bf16);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
