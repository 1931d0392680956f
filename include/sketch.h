/*
 * sketch.h -- C ABI of the MI355X (gfx950) UltraSketchLLM sketch library.
 *
 * Method: "UltraSketchLLM: Sub-1-Bit LLM Compression via Sketch and
 * Hardware-Friendly Operators" (gist.science explainer, "Resumen Técnico").
 *   Metodología §1 (AbsMaxMin sketch): every weight of a row block is hashed
 *     to a bucket; a bucket keeps the weight of minimum absolute value among
 *     its colliders.
 *   Metodología §2 (importance): E[a^2]-style importance scales the choice;
 *     here a per-input-column factor on the comparison key.
 *   Metodología §4 (matrix operators): compression is a MIN reduction through
 *     a one-hot projection P; decompression is W_hat = S * P^T.
 *   Resultados (compression efficiency): 0.5 bits per weight.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers named *_dev, and every tensor argument (W, importance, tables,
 *    X, Y, proj, workspace, status_dev), are DEVICE pointers on the current
 *    HIP device.  `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).  The caller allocates and owns all memory; the library
 *    allocates nothing (it holds a few bytes of static device memory per
 *    device, see sketch_encode).
 *  - Every call that takes a stream only enqueues work and returns; nothing
 *    synchronises the host, except sketch_encode without a status word
 *    (status_dev == NULL), which waits for its stream.  Host-side validation
 *    errors are returned before anything is enqueued; a failed kernel launch
 *    returns SKETCH_EDEVICE.
 *  - The two operations of the method are sketch_encode (W, importance, bpw,
 *    seed -> tables) and sketch_matmul (tables, X -> Y).  Both also take the
 *    projection `proj` (below), which the plain two-call form
 *    encode(W, importance, bpw, seed) -> tables / matmul(tables, X) -> Y
 *    does not have: the library allocates nothing, so the index form of P,
 *    shared by every linear of one shape, lives in a caller buffer built once
 *    by sketch_projection_build instead of being rebuilt (or rehashed per
 *    weight) inside every call.
 *  - W is [M][N] row-major (out x in, the nn.Linear weight layout).  A row
 *    block b covers rows [b*R, (b+1)*R).  Local index inside a block:
 *    l = r*N + j.  Tables are [M/R][Bg] binary16 bit patterns.
 *  - X is [batch][N] row-major; Y is [batch][M] float32; Y = X * W_hat^T.
 *  - Tensor pointers must be 16-byte aligned.
 *  - The library keeps no state between calls and is reentrant; calls on
 *    different streams may run concurrently as long as they do not write the
 *    same memory.
 */
#ifndef SUB_BIT_WEIGHT_SKETCH_H
#define SUB_BIT_WEIGHT_SKETCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SKETCH_OK = 0,
    SKETCH_EINVAL = -1,   /* bad parameters, shapes, pointers or importance */
    SKETCH_ERANGE = -2,   /* a weight is NaN/Inf or rounds to binary16 infinity */
    SKETCH_EDEVICE = -3,  /* a HIP call or kernel launch failed */
    SKETCH_ESMALL = -4,   /* a caller buffer (projection, workspace) is too small */
    SKETCH_ENOSPACE = -5  /* the call needs more scratch than sketch_matmul_noalloc holds */
} sketch_status;

typedef enum { SKETCH_F32 = 0, SKETCH_BF16 = 1, SKETCH_F16 = 2 } sketch_dtype;

/* Which collider a bucket keeps (Metodología §1 keeps the minimum |w|; the
 * plain-language part of the page keeps the largest).  Key = |w| * imp[j]
 * as one binary32 multiply; equal keys go to the smallest local index. */
typedef enum { SKETCH_ABSMIN = 0, SKETCH_ABSMAX = 1 } sketch_rule;

typedef struct {
    int64_t M, N;          /* weight shape [M][N] */
    int32_t R;             /* rows per block; M % R == 0 */
    double bpw;            /* bits per weight; Bg = R*N*bpw/16 must be an integer >= 1 */
    uint32_t seed;         /* hash seed */
    sketch_rule rule;
    sketch_dtype w_dtype;  /* dtype of W given to sketch_encode */
    int32_t rows;          /* sketch rows (hash functions), 1..SKETCH_MAX_ROWS; 0 means 1 */
    /* Importance-aware allocation (see below); NULL / 0 for the uniform sketch. */
    const uint32_t* block_offsets;  /* DEVICE [M/R + 1] table offsets, or NULL */
    int32_t block_bg_max;           /* largest block count of that allocation */
    int32_t bucket_bits;            /* 16 (binary16 buckets; 0 means 16) or 4 (4-bit buckets, below) */
} sketch_params;

/*
 * Multi-row sketch (rows > 1), Metodología §1 (multi-row design: several
 * independent hash functions, each with its own sketch row; decompression
 * takes the Max over the rows).  Same bit budget and table layout: each
 * block's Bg buckets are split into `rows` segments of Bg/rows (Bg % rows
 * must be 0); row rho hashes with seed + rho into its segment and keeps the
 * same winner per bucket as the single-row sketch.  W_hat[i][j] is the row
 * bucket of largest magnitude (SKETCH_ABSMIN; smallest for SKETCH_ABSMAX),
 * the first row among equal magnitudes.  W_hat is not linear in the tables,
 * so the product decodes every weight instead of factoring through P^T x:
 * it is compute-bound, not HBM-bound.  A multi-row projection is a different
 * buffer (sketch_projection_bytes / _build with the same rows).
 */
#define SKETCH_MAX_ROWS 16

/*
 * Importance-aware space allocation (block_offsets != NULL), Metodología §2:
 * rows of higher importance (expected squared activation E[a^2]) get more
 * sketch space.  Row block b owns Bg_b = off[b+1] - off[b] buckets at
 * tables[off[b] ..], with off = block_offsets (uint32, device, M/R + 1
 * entries, off[0] = 0, each Bg_b in 1..block_bg_max, off[M/R] <= (M/R)*Bg:
 * the uniform budget of sketch_layout).  Block b hashes with the same
 * function reduced to its own count:
 *     k_b(l) = (u64(hash32((u32)(l*0x9E3779B1) ^ seed)) * Bg_b) >> 32,
 * and keeps the same winner per bucket as the uniform sketch.  The
 * projection of an allocated sketch holds the 32-bit hash of every local
 * index (it does not depend on the counts; sketch_projection_bytes / _build
 * with block_offsets set).  rows must be 1; block_bg_max <= SKETCH_MAX_BG.
 * Block counts the device finds invalid make sketch_encode set
 * SKETCH_FLAG_ALLOCATION (that block's tables are not written) and
 * sketch_matmul / sketch_decode write NaN for that block's rows.  The
 * per-block hash range makes W_hat no longer share one P across blocks, so
 * the products decode every weight (compute-bound, like the multi-row
 * sketch).  sketch_block_importance and sketch_alloc_plan compute the counts.
 */
/*
 * 4-bit buckets (bucket_bits == 4), Resultados (0.5 bits per weight combined
 * with 4-bit quantization): a block has Bg = R*N*bpw/4 buckets (8 weights
 * per bucket at 0.5 bpw; Bg must be an even integer), each a signed code q in
 * [-7, 7], and one binary16 scale s.  The winner of a bucket is chosen as in
 * the binary16 sketch; s = binary16(max |winner| / 7) (float32, correctly
 * rounded); q = clamp(rint(w / s), -7, 7) for the winner w (float32 division,
 * ties to even), 0 for an empty bucket or s == 0; W_hat = q * s.  The
 * `tables` buffer of sketch_layout's table_bytes holds the codes, two per
 * byte (even bucket in the low nibble, block b at byte b*Bg/2), then the nb
 * binary16 scales at byte offset align256(nb*Bg/2).  The projection is the
 * binary16 sketch's for Bg buckets.  rows must be 1 and block_offsets NULL.
 * The products decode every weight and apply s once per output.
 */
#define SKETCH_MAX_BG4 16384           /* 4-bit buckets per block */

/* Encode status flag bits written by the device into *status_dev. */
#define SKETCH_FLAG_WEIGHT_RANGE 0x1   /* some weight NaN/Inf or |w| >= 65520 */
#define SKETCH_FLAG_IMPORTANCE 0x2     /* some importance NaN, Inf or negative */
#define SKETCH_FLAG_PROJECTION 0x4     /* proj was built for other parameters */
#define SKETCH_FLAG_ALLOCATION 0x8     /* some block_offsets entry out of range */

/* Limits of this implementation (SKETCH_EINVAL beyond them). */
#define SKETCH_MAX_BG 16384            /* buckets per block (LDS-resident table) */
#define SKETCH_MAX_N 65535             /* input columns (16-bit column indices) */

/*
 * sketch_layout -- bit budget and table layout (host only, pure).
 * Budget: Bg = R*N*bpw/16 binary16 buckets per block (0.5 bpw = one bucket per
 * 32 weights); num_blocks = M/R; table_bytes = num_blocks*Bg*2.
 * With 4-bit buckets, Bg = R*N*bpw/4 and table_bytes = align256(num_blocks*Bg/2)
 * + num_blocks*2 (codes, then scales).
 * Any output pointer may be NULL.  Returns SKETCH_EINVAL if M % R != 0, Bg is
 * not a positive integer, R*N*sizeof(w) >= 2^32 (R*N >= 2^31 for 16-bit
 * weights, 2^30 for float32: a block's bytes are addressed with 32-bit
 * offsets), N > SKETCH_MAX_N or Bg > SKETCH_MAX_BG.
 */
sketch_status sketch_layout(const sketch_params* p, int64_t* num_blocks, int64_t* Bg,
                            size_t* table_bytes);

/*
 * The projection P (Metodología §4) in index form, the first level of the
 * "two-level cache" the page mentions for P: it depends only on (R, N, Bg,
 * seed), so one buffer serves every block and every linear of that shape.
 * Contents (built on the device): a header, the forward map
 * k(l) = (u64(hash32((u32)(l*0x9E3779B1) ^ seed)) * Bg) >> 32 for every
 * local index l (hash32 = MurmurHash3's fmix32), and its inverse as a CSR:
 * for every (r, k) the columns j with k(r*N + j) = k, ascending.
 *
 * sketch_projection_bytes: size of the buffer (host only).
 * sketch_projection_build: fills `proj` (device, proj_bytes >= the size) on
 *   `stream`.  Returns SKETCH_ESMALL if proj_bytes is too small.
 *
 * The calls that take `proj` read at most sketch_projection_bytes(p) bytes
 * of it and check its header on the device: a projection built for other
 * parameters (shape or seed) makes sketch_encode set
 * SKETCH_FLAG_PROJECTION, and sketch_matmul and sketch_decode write NaN to
 * every output, provided the buffer is at least that many bytes long
 * (shorter buffers are a caller error with undefined results).
 */
sketch_status sketch_projection_bytes(const sketch_params* p, size_t* bytes);
sketch_status sketch_projection_build(const sketch_params* p, void* proj, size_t proj_bytes,
                                      void* stream);

/*
 * sketch_encode -- compression (Metodología §1, §2, §4).
 *   W          [M][N] of p->w_dtype (float32, bfloat16 or binary16 bits).
 *   importance [N] float32, or NULL for all ones.  Must be finite and >= 0.
 *   proj       built by sketch_projection_build for the same parameters.
 *   tables     [M/R][Bg] uint16 output (binary16 bits).  Bucket = binary16
 *              round-to-nearest-even of the winning weight; +0 if empty.
 *   status_dev one device int32 that the kernel ORs SKETCH_FLAG_* bits into.
 *              The caller zeroes it before the first call and reads it after
 *              the stream has reached this call; sketch_encode_status()
 *              turns the flags into a status.  When flags are set, the
 *              affected tables are unspecified.
 *              NULL: the call uses a status word of its own (one per device,
 *              held by the library until the process ends), waits for
 *              `stream` and returns sketch_encode_status() of the flags:
 *              SKETCH_ERANGE for out-of-range weights, SKETCH_EINVAL for bad
 *              importance or projection.  Such calls are serialised by a
 *              process-wide lock; they cannot be captured into a HIP graph
 *              (the wait fails with SKETCH_EDEVICE).
 * Asynchronous on `stream` when status_dev != NULL.  Returns SKETCH_EINVAL
 * for bad parameters or NULL/misaligned pointers.
 * Beyond the two-call form, this call takes `proj` (see the conventions
 * above) and, with a status word, reports weight-range and importance
 * problems through it instead of its return value, so that it never has to
 * wait for the device.
 */
sketch_status sketch_encode(const sketch_params* p, const void* proj, const void* W,
                            const float* importance, uint16_t* tables, int32_t* status_dev,
                            void* stream);

/* Flags read back from status_dev -> SKETCH_OK, SKETCH_ERANGE (weights) or
 * SKETCH_EINVAL (importance or projection). */
sketch_status sketch_encode_status(int32_t flags);

/*
 * sketch_workspace_bytes -- device scratch sketch_matmul needs for `batch`
 * rows of X of dtype x_dtype (0 when none is needed).  Host only.  It takes
 * x_dtype because the dtype picks the product path (matrix cores or not),
 * and with it whether Z is staged in the workspace.
 * The workspace holds Z = P^T x for the large-problem path; its contents
 * need no initialisation.  Calls that overlap in time need separate
 * workspaces.  For the prefill of multi-row sketches (rows > 1, batch > 16)
 * the workspace is optional: with the bytes reported here (batch x M
 * floats per extra part, when the product's tiles would leave compute
 * units idle) the product splits K over more workgroups and adds the parts
 * in a second launch, in a fixed order; with less it runs unsplit.  The two
 * forms differ only in float32 accumulation rounding.
 */
sketch_status sketch_workspace_bytes(const sketch_params* p, int64_t batch, sketch_dtype x_dtype,
                                     size_t* bytes);

/*
 * sketch_matmul -- Y = X * W_hat^T with W_hat = S * P^T never materialised
 * (Metodología §4).
 *   tables  [M/R][Bg] from sketch_encode with the same parameters.
 *   X       [batch][N] of x_dtype; Y [batch][M] float32 (overwritten).
 *   workspace / workspace_bytes: at least sketch_workspace_bytes(...) bytes
 *           (may be NULL when that is 0; optional for the multi-row
 *           prefill, see sketch_workspace_bytes).
 * Paths: batch <= 16, or any non-bfloat16 operand: the factorized product
 * Y[t][bR+r] = sum_k S[b][k] * Z[t][r][k] with Z = P^T x (float32
 * accumulation).  batch > 16 with bfloat16 W and X: Ŵ tiles decoded into LDS
 * and multiplied on bf16 matrix cores with float32 accumulation (buckets of
 * bfloat16 weights are exact in bfloat16).
 * Asynchronous on `stream`; never synchronises.  NaN/Inf in X propagate.
 * batch == 0 or M == 0 is a no-op returning SKETCH_OK.
 * Beyond the two-call form, this call takes `proj` (see the conventions
 * above) and a caller workspace (the library allocates nothing).
 */
sketch_status sketch_matmul(const sketch_params* p, const void* proj, const uint16_t* tables,
                            const void* X, sketch_dtype x_dtype, int64_t batch, float* Y,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * sketch_matmul_noalloc -- sketch_matmul for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, paths and results as
 * sketch_matmul, without the workspace: when the product needs one (see
 * sketch_workspace_bytes; the optional one of the multi-row prefill only
 * when it fits) it uses a scratch array of
 * SKETCH_NOALLOC_SCRATCH_BYTES that the library holds in static device
 * memory, one copy per GPU, kept until the process ends.  The call itself
 * allocates nothing (no hipMalloc, no allocating library routine).
 * Returns SKETCH_ENOSPACE, before anything is enqueued, when the product
 * needs more scratch than that.  Every call on one GPU shares that GPU's
 * scratch: calls that overlap in time on one GPU (several streams or host
 * threads) race and give undefined results; calls ordered on one stream
 * are safe (nothing in the scratch needs clearing between calls).
 */
#define SKETCH_NOALLOC_SCRATCH_BYTES (8u << 20)
sketch_status sketch_matmul_noalloc(const sketch_params* p, const void* proj, const uint16_t* tables,
                                    const void* X, sketch_dtype x_dtype, int64_t batch, float* Y, void* stream);

/*
 * Grouped decode product -- several linears, each with its own input token
 * and output, multiplied in one pass (Metodología §4, the factorised product
 * y[b*R + r] = sum_k S[b][k] * Z[r][k], Z = P^T x, of every linear): the
 * linears of a decoder layer for one token step, or those of a whole model.
 * Taken one by one, such products are too small to keep the memory system
 * busy; grouped, all their bucket tables form one stream.
 *
 * Each item: a uniform single-row sketch (rows 1, no block_offsets), R in
 * {2, 4, 8}, N * sizeof(x) <= 120 KiB (N <= 61440 for 16-bit x, N <= 30720
 * for float32); its projection, tables, x ([N], one token, of the group's
 * x_dtype) and y ([M] float32, overwritten), all device pointers, 16-byte
 * aligned.  At most SKETCH_GROUP_MAX_ITEMS items, all with one bucket
 * format:
 *   - binary16 buckets (bucket_bits 16), Bg a multiple of 32;
 *   - 4-bit codes (bucket_bits 4; Resultados, 0.5 bpw with 4-bit
 *     quantization), Bg a multiple of 128: the same factorisation over the
 *     Bg codes of a block, y[b*R + r] = s_b * sum_k q[b][k] * Z[r][k], with
 *     the codes as exact binary16 operands and the block scale s_b applied
 *     once per output; tables is the buffer sketch_encode wrote (codes,
 *     then the block scales at the offset sketch_layout's notes give).
 * Other items, or both formats in one group, give SKETCH_EINVAL (use
 * sketch_matmul for them).
 *
 * sketch_group_bytes (host only): sizes of the plan and of the workspace.
 * sketch_group_plan: writes the plan of this exact list of items (their
 *   pointers and shapes, and how the tile stream is split over the waves of
 *   the current device) into `plan` (device, plan_bytes), asynchronously on
 *   `stream`; it allocates nothing.  A plan is reused for every call with
 *   the same items (e.g. one per token step whose buffers it names).
 * sketch_matmul_group: the products of the items, asynchronously on
 *   `stream`, with the plan built for these same items on this device and a
 *   workspace of at least the stated size (contents need no initialisation;
 *   calls that overlap in time need separate workspaces).  The result per
 *   item is that of sketch_matmul within the same tolerance (float32
 *   accumulation of exact binary16 hi + lo products; the power-of-two scale
 *   of an item bounds |Z| by N * max |x|, so results can differ from
 *   sketch_matmul's in the last bits); a projection built for other parameters makes that item's
 *   outputs NaN, and a non-finite x makes them non-finite.
 */
#define SKETCH_GROUP_MAX_ITEMS 65536
typedef struct {
    const sketch_params* p;   /* host pointer to the item's parameters */
    const void* proj;         /* device: projection built for p */
    const uint16_t* tables;   /* device: [M/R][Bg] binary16 bits, or the 4-bit tables buffer */
    const void* x;            /* device: [N] of the group's x_dtype */
    float* y;                 /* device: [M] float32 */
} sketch_group_item;

sketch_status sketch_group_bytes(const sketch_group_item* items, int32_t count, sketch_dtype x_dtype,
                                 size_t* plan_bytes, size_t* workspace_bytes);
sketch_status sketch_group_plan(const sketch_group_item* items, int32_t count, sketch_dtype x_dtype, void* plan,
                                size_t plan_bytes, void* stream);
sketch_status sketch_matmul_group(const sketch_group_item* items, int32_t count, sketch_dtype x_dtype,
                                  const void* plan, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sketch_decode -- materialise W_hat = S * P^T (Metodología §4,
 * decompression): W_hat[i][j] = S[i/R][k((i % R)*N + j)], each weight's
 * bucket index read from the projection's forward map.
 *   proj     built by sketch_projection_build for the same parameters (see
 *            the projection notes above for other ones).
 *   tables   [M/R][Bg] binary16 bits, from sketch_encode with the same
 *            parameters.
 *   out      [M][N] of out_dtype, overwritten: SKETCH_F16 = the bucket bits,
 *            SKETCH_F32 = the bucket's exact value, SKETCH_BF16 = the value
 *            rounded to nearest even (exact for buckets of bfloat16 weights).
 * Asynchronous on `stream`.  M == 0 is a no-op.  SKETCH_EINVAL for bad
 * parameters, an unknown out_dtype or NULL/misaligned pointers.
 */
sketch_status sketch_decode(const sketch_params* p, const void* proj, const uint16_t* tables, void* out,
                            sketch_dtype out_dtype, void* stream);

/*
 * sketch_decode_hashed -- the same W_hat, element for element, computed the
 * way a naive hash-based sketch decompresses: every weight's bucket index is
 * hashed from its local index and its bucket is read from the table in
 * memory.  It is the baseline of the decompression speed comparison in
 * "Resumen Técnico" › Resultados Experimentales › Latencia de Sobrecarga,
 * kept to measure that ratio; it needs no projection.  Arguments, output and
 * errors as sketch_decode.
 */
sketch_status sketch_decode_hashed(const sketch_params* p, const uint16_t* tables, void* out,
                                   sketch_dtype out_dtype, void* stream);

/*
 * sketch_block_importance -- the importance of every row block for the
 * allocation (Metodología §2, E[a^2] as the importance metric), read as the
 * expected squared output of the block's rows for independent zero-mean
 * inputs with second moments a2:
 *     scores[b] = sum over rows i of block b of sum_j W[i][j]^2 * a2[j].
 *   W       [M][N] of p->w_dtype (device).
 *   a2      [N] float32 (device): E[x_j^2] of the layer's inputs, >= 0.
 *   scores  [M/R] float32 output (device), summed in float32 in a fixed
 *           order (deterministic; not bit-identical to a float64 sum).
 * Only M, N, R and w_dtype of p are used.  Asynchronous on `stream`.
 */
sketch_status sketch_block_importance(const sketch_params* p, const void* W, const float* a2, float* scores,
                                      void* stream);

/*
 * sketch_alloc_plan -- bucket counts from block importances (host only).
 * Each of the nb blocks gets `lo` buckets; the rest of `total` is shared in
 * proportion to scores[b] by largest remainder: quota
 * q_b = ((double)(total - nb*lo) * scores[b]) / sum(scores) (sum in double,
 * b ascending), floor(q_b) each, the leftover units to the largest
 * fractional parts (ties: lower block; a unit of rounding overshoot is taken
 * back from the smallest, ties: higher block); all scores zero gives equal
 * shares.  Writes offsets[0..nb] (offsets[0] = 0, offsets[nb] = total) and
 * *bg_max (may be NULL).  total = nb * Bg keeps the uniform bit budget.
 * SKETCH_EINVAL for nb < 1, lo < 1, total < nb*lo, total >= 2^32, a
 * negative or non-finite score, or a count above SKETCH_MAX_BG.
 */
sketch_status sketch_alloc_plan(int64_t nb, int64_t total, int64_t lo, const double* scores, uint32_t* offsets,
                                int32_t* bg_max);

/* Static, human-readable name of a status code. */
const char* sketch_status_str(sketch_status s);

#ifdef __cplusplus
}
#endif
#endif
