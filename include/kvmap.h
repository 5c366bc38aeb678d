/*
 * libkvmap -- closed-form cross-model KV-cache mapping on AMD Instinct MI355X (gfx950).
 *
 * The mapping (Heo et al., "Cross-Model KV Cache Transfer in LLM Families"), as the
 * pages describe it:
 *   K_hat_t = rope_tgt( strip_rope_src(K_s) . W_K + b_K ),   V_hat_t = V_s . W_V + b_V
 * with one ridge map per target (layer, KV head), fed by the top-k selected source
 * layers' keys/values of ALL source KV heads concatenated into one feature row
 * (VeloxQuant-MLX "Cross-Model KV Transfer", section "The mapping"; KVBridge README,
 * "What ships" and "System design").  The fit side keeps only centered sufficient
 * statistics merged batchwise with Chan/Welford updates and solves
 * W = (X^T X + lambda I)^-1 X^T Y, b = Ybar - Xbar W (KVBridge README, fitting section
 * headed "Loading"; reactapp.top article, section "Eine lineare Bruecke reicht").
 *
 * Conventions used by every call
 *   L_src, L_tgt  source / target layer counts      H = H_kv   KV heads (matched)
 *   d             head dim (64 or 128)              T          cached tokens
 *   k             selected source layers per target layer
 *   F = k*H*d     feature width of one row          N = H*d    output width per target layer
 *   Cache layout  [layer][kv_head][token][dim], dim fastest (the order of the
 *                 voidwest.dev "Before Mapping KV Caches" snapshot, "what became
 *                 first-class"); keys stored rotated, as the model stores them.
 *   Feature order row column (j*H + h)*d + e = selected rank j (order of layer_sel[t]),
 *                 source head h, dim e.
 *   Output order  column n = h*d + e of target layer t goes to tgt[t][h][token][e].
 *   Map layout    W[t] is OUTPUT-major [N][F]: row n holds the F weights of output
 *                 column n (the transpose of the logical F x N matrix).  b[t] is [N].
 *   RoPE          half-split pairs (i, i + d/2), angle (pos0 + token) * theta^(-2i/d);
 *                 the interleaved form is refused, as VeloxQuant-MLX's "honesty crux"
 *                 item 7 refuses it.  Angles and their sines/cosines are formed in
 *                 float64 and stored as float32 tables.
 *   dtype         KVMAP_DTYPE_BF16: caches, maps and biases bf16, fp32 accumulation,
 *                 bf16 outputs (round-to-nearest-even);  KVMAP_DTYPE_F32: all fp32.
 *
 * Memory and streams
 *   Pointers named "device" are HIP device memory owned by the caller; the library
 *   never frees them.  `stream` is a hipStream_t passed as void* (NULL = the null
 *   stream).  Device work is enqueued asynchronously on it.  One context must not be
 *   used from two host threads at once, and calls that share a context should be
 *   issued on one stream (or the caller orders them): the context's workspace and
 *   tables are shared by its calls.
 *
 * Errors
 *   Every call returns a kvmap_status.  All argument, shape and dtype validation
 *   happens on the host before any device work; a refused call leaves outputs
 *   untouched.  kvmap_last_error() returns a thread-local detail string for the
 *   most recent failure on the calling thread.
 */
#ifndef KVMAP_H
#define KVMAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVMAP_VERSION 100 /* 1.0.0 */

typedef enum {
    KVMAP_OK = 0,
    KVMAP_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad enum, lambda < 0, ...        */
    KVMAP_ERR_SHAPE = 2,            /* inconsistent sizes, layer_sel out of range/dup */
    KVMAP_ERR_UNSUPPORTED = 3,      /* valid but outside the matched-KV regime        */
    KVMAP_ERR_NONFINITE = 4,        /* KVMAP_FLAG_CHECK_FINITE found NaN/Inf          */
    KVMAP_ERR_NOT_SPD = 5,          /* ridge system not positive definite             */
    KVMAP_ERR_DEVICE = 6,           /* HIP runtime / launch error                     */
    KVMAP_ERR_OUT_OF_MEMORY = 7     /* workspace allocation failed                    */
} kvmap_status;

typedef enum { KVMAP_DTYPE_BF16 = 0, KVMAP_DTYPE_F32 = 1 } kvmap_dtype;

typedef enum {
    KVMAP_ROPE_HALF_SPLIT = 0,  /* pairs (i, i + d/2): supported               */
    KVMAP_ROPE_INTERLEAVED = 1  /* pairs (2i, 2i + 1): refused (UNSUPPORTED)   */
} kvmap_rope_style;

/* Flags for kvmap_apply. */
#define KVMAP_FLAG_CHECK_FINITE 0x1u /* after mapping, scan tgt_k/tgt_v; any NaN/Inf
                                         returns KVMAP_ERR_NONFINITE (synchronises the
                                         stream). The outputs are written regardless.   */
#define KVMAP_FLAG_TIMING 0x2u       /* record HIP events around each kernel launch on
                                         `stream`; read with kvmap_last_timings().       */

typedef struct kvmap_ctx kvmap_ctx;

typedef struct {
    int32_t L_src, L_tgt, H_kv, head_dim, k;
    int64_t T;
    int32_t dtype; /* kvmap_dtype */
} kvmap_dims;

typedef struct {
    double theta;            /* RoPE base of the model, > 0 (not read when inv_freq is given) */
    int64_t pos0;            /* absolute position of token 0 (>= 0)                          */
    int32_t style;           /* kvmap_rope_style; only KVMAP_ROPE_HALF_SPLIT                  */
    const double* inv_freq;  /* optional host [head_dim/2]: the model's own rotary frequencies
                                f_i (finite, >= 0), angle (pos0 + t) * f_i, instead of
                                theta^(-2i/d) (KVBridge README "What ships": exact RoPE from the
                                factors each model emits).  NULL = theta^(-2i/d).  Read during
                                the call only.                                                 */
} kvmap_rope;

/* ---- status / version ------------------------------------------------------------ */

/* Static string naming a status code. Never NULL. */
const char* kvmap_status_string(int status);
/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* kvmap_last_error(void);
/* KVMAP_VERSION of the built library. */
int kvmap_version(void);

/* ---- context ----------------------------------------------------------------------- */

/* Create a context bound to HIP device `device`.  The context owns the RoPE-table cache,
 * the de-rotated-key workspace and small scratch; it allocates on first use and keeps
 * what it allocated until kvmap_destroy.  Returns KVMAP_ERR_DEVICE if the device does not
 * exist or is not gfx950. *out is NULL on failure. */
int kvmap_create(kvmap_ctx** out, int device);
/* Free everything the context owns (synchronises its device first). NULL is a no-op. */
int kvmap_destroy(kvmap_ctx* ctx);
/* Pre-allocate the workspace and the selection buffers kvmap_apply needs for `dims`, so
 * that applies of those dims (or smaller) allocate nothing and never wait for the device
 * to grow them.  `dims` is checked first, exactly as kvmap_validate_apply checks it
 * (SHAPE / UNSUPPORTED / INVALID_ARGUMENT; layer_sel and the RoPE descriptors are not
 * involved), so a zeroed or otherwise invalid struct is refused before any arithmetic on
 * it; then a NULL ctx is INVALID_ARGUMENT.  Synchronous. */
int kvmap_reserve(kvmap_ctx* ctx, const kvmap_dims* dims);

/* ---- apply (the hot path) ---------------------------------------------------------- */

/* Host-only validation of an apply call: shapes, dtype, RoPE descriptors, and layer_sel
 * (host int32 [L_tgt][k]: every entry in [0, L_src), entries of one row distinct).
 * Refusals, following the matched-KV scope of the pages (VeloxQuant-MLX "honesty crux"
 * item 7; KVBridge README "Scope and limitations"):
 *   SHAPE        L_src, L_tgt, H_kv, k < 1; T < 1; k > L_src; odd head_dim;
 *                layer_sel entry out of range or repeated within a row
 *   UNSUPPORTED  head_dim not 64 or 128; k > 64; style not half-split; dtype unknown
 *   INVALID_ARGUMENT  NULL pointer; theta <= 0 or not finite; pos0 < 0;
 *                pos0 + T beyond 2^31
 * Needs no device. */
int kvmap_validate_apply(const kvmap_dims* dims, const int32_t* layer_sel,
                         const kvmap_rope* rope_src, const kvmap_rope* rope_tgt);
/* Host-only checks of the buffers of an apply call, taken as addresses (nothing is read):
 * dims as in kvmap_validate_apply; then INVALID_ARGUMENT for a NULL pointer, a pointer not
 * 16-byte aligned, an output range overlapping an input range, or tgt_k overlapping tgt_v
 * (ranges from the layouts and sizes of kvmap_apply).  kvmap_apply runs exactly these checks
 * before any device work.  Needs no device. */
int kvmap_validate_apply_buffers(const kvmap_dims* dims, const void* src_k, const void* src_v,
                                 const void* W_k, const void* b_k, const void* W_v, const void* b_v,
                                 const void* tgt_k, const void* tgt_v);

/* Map a source KV cache into the target model's cache (the whole apply step).
 *   src_k, src_v  device [L_src][H][T][d]   stored source cache (keys rotated by the
 *                                           source model at positions rope_src->pos0 + t)
 *   layer_sel     HOST   int32 [L_tgt][k]   selected source layers per target layer
 *   W_k, W_v      device [L_tgt][N][F]      output-major maps
 *   b_k, b_v      device [L_tgt][N]
 *   tgt_k, tgt_v  device [L_tgt][H][T][d]   written completely; keys rotated by the
 *                                           target model at positions rope_tgt->pos0 + t
 * For every target layer t, token p and output column n = h*d + e:
 *   X_K[p, (j*H + h')*d + e'] = strip_rope_src(src_k[layer_sel[t][j]][h'][p])[e']
 *   X_V[p, (j*H + h')*d + e'] = src_v[layer_sel[t][j]][h'][p][e']
 *   tgt_k[t][h][p] = rope_tgt( (X_K W_k[t]^T + b_k[t])[p, h*d : h*d + d] )
 *   tgt_v[t][h][p][e] = (X_V W_v[t]^T + b_v[t])[p, h*d + e]
 * Inputs must not overlap outputs; all pointers 16-byte aligned.
 * Asynchronous on `stream`: the host returns without waiting for the device, also when
 * layer_sel differs from the previous call's (the context keeps the last 8 distinct
 * selections on the device; a new one is uploaded from pinned staging with an
 * asynchronous copy, and layer_sel is read during the call only).  The host waits only in
 * these cases: KVMAP_FLAG_CHECK_FINITE (it reads the count back); growth of the workspace
 * or of the selection buffers (both pre-sized by kvmap_reserve), which waits for the device
 * before it frees the old buffers; a 9th distinct RoPE table
 * (theta or frequency list, pos0, head_dim), which evicts the least recently used one
 * after the device is idle; and a 9th distinct selection queued while the upload of the
 * selection it replaces has not yet run.  In bf16 the de-rotated
 * keys are rounded to bf16 before the map (fp32 accumulation, bf16 output).  bf16 caches of
 * up to 128 tokens take a kernel that streams the maps (the apply is bound by reading W
 * there).  Where its K reduction is split over workgroups, or its tiles hold 16 or 32 tokens,
 * its fp32 partial sums live in the workspace and a second kernel adds them in a fixed order
 * with the bias and the target RoPE; otherwise each workgroup finishes its rows itself.
 * Either way repeated calls give identical outputs. */
int kvmap_apply(kvmap_ctx* ctx, const kvmap_dims* dims,
                const void* src_k, const void* src_v, const int32_t* layer_sel,
                const void* W_k, const void* b_k, const void* W_v, const void* b_v,
                const kvmap_rope* rope_src, const kvmap_rope* rope_tgt,
                void* tgt_k, void* tgt_v, void* stream, uint32_t flags);

/* Durations (ms) of the kernels the last KVMAP_FLAG_TIMING apply on this context
 * launched, measured with HIP events recorded on the apply's stream:
 *   ms[0] RoPE-table build (0 if cached), ms[1] key de-rotation producer,
 *   ms[2] map GEMM (K and V of all target layers: one launch; for bf16 caches of up to 128
 *         tokens the short-cache kernel and, where it runs, the reduce that adds its partial
 *         sums).
 * Synchronises on the events.  n_ms must be >= 3. */
int kvmap_last_timings(kvmap_ctx* ctx, float* ms, int n_ms);
/* The same durations for an earlier timed apply: back = 0 is the most recent, up to 127 back
 * (the context keeps the events of the last 128 KVMAP_FLAG_TIMING applies), so a run of timed
 * applies can be queued with no host wait between them and read afterwards.  INVALID_ARGUMENT
 * when that apply is not held.  Synchronises on its events. */
int kvmap_timings(kvmap_ctx* ctx, int32_t back, float* ms, int n_ms);

/* ---- RoPE recode (identity map) ---------------------------------------------------- */

/* Re-encode a key cache from the source model's RoPE to the target's without a map:
 *   dst[r][t][:] = rope(strip(src[r][t][:], pos0_s + t, theta_s), pos0_t + t, theta_t)
 * for every row r (layers x heads flattened), which is one rotation of every pair
 * (e, e + d/2) by (pos0_t + t) f_t,e - (pos0_s + t) f_s,e, f_e = theta^(-2e/d)
 * (VeloxQuant-MLX "Cross-Model KV Transfer", section "Metal kernel": the strip and the
 * target rotation turn one pair at one position, so one rotation by the difference of the
 * two angles does both).  The angle is formed in float64 into a cached fp32
 * cos/sin table [T][d/2] (built on first use of the (theta, pos0) pair, like the apply's
 * tables); the rotation runs in fp32 and is rounded once to `dtype`.
 *   src, dst  device [rows][T][head_dim], row-major, bf16 or fp32, 16-byte aligned, not
 *             overlapping (dst is fully overwritten)
 *   head_dim  64 or 128;  rope styles must be half-split;  T <= 2^31, pos0 + T <= 2^31
 * Asynchronous on `stream`.  Errors: INVALID_ARGUMENT (NULLs, alignment, overlap, bad rope
 * fields), UNSUPPORTED (dtype, head_dim, rope style), SHAPE (rows < 1, T < 1 or too large);
 * nothing is written on a refused call. */
int kvmap_recode(kvmap_ctx* ctx, int32_t rows, int64_t T, int32_t head_dim, int32_t dtype,
                 const void* src, void* dst, const kvmap_rope* rope_src, const kvmap_rope* rope_tgt,
                 void* stream);

/* ---- fit-side statistics ----------------------------------------------------------- */

/* Rows of calibration caches for kvmap_gram (KVBridge README "What ships": cross-head
 * features of the selected layers; VeloxQuant-MLX "Cross-Model KV Transfer", "The mapping":
 * keys are moved to content space with the model's own rotation before any statistics):
 *   out[t][(j * H + h) * head_dim + e] = strip(cache[layers[j]][h][t][:], pos0 + t, theta)[e]
 * for j < n_layers (the order given), or the plain value when rope == NULL (values, or keys
 * already in content space).
 *   cache   device [L][H][T][head_dim], bf16 or fp32;  out  device [T][n_layers * H * head_dim]
 *   layers  host [n_layers], each in [0, L), 1 <= n_layers <= 128;  head_dim 64 or 128
 * Pointers 16-byte aligned, out not overlapping the cache.  Asynchronous on `stream`.
 * Errors: SHAPE, UNSUPPORTED, INVALID_ARGUMENT (nothing written). */
int kvmap_cache_rows(kvmap_ctx* ctx, const void* cache, int32_t L, int32_t H, int64_t T, int32_t head_dim,
                     int32_t dtype, const int32_t* layers, int32_t n_layers, const kvmap_rope* rope, void* out,
                     void* stream);

/* Centered sufficient statistics of a stream of (x, y) rows, x in R^p, y in R^q:
 *   n       rows merged so far (host integer, updated by the calls)
 *   mean_x  device fp32 [p],  mean_y device fp32 [q]
 *   M_xx    device fp32 [p][p]  = sum (x - mean_x)(x - mean_x)^T   (unnormalised, both
 *                                 triangles stored)
 *   M_xy    device fp32 [p][q]  = sum (x - mean_x)(y - mean_y)^T
 *   ss_y    device fp32 [q] or NULL = sum (y - mean_y)^2 per column (the diagonal of the
 *           y-y co-moments, which the fit itself never needs; layer scoring takes the total
 *           sum of squares from it).  NULL: not kept.  States merged together must agree
 *           on keeping it.
 * Buffers are caller-allocated device memory, 16-byte aligned; the struct only points at
 * them. */
typedef struct {
    int64_t n;
    int32_t p, q;
    float* mean_x;
    float* mean_y;
    float* M_xx;
    float* M_xy;
    float* ss_y;
    int32_t xx_block;  /* 0: M_xx is the whole [p][p].  b > 0 (a multiple of 4 dividing p): only
                          the p / b diagonal blocks of b x b features are kept, compactly as
                          [p / b][b][b]; for features split into groups (the layers of a
                          selection stage) that need their own co-moments but share Y.  Block g
                          is then a whole state of its own, viewed as p = b, mean_x + g b,
                          M_xx + g b^2, M_xy + g b q (same mean_y, ss_y, n, q) -- the form the
                          ridge calls take (they refuse a blocked state).                    */
} kvmap_gram_state;

/* Zero the state's device arrays on `stream` and set n = 0. */
int kvmap_gram_reset(kvmap_ctx* ctx, kvmap_gram_state* st, void* stream);

/* Merge one batch of n_b rows into st (Chan/Welford pairwise update, KVBridge README
 * fitting section):  X device [n_b][p], Y device [n_b][q], row-major, in `dtype`
 * (bf16 or fp32).  The batch's co-moments M_b about its own mean are formed from
 * shifted values x - c (the batch mean m of x - c is removed exactly), then
 *   delta = mean_b - mean,  mean += delta * n_b / n',  M += M_b + (n * n_b / n') delta delta^T
 * with n' = n + n_b.  bf16 batches: c is the batch's column mean rounded to bf16 when the
 * state is empty, else the running mean rounded to bf16 (so a merging batch is read once
 * before its co-moments); x - c is then exact in fp32, split into bf16 hi + lo, and the
 * co-moments come from three bf16 matrix-core passes (hi hi + hi lo + lo hi) with fp32
 * accumulation; batches of more than 16384 rows are merged in sub-batches of at most 16384
 * rows.  fp32 batches: fp32 mean,
 * fp32 matrix cores.  The context keeps the shifted operands of one sub-batch as scratch
 * ((p + q) * ceil(rows / 32) * 128 bytes, allocated on first use).  n_b = 0 is a no-op.
 * p, q must be multiples of 4 and <= 65536, n_b <= 2^31.  Asynchronous on `stream`;
 * st->n is updated on the host at once. */
int kvmap_gram(kvmap_ctx* ctx, const void* X, const void* Y, int64_t n_b, int32_t dtype,
               kvmap_gram_state* st, void* stream);

/* Host-only checks of a kvmap_gram / kvmap_gram_noalloc call, on the state and the batch
 * addresses (nothing is read): the state's dims and arrays (SHAPE / INVALID_ARGUMENT), dtype
 * (UNSUPPORTED), n_b in [0, 2^31] (SHAPE), and for n_b > 0 non-NULL, 16-byte aligned X and Y
 * whose ranges ([n_b][p] and [n_b][q] in dtype) overlap none of the state's arrays
 * (INVALID_ARGUMENT).  The statistics calls run exactly these checks, after their context
 * check, before any device work.  Needs no device. */
int kvmap_validate_gram(const kvmap_gram_state* st, const void* X, const void* Y, int64_t n_b, int32_t dtype);

/* kvmap_gram for callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, checks and result as kvmap_gram,
 * but the scratch (split partial sums, shift, means, deltas and the bf16 hi/lo operands of a
 * sub-batch) is a static device array of KVMAP_STATIC_SCRATCH_BYTES = 64 MiB that the library
 * holds on every GPU it runs on until the process ends; the call itself allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).  bf16 batches are merged in
 * sub-batches of as many rows (a multiple of 32, at most 16384) as fit next to the fixed part
 * of (2 * 64 + 3) * (p + q) floats -- 1664 rows at p 8192, q 1024 -- so results match
 * kvmap_gram bit for bit whenever a batch fits one such sub-batch, and to fp32 rounding of a
 * different merge order otherwise; fp32 batches need no per-row scratch.  Refused with
 * KVMAP_ERR_UNSUPPORTED (nothing done) when p + q is too large for even 32 rows (more than
 * about 100,000 at 64 MiB).  The array is shared by every call on one GPU, from any
 * context or thread: calls that overlap on one GPU (queued on different streams, or from
 * two threads) race and give wrong results -- the caller orders them.  Asynchronous on
 * `stream`; st->n is updated on the host at once. */
int kvmap_gram_noalloc(kvmap_ctx* ctx, const void* X, const void* Y, int64_t n_b, int32_t dtype,
                       kvmap_gram_state* st, void* stream);

/* dst <- Chan merge of dst and src (statistics of disjoint samples; same p, q, xx_block and
 * ss_y choice): the pairwise update kvmap_gram applies to each batch, with src as the batch
 *   n' = n_dst + n_src,  delta = mean_src - mean_dst,  mean_dst += delta * n_src / n',
 *   M_dst += M_src + (n_dst * n_src / n') delta_x delta_y^T   (likewise M_xx and ss_y)
 * -- the mergeable form of the centered statistics that lets shards of calibration data be
 * accumulated apart and combined (KVBridge README, fitting section headed "Loading": only
 * centered statistics are kept and merged with Chan/Welford updates; "What ships": the
 * statistics are reduced across workers).  Merging an empty state is the identity.
 * INVALID_ARGUMENT when any array of dst overlaps any array of src (or one keeps ss_y and the
 * other does not); SHAPE when p, q or xx_block differ.  Asynchronous on `stream`. */
int kvmap_gram_merge(kvmap_ctx* ctx, kvmap_gram_state* dst, const kvmap_gram_state* src,
                     void* stream);

/* ---- ridge solve (host, fp64) ------------------------------------------------------ */

/* Closed-form ridge from statistics held in host memory (fp32 as kept on the device):
 *   W = (M_xx + lambda I)^-1 M_xy,  b = mean_y - mean_x W
 * (KVBridge README, fitting section headed "Loading": the closed-form ridge solve from the
 * centered statistics; reactapp.top article, section "Eine lineare Bruecke reicht": the
 * ridge demo centres x and y, adds lambda = 0.01 to the Gram and takes the intercept from the
 * means, so the intercept is not penalised)
 * solved by blocked Cholesky in float64 on `n_threads` host threads (0 = all cores; at most one
 * per 64 rows of p, so small systems run on fewer).
 * W_out is written OUTPUT-major [q][p] (the layout kvmap_apply takes), b_out [q], both
 * fp32 host.  M_xx is read from its upper triangle.  Returns KVMAP_ERR_NOT_SPD if the
 * factorisation meets a non-positive pivot, INVALID_ARGUMENT for lambda < 0 or NULLs,
 * OUT_OF_MEMORY if the host cannot hold the fp64 system (p^2 + p q doubles); if the system
 * refuses threads, the solve runs on those that did start. */
int kvmap_ridge_solve_host(int32_t p, int32_t q, const float* mean_x, const float* mean_y,
                           const float* M_xx, const float* M_xy, double lambda,
                           float* W_out, float* b_out, int n_threads);

/* Same solve (same passages), from a device state: copies mean_x, mean_y, M_xx, M_xy to the
 * host on `stream`,
 * synchronises, and solves on all host cores.  Synchronous; OUT_OF_MEMORY also when the host
 * cannot hold the fp32 copy of the statistics. */
int kvmap_ridge_solve(kvmap_ctx* ctx, const kvmap_gram_state* st, double lambda,
                      float* W_out, float* b_out, void* stream);

/* Same solve (same passages) on the device in float64 (no copy of the statistics to the
 * host): blocked
 * Cholesky of sym(M_xx) + lambda I (read from M_xx's upper triangle) with 64-wide blocks,
 * then forward and back substitution for the q right-hand sides, then b = mean_y - mean_x W.
 *   W_out  device [q][p] output-major (the layout kvmap_apply takes for one target layer),
 *   b_out  device [q], both in `dtype` (bf16: rounded to nearest even; fp32), 4-byte aligned,
 *          not overlapping each other or the state.
 * The context keeps an fp64 scratch of (P^2 + P Q + Q + 64 P) * 8 bytes, P and Q being p and q
 * rounded up to multiples of 128 (580 MiB at p 8192, q 1024), allocated on first use.  Synchronous:
 * returns after the solve, KVMAP_ERR_NOT_SPD if a pivot was not positive and finite (the
 * outputs are then undefined), INVALID_ARGUMENT / UNSUPPORTED on refused arguments (nothing
 * written).  A state of fewer rows than features has a large null space, and the rounding
 * error of its fp32 statistics can exceed a small lambda in spectral norm (about 13 at p 65,536
 * from 2,048 rows): sym(M_xx) + lambda I is then indefinite, and refused as above. */
int kvmap_ridge_solve_device(kvmap_ctx* ctx, const kvmap_gram_state* st, double lambda, void* W_out,
                             void* b_out, int32_t dtype, void* stream);

/* In-sample R^2 of that ridge fit, pooled over groups of `group` consecutive y columns
 * (one target KV head's head_dim outputs: the per-head score of the layer selection, KVBridge
 * README "What ships": each source layer is scored alone, by R^2 averaged over heads).  For group g
 *   R^2_g = 1 - sum_c RSS_c / sum_c ss_y[c]   over its columns c,
 *   RSS_c = sum_rows (y_c - yhat_c)^2 = ss_y[c] - w_c . M_xy[:, c] - lambda |w_c|^2,
 * the last form following from (M_xx + lambda I) w_c = M_xy[:, c]; it needs the state's
 * ss_y (INVALID_ARGUMENT without it).  The solve is the fp64 one of kvmap_ridge_solve_device
 * (same scratch, plus q doubles).  r2_out: device fp64 [q / group], 8-byte aligned; NaN for a
 * group whose total sum of squares is 0.  group must divide q (SHAPE).  Synchronous;
 * KVMAP_ERR_NOT_SPD as kvmap_ridge_solve_device. */
int kvmap_ridge_r2(kvmap_ctx* ctx, const kvmap_gram_state* st, double lambda, int32_t group, double* r2_out,
                   void* stream);

/* Batched forms of the two device solves above: n >= 1 states of one (p, q), host arrays of
 * n state pointers and n output pointers (the outputs of different systems must not overlap).
 * The library solves up to 16 systems together: every kernel of the factorisation and the
 * substitutions covers all of them, so the serial chain of 64-wide block steps is paid once per
 * batch; the scratch grows to the batch's size (as many systems as fit in about 16 GiB, at least
 * one).  Synchronous; validation of all n before any device work; KVMAP_ERR_NOT_SPD names the
 * first system that failed (outputs of systems in earlier batches are then already written). */
int kvmap_ridge_solve_device_batch(kvmap_ctx* ctx, const kvmap_gram_state* const* states, int32_t n, double lambda,
                                   void* const* W_out, void* const* b_out, int32_t dtype, void* stream);
int kvmap_ridge_r2_batch(kvmap_ctx* ctx, const kvmap_gram_state* const* states, int32_t n, double lambda,
                         int32_t group, double* const* r2_out, void* stream);

/* ---- end-to-end fit: layer selection, then the maps (KVBridge README, fitting section
 * headed "Loading": a two-stage, multi-pass fit over re-iterable calibration data that keeps
 * only centered statistics and bounds memory by blocks of target layers) -------------------
 *
 * Stage 1, selection: for every target layer t and source layer s, single-source ridge maps
 *   from all H*d features of source layer s to all H*d outputs of target layer t, for K and
 *   for V; the in-sample R^2 pooled per target head, averaged over heads and {K, V}, scores
 *   the pair; the k best s per t win (ties to the lower index), kept ascending ("What ships":
 *   the k best-scoring source layers become the concatenated features).  One Gram state per
 *   (group of source layers, K/V) against the rows of a block of target layers: X = the
 *   group's rows (as many layers as fit 65,536 features), Y = the block's rows
 *   (q = block*H*d), M_xx block-diagonal with one H*d block per source layer (xx_block).
 * Stage 2, maps: per (target layer, K/V) the statistics of the selected layers' rows
 *   (p = k*H*d) against the target layer's rows (q = H*d), solved on the device in fp64 into
 *   the apply's layout.
 * One-pass mode (the default when L_src*H*d <= 65,536 and L_tgt*H*d <= 65,536, select_block
 *   covering every target layer, no given selection, two_pass = 0): the stage-1 state keeps the
 *   FULL source Gram (all pairs of source layers) instead of its diagonal blocks, so every map's
 *   statistics are blocks of the stage-1 statistics; the maps are gathered and solved right
 *   after the selection, at the end of the single pass -- one pass over the calibration data.
 * Keys enter every statistic in content space: each model's own RoPE is stripped first
 * (VeloxQuant-MLX "The mapping").  Rows are tokens; columns follow kvmap_cache_rows.
 *
 * Protocol: kvmap_fit_next_pass ends the open pass (if any) and opens the next one; the
 * caller then feeds the SAME calibration sequences, in any order, with kvmap_fit_add, and
 * calls kvmap_fit_next_pass again, until it reports stage 0 (done).  Every pass must see the
 * same number of tokens (SHAPE otherwise). */
typedef struct {
    int32_t L_src, L_tgt, H_kv, head_dim, k;
    int32_t dtype;         /* kvmap_dtype of the calibration caches                          */
    int32_t out_dtype;     /* kvmap_dtype of W and b                                          */
    int32_t select_block;  /* target layers per selection pass; 0 = as many as fit one state
                              (block*H*d <= 65536, <= 128 layers)                              */
    int32_t map_block;     /* target layers per map pass; 0 = all                             */
    int32_t given_sel;     /* nonzero: layer_sel is an input and there is no selection stage;
                              it is read (synchronously) by kvmap_fit_create                   */
    int32_t two_pass;      /* nonzero: never the one-pass mode (see below)                      */
    double theta_src;      /* RoPE bases of the two models (> 0; not read where the matching
                              inv_freq is given)                                               */
    double theta_tgt;
    double lambda;         /* ridge penalty on the unnormalised centered Gram (>= 0)          */
    int32_t* layer_sel;    /* device [L_tgt][k] int32: written by stage 1, or read (given_sel) */
    double* scores;        /* device [L_tgt][L_src] fp64 selection scores, or NULL            */
    void* W_k;             /* device [L_tgt][H*d][k*H*d] output-major, out_dtype              */
    void* b_k;             /* device [L_tgt][H*d], out_dtype                                   */
    void* W_v;
    void* b_v;
    const double* inv_freq_src;  /* optional host [head_dim/2] rotary frequencies of each model
                                    (see kvmap_rope); copied by kvmap_fit_create; NULL = theta  */
    const double* inv_freq_tgt;
} kvmap_fit_config;

typedef struct {
    int32_t stage;         /* 1 selection, 2 maps, 0 done                                     */
    int32_t t_begin;       /* target layers of this pass: [t_begin, t_end)                    */
    int32_t t_end;
    int32_t pass;          /* 0-based index of this pass among all passes                      */
    int32_t passes;        /* total passes of the fit                                          */
} kvmap_fit_pass;

typedef struct kvmap_fit kvmap_fit;

/* Validate cfg and create a fit on ctx (the fit uses ctx's scratch: one fit per context at a
 * time).  Device memory is allocated per stage: stage 1 holds, per K/V and source group,
 * 4*(p + 2q + p*N + p*q) bytes (p = group layers * N, N = H*d, q = block*N), stage 2 holds
 * 2*block states of 4*(F + N + F^2 + F*N) bytes (F = k*N), plus row buffers of T rows.
 * After a failed call the fit is not usable: destroy it.  With
 * given_sel the selection is copied to the host and checked (distinct, in range) here.
 * Synchronous. */
int kvmap_fit_create(kvmap_ctx* ctx, const kvmap_fit_config* cfg, kvmap_fit** out);
/* End the open pass (stage 1: score its block; the last stage-1 pass also selects and
 * writes layer_sel / scores; stage 2: solve its block's maps into W / b) and open the next.
 * Synchronous.  *info describes the pass now open (stage 0: the fit is complete). */
int kvmap_fit_next_pass(kvmap_fit* fit, kvmap_fit_pass* info, void* stream);
/* Feed one calibration sequence of T tokens at positions pos0 .. pos0 + T - 1 to the open
 * pass: src_k/src_v device [L_src][H][T][d], tgt_k/tgt_v device [L_tgt][H][T][d], keys stored
 * rotated by their model, in cfg.dtype, 16-byte aligned.  Asynchronous on `stream`. */
int kvmap_fit_add(kvmap_fit* fit, const void* src_k, const void* src_v, const void* tgt_k, const void* tgt_v,
                  int64_t T, int64_t pos0, void* stream);
/* Free the fit's device memory (synchronises the device). NULL is a no-op. */
int kvmap_fit_destroy(kvmap_fit* fit);

#ifdef __cplusplus
}
#endif

#endif /* KVMAP_H */
