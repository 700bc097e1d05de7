/*
 * fsa.h -- C ABI of libfsa: frame-aligned windowed sparse attention on
 * AMD Instinct MI355X (gfx950).
 *
 * Source of the method: the page "HeyGen 与 Google Cloud：将 Avatar IV 部署到
 * TPU" (news.xcc.im/article/5328), English text. Citations name its section
 * and paragraph (figure captions are not counted as paragraphs).
 *
 * The operation. A chunk of F video frames of T tokens each (N = F*T tokens,
 * frame-major: token n lies in frame n / T) is attended head by head. Queries
 * of frame f see the keys of the frames in
 *     S(f) = { g : 0 <= g < F, |g - f| <= window }  U  { ref_frame }
 * and nothing else ("Deleting the Mask" ¶1), with scores scale * <q_i, k_j>
 * and a softmax over that slice:
 *     O_i = sum_j softmax_j(scale * q_i . k_j) v_j ,  j in frames S(f(i)).
 * The window is clipped at the chunk edges; the reference frame is joined as
 * a set union; the reference frame's own queries see only their own slice;
 * there is no causal masking inside a frame.
 *
 * Route (changes rounding only, never the exact result):
 *  - tiling in blocks that are multiples of 16 tokens and divide T, so each
 *    (query block, key block) tile is entirely inside or outside the mask and
 *    the reference frame is just more full blocks in one pass
 *    ("Deleting the Mask" ¶2);
 *  - keys centred by their mean over the chunk, and a per-row softmax shift
 *    fixed in advance at the Cauchy-Schwarz bound
 *    scale * ||q_i|| * max_{j in slice} ||k_j - mu||, which removes the
 *    running-max rescale ("Unchaining the Softmax" ¶2, ¶3);
 *  - heads whose bound is loose (largest row bound > FSA_ELIG_BETA) use the
 *    online softmax inside the same kernel ("Unchaining the Softmax" ¶3);
 *  - bf16 inputs: the P.V product takes P rounded to bf16, fp32 accumulation
 *    ("Proving the Pixels Didn't Change" ¶2).
 *
 * Cross-attention. A plan made by fsa_plan_create_cross attends every query
 * of the chunk to all M tokens of a separate reference set (K and V of
 * [B][H][M][d]) through the same kernels: the pipeline runs several
 * attention variants, each with a kernel built for its shape ("The
 * Workload, and the Port" ¶2). The same route applies: reference keys
 * centred on their own mean, a fixed per-row shift from the Cauchy-Schwarz
 * bound over the whole reference set, and the online softmax for loose heads
 * (or frames, under FSA_MODE_AUTO_FRAME).
 *
 * Layout. Q, K, V, O are [B][H][N][d] contiguous, d fastest, in the dtype
 * given by the shape; base pointers 16-byte aligned; device memory. For a
 * cross plan K and V are [B][H][M][d].
 *
 * Ownership. The caller owns Q, K, V, O and the workspace (device memory of
 * fsa_workspace_bytes() bytes, 256-byte aligned). The library never frees
 * them, never writes K, and never allocates device memory in fsa_bounds,
 * fsa_forward or fsa_attention. A plan is host memory only.
 *
 * Errors. Every call validates its arguments synchronously before any
 * launch and returns a status; nothing is launched on an error. Kernel faults
 * surface at the caller's next synchronisation. fsa_last_error() gives the
 * calling thread's last error detail. No C++ exception crosses the ABI.
 *
 * Streams. Work is enqueued on the given HIP stream (0 = the null stream)
 * and is asynchronous to the host unless stated.
 */
#ifndef FSA_H
#define FSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FSA_OK = 0,
    FSA_ERR_INVALID_ARG = -1,   /* a value outside its documented range */
    FSA_ERR_UNSUPPORTED = -2,   /* a valid request this build cannot do   */
    FSA_ERR_WORKSPACE = -3,     /* workspace missing, too small, unaligned */
    FSA_ERR_HIP = -4,           /* a HIP runtime call failed              */
    FSA_ERR_NOMEM = -5          /* host allocation failed                 */
} fsa_status;

typedef enum { FSA_BF16 = 0, FSA_F32 = 1 } fsa_dtype;

typedef enum {
    FSA_MODE_AUTO = 0,          /* per head: fixed max if eligible, else online */
    FSA_MODE_ONLINE_ONLY = 1,   /* every head online (the A/B baseline)         */
    FSA_MODE_FIXED_ONLY = 2,    /* every head fixed max (tests: shows why the
                                   fallback exists; loose heads underflow)      */
    FSA_MODE_AUTO_FRAME = 3,    /* per (head, frame): fixed max where every row of
                                   the frame has its bound within FSA_ELIG_BETA,
                                   else online                                   */
    FSA_MODE_AUTO_ROWS = 4,     /* per block of query rows: fixed max where every
                                   row of the block has its gap bound within
                                   FSA_GAP_LIMIT, else online                    */
    FSA_MODE_RECORD_PMAX = 0x100 /* flag OR'ed into a mode (bf16 plans): the
                                   forward also records the largest probability
                                   its fixed route forms into the workspace's
                                   pmax (a check that the fixed shift bounds
                                   every logit: it must not exceed 1 + 2^-8)   */
} fsa_mode;

/* Eligibility threshold on a head's largest row bound, in logit units. */
#define FSA_ELIG_BETA 32.0f
/* Limit on a row's gap bound (FSA_MODE_AUTO_ROWS), in logit units: twice
   FSA_ELIG_BETA, the largest gap between the fixed max and a row's true max
   that the per-head check allows (the logits of a row lie within +-B_i). */
#define FSA_GAP_LIMIT 64.0f
/* Limit, in log2 units, on c ||q_i|| R_S(f) (c = scale * log2 e) for the
   forward's scaled fixed route: a wave of the fixed route whose rows all stay
   within it scores q'_i = bf16(c q_i) against the bound taken on q'_i (one
   exp per probability, no vector arithmetic before it); rounding c q_i moves
   each exponent by at most 2^-9 times this, 2^-4, beyond a part common to the
   row that cancels. Other fixed waves apply the scale per score, exactly.
   ("Unchaining the Softmax" para. 2: the fixed max from precomputed norms.) */
#define FSA_SCALED_LIMIT 32.0f
/* Largest frame count a plan accepts. */
#define FSA_MAX_FRAMES 255

typedef struct {
    int32_t B, H;        /* batch, heads (>= 1)                                */
    int32_t F, T;        /* frames (1..FSA_MAX_FRAMES), tokens per frame
                            (multiple of 16)                                   */
    int32_t d;           /* head width: 64 or 128                              */
    int32_t window;      /* frames on each side of the query frame (>= 0)      */
    int32_t ref_frame;   /* reference frame, 0 <= ref_frame < F                */
    int32_t bq, bk;      /* tile-list block sizes: multiples of 16 dividing T;
                            0 = choose                                         */
    int32_t dtype;       /* fsa_dtype of Q, K, V, O                            */
} fsa_shape;

typedef struct fsa_plan fsa_plan;   /* opaque, host memory only */

/* Byte offsets of the bound products inside a workspace. */
typedef struct {
    size_t mu;      /* key mean, float [B][H][d]                               */
    size_t qnorm;   /* ||q_i||, float [B][H][N]                                */
    size_t rframe;  /* max_{j in frame g} ||k_j - mu||, float [B][H][F]; for a
                       cross plan one value per head over the M reference
                       keys, float [B][H][1]                                   */
    size_t rslice;  /* max over the frames of S(f) of rframe, float [B][H][F]  */
    size_t stat;    /* scale * max_i ||q_i|| rslice(f(i)), float [B][H]        */
    size_t elig;    /* 1 if stat <= FSA_ELIG_BETA else 0, uint8 [B][H]         */
    size_t statf;   /* per frame f: scale * max_{i in f} ||q_i|| rslice(f),
                       float [B][H][F]                                         */
    size_t eligf;   /* 1 if statf <= FSA_ELIG_BETA else 0, uint8 [B][H][F]     */
    size_t dslice;  /* mean key of the slice S(f) minus mu, float [B][H][F][d]
                       (a cross plan: the mean of all M keys minus their mu)   */
    size_t pmax;    /* float [1]: the largest probability the fixed route formed
                       (before rounding to bf16) in the forward launches run
                       with FSA_MODE_RECORD_PMAX since fsa_bounds last wrote
                       ws (which sets it to 0)                                 */
    size_t total;   /* bytes needed (== fsa_workspace_bytes)                   */
} fsa_ws_layout;

/*
 * fsa_plan_create -- build the frame-aligned tile list for a shape
 * ("Deleting the Mask" ¶2): q-blocks of bq tokens and k-blocks of bk tokens,
 * both multiples of 16 that divide T, so no block straddles a frame. Tile
 * (qb, kb) is live iff the frame of kb is in S(frame of qb); a live tile is
 * full by construction. Rows in ascending qb, columns in ascending kb.
 * Host work only (no HIP call); *out is owned by the caller and freed with
 * fsa_plan_destroy. Errors: FSA_ERR_INVALID_ARG (NULL pointers, B, H, F or
 * T < 1, window < 0, ref_frame outside [0,F), bq or bk neither 0 nor a
 * multiple of 16 dividing T, dtype not an fsa_dtype), FSA_ERR_UNSUPPORTED
 * (T % 16 != 0, d not 64 or 128, F above FSA_MAX_FRAMES, B*H*N*d above
 * 2^31 - 1 elements per tensor), FSA_ERR_NOMEM.
 */
fsa_status fsa_plan_create(const fsa_shape* shape, fsa_plan** out);

/*
 * fsa_plan_create_cross -- a plan for cross-attention of the chunk's F*T
 * query tokens to M reference tokens: every query row sees every reference
 * key ("The Workload, and the Port" ¶2: one kernel per attention variant; the
 * key set is not frame-structured, so each frame's slice is the whole set and
 * every tile is live and full). shape->window and shape->ref_frame must be 0;
 * shape->bk, if not 0, is a multiple of 16 dividing M. fsa_bounds and
 * fsa_forward then take K and V of [B][H][M][d]; the bounds centre the
 * reference keys on their own mean and bound every row by
 * scale * ||q_i|| * max_j ||k_j - mu|| over the whole set ("Unchaining the
 * Softmax" ¶2-¶3). Errors: as fsa_plan_create, plus FSA_ERR_INVALID_ARG
 * (M <= 0, window or ref_frame not 0), FSA_ERR_UNSUPPORTED (M % 16 != 0,
 * B*H*M*d above 2^31 - 1 elements).
 */
fsa_status fsa_plan_create_cross(const fsa_shape* shape, int32_t M, fsa_plan** out);
void fsa_plan_destroy(fsa_plan* plan);

/* The shape a plan was built for, with bq and bk resolved. */
fsa_status fsa_plan_shape(const fsa_plan* plan, fsa_shape* out);

/*
 * fsa_plan_export -- copy the tile list out in CSR form (host arrays).
 * row_ptr: int32[n_qblocks + 1]; col_idx: int32[nnz]; qframe: int32[n_qblocks]
 * (frame of each q-block); runs: int32[n_qblocks * 4], per q-block up to two
 * maximal ranges of consecutive live k-blocks as key-token ranges
 * {start0, end0, start1, end1} (unused range = {0, 0}). Any array pointer may
 * be NULL (skipped); n_qblocks and nnz (may be NULL) receive the sizes, so a
 * call with all arrays NULL is a size query.
 */
fsa_status fsa_plan_export(const fsa_plan* plan, int32_t* row_ptr, int32_t* col_idx,
                           int32_t* qframe, int32_t* runs,
                           int32_t* n_qblocks, int64_t* nnz);

/* Valid (query, key) pairs of one (batch, head): T^2 * sum_f |S(f)|, or
   N * M for a cross plan. -1 for a NULL plan. */
int64_t fsa_plan_valid_pairs(const fsa_plan* plan);

/* Key (and value) tokens per (batch, head) the plan's K and V hold: N = F*T,
   or M for a cross plan. -1 for a NULL plan. */
int64_t fsa_plan_key_tokens(const fsa_plan* plan);

/*
 * fsa_plan_row_block -- query rows one workgroup of the bf16 forward kernel
 * computes for this plan: consecutive rows of one frame, 256 (8 waves of 32
 * rows, one workgroup per CU sharing each staged key chunk) or 128 (4 waves,
 * two workgroups per CU). FSA_MODE_AUTO_ROWS decides the route per such
 * block. 1 for an fp32 plan (one row per thread), -1 for a NULL plan. The
 * geometry changes only how rows are grouped, never the result's arithmetic
 * per row ("Unchaining the Softmax" ¶3: block shapes re-tuned with the
 * softmax).
 */
int32_t fsa_plan_row_block(const fsa_plan* plan);

/*
 * fsa_plan_set_row_block -- replace the plan's own choice of row block
 * (rows = 128 or 256; 0 restores the plan's choice; an fp32 plan accepts only
 * 0 or 1). For measurement and tests. Not thread-safe against calls using the
 * same plan; plans cached by fsa_attention are never changed.
 * Errors: FSA_ERR_INVALID_ARG (NULL plan, another value).
 */
fsa_status fsa_plan_set_row_block(fsa_plan* plan, int32_t rows);

/* Workspace size in bytes for this plan, and where each product lives. */
size_t fsa_workspace_bytes(const fsa_plan* plan);
fsa_status fsa_workspace_layout(const fsa_plan* plan, fsa_ws_layout* out);

/*
 * fsa_bounds -- per (batch, head): key mean mu over all N keys (fp32, fixed
 * reduction order), per-frame max ||k_j - mu|| (fp32, from the keys as
 * given), per-slice max, row norms ||q_i||, the head statistic and its
 * eligibility flag ("Unchaining the Softmax" ¶2, ¶3), and per slice the
 * offset of its mean key from mu (dslice) for the gap bound of
 * FSA_MODE_AUTO_ROWS. Q and K are only read (no centred copy of K is
 * written); results go to ws.
 * scale > 0 and finite. Deterministic: no atomics, fixed reduction trees.
 * Errors: FSA_ERR_INVALID_ARG (NULL plan/pointers, bad scale),
 * FSA_ERR_WORKSPACE (ws NULL or not 256-byte aligned), FSA_ERR_HIP.
 */
fsa_status fsa_bounds(const fsa_plan* plan, const void* Q, const void* K, void* ws,
                      float scale, hipStream_t stream);

/*
 * fsa_forward -- the attention itself, one launch. Reads Q, K, V and the
 * bound products in ws (mu, qnorm, rslice, elig, eligf, dslice) written by
 * fsa_bounds (or fsa_bounds_after_prep) for the same plan, inputs and scale;
 * writes O. Per (batch, head), mode picks the
 * route: AUTO takes the fixed max where elig = 1 and the online softmax
 * elsewhere (the per-head check of "Unchaining the Softmax" ¶3); AUTO_FRAME
 * decides per (batch, head, frame) from eligf instead, a finer check that is
 * as safe (every row of the frame has its bound within FSA_ELIG_BETA) and
 * keeps the frames of a loose head that never see its outlier keys on the
 * fixed route. AUTO_ROWS decides per block of query rows (a run of at most
 * 256 consecutive rows of one frame, the rows one workgroup computes; one row
 * in the fp32 kernel) from each row's gap bound
 * G_i = B_i - scale q_i.(dslice(f)), B_i the row's Cauchy-Schwarz bound: a
 * row's largest logit is at least the mean of its logits over its slice
 * ("Unchaining the Softmax" ¶3: each row sees its own slice), so the fixed max
 * exceeds it by at most G_i <= 2 B_i. A block takes the fixed max when every
 * row has G_i <= FSA_GAP_LIMIT, which is the gap the per-head check allows,
 * so the guarantee is the same row by row while looser heads keep most of
 * their rows on the fixed route. Both routes score the keys as given. The fixed-max route shifts
 * row i by its Cauchy-Schwarz bound on the centred scores plus scale q_i.mu:
 * centring by mu moves every score of the row by that same amount, so the
 * softmax is unchanged and the shift bounds the raw scores ("Unchaining the
 * Softmax" ¶2, ¶3). O must not overlap Q, K, V or ws.
 * Errors: FSA_ERR_INVALID_ARG (NULL pointers, bad scale or mode, misaligned
 * tensors, O overlapping an input), FSA_ERR_WORKSPACE, FSA_ERR_HIP.
 */
fsa_status fsa_forward(const fsa_plan* plan, const void* Q, const void* K, const void* V,
                       void* O, const void* ws, float scale, int32_t mode, hipStream_t stream);

/*
 * fsa_copy_eligibility -- copy the B*H eligibility flags (uint8, 1 = the head
 * takes the fixed-max route under AUTO; index b*H + h) that fsa_bounds wrote
 * into ws, to host memory at host_out (caller-owned, at least B*H bytes). The
 * copy is ordered on `stream` after the work already queued there, and the
 * call returns once the flags are on the host (it synchronizes the stream).
 * The flag is the per-head check of "Unchaining the Softmax" ¶3: the head's
 * largest row bound is at most FSA_ELIG_BETA.
 * Errors: FSA_ERR_INVALID_ARG (NULL plan or host_out), FSA_ERR_WORKSPACE (ws
 * NULL or not 256-byte aligned), FSA_ERR_HIP (copy or synchronization failed,
 * including a fault of earlier work on the stream).
 */
fsa_status fsa_copy_eligibility(const fsa_plan* plan, const void* ws, uint8_t* host_out,
                                hipStream_t stream);

/*
 * fsa_attention -- fsa_bounds then fsa_forward with a plan built for the
 * given shape and cached per shape (bq = bk = 0, the cache is guarded by a
 * mutex; this is the only call that allocates, host memory, on a cache miss).
 * ws must hold at least fsa_workspace_bytes() of that plan (ws_bytes says how
 * much it holds). Errors as fsa_plan_create, fsa_bounds and fsa_forward.
 */
fsa_status fsa_attention(const void* Q, const void* K, const void* V, void* O,
                         int32_t F, int32_t T, int32_t window, int32_t ref_frame,
                         float scale, int32_t B, int32_t H, int32_t d, int32_t dtype,
                         int32_t mode, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes fsa_attention needs for this shape (0 on invalid input). */
size_t fsa_attention_workspace_bytes(int32_t F, int32_t T, int32_t window, int32_t ref_frame,
                                     int32_t B, int32_t H, int32_t d, int32_t dtype);

/*
 * fsa_cross_attention -- fsa_bounds then fsa_forward with a cross plan
 * (fsa_plan_create_cross, bq = bk = 0) cached per shape: O [B][H][F*T][d] of
 * the queries Q [B][H][F*T][d] attending to all M reference tokens of
 * Kr, Vr [B][H][M][d]. Same ownership, workspace and error rules as
 * fsa_attention; FSA_ERR_INVALID_ARG also for M <= 0.
 */
fsa_status fsa_cross_attention(const void* Q, const void* Kr, const void* Vr, void* O,
                               int32_t F, int32_t T, int32_t M, float scale, int32_t B,
                               int32_t H, int32_t d, int32_t dtype, int32_t mode, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/* Workspace bytes fsa_cross_attention needs for this shape (0 on invalid input). */
size_t fsa_cross_attention_workspace_bytes(int32_t F, int32_t T, int32_t M, int32_t B, int32_t H,
                                           int32_t d, int32_t dtype);

/*
 * fsa_attention_static -- for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * fsa_bounds then fsa_forward on `plan` (made beforehand by
 * fsa_plan_create or fsa_plan_create_cross, so this call allocates nothing,
 * host or device), with a workspace that is a static device array of
 * FSA_STATIC_WS_BYTES inside the library instead of the caller's. Each GPU
 * holds its own copy until the process ends. Every call on a GPU shares that
 * GPU's array and leaves its contents behind (nothing in it needs to start at
 * zero: fsa_bounds writes every product the forward reads), so calls that
 * overlap on one GPU (other threads, other streams) race; serialize them.
 * Same arguments, layout and checks as fsa_attention with the plan given.
 * Errors: FSA_ERR_WORKSPACE (the plan's workspace exceeds
 * FSA_STATIC_WS_BYTES), FSA_ERR_HIP (no current device, or the array's
 * address could not be taken), and those of fsa_bounds and fsa_forward.
 */
#define FSA_STATIC_WS_BYTES (16u << 20)
fsa_status fsa_attention_static(const fsa_plan* plan, const void* Q, const void* K, const void* V,
                                void* O, float scale, int32_t mode, hipStream_t stream);

/* Drop every cached plan of fsa_attention and fsa_cross_attention. Safe to
   call while other threads are inside those calls: a call keeps the plan it
   looked up until it returns. */
void fsa_cache_clear(void);

/*
 * The producer of the attention's inputs ("Layout Is the ABI" ¶2: the chain
 * of normalization, rotary embeddings, projections and head packing that
 * feeds attention is fused into one kernel writing its consumer's layout).
 * Per token n of the chunk (C = H*d channels; frame-major on a latent grid of
 * grid_h x grid_w patches per frame, T = grid_h*grid_w):
 *   x_hat = x / sqrt(mean_c x_c^2 + 1e-6) * gamma;  y = W x_hat;
 *   q, k, v = channels [0,C), [C,2C), [2C,3C) of y; head h = [h*d, (h+1)*d);
 *   q and k turned by the 3-D rotary embedding of the token's (frame t,
 *   row y, column x): the head splits into bands of d/4 (t), 3d/8 (y) and
 *   3d/8 (x) channels, and inside a band of n_b channels with coordinate p,
 *   channel pair (2i, 2i+1) turns by p * 10000^(-2i/n_b) radians.
 * The bounds' inputs come out of the same kernel: ||q_i|| of the rounded
 * queries and per-tile column sums of the rounded keys ("Unchaining the
 * Softmax" ¶2), so fsa_bounds_after_prep replaces fsa_bounds and no longer
 * reads Q.
 */

/* Bytes of the packed producer weights for H heads of width d: 3*C*C bf16. */
size_t fsa_prep_weight_bytes(int32_t H, int32_t d);

/*
 * fsa_prep_pack_weights -- fold the RMSNorm weight into the projection once:
 * Wp[o][c] = bf16(W[o][c] * gamma[c]). W: bf16 [3C][C] (output channel major:
 * rows [0,C) queries, [C,2C) keys, [2C,3C) values), gamma: float [C], Wp:
 * bf16 [3C][C] (fsa_prep_weight_bytes), device memory, caller-owned, Wp not
 * overlapping W. Errors: FSA_ERR_INVALID_ARG (NULL, misaligned, H < 1,
 * overlap), FSA_ERR_UNSUPPORTED (d != 128), FSA_ERR_HIP.
 */
fsa_status fsa_prep_pack_weights(const void* W, const float* gamma, void* Wp, int32_t H,
                                 int32_t d, hipStream_t stream);

/*
 * fsa_prep -- Q, K, V [B][H][F*T][d] bf16 of the tokens X [B][F*T][C] bf16
 * under the packed weights Wp, for a self-attention plan of d = 128, bf16;
 * also writes the row norms ||q_i|| (the workspace's qnorm) and the keys'
 * per-tile column sums (private workspace) for fsa_bounds_after_prep.
 * Outputs must not overlap each other, X, Wp or ws. Errors:
 * FSA_ERR_INVALID_ARG (NULL, misaligned, overlap, grid_h*grid_w != T),
 * FSA_ERR_UNSUPPORTED (a cross plan, d != 128 or not bf16),
 * FSA_ERR_WORKSPACE, FSA_ERR_HIP.
 */
fsa_status fsa_prep(const fsa_plan* plan, int32_t grid_h, int32_t grid_w, const void* X,
                    const void* Wp, void* Q, void* K, void* V, void* ws, hipStream_t stream);

/*
 * fsa_bounds_after_prep -- what fsa_bounds computes (mu, radii, statistics,
 * flags in ws), from the statistics fsa_prep left in ws and one read of K.
 * Call it after fsa_prep on the same plan, K and workspace; then fsa_forward.
 * Errors as fsa_bounds, and FSA_ERR_UNSUPPORTED as fsa_prep.
 */
fsa_status fsa_bounds_after_prep(const fsa_plan* plan, const void* K, void* ws, float scale,
                                 hipStream_t stream);

const char* fsa_status_string(fsa_status status);
/* Detail of the calling thread's last failed call ("" if none). */
const char* fsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FSA_H */
