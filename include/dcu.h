/*
 * dcu.h -- C ABI of the selective token cache library for MI355X (gfx950).
 *
 * The library implements, as hand-written HIP kernels, one denoising step of Dynamic Cache
 * Updating (DCU) for masked-diffusion LLMs and the Frechet-profile commit rule that ends the step:
 *
 *   dcu_budget           per-layer recompute budgets from the previous step's layer means
 *   dcu_distance         per-token cosine distance between a layer's input now and its cached input
 *                        from the previous step, plus the per-group mean (layer dynamics)
 *   dcu_distance_rows    the same on listed rows only, with the cache roll (closed-loop layers)
 *   dcu_select           per-sequence top-B selection by distance, united with forced windows
 *   dcu_selective_layer  QKV / attention / output projection / SwiGLU FFN on the selected rows only,
 *                        with K/V and output rows scattered back into caller-owned caches
 *   dllm_confidence      per-position softmax confidence and argmax over the vocabulary
 *   frechet_commit       sort, prefix sum and the Frechet margin rule -> how many positions commit
 *   dllm_commit          the same with the factor, threshold or per-position threshold rule
 *   dllm_apd             adaptive-parallel-decoding signals and per-position thresholds
 *   dllm_commit_positions  committed positions -> the next step's key positions
 *   dcu_v_features, dcu_attention_context  other distance features (Value vectors, attention
 *                        contexts of every row)
 *   dcu_pack_weights, dcu_pack_gate_up, dcu_pack_qkv   the projections' blocked weight layout (set-up)
 *
 * Sources: "Dynamic-dLLM: Dynamic Cache-Budget and Adaptive Parallel Decoding for Training-Free
 * Acceleration of Diffusion LLM" (reading notes), Key designs 1-2; "Fast-dLLM++: Frechet Profile
 * Decoding for Faster Diffusion LLM Inference" (reading notes), Key designs 1-3.
 *
 * Conventions (every entry point):
 *  - Every pointer is a DEVICE pointer to caller-owned memory, row-major and contiguous, aligned
 *    to 16 bytes, unless stated otherwise. bf16 tensors are raw 16-bit patterns.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue work and return;
 *    outputs are valid once the stream reaches that point; inputs must stay alive until then.
 *  - The library never allocates device memory and keeps no pointer past a call. Its one piece of
 *    mutable global state is the scratch of dcu_selective_layer_noalloc (a device array per GPU,
 *    see there); every other call is reentrant and thread-safe. Outputs must not alias inputs
 *    except for the documented in/out buffers.
 *  - All argument checks happen on the host before any launch: a non-zero status means nothing
 *    was enqueued, except DCU_EHIP, which reports a failed launch.
 *  - NaN or Inf inputs are a caller error; the results are then unspecified.
 */
#ifndef DCU_H
#define DCU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DCU_OK = 0,
  DCU_EINVAL = 1,       /* null pointer, non-positive size, value out of range            */
  DCU_EUNSUPPORTED = 2, /* a valid request outside what the kernels implement (see below) */
  DCU_EWORKSPACE = 3,   /* workspace missing or smaller than the *_workspace query says   */
  DCU_EHIP = 4          /* a kernel launch failed (hipGetLastError has the detail)        */
};

enum { DCU_F32 = 0, DCU_BF16 = 1 };

/* Text for a status code (static storage; never NULL). */
const char* dcu_status_string(int status);
/* Library version, major*10000 + minor*100 + patch. */
int dcu_version(void);

/*
 * dcu_budget -- per-layer budgets of one step.
 * Dynamic-dLLM notes, Key design 1 (DCU), budget equation: the total T = b_layer * L of each
 * sequence is split across the L layers in proportion to the previous step's layer means.
 *
 * s_prev  [L, B] fp32 layer means of the previous step, layer-major (each layer's dcu_distance
 *         call writes its B means contiguously), or NULL for "no previous step". A mean is never
 *         negative (an average of distances in [0, 2]); a negative entry is read as 0.
 * budget  [B, L] int32 out. Each row sums to exactly T: floor of T*s/sum(s) plus one for the
 *         largest remainders (ties to the lower layer), computed in IEEE fp64 in a fixed order.
 *         A NULL s_prev, or a row whose means sum to 0, gives b_layer to every layer.
 * Errors: EINVAL if budget is NULL, B <= 0, L <= 0, b_layer < 0 or b_layer*L overflows int32;
 *         EUNSUPPORTED if L > 1024.
 */
int dcu_budget(const float* s_prev, int32_t B, int32_t L, int32_t b_layer, int32_t* budget,
               void* stream);

/*
 * dcu_distance -- token cosine distance and group mean.
 * Dynamic-dLLM notes, Key design 1 (DCU): d_i = 1 - <x_i^t, x_i^{t+1}> / (|x_i^t| |x_i^{t+1}|)
 * between a token's layer input now (x_cur) and at the previous step (x_prev); the layer dynamics
 * s = (1/N) sum_i d_i.
 *
 * x_cur, x_prev  [G, N, d] of dtype DCU_BF16 or DCU_F32 (G groups, e.g. sequences or layers).
 * dist           [G, N] fp32 out. Accumulated in fp64; bitwise-identical rows give exactly 0,
 *                two zero rows give 0, exactly one zero row gives 1; clamped to [0, 2].
 * mean           [G] fp32 out, or NULL: (sum over the fp32 dist of the group, in fp64) / N.
 * Errors: EINVAL on NULL x_cur/x_prev/dist or G, N, d <= 0 or a bad dtype;
 *         EUNSUPPORTED if d is not a multiple of 8 (bf16) or 4 (fp32), or a pointer is not
 *         16-byte aligned.
 */
int dcu_distance(const void* x_cur, const void* x_prev, int32_t dtype, int64_t G, int64_t N,
                 int64_t d, float* dist, float* mean, void* stream);

/*
 * dcu_distance_rows -- dcu_distance when only listed rows can have changed (closed-loop layers).
 * Dynamic-dLLM notes, Key design 2 (a token not updated at layer l keeps its cached output, so its
 * input to layer l+1 is unchanged and its distance there is 0): when layer l+1's input is layer l's
 * output buffer, only the rows layer l scattered can differ from the cached input, so only those
 * are read.
 * x_cur, x_prev  [B, N, d] (dtype DCU_BF16 or DCU_F32), not overlapping. Every row not listed must
 *                be bitwise equal in both (the caller's guarantee; its distance is reported as 0).
 * sel_idx, sel_count  [B, N] / [B] int32: the listed positions of each sequence (each at most
 *                once; counts clamped to [0, N]; entries outside [0, N) skipped), e.g. the previous
 *                layer's dcu_select output.
 * dist     [B, N] fp32 out: bit for bit dcu_distance's value on every row under that guarantee.
 * roll     non-zero: afterwards each listed row of x_cur is copied into x_prev (the cache roll of
 *          the rows that changed; the others are already equal).
 * The layer mean is then available from dcu_select (mean argument), which reads every distance.
 * One launch: each workgroup marks its sequence's listed positions in an LDS bitmap and writes
 * 0 for the unlisted positions it covers.
 * Errors: EINVAL on NULL pointers, B, N, d <= 0 or a bad dtype; EUNSUPPORTED if d is not a
 *         multiple of 8 (bf16) or 4 (fp32), a pointer is not 16-byte aligned, B > 65535 or
 *         N > 65536.
 */
int dcu_distance_rows(const void* x_cur, void* x_prev, int32_t dtype, int64_t B, int64_t N,
                      int64_t d, const int32_t* sel_idx, const int32_t* sel_count, float* dist,
                      int32_t roll, void* stream);

/*
 * dcu_select -- recompute set of one layer for each sequence.
 * Dynamic-dLLM notes, Key design 1 (top-B tokens by distance are recomputed, the rest reuse their
 * cached values) and Key design 2 (forced update window around each key token unmasked at the
 * previous step; the remaining budget is spent outside the window).
 *
 * dist      [B, N] fp32 distances of this layer (from dcu_distance).
 * budgets   [B, L] int32; column `layer` is this layer's budget b (negative values count as 0).
 * key_pos   [B, P] int32 positions unmasked at the previous step; values outside [0, N) are
 *           ignored (-1 = unused). May be NULL when P == 0.
 * b_window  window size: positions [p - b_window/2, p - b_window/2 + b_window - 1] clipped to
 *           [0, N) are always selected (b_window/2 rounds down).
 * sel_idx   [B, N] int32 out: ascending positions W u A, where A is the top-min(b, |C|) of the
 *           candidates C = {i not in W : dist_i > 0} ranked by (dist desc, position asc).
 *           Entries past sel_count[b] are set to -1.
 * sel_count [B] int32 out.
 * mean      [B] fp32 out, or NULL: the layer dynamics s of each sequence (Key design 1), bit for
 *           bit what dcu_distance writes to its `mean` for the same dist (same fp64 sums, same
 *           order), so a step can take s here and call dcu_distance with mean = NULL (one launch
 *           fewer per layer).
 * Errors: EINVAL on NULL pointers, B, N, L <= 0, P < 0, b_window < 0, layer outside [0, L);
 *         EUNSUPPORTED if N > 8192.
 */
int dcu_select(const float* dist, const int32_t* budgets, int32_t L, int32_t layer,
               const int32_t* key_pos, int32_t P, int32_t B, int32_t N, int32_t b_window,
               int32_t* sel_idx, int32_t* sel_count, float* mean, void* stream);

/*
 * dcu_pack_weights -- write one projection matrix in the blocked layout the layer reads.
 * (A data layout of this library, not an operation of the method: the projections of a layer are
 * the matrices of the pre-norm transformer layer below.)
 * w      [rows, cols] bf16 row-major: an [out, in] projection matrix. Not modified.
 * out    rows * cols bf16, caller-owned, must not overlap w. Block (g, t) holds rows
 *        16g .. 16g+15 and columns 64t .. 64t+63 at element offset (g * (cols/64) + t) * 1024;
 *        inside a block, columns 64t+8c .. 64t+8c+7 of row 16g+r sit at element offset
 *        (16c + r) * 8. A pure permutation (no arithmetic); the device buffers must stay valid
 *        until the work on `stream` completes.
 * Errors: EINVAL on NULL pointers or rows, cols <= 0; EUNSUPPORTED if rows % 16 != 0,
 *         cols % 64 != 0, rows * cols >= 2^40, or a pointer not 16-byte aligned.
 */
int dcu_pack_weights(const void* w, int32_t rows, int32_t cols, void* out, void* stream);

/*
 * dcu_pack_gate_up -- the gate and up matrices of the SwiGLU FFN as one blocked matrix.
 * (A data layout of this library, as dcu_pack_weights.)
 * w_gate, w_up  [F, d] bf16 row-major each. Not modified.
 * out    2 * F * d bf16, caller-owned, overlapping neither input: the [2F, d] matrix whose 16-row
 *        groups alternate gate group g, up group g (rows 32g .. 32g+15 = gate rows 16g .. 16g+15,
 *        rows 32g+16 .. 32g+31 = up rows 16g .. 16g+15), written in the blocked layout of
 *        dcu_pack_weights. (The gate and up rows of the same outputs sit next to each other, so the
 *        FFN's weight stream is one contiguous range per tile.)
 * Errors: EINVAL on NULL pointers or F, d <= 0; EUNSUPPORTED if F % 16 != 0, d % 64 != 0,
 *         2 * F * d >= 2^40, or a pointer not 16-byte aligned.
 */
int dcu_pack_gate_up(const void* w_gate, const void* w_up, int32_t F, int32_t d, void* out,
                     void* stream);

/*
 * dcu_pack_qkv -- W_qkv in the blocked layout for a layer with rotary position embedding.
 * (A data layout of this library, as dcu_pack_weights. Rotary embedding is not part of the
 * Dynamic-dLLM notes; it belongs to the LLaMA-family models, LLaDA among them, that the notes'
 * diffusion LLMs are built on, and turns each pair (i, i + head_dim/2) of a head's q and k.)
 * w_qkv  [3d, d] bf16 row-major, rows Wq | Wk | Wv. Not modified.
 * out    3 * d * d bf16, caller-owned, must not overlap w_qkv: the blocked layout of
 *        dcu_pack_weights applied to the matrix whose Q and K rows are reordered inside every head
 *        in groups of 16 (with h = head_dim/2: head dims 0..15, h..h+15, 16..31, h+16..h+31, ...),
 *        so that the two dims of a rotation pair are outputs 16 apart within one 32-row group; the
 *        V rows keep their order.
 * Errors: EINVAL on NULL pointers, d or head_dim <= 0, d % head_dim != 0; EUNSUPPORTED if
 *         head_dim not in {32, 64, 128}, d % 64 != 0, 3 * d * d >= 2^40, or a pointer not 16-byte
 *         aligned.
 */
int dcu_pack_qkv(const void* w_qkv, int32_t d, int32_t head_dim, void* out, void* stream);

/* dcu_layer.weight_layout: the layouts the layer accepts. BLOCKED: all matrices from
 * dcu_pack_weights / dcu_pack_gate_up, no rotary embedding (rope_theta must be 0). BLOCKED_ROPE:
 * W_qkv from dcu_pack_qkv, the rest as BLOCKED, rotary embedding with base rope_theta (> 0). */
#define DCU_WEIGHTS_BLOCKED 1
#define DCU_WEIGHTS_BLOCKED_ROPE 2

/*
 * One pre-norm transformer layer (bf16 weights; W[out, in] below means the [out, in] matrix
 * written in the blocked layout of dcu_pack_weights):
 *   xn = RMSNorm(x; g_attn), [q|k|v] = xn W_qkv^T, o = softmax(q K^T / sqrt(head_dim)) V per head
 *   over all N cached rows (no mask), a = x + o W_o^T, an = RMSNorm(a; g_ffn),
 *   y = a + (silu(an W_gate^T) * (an W_up^T)) W_down^T.
 * With DCU_WEIGHTS_BLOCKED_ROPE, q and k of a row at position p (its index in the sequence) are
 * rotated before k is cached and attention runs: in every head, dims i and i + head_dim/2 turn by
 * p * rope_theta^(-2i/head_dim) radians (x_i cos - x_{i+h} sin, x_{i+h} cos + x_i sin). The cache
 * holds rotated keys in the standard [head, dim] order.
 */
typedef struct {
  int32_t d;          /* model width, = n_heads * head_dim          */
  int32_t n_heads;
  int32_t head_dim;   /* 32, 64 or 128                                */
  int32_t ffn;        /* FFN width F                                  */
  float rms_eps;
  const void* w_qkv;  /* bf16 [3d, d] blocked: rows Wq | Wk | Wv      */
  const void* w_o;    /* bf16 [d, d] blocked                          */
  const void* w_gate_up; /* bf16 [2F, d]: gate and up, dcu_pack_gate_up */
  const void* w_down; /* bf16 [d, F] blocked                          */
  const void* g_attn; /* bf16 [d] RMSNorm gain before attention       */
  const void* g_ffn;  /* bf16 [d] RMSNorm gain before the FFN         */
  int32_t weight_layout; /* DCU_WEIGHTS_BLOCKED or DCU_WEIGHTS_BLOCKED_ROPE */
  float rope_theta;   /* rotary base (BLOCKED_ROPE), 0 with BLOCKED     */
} dcu_layer;

/* Workspace bytes dcu_selective_layer needs for these shapes (max_rows <= 0 means B*N). */
size_t dcu_selective_layer_workspace(const dcu_layer* w, int32_t B, int32_t N, int32_t max_rows);

/*
 * dcu_selective_layer -- recompute the selected rows of one layer.
 * Dynamic-dLLM notes, Key design 1 (DCU): only the selected tokens are recomputed; every other
 * token keeps its cached K, V and output. Attention is bidirectional over all cached rows.
 *
 * x_in      [B, N, d] bf16 layer input (only selected rows are read).
 * sel_idx   [B, N] int32 ascending positions and sel_count [B] int32 (from dcu_select), or both
 *           NULL for every row (dense mode). Counts are clamped to [0, N]. A listed position
 *           outside [0, N) (e.g. a -1 pad) is skipped: nothing is read or written for it, and it
 *           is not counted in rows_done.
 * max_rows  host-side upper bound on sum(sel_count) used to size the workspace (<= 0: B*N).
 *           If the device counts exceed it, only the first max_rows entries in (sequence,
 *           position) order are processed; rows_done shows what was recomputed.
 * k_cache, v_cache  [B, N, n_heads, head_dim] bf16 IN/OUT: selected rows are overwritten before
 *           attention reads the cache; other rows are untouched.
 * y_out     [B, N, d] bf16 IN/OUT: selected rows get the layer output; other rows are untouched.
 * workspace device scratch of at least dcu_selective_layer_workspace() bytes (256-byte aligned),
 *           owned by the caller; its contents on entry do not matter. Calls that share a
 *           workspace must be ordered (same stream): it holds the row map, activations and
 *           split-K partial tiles of one call.
 * rows_done [B] int32 out, or NULL: the number of rows of each sequence actually recomputed
 *           (listed positions inside [0, N) among the entries that fit in max_rows).
 * Results are bitwise reproducible for a given device: every reduction runs in a fixed order.
 * Errors: EINVAL on NULL pointers or non-positive sizes, only one of sel_idx/sel_count NULL,
 *         d != n_heads*head_dim, rms_eps < 0, rope_theta not 0 with DCU_WEIGHTS_BLOCKED or not
 *         positive and finite with DCU_WEIGHTS_BLOCKED_ROPE; EUNSUPPORTED if weight_layout is
 *         neither, head_dim not in {32, 64, 128}, d or ffn not a multiple of 64, N > 65536, B > 4096, B*N > 2^28, or a pointer not 16-byte
 *         aligned;
 *         EWORKSPACE if the workspace is too small or not 256-byte aligned.
 */
int dcu_selective_layer(const dcu_layer* w, const void* x_in, const int32_t* sel_idx,
                        const int32_t* sel_count, int32_t B, int32_t N, int32_t max_rows,
                        void* k_cache, void* v_cache, void* y_out, void* workspace,
                        size_t workspace_bytes, int32_t* rows_done, void* stream);

/*
 * dcu_selective_layer_noalloc -- dcu_selective_layer for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same computation (same kernels, same results bit for bit) with its scratch in a device
 * array the library owns instead of a caller workspace; it calls no allocating routine.
 * The array holds DCU_NOALLOC_SCRATCH_BYTES on every GPU the library runs on, until the process
 * ends; its address is looked up on the first call for a device (the device of `stream`).
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and must be ordered by the caller. Its contents on entry do not matter.
 * Arguments, outputs and errors as dcu_selective_layer, plus EWORKSPACE when the scratch these
 * shapes need (dcu_selective_layer_workspace(w, B, N, max_rows)) exceeds
 * DCU_NOALLOC_SCRATCH_BYTES: a LLaDA-8B-shaped layer (d 4096, 32 heads of 128, FFN 12288) fits
 * with max_rows <= 64 (one sequence: budget 32 + window 32) up to N = 8192; pass max_rows.
 */
#define DCU_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int dcu_selective_layer_noalloc(const dcu_layer* w, const void* x_in, const int32_t* sel_idx,
                                const int32_t* sel_count, int32_t B, int32_t N, int32_t max_rows,
                                void* k_cache, void* v_cache, void* y_out, int32_t* rows_done,
                                void* stream);

/*
 * dcu_attention_context -- the attention context of every row of a layer, for an attention-context
 * distance. (DyLLM, in the pages' listing of related papers, finds its salient tokens by the cosine
 * similarity of attention contexts between adjacent denoising steps; apply dcu_distance to ctx_out
 * and the previous step's contexts.)
 * For every row of x_in: xn = RMSNorm(x; g_attn), q = xn W_q^T (rotated by the row's position with
 * DCU_WEIGHTS_BLOCKED_ROPE), ctx = softmax(q K^T / sqrt(head_dim)) V per head over the N cached
 * rows of its sequence, with W_q the rows 0 .. d-1 of the layer's blocked W_qkv.
 * x_in      [B, N, d] bf16.
 * k_cache, v_cache  [B, N, n_heads, head_dim] bf16, read only (the caches as given; not updated).
 * ctx_out   [B, N, d] bf16 out (heads contiguous), caller-owned.
 * workspace at least dcu_selective_layer_workspace(w, B, N, B*N) bytes, 256-byte aligned.
 * Errors: as dcu_selective_layer; EINVAL on a NULL x_in, cache or ctx_out.
 */
int dcu_attention_context(const dcu_layer* w, const void* x_in, int32_t B, int32_t N,
                          const void* k_cache, const void* v_cache, void* ctx_out, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * dcu_v_features -- the Value vectors of every row of a layer, for the V-feature distance.
 * (The alternative distance feature of the dLLM-Cache design the Dynamic-dLLM notes compare their
 * input proxy against: the cosine distance is taken between this step's Value vectors, recomputed
 * for all N rows, and the cached ones; apply dcu_distance to v_out and the V cache.)
 * v_out = RMSNorm(x; g_attn) W_v^T for all B*N rows, [B, N, d] bf16 (the V-cache row layout), with
 * W_v the rows 2d .. 3d-1 of the layer's blocked W_qkv.
 * workspace  at least dcu_selective_layer_workspace(w, B, N, B*N) bytes, 256-byte aligned.
 * Errors: as dcu_selective_layer (layer shape, alignment, workspace).
 */
int dcu_v_features(const dcu_layer* w, const void* x_in, int32_t B, int32_t N, void* v_out,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * dcu_selective_layer_staged -- dcu_selective_layer with per-stage timing marks, for measurement.
 * Identical work and results; additionally records the caller-created hipEvent_t events[0] before
 * the first kernel and events[i] after stage i on `stream`, for the DCU_LAYER_STAGES stages
 *   1 row offsets and map + gather + RMSNorm, 2 QKV projection + K/V scatter,
 *   3 its split-tail fixup, 4 attention (+ split combine), 5 output projection + residual,
 *   6 its fixup (empty when the split tiles are finished inside stage 7: rows of up to 4096
 *   values, or of up to 8192 under a row bound of at most 64), 7 RMSNorm, 8 gate/up projection +
 *   SwiGLU, 9 its fixup, 10 down projection + residual + scatter, 11 its fixup.
 *   Under a row bound (max_rows) of at most 64 with rows of up to 8192 values (rotary head_dim up
 *   to 128), stage 2 also does the work of stage 1, which is then empty, and stage 3 is empty.
 * (A fixup kernel finishes the tiles whose K range was split over idle workgroups; it exits at
 * once when the projection did not split.)
 * events may be NULL (then this is dcu_selective_layer); otherwise n_events must be at least
 * DCU_LAYER_STAGES + 1 (EINVAL), and a NULL entry skips that mark (each recorded event costs a
 * few microseconds of device time, so a caller timing one stage passes only its two events).
 * A failed event record returns DCU_EHIP.
 */
#define DCU_LAYER_STAGES 11
int dcu_selective_layer_staged(const dcu_layer* w, const void* x_in, const int32_t* sel_idx,
                               const int32_t* sel_count, int32_t B, int32_t N, int32_t max_rows,
                               void* k_cache, void* v_cache, void* y_out, void* workspace,
                               size_t workspace_bytes, int32_t* rows_done, void* stream,
                               void* const* events, int32_t n_events);

/*
 * dllm_confidence -- confidence and argmax of each candidate position.
 * Fast-dLLM++ notes, Key designs (overall framework): each masked position takes the argmax of its
 * predicted distribution and that argmax's probability as its confidence c_i.
 *
 * logits  [R, ld] of dtype DCU_BF16 or DCU_F32; the first V columns of each row are used.
 * conf    [R] fp32 out: 1 / sum_v exp(z_v - max z) (temperature 1; fp64 row accumulation).
 * token   [R] int32 out: the lowest index attaining max z.
 * Errors: EINVAL on NULL pointers, R <= 0, V <= 0, ld < V, bad dtype; EUNSUPPORTED if ld is not
 *         a multiple of 8 (bf16) or 4 (fp32), or V > 2^31 - 1.
 */
int dllm_confidence(const void* logits, int32_t dtype, int64_t R, int64_t V, int64_t ld,
                    float* conf, int32_t* token, void* stream);

/*
 * frechet_commit -- how many candidates commit this step.
 * Fast-dLLM++ notes, Key design 1 (Theorem 4.1: L_n = max{0, sum_{j<=n} c_(j) - (n-1)},
 * U_n = 1 - c_(n)) and Key design 2 (n* = max{n : L_n - U_n > delta}, else 1).
 *
 * conf      [B, m] fp32 confidences; only the first m_valid[b] slots of row b are candidates.
 * m_valid   [B] int32 (values clamped to [0, m]), or NULL for m everywhere.
 * delta     margin, >= 0.
 * n_commit  [B] int32 out: n* (0 when a row has no candidates).
 * order     [B, m] int32 out: candidate slots sorted by (conf desc, slot asc); the first
 *           n_commit[b] commit; entries past m_valid[b] are -1.
 * Prefix sums are fp64 and exact whenever every c is 0 or in [2^-17, 1] (always true for
 * dllm_confidence outputs); otherwise they are taken sequentially in sorted order.
 * Errors: EINVAL on NULL conf/n_commit/order, B <= 0, m <= 0, delta < 0 or NaN;
 *         EUNSUPPORTED if m > 8192.
 */
int frechet_commit(const float* conf, const int32_t* m_valid, int32_t B, int32_t m, double delta,
                   int32_t* n_commit, int32_t* order, void* stream);

/*
 * dllm_commit -- frechet_commit under a choice of rule, for comparing the rules on the same step.
 * Fast-dLLM++ notes, motivation (the two rules of Fast-dLLM's confidence-aware parallel decoding,
 * which the Frechet rule generalises) and Key designs 1-2:
 *   DCU_COMMIT_FRECHET    param = delta >= 0: exactly frechet_commit;
 *   DCU_COMMIT_FACTOR     param = f: n* = max{n : (n+1)(1 - c_(n)) < f} (fp64), else 1;
 *   DCU_COMMIT_THRESHOLD  param = tau: every candidate with c_i >= tau (fp64), at least 1; these
 *                         are the first n* entries of `order`;
 *   DCU_COMMIT_TAU        per-candidate thresholds tau [B, m] fp32 (adaptive parallel decoding,
 *                         Dynamic-dLLM notes Key design 3, from dllm_apd): every candidate with
 *                         c_i >= tau_i commits (fp32 compare), at least 1 (the most confident);
 *                         `order` lists the passing candidates first, then the others, each group
 *                         by (conf desc, slot asc); param is ignored.
 * tau is read only for DCU_COMMIT_TAU (NULL otherwise). Other arguments, outputs (n_commit is 0 for
 * a row without candidates; for the first three rules order is frechet_commit's) and limits as
 * frechet_commit.
 * Errors: EINVAL on NULL conf/n_commit/order, B <= 0, m <= 0, an unknown rule, a NaN or infinite
 *         param, delta < 0, or DCU_COMMIT_TAU without tau; EUNSUPPORTED if m > 8192.
 */
#define DCU_COMMIT_FRECHET 0
#define DCU_COMMIT_FACTOR 1
#define DCU_COMMIT_THRESHOLD 2
#define DCU_COMMIT_TAU 3
int dllm_commit(const float* conf, const int32_t* m_valid, int32_t B, int32_t m, int32_t rule,
                double param, const float* tau, int32_t* n_commit, int32_t* order, void* stream);

/*
 * dllm_commit_positions -- the positions committed this step, as the next step's key positions.
 * Dynamic-dLLM notes, Key design 2: the forced window sits around each position unmasked at the
 * previous step; this closes the loop from a commit to the next step's dcu_select.
 * order, n_commit  [B, m] / [B] int32 from frechet_commit or dllm_commit.
 * slot_pos  [B, m] int32: the sequence position of each candidate slot.
 * key_pos   [B, P] int32 out: the positions of the first min(n_commit[b], P) committed slots (the
 *           most confident first), -1 after them.
 * Errors: EINVAL on NULL pointers or B, m, P <= 0.
 */
int dllm_commit_positions(const int32_t* order, const int32_t* n_commit, const int32_t* slot_pos,
                          int32_t B, int32_t m, int32_t P, int32_t* key_pos, void* stream);

/*
 * dllm_apd -- adaptive-parallel-decoding signals and per-position thresholds of one step.
 * Dynamic-dLLM notes, Key design 3: with z the softmax distribution (temperature 1) of a position,
 * concentration c = 1 - max_{v != argmax} z_v, temporal instability H = 1 - cos(z^t, z^{t+1})
 * against the previous step's distribution, and tau^t = tau^{t+1} - alpha c + beta H.
 *
 * logits       [R, ld] of dtype DCU_BF16 or DCU_F32, this step; the first V columns are used.
 * logits_prev  the same positions' logits of the previous step (same shape and dtype), or NULL at
 *              the first step (then H = 0).
 * alpha, beta  >= 0 (the page leaves them open).
 * tau          [R] fp32 in/out: tau^{t+1} in (initialise near 0.9), tau^t out.
 * zmax         [R] fp32 in/out: in, the previous step's row max of logits_prev (read only when
 *              logits_prev is given; it is what this call wrote last step); out, this step's.
 * conf, token  [R] out: the largest probability and its (lowest) index, as dllm_confidence.
 * c_conc, h_instab  [R] fp32 out, or NULL: c and H.
 * Sums of exponentials are fp32 per 8 terms, fp64 across them; the cosine uses
 * D / sqrt(Q P) with D = sum e q, Q = sum e^2, P = sum q^2 (e, q the unnormalised softmax terms).
 * Errors: EINVAL on NULL logits/tau/zmax/conf/token, R <= 0, V <= 0, ld < V, a bad dtype, alpha
 *         or beta negative, NaN or infinite; EUNSUPPORTED if ld is not a multiple of 8 (bf16) or
 *         4 (fp32), a pointer is not 16-byte aligned, or V > 2^31 - 17.
 */
int dllm_apd(const void* logits, const void* logits_prev, int32_t dtype, int64_t R, int64_t V,
             int64_t ld, float alpha, float beta, float* tau, float* zmax, float* conf,
             int32_t* token, float* c_conc, float* h_instab, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DCU_H */
