/*
 * nhmamba.h -- C ABI of libnhmamba, the Nemotron-H Mamba2 mixer block on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  The mixer block of the Nemotron-H language model whose
 * configuration is printed on the issue page "feat(nemotron_voicechat): load
 * the VoiceChat checkpoint and run offline duplex inference ... #1374",
 * section "config.json" (text_config: hidden_size 4480, mamba_num_heads 128,
 * mamba_head_dim 80, ssm_state_size 128, n_groups 8, conv_kernel 4,
 * use_conv_bias true, mamba_proj_bias false, layer_norm_epsilon 1e-5, and the
 * 4-bit group-64 quantization of the mixer projections).  The block is
 *     out = x + out_proj( RMSNormGated( SSM( silu(conv1d(xBC)) ), z ) ),
 *     [z | xBC | dt_raw] = in_proj( RMSNorm(x) ),
 * the standard Mamba2 mixer (Dao & Gu 2024, "Transformers are SSMs").  Two
 * modes are exported, which the docs page "Nemotron VoiceChat", section
 * "Offline timeline", says give the same tokens: a cached per-position step
 * and a full-history recompute (here a chunked SSD scan).
 *
 * Conventions for every entry point.
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing; scratch memory is a caller-provided workspace whose
 *    size is returned by nh_*_workspace_bytes.
 *  - bf16 tensors are passed as uint16_t bit patterns; fp32 as float.
 *  - Tensor pointers must be 16-byte aligned (NH_ERR_MISALIGNED otherwise);
 *    row strides ("ld", in elements) must keep every row 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work; they never synchronise the host.
 *  - Arguments are validated before anything is enqueued.  On failure the
 *    call returns a non-zero nh_status, enqueues nothing and changes nothing;
 *    nh_last_error() then returns a message (thread-local).  NH_ERR_HIP means
 *    a launch failed; device memory may then be partially written.
 *  - Weights are read-only and may be shared by concurrent calls.  A state
 *    (nh_mamba_state) and a workspace must not be used by two calls that can
 *    run at the same time.
 *  - Results are deterministic for fixed inputs on a fixed device (no
 *    floating-point atomics).
 *  - Internal operands are fp16 where noted.  The chunked scan and the W4
 *    GEMM need their activations within the fp16 range (|v| < 65504), and
 *    magnitudes below 2^-14 keep only fp16 subnormal precision.  The W4 GEMM
 *    dequantises exactly for scales 2^-17 <= |s| <= 8188 (or s = 0).
 *  - W4 GEMV activations are staged in fp16 chunks of 32.  nh_w4_gemv (and
 *    the MLP down and attention o_proj projections) scale each chunk by an
 *    exact power of two, so every finite bf16 input is exact.  The pre-normed
 *    projections stage u = x / rms(x) * w, with |u| <= sqrt(d) max|w|.  These
 *    are in_proj, MLP up, attention q/k/v, the heads and out_proj.  They need
 *    max|w| < 978 for the hidden-size norms and < 1830 for the gated norm.
 *    None of these ranges is checked at run time.
 */
#ifndef NHMAMBA_H
#define NHMAMBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NH_OK = 0,
    NH_ERR_INVALID_ARGUMENT = 1,   /* NULL pointer, negative size, bad enum */
    NH_ERR_UNSUPPORTED_SHAPE = 2,  /* dims outside the supported set */
    NH_ERR_MISALIGNED = 3,         /* pointer or stride not 16-byte aligned */
    NH_ERR_WORKSPACE_TOO_SMALL = 4,
    NH_ERR_HIP = 5                 /* a HIP launch reported an error */
} nh_status;

typedef enum { NH_BF16 = 0, NH_F32 = 1 } nh_dtype;

/* Block dimensions.  Supported set: hidden 4480, n_heads 128, head_dim 80,
 * d_state 128, n_groups 8, conv_k 4 (text_config, issue page "config.json");
 * chunk (scan chunk length Q) 1..256; eps > 0 (1e-5 in text_config). */
typedef struct {
    int hidden, n_heads, head_dim, d_state, n_groups, conv_k, chunk;
    float eps;
} nh_mamba_dims;

/* Affine 4-bit weight matrix in the MLX layout (issue page "config.json":
 * group_size 64, bits 4; a quantized linear carries .scales).
 *   W[n][k] = scales[n][k/64] * q[n][k] + biases[n][k/64],
 *   q[n][k] = (qweight[n][k/8] >> 4*(k%8)) & 15   (lowest nibble first).
 * qweight: u32 [n_out][k_in/8]; scales, biases: bf16 [n_out][k_in/64].
 * Requirements: group_size == 64, k_in % 64 == 0, k_in <= 16384, and the
 * packed matrix under 2 GiB (n_out * k_in / 2 < 2^31 bytes). */
typedef struct {
    const uint32_t *qweight;
    const uint16_t *scales;
    const uint16_t *biases;
    int n_out, k_in, group_size;
} nh_w4_matrix;

/* Weights of one block (mamba_proj_bias false: the projections have no bias). */
typedef struct {
    const uint16_t *norm_w;   /* bf16 [hidden]: pre-norm weight */
    nh_w4_matrix in_proj;     /* [2*d_inner + 2*G*N + H][hidden] = [22656][4480] */
    const uint16_t *conv_w;   /* bf16 [conv_dim][conv_k], tap conv_k-1 multiplies the newest
                                 input (the [channels, 4, 1] layout of the issue page,
                                 "Network 2", flattened) */
    const uint16_t *conv_b;   /* bf16 [conv_dim] (use_conv_bias true) */
    const float *dt_bias;     /* f32 [n_heads] */
    const float *A_log;       /* f32 [n_heads]; A = -exp(A_log) */
    const float *D;           /* f32 [n_heads] */
    const uint16_t *gnorm_w;  /* bf16 [d_inner]: gated-norm weight */
    nh_w4_matrix out_proj;    /* [hidden][d_inner] = [4480][10240] */
} nh_mamba_weights;

/* Per-sequence recurrent state of one block (the "Mamba2 state" a session
 * keeps per position, docs page "Nemotron VoiceChat", "Online session"). */
typedef struct {
    uint16_t *conv_state; /* bf16 [batch][conv_k-1][conv_dim]; row 0 oldest */
    float *ssm_state;     /* f32 [batch][n_heads][head_dim][d_state], d_state fastest */
} nh_mamba_state;

/* ------------------------------------------------------------- library */

/* The message of the calling thread's last failed call (thread-local; empty
 * after a success).  Bad arguments are rejected at the boundary, before any
 * work, as the session calls of the docs page "Nemotron VoiceChat", section
 * "Online session", reject bad input. */
const char *nh_last_error(void);
/* Library name, version and target (gfx950). */
const char *nh_version(void);
/* The hybrid_override_pattern of text_config (issue page, section
 * "config.json"): 'M' Mamba2, '*' attention, '-' MLP, 56 layers. */
const char *nh_hybrid_pattern(void);

/* Measurement hook for the per-position step (docs page, section
 * "Performance": the language stage's time per position is the figure of
 * merit).  events: NULL (off) or an array of n >= 6 hipEvent_t
 * created by the caller.  While set, every nh_mamba_block_step call on this
 * thread records events[2i] on its stream right before kernel i (0: fused
 * pre-norm/in_proj/conv, 1: SSM step + gated-norm partial sums, 2: gated
 * norm/out_proj/residual) and launches that kernel with events[2i+1] stamped
 * at its own end (hipExtLaunchKernelGGL), so hipEventElapsedTime(events[2i],
 * events[2i+1]) is the kernel's duration plus its dispatch.  Returns NH_ERR_INVALID_ARGUMENT for n < 6 or a
 * NULL event. */
nh_status nh_profile_events(void *const *events, int n);

/* ---------------------------------------------------------- primitives */

/* y = W x (+ residual): the W4 dequantising matrix-vector product for small
 * batches, the per-position decode of the in_proj / out_proj rows of the
 * scope (issue page, section "config.json": 4-bit, group 64; docs page,
 * "Online session": one position at a time).  x: [batch][k_in] of x_dtype
 * (fp32 values are rounded to bf16, the activation precision of every
 * projection here); residual: nullable, [batch][n_out] of res_dtype; y:
 * [batch][n_out] of y_dtype (fp32 accumulation, one rounding at the end).
 * Any finite x (each 32-value chunk is staged in fp16 after an exact
 * power-of-two scaling).  batch 1..4. */
nh_status nh_w4_gemv(const nh_w4_matrix *W, const void *x, nh_dtype x_dtype, int batch,
                     const void *residual, nh_dtype res_dtype,
                     void *y, nh_dtype y_dtype, void *stream);

/* Y = X W^T (+ residual): the W4 matrix product for whole sequences, the
 * full-history recompute's in_proj / out_proj (docs page "Nemotron
 * VoiceChat", section "Offline timeline"; issue page, section "config.json":
 * 4-bit, group 64).  X: bf16 [M][k_in] (|x| < 65504); residual: nullable
 * [M][n_out] of res_dtype; Y: [M][n_out] of y_dtype.  M >= 1.  Needs
 * nh_w4_gemm_workspace_bytes(M, k_in) bytes of workspace.  Matrix-core
 * arithmetic; W is dequantised exactly for 2^-17 <= |scale| <= 8188, and
 * the products are exact with fp32 accumulation; for asymmetric groups the
 * offset term (beta + 8 s) * sum(x over the group) is formed and added in
 * fp32. */
size_t nh_w4_gemm_workspace_bytes(int M, int k_in);
nh_status nh_w4_gemm(const nh_w4_matrix *W, const uint16_t *X, int M,
                     const void *residual, nh_dtype res_dtype,
                     void *Y, nh_dtype y_dtype, void *ws, size_t ws_bytes, void *stream);

/* u = RMSNorm(x) * w, rounded to bf16: the block's pre-norm (issue page,
 * section "config.json": layer_norm_epsilon 1e-5).  x: [rows][d] of x_dtype;
 * w, u: bf16.  RMS over the d values of a row, eps inside the square root. */
nh_status nh_rmsnorm(const void *x, nh_dtype x_dtype, const uint16_t *w, uint16_t *u,
                     int rows, int d, float eps, void *stream);

/* The front of one block step as one fused kernel: u = RMSNorm(x) * norm_w
 * (bf16), zxbcdt = in_proj(u) (W4 GEMV, fp32 sums), split into z | xBC | dt_raw
 * (Nemotron-H issue page, section "config.json": d_inner 10240, 8 groups x
 * state 128, 128 heads); xBC goes through the conv step (as nh_conv1d_step,
 * state shifted in place) and SiLU.  x: [batch][hidden] of x_dtype; outputs
 * bf16: z [batch][d_inner], xc [batch][conv_dim] (x | B | C after conv and
 * SiLU), dt_raw [batch][n_heads].  Uses w->norm_w, in_proj, conv_w, conv_b
 * and state->conv_state only.  batch 1..4; outputs may not alias x. */
nh_status nh_inproj_conv_step(const nh_mamba_dims *d, const nh_mamba_weights *w,
                              nh_mamba_state *state, const void *x, nh_dtype x_dtype,
                              uint16_t *z, uint16_t *xc, uint16_t *dt_raw, int batch,
                              void *stream);

/* One position of the causal depthwise conv1d (kernel k, with bias) + SiLU
 * (issue page, section "config.json": conv_kernel 4, use_conv_bias true;
 * section "Network 2": the [channels, 4, 1] weight layout).
 * xbc: bf16, row b at xbc + b*ld (channels values); conv_state: bf16
 * [batch][k-1][channels], row 0 oldest, updated in place (shifted by one,
 * the new input appended); w: bf16 [channels][k], tap k-1 newest; b: bf16
 * [channels]; out: bf16 [batch][channels].  k == 4. */
nh_status nh_conv1d_step(const uint16_t *xbc, long ld, uint16_t *conv_state,
                         const uint16_t *w, const uint16_t *b, uint16_t *out,
                         int batch, int channels, int k, void *stream);

/* The same conv over T positions (the full-history recompute, docs page,
 * section "Offline timeline").  xbc row (b, t) at xbc + (b*T + t)*ld;
 * state_in: nullable bf16 [batch][k-1][channels] (NULL = zeros);
 * state_out: nullable, receives the last k-1 pre-conv rows (may not alias
 * state_in); out: bf16 [batch][T][channels]. */
nh_status nh_conv1d_seq(const uint16_t *xbc, long ld, int T, const uint16_t *state_in,
                        uint16_t *state_out, const uint16_t *w, const uint16_t *b,
                        uint16_t *out, int batch, int channels, int k, void *stream);

/* One position of the selective SSM (issue page, section "config.json":
 * mamba_num_heads 128, mamba_head_dim 80, ssm_state_size 128, n_groups 8;
 * docs page, "Online session": the state carried from position to
 * position).  xc: bf16 [batch][conv_dim], the
 * post-conv x | B | C; dt_raw: bf16, row b at dt_raw + b*ld_dt (n_heads
 * values).  dt = softplus(dt_raw + dt_bias), A = -exp(A_log); for head h
 * (group g = h / (n_heads/n_groups)):
 *   S[h][p][:] = exp(dt*A) * S[h][p][:] + dt * x[h*P+p] * B[g][:]
 *   y[h*P+p]   = C[g][:] . S[h][p][:] + D[h] * x[h*P+p]
 * ssm_state: f32 [batch][H][P][N], updated in place; y: [batch][d_inner] of
 * y_dtype.  batch 1..64. */
nh_status nh_ssm_step(const nh_mamba_dims *d, const uint16_t *xc, const uint16_t *dt_raw,
                      long ld_dt, const float *dt_bias, const float *A_log, const float *D,
                      float *ssm_state, void *y, nh_dtype y_dtype, int batch, void *stream);

/* The same recurrence over T positions (docs page, "Offline timeline": the
 * full-history recompute gives the cached step's tokens), computed as a
 * chunked SSD scan with
 * chunk length d->chunk (intra-chunk quadratic form, chunk states, sequential
 * state passing; Dao & Gu 2024).  Equals the per-position recurrence up to
 * rounding for every chunk length.
 * xc: bf16 [batch][T][conv_dim]; dt_raw: bf16, row (b, t) at
 * dt_raw + (b*T + t)*ld_dt; h0: nullable f32 [batch][H][P][N] (NULL = zero
 * state); h_final: nullable, receives the state after position T-1 (may
 * alias h0); y: [batch][T][d_inner] of y_dtype.
 * ws: caller-owned device workspace of at least
 * nh_ssd_scan_workspace_bytes(d, batch, T) bytes (16-byte aligned), which
 * receives the per-group C.B^T tiles of every chunk (at most 8 KiB per
 * position, for chunks of at most 16 rows); for chunks of at least 128 rows
 * in sequences of at least 64 positions also B and C in the matrix-core
 * operand order and each head's per-chunk decay tables (about 8 KiB per
 * position in all at chunk 256; never above 10 KiB per position).  Its
 * contents on return are
 * unspecified.  A smaller ws fails with NH_ERR_WORKSPACE_TOO_SMALL before
 * any launch. */
size_t nh_ssd_scan_workspace_bytes(const nh_mamba_dims *d, int batch, int T);
nh_status nh_ssd_chunk_scan(const nh_mamba_dims *d, const uint16_t *xc, const uint16_t *dt_raw,
                            long ld_dt, int T, const float *dt_bias, const float *A_log,
                            const float *D, const float *h0, float *h_final, void *y,
                            nh_dtype y_dtype, int batch, void *ws, size_t ws_bytes,
                            void *stream);

/* Gated RMSNorm (issue page, section "config.json": n_groups 8,
 * layer_norm_epsilon 1e-5; Mamba2's norm before out_proj): g = y * silu(z);
 * every block of `group` channels is normalised by its own RMS (eps inside
 * the root) and multiplied by its slice of w.  y: [rows][d] of y_dtype; z:
 * bf16, row r at z + r*ld_z; w: bf16 [d]; out: bf16 [rows][d].
 * d % group == 0, group % 8 == 0, group <= 8192. */
nh_status nh_rmsnorm_gated(const void *y, nh_dtype y_dtype, const uint16_t *z, long ld_z,
                           const uint16_t *w, uint16_t *out, int rows, int d, int group,
                           float eps, void *stream);

/* ----------------------------------------------------------- model top */

/* One MLP layer of the hybrid stack, per position, for `batch` sequences
 * (issue page, section "config.json": the '-' layers of hybrid_override_pattern
 * are MLPs with intermediate_size 15680 and mlp_bias false, quantized like the
 * mixer projections; the pages do not name the activation, and squared ReLU,
 * Nemotron-H's, is the reading taken):
 *   u = bf16(RMSNorm(x) * norm_w), h = bf16(relu(up u)^2), out = x + down h
 * with fp32 sums.  up: [inter][4480], down: [4480][inter], inter % 64 == 0
 * and <= 16384; x: [batch][4480] of x_dtype; out: [batch][4480] of out_dtype
 * (may not alias x).  ws: at least nh_mlp_workspace_bytes(inter, batch)
 * bytes (holds h).  batch 1..4; every pointer 16-byte aligned.  Errors
 * before any launch as for the other entry points. */
size_t nh_mlp_workspace_bytes(int inter, int batch);
nh_status nh_mlp_step(const uint16_t *norm_w, const nh_w4_matrix *up, const nh_w4_matrix *down, float eps,
                      const void *x, nh_dtype x_dtype, void *out, nh_dtype out_dtype, int batch,
                      void *ws, size_t ws_bytes, void *stream);

/* The language model's input row for `batch` positions (issue page, section
 * "Network 2": embed_tokens row of the previous text id, plus the projected
 * audio frame, plus function_channel_weight (2.0 in the config) times the
 * embed_tokens row of the previous function id):
 *   out[b] = E[text_ids[b]] + audio[b] + function_weight * E[function_ids[b]]
 * with E rows dequantised to fp32 (E[n][k] = s q + b, one rounding) and the
 * sums taken in fp32 in that order.  E: any W4 matrix (k_in = the hidden
 * size for the model); text_ids, function_ids: int32 [batch] device arrays;
 * audio: [batch][k_in] of audio_dtype; out: f32 [batch][k_in].  An id
 * outside 0 .. n_out-1 gives a row of NaN (no out-of-table read).
 * batch 1 .. 4096; every pointer 16-byte aligned; function_weight finite.
 * Errors before any launch: NH_ERR_UNSUPPORTED_SHAPE, NH_ERR_MISALIGNED,
 * NH_ERR_INVALID_ARGUMENT. */
nh_status nh_fused_embedding(const nh_w4_matrix *E, const int32_t *text_ids,
                             const int32_t *function_ids, const void *audio,
                             nh_dtype audio_dtype, float function_weight, int batch,
                             float *out, void *stream);

/* One attention layer of the hybrid stack, per position, for `batch`
 * sequences (issue page, section "config.json": the '*' layers of
 * hybrid_override_pattern, num_attention_heads 40, num_key_value_heads 8,
 * head_dim 128, attention_bias false; the projections are 4-bit group-64 like
 * the mixer's; no positional encoding is named, so none is applied).  The
 * docs page "Nemotron VoiceChat", section "Online session", keeps the
 * attention key/value caches across positions.  With fp32 sums:
 *   u = bf16(RMSNorm(x) * norm_w),
 *   q = bf16(q_proj u), k = bf16(k_proj u), v = bf16(v_proj u),
 *   k and v are written into the cache at index positions[b],
 *   o[h] = bf16(softmax_t(q[h] . K[h/5][t] / sqrt(128)) V[h/5]) over cache
 *          indices t = 0 .. positions[b] (query head h reads key/value head
 *          h / 5),
 *   out = x + o_proj o.
 * positions: int32 [batch] DEVICE array, the cache index of this position per
 * sequence (the caller advances it; indices below it must hold the earlier
 * positions' k and v).  A position outside 0 .. max_len-1 writes nothing to
 * the cache and gives a row of NaN in out.  x: [batch][4480] of x_dtype; out:
 * [batch][4480] of out_dtype (may not alias x).  ws: at least
 * nh_attention_workspace_bytes(batch) bytes, contents on return unspecified.
 * batch 1..4; every pointer 16-byte aligned.  Five kernels on `stream`.
 * Errors before any launch: NH_ERR_UNSUPPORTED_SHAPE (projection shapes,
 * max_len outside 1 .. 2^22, batch), NH_ERR_WORKSPACE_TOO_SMALL,
 * NH_ERR_MISALIGNED, NH_ERR_INVALID_ARGUMENT (NULL pointer, dtype, eps <= 0,
 * out == x). */
typedef struct {
    const uint16_t *norm_w;   /* bf16 [hidden]: pre-norm weight */
    nh_w4_matrix q_proj;      /* [40*128][hidden] = [5120][4480] */
    nh_w4_matrix k_proj;      /* [8*128][hidden] = [1024][4480] */
    nh_w4_matrix v_proj;      /* [1024][4480] */
    nh_w4_matrix o_proj;      /* [hidden][5120] = [4480][5120] */
} nh_attention_weights;

/* Key/value cache of one attention layer; k and v: bf16
 * [batch][8][max_len][128] each (key/value head, then cache index, then the
 * head dimension), owned by the caller. */
typedef struct {
    uint16_t *k, *v;
    int max_len;
} nh_kv_cache;

size_t nh_attention_workspace_bytes(int batch);
nh_status nh_attention_step(const nh_attention_weights *w, const nh_kv_cache *cache,
                            const int32_t *positions, const void *x, nh_dtype x_dtype, void *out,
                            nh_dtype out_dtype, int batch, float eps, void *ws, size_t ws_bytes,
                            void *stream);

/* The attention core of nh_attention_step on its own (same kernels): for
 * every sequence b and query head h,
 *   o[b][h] = bf16(softmax_t(q[b][h] . K[b][h/5][t] / sqrt(128)) V[b][h/5])
 * over cache indices t = 0 .. positions[b], with fp32 scores and sums.
 * q, o: bf16 [batch][40][128]; cache and positions as in nh_attention_step
 * (the cache already holds index positions[b]; nothing is written to it).  A
 * position outside 0 .. max_len-1 gives a row of NaN.  ws: at least
 * nh_attention_decode_workspace_bytes(batch) bytes.  batch 1..64; errors
 * before any launch as for nh_attention_step. */
size_t nh_attention_decode_workspace_bytes(int batch);
nh_status nh_attention_decode(const uint16_t *q, const nh_kv_cache *cache, const int32_t *positions,
                              uint16_t *o, int batch, void *ws, size_t ws_bytes, void *stream);

/* One position of the language model (issue page, section "Network 2"): the
 * fused input row, the 56 layers of hybrid_override_pattern in order, norm_f,
 * both heads and their greedy ids.  'M' layers run nh_mamba_block_step
 * (state updated in place), '-' layers nh_mlp_step, '*' layers
 * nh_attention_step (cache written at positions[b]).  The residual stream
 * between layers is fp32. */
typedef struct {
    const uint16_t *norm_w;   /* bf16 [hidden] */
    nh_w4_matrix up;          /* [inter][hidden] */
    nh_w4_matrix down;        /* [hidden][inter] */
} nh_mlp_weights;

typedef struct {
    nh_w4_matrix embed;                 /* [vocab][hidden]: embed_tokens */
    const nh_mamba_weights *mamba;      /* host array, one per 'M' of the pattern (27) */
    const nh_mlp_weights *mlp;          /* host array, one per '-' of the pattern (25) */
    const nh_attention_weights *attn;   /* host array, one per '*' of the pattern (4) */
    const uint16_t *norm_f;             /* bf16 [hidden] */
    nh_w4_matrix lm_head, function_head; /* [vocab][hidden] each */
    float function_weight;              /* function_channel_weight, 2.0 in the config */
} nh_lm_weights;

/* Workspace bytes of nh_lm_step for MLP width `inter` at this batch (0 on bad
 * arguments). */
size_t nh_lm_workspace_bytes(const nh_mamba_dims *d, int inter, int batch);
/* states: host array, one per 'M' layer, updated in place.  caches: host
 * array, one per '*' layer; positions: int32 [batch] device array, the cache
 * index of this position (shared by the 4 attention layers; the caller
 * advances it).  text_ids,
 * function_ids: int32 [batch] (the previous ids); audio: [batch][hidden] of
 * audio_dtype; hidden_out: nullable f32 [batch][hidden] (the stream before
 * norm_f); text_out, function_out: int32 [batch] (greedy ids as in
 * nh_head_argmax).  batch 1..4; every pointer 16-byte aligned. */
nh_status nh_lm_step(const nh_mamba_dims *d, const nh_lm_weights *w, nh_mamba_state *states,
                     const nh_kv_cache *caches, const int32_t *positions,
                     const int32_t *text_ids, const int32_t *function_ids, const void *audio,
                     nh_dtype audio_dtype, int batch, float *hidden_out, int32_t *text_out,
                     int32_t *function_out, void *ws, size_t ws_bytes, void *stream);

/* Final norm, one output head and the greedy id for `batch` positions
 * (issue page, section "Network 2": after the last layer the hidden state
 * goes through norm_f, then through lm_head and function_head, both 4-bit
 * [4480 -> 131072] matrices without a linear bias; the text and function ids
 * are the argmax of the last position, with no sampling).  Call it once per
 * head.
 *   h = bf16(x / rms(x) * norm_w)   (RMS over the 4480 values, eps inside
 *                                    the root)
 *   logits[b][n] = W[n] . h[b]      (fp32 accumulation)
 *   ids[b] = the smallest n holding the largest logits[b][n]; NaN logits
 *            are never chosen, and a row of NaN logits gives -1.
 * W: k_in == 4480, n_out 1 .. 524288; x: [batch][4480] of x_dtype; norm_w:
 * bf16 [4480]; logits: nullable f32 [batch][n_out] (NULL: not stored);
 * ids: int32 [batch]; ws: caller-owned device workspace of at least
 * nh_head_workspace_bytes(batch) bytes, contents on return unspecified.
 * batch 1..4.  Every pointer 16-byte aligned.  Two kernels on `stream`; the
 * ids are bitwise deterministic.  Errors (checked before any launch):
 * NH_ERR_UNSUPPORTED_SHAPE for k_in, n_out or batch outside these ranges,
 * NH_ERR_WORKSPACE_TOO_SMALL, NH_ERR_MISALIGNED, NH_ERR_INVALID_ARGUMENT for
 * NULL pointers, an unknown dtype or eps <= 0. */
size_t nh_head_workspace_bytes(int batch);
nh_status nh_head_argmax(const nh_w4_matrix *W, const void *x, nh_dtype x_dtype,
                         const uint16_t *norm_w, float eps, int batch, float *logits,
                         int32_t *ids, void *ws, size_t ws_bytes, void *stream);

/* -------------------------------------------------------------- blocks */

#define NH_MODE_STEP 0
#define NH_MODE_SEQ 1

/* Workspace bytes for nh_mamba_block_step (mode NH_MODE_STEP, T ignored) or
 * nh_mamba_block_seq (NH_MODE_SEQ) at this batch and T; 0 on bad arguments.
 * (Each entry point that needs scratch has its own size function: the sizes
 * depend on different arguments.) */
size_t nh_block_workspace_bytes(const nh_mamba_dims *d, int batch, int T, int mode);

/* One position of the whole Mamba2 block for `batch` independent sequences
 * (docs page, "Online session": the cached per-position step; issue page,
 * "config.json": the block's dimensions):
 * out = x + mixer(RMSNorm(x)), state updated in place.
 * x: [batch][hidden] of x_dtype; out: [batch][hidden] of out_dtype (may not
 * alias x).  Storage points: the normalised input, the in_proj output, the
 * conv output, y and the gated-norm output are rounded to bf16; dt, the
 * state and the out_proj accumulator are fp32.  batch 1..4. */
nh_status nh_mamba_block_step(const nh_mamba_dims *d, const nh_mamba_weights *w,
                              nh_mamba_state *state, const void *x, nh_dtype x_dtype,
                              void *out, nh_dtype out_dtype, int batch,
                              void *ws, size_t ws_bytes, void *stream);

/* nh_mamba_block_step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same computation, kernels and results as nh_mamba_block_step,
 * but the step workspace is the library's own file-scope device array
 * (1 MiB per GPU, held until the process ends), so no workspace argument
 * is taken and nothing is allocated or freed.  Every call on one GPU shares
 * that GPU's array: calls that can overlap on one GPU (two streams, two
 * threads) race and must be serialised by the caller.  The array keeps the
 * last call's contents; nothing in it has to start at zero.  batch 1..4
 * (NH_ERR_UNSUPPORTED_SHAPE above that, the array's limit); other errors as
 * nh_mamba_block_step; NH_ERR_HIP if the array's address cannot be looked up
 * on the current device. */
nh_status nh_mamba_block_step_noalloc(const nh_mamba_dims *d, const nh_mamba_weights *w,
                                      nh_mamba_state *state, const void *x, nh_dtype x_dtype,
                                      void *out, nh_dtype out_dtype, int batch, void *stream);

/* The whole block over T positions (full-history recompute, docs page,
 * section "Offline timeline") with the same
 * storage points.  init: nullable (NULL = zero conv and SSM state);
 * final_state: nullable, receives the state after position T-1 (its
 * buffers may be init's).  x: [batch][T][hidden]; out: [batch][T][hidden]. */
nh_status nh_mamba_block_seq(const nh_mamba_dims *d, const nh_mamba_weights *w,
                             const nh_mamba_state *init, nh_mamba_state *final_state,
                             const void *x, nh_dtype x_dtype, int T, void *out,
                             nh_dtype out_dtype, int batch, void *ws, size_t ws_bytes,
                             void *stream);

/* A stack of n_layers Mamba2 blocks applied in order (issue page,
 * "config.json", hybrid_override_pattern: the M layers of the
 * hybrid pattern; attention and MLP layers are not part of this library and
 * act as identity between them).  The residual stream between blocks is
 * fp32: layer i reads layer i-1's output and writes
 * outs + i*batch*T*hidden (f32).  weights, states: host arrays of n_layers
 * entries (states[i] is used in place by the step, and as init/final by the
 * seq mode; a NULL states pointer in seq mode means zero initial state and
 * no write-back).  mode NH_MODE_STEP requires T == 1. */
nh_status nh_mamba_stack(const nh_mamba_dims *d, const nh_mamba_weights *weights,
                         nh_mamba_state *states, int n_layers, int mode,
                         const void *x, nh_dtype x_dtype, int T, float *outs, int batch,
                         void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NHMAMBA_H */
