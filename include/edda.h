/*
 * edda.h — C ABI of libedda.so: Whisper-large-v3 encoder self-attention and
 * speculative block-verification attention on AMD MI355X (gfx950).
 *
 * What the library computes (the pages it follows):
 *  - "audio.cpp PR #1223, Add Edda ASR", PR description and encoder commit
 *    message: the encoder packs Q, K and V into one projection and runs flash
 *    attention over fp16 K/V instead of materializing fp32 scores for all 1500
 *    frames of a 30 s window.
 *  - "higgs-audio-v3-stt-GGUF" model card, architecture note: 4 s chunks are
 *    encoded independently with within-chunk attention, and valid frames must
 *    not attend to padding.
 *  - "BuzzASR/danish discussion #1", first reply: the encoder is bidirectional.
 *  - "audio.cpp PR #1223", commit messages: the decoder verifies an anchor plus
 *    up to 15 drafted tokens in one pass over KV slots indexed by position;
 *    beams share one token-tree KV cache whose mask row admits only a beam's
 *    ancestors.
 *  - llama.cpp DSpark diff, src/models/dflash.cpp ("cache-aware, non-causal
 *    attention"): one attention call takes Q, K, V, the output projection and
 *    the score scale together.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers to IEEE binary16 (fp16) unless noted,
 *    row-major, 16-byte aligned. Geometry is fixed: d_model 1280, 20 heads of 64.
 *  - The caller owns every buffer (inputs, outputs, workspaces). The library
 *    never allocates, frees or synchronizes; it keeps no state between calls
 *    except the calling thread's last error text. Calls only enqueue work on
 *    `stream` (a hipStream_t passed as void*; NULL = the null stream) and return.
 *  - Arguments are validated on the host before anything is enqueued; an
 *    invalid call returns a non-zero status, enqueues nothing and sets the text
 *    returned by edda_last_error(). Nothing falls back silently.
 *  - WEIGHT LAYOUT. Every weight matrix argument is output-feature major
 *    ("Linear" layout, [out_features, in_features], row n = the inputs of
 *    output feature n), the layout Whisper checkpoints store q/k/v/out
 *    projections in; both GEMM operands are then K-contiguous. This replaces
 *    the math layout y = x * W with W [in, out]: the packed QKV weight is
 *    passed as w_qkv [3840, 1280] = W_qkv^T, NOT as the [1280, 3840] matrix
 *    whose column blocks are Q | K | V, and the output projection as
 *    w_o [1280, 1280] = W_o^T. A math-layout matrix must be transposed once
 *    at load time. The two layouts have the same element count, so passing
 *    the untransposed matrix is not detected and gives wrong results.
 *  - Arithmetic: fp16 operands, fp32 accumulation and fp32 softmax, fp16
 *    results rounded to nearest even. The score scale is 1/sqrt(64) = 1/8.
 *  - Calls on different streams may run concurrently when their output and
 *    workspace buffers do not overlap.
 */
#ifndef EDDA_H
#define EDDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EDDA_D_MODEL 1280
#define EDDA_N_HEADS 20
#define EDDA_HEAD_DIM 64
#define EDDA_QKV_COLS (3 * EDDA_D_MODEL)
#define EDDA_MAX_VERIFY_QUERIES 16
#define EDDA_D_FF 5120
/* Leading bytes of the verification workspace that hold its arrival counters. */
#define EDDA_VERIFY_COUNTER_BYTES 16384
/* Most heads edda_verify_attn_ex handles (head_dim is always 64). */
#define EDDA_MAX_VERIFY_HEADS 64

typedef enum {
  EDDA_OK = 0,
  EDDA_ERR_INVALID_ARGUMENT = 1, /* null pointer, size out of range            */
  EDDA_ERR_UNSUPPORTED = 2,      /* valid request the library does not handle */
  EDDA_ERR_MISALIGNED = 3,       /* a pointer is not 16-byte aligned           */
  EDDA_ERR_WORKSPACE = 4,        /* workspace missing or too small             */
  EDDA_ERR_HIP = 5               /* the HIP runtime reported a launch error    */
} edda_status;

/*
 * Packed QKV projection: qkv = x * W_qkv + b_qkv.
 * (audio.cpp PR #1223: the encoder "packs QKV" — one projection instead of three.)
 *
 *  x      [rows, 1280]   fp16, row-major.
 *  w_qkv  [3840, 1280]   fp16, row-major, output-feature major ("Linear" layout:
 *                        row n holds the 1280 input weights of output column n).
 *                        Rows 0..1279 are Q, 1280..2559 K, 2560..3839 V; inside
 *                        each third, head h owns rows 64h..64h+63. This is the
 *                        stacked q/k/v projection weight of a Whisper layer;
 *                        mathematically W_qkv = w_qkv^T, a [1280, 3840] matrix.
 *  b_qkv  [3840] fp16, or NULL for no bias (Whisper has no K bias: pass zeros).
 *  qkv    [rows, 3840]   fp16 output, row-major, columns Q | K | V.
 *  rows   >= 1.
 * Errors: NULL x/w_qkv/qkv or rows < 1 -> EDDA_ERR_INVALID_ARGUMENT; a pointer
 * not 16-byte aligned -> EDDA_ERR_MISALIGNED; launch failure -> EDDA_ERR_HIP.
 */
edda_status edda_qkv_pack(const void* x, int64_t rows, const void* w_qkv, const void* b_qkv,
                          void* qkv, void* stream);

/*
 * Encoder self-attention followed by the output projection, for `batch`
 * windows of `seq_len` rows each (flash attention: the score matrix is never
 * stored; "audio.cpp PR #1223" encoder commit message).
 *
 *  qkv        [batch*seq_len, 3840] fp16 from edda_qkv_pack (window b occupies
 *             rows b*seq_len .. b*seq_len+seq_len-1).
 *  chunk_len  0: full bidirectional attention inside each window.
 *             c in [1, seq_len]: block-diagonal — query row i of a window admits
 *             only keys of its own chunk [c*floor(i/c), c*floor(i/c)+c)
 *             ("higgs-audio-v3-stt-GGUF", chunked encoder note).
 *  valid_len  HOST int32[batch], or NULL (= seq_len for every window). Keys at
 *             positions >= valid_len[b] are masked in window b; every query
 *             row, padded or not, is still computed. Each value in [1, seq_len].
 *             A query row whose admitted key set is empty gets O = 0.
 *  w_o        [1280, 1280] fp16, output-feature major (Linear layout; W_o = w_o^T).
 *  b_o        [1280] fp16 or NULL.
 *  y          [batch*seq_len, 1280] fp16 output: y = O * W_o + b_o, where O
 *             holds head h's attention output in columns 64h..64h+63.
 *  workspace  device scratch of at least edda_encoder_workspace_bytes(batch,
 *             seq_len) bytes (holds O); contents on entry are ignored.
 * Errors: EDDA_ERR_INVALID_ARGUMENT for NULL required pointers, batch < 1,
 * seq_len < 1, chunk_len outside {0} U [1, seq_len], valid_len[b] outside
 * [1, seq_len]; EDDA_ERR_MISALIGNED; EDDA_ERR_WORKSPACE; EDDA_ERR_HIP.
 */
edda_status edda_encoder_attn(const void* qkv, int32_t batch, int32_t seq_len, int32_t chunk_len,
                              const int32_t* valid_len, const void* w_o, const void* b_o, void* y,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The attention core of edda_encoder_attn without the output projection:
 * o = concat_h softmax(Q_h K_h^T / 8, masked) V_h, flash-style (scores never
 * stored). Arguments as for edda_encoder_attn; o is [batch*seq_len, 1280] fp16
 * with head h in columns 64h..64h+63.
 * Errors as for edda_encoder_attn (no workspace is needed).
 */
edda_status edda_flash_attn(const void* qkv, int32_t batch, int32_t seq_len, int32_t chunk_len,
                            const int32_t* valid_len, void* o, void* stream);

/* Bytes of workspace edda_encoder_attn needs (0 if the shape is invalid). */
size_t edda_encoder_workspace_bytes(int32_t batch, int32_t seq_len);

/*
 * Block-verification attention: n_q query tokens (the anchor plus up to 15
 * drafted tokens, or one token per beam) attend to a KV cache whose slot j
 * holds position j ("audio.cpp PR #1223": KV slots indexed by position; beams
 * share a token-tree cache whose mask rows admit only ancestors). Also serves
 * cross-attention over the encoder output (mask_rows = NULL).
 *
 *  q          [n_q, 20, 64] fp16 query projections (unscaled).
 *  n_q        in [1, 16].
 *  k, v       [n_kv, 20, 64] fp16, row j = cache slot j.
 *  n_kv       >= 1.
 *  mask_rows  DEVICE uint32 [n_q][ceil(n_kv/32)]; bit (j % 32) of word j / 32
 *             of row t set = query t admits slot j. NULL = every slot admitted.
 *             Causal verification of a block in the last n_q slots sets bits
 *             0 .. n_kv-n_q+t of row t. Contents are not validated; a row with
 *             no admitted slot gets O = 0. Bits at j >= n_kv are ignored.
 *  o          [n_q, 20, 64] fp16 output: o[t,h] = softmax_j(q[t,h].k[j,h]/8) v[j,h]
 *             over the admitted slots j.
 *  workspace  device scratch of at least edda_verify_workspace_bytes(n_q, n_kv)
 *             bytes (may be NULL / 0 bytes when that returns 0). It holds per-head
 *             arrival counters in its first EDDA_VERIFY_COUNTER_BYTES bytes, then the
 *             fp32 partial results of the key splits. The counter bytes must be zero
 *             before the first call that uses the workspace (e.g. one hipMemset after
 *             allocating it);
 *             every call leaves them zero again, so captured graphs may replay it.
 *             Calls that share a workspace must not overlap (same stream, or ordered).
 * Errors: EDDA_ERR_INVALID_ARGUMENT (NULL q/k/v/o, n_q outside [1,16], n_kv < 1),
 * EDDA_ERR_MISALIGNED (q/k/v/o not 16-byte aligned, mask_rows not 4-byte
 * aligned), EDDA_ERR_WORKSPACE, EDDA_ERR_HIP.
 */
edda_status edda_verify_attn(const void* q, int32_t n_q, const void* k, const void* v, int32_t n_kv,
                             const uint32_t* mask_rows, void* o, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * edda_verify_attn without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It allocates nothing (no hipMalloc, hipFree or allocating library call); the
 * split results of caches above 512 keys go to a static device array of
 * EDDA_NOALLOC_SCRATCH_BYTES bytes inside the library (one copy per GPU, held until the
 * process ends), whose device address is looked up on the first call on each device; that
 * first call also clears the array's arrival counters with a kernel on its stream, and every
 * call leaves them zero again.
 *  Arguments and result as for edda_verify_attn; n_kv at most EDDA_NOALLOC_MAX_KV.
 *  Every call on one GPU shares that GPU's array: calls that overlap on one GPU (different
 *  streams, or graphs replayed concurrently) race and give wrong results; order them. The first
 *  call on a device must also complete or be ordered before calls on other streams.
 * Errors: as edda_verify_attn; EDDA_ERR_UNSUPPORTED for n_kv > EDDA_NOALLOC_MAX_KV;
 * EDDA_ERR_HIP if the array's address cannot be obtained.
 */
#define EDDA_NOALLOC_MAX_KV 8192
#define EDDA_NOALLOC_SCRATCH_BYTES (EDDA_VERIFY_COUNTER_BYTES + 64 * 16 * 20 * 66 * 4)
edda_status edda_verify_attn_noalloc(const void* q, int32_t n_q, const void* k, const void* v, int32_t n_kv,
                                     const uint32_t* mask_rows, void* o, void* stream);

/* Bytes of workspace edda_verify_attn needs: 0 for caches of at most 512 keys (one workgroup
 * per head) or an invalid shape; longer caches split the keys into 128-key ranges, one
 * workgroup each, whose fp32 partial results the last workgroup of each head to finish merges
 * in the same launch: EDDA_VERIFY_COUNTER_BYTES + splits * n_q * 20 * 66 * 4 bytes. (The
 * counter region serves up to EDDA_MAX_VERIFY_HEADS heads.) */
size_t edda_verify_workspace_bytes(int32_t n_q, int32_t n_kv);

/* ------------------------------------------------------------------------------------
 * The rest of the encoder around the attention path. The pages time the whole encoder of
 * a 30 s window ("audio.cpp PR #1223", encoder commit message) and count its 32 layers
 * ("BuzzASR/danish discussion #1"); they do not spell out the layer. It follows the public
 * Whisper-large-v3 architecture: pre-norm residual layers
 *   x1 = x + Attn(LN1(x)),  y = x1 + GELU(LN2(x1) W1 + b1) W2 + b2   (hidden width 5120),
 * LayerNorm with eps 1e-5 and the exact GELU x * Phi(x); a stem of two kernel-3 convolutions
 * (128 mel bins -> 1280, then stride 2) each followed by GELU, plus a positional table.
 * ------------------------------------------------------------------------------------ */

typedef enum { EDDA_ACT_NONE = 0, EDDA_ACT_GELU = 1 } edda_activation;

/*
 * Fused linear layer: y = act(x * W + bias) + residual.
 *
 *  x            [rows, in_features] fp16.
 *  w            [out_features, in_features] fp16, output-feature major (Linear layout;
 *               W = w^T).
 *  bias         [out_features] fp16 or NULL.
 *  activation   EDDA_ACT_NONE or EDDA_ACT_GELU (exact, x * Phi(x)), applied before the
 *               residual is added.
 *  residual     [residual_rows, out_features] fp16 or NULL; output row r adds residual row
 *               r % residual_rows (residual_rows = rows for an ordinary residual; a smaller
 *               period repeats one table, e.g. positions, over stacked windows). It may be
 *               y itself (in-place residual); it must not overlap y otherwise.
 *  y            [rows, out_features] fp16; must not overlap x.
 *  in_features, out_features: multiples of 64; rows >= 1.
 * One rounding to fp16 at the end (fp32 accumulation, bias, activation and residual).
 * Errors: EDDA_ERR_INVALID_ARGUMENT (NULL x/w/y, sizes out of range, unknown activation,
 * residual_rows < 1 when residual is given), EDDA_ERR_UNSUPPORTED (a feature count not a
 * multiple of 64), EDDA_ERR_MISALIGNED, EDDA_ERR_HIP.
 */
edda_status edda_linear(const void* x, int64_t rows, int32_t in_features, const void* w,
                        int32_t out_features, const void* bias, int32_t activation, const void* residual,
                        int64_t residual_rows, void* y, void* stream);

/*
 * LayerNorm over the last dimension: y = (x - mean) / sqrt(var + 1e-5) * gamma + beta with
 * the biased variance, statistics in fp32.
 *  x, y         [rows, features] fp16 (y may equal x).
 *  gamma, beta  [features] fp16.
 *  features     a multiple of 256, at most 4096 (1280 for this model).
 * Errors: EDDA_ERR_INVALID_ARGUMENT, EDDA_ERR_UNSUPPORTED (features), EDDA_ERR_MISALIGNED,
 * EDDA_ERR_HIP.
 */
edda_status edda_layer_norm(const void* x, int64_t rows, int32_t features, const void* gamma,
                            const void* beta, void* y, void* stream);

/* Weights of one encoder layer, all fp16 device pointers, Linear layout ([out, in]). */
typedef struct {
  const void* ln1_gamma;  /* [1280] */
  const void* ln1_beta;   /* [1280] */
  const void* w_qkv;      /* [3840, 1280], as for edda_qkv_pack */
  const void* b_qkv;      /* [3840] or NULL */
  const void* w_o;        /* [1280, 1280] */
  const void* b_o;        /* [1280] or NULL */
  const void* ln2_gamma;  /* [1280] */
  const void* ln2_beta;   /* [1280] */
  const void* w_fc1;      /* [5120, 1280] */
  const void* b_fc1;      /* [5120] or NULL */
  const void* w_fc2;      /* [1280, 5120] */
  const void* b_fc2;      /* [1280] or NULL */
} edda_encoder_layer_weights;

/*
 * One pre-norm encoder layer over `batch` windows of `seq_len` rows:
 *   h = LN1(x); o = attention(h W_qkv + b_qkv) (as edda_flash_attn, with chunk_len and
 *   valid_len); x1 = x + o W_o + b_o; y = x1 + GELU(LN2(x1) W1 + b1) W2 + b2.
 *  x, y       [batch*seq_len, 1280] fp16; y may equal x (in-place layer).
 *  chunk_len, valid_len: as for edda_encoder_attn.
 *  weights    host pointer to the layer's weight pointers; every LayerNorm and matrix
 *             pointer is required, biases may be NULL.
 *  workspace  at least edda_encoder_layer_workspace_bytes(batch, seq_len) device bytes
 *             (holds h, QKV / the MLP hidden layer, O, x1); contents on entry ignored.
 * Errors: as for edda_encoder_attn.
 */
edda_status edda_encoder_layer(const void* x, int32_t batch, int32_t seq_len, int32_t chunk_len,
                               const int32_t* valid_len, const edda_encoder_layer_weights* weights, void* y,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace edda_encoder_layer needs: batch*seq_len*(5120 + 1280 + 1280)*2
 * (0 if the shape is invalid). */
size_t edda_encoder_layer_workspace_bytes(int32_t batch, int32_t seq_len);

/*
 * Convolutional stem: y = GELU(conv2(GELU(conv1(mel)))) + pos, per window.
 *  mel       [batch, n_mels, n_frames] fp16, channel-major per window (a log-mel
 *            spectrogram as usually stored).
 *  conv1_w   [1280, 3 * n_mels] fp16: column tap*n_mels + c holds the weight of input
 *            channel c at tap (frame t + tap - 1); i.e. a [1280, n_mels, 3] convolution
 *            weight with its last two axes swapped and flattened.
 *  conv2_w   [1280, 3 * 1280] likewise; conv2 has stride 2 (frame 2t + tap - 1).
 *  conv1_b, conv2_b  [1280] fp16 or NULL.
 *  pos       [(n_frames + 1) / 2, 1280] fp16 positional table, added to every window.
 *  y         [batch * (n_frames + 1) / 2, 1280] fp16.
 *  n_mels    a multiple of 64 (128 for large-v3); n_frames >= 1 (3000 for 30 s).
 *  workspace at least edda_encoder_stem_workspace_bytes(batch, n_mels, n_frames) bytes.
 * Convolutions use padding 1 (zero frames outside the window).
 * Errors: EDDA_ERR_INVALID_ARGUMENT, EDDA_ERR_UNSUPPORTED (n_mels), EDDA_ERR_MISALIGNED,
 * EDDA_ERR_WORKSPACE, EDDA_ERR_HIP.
 */
edda_status edda_encoder_stem(const void* mel, int32_t batch, int32_t n_mels, int32_t n_frames,
                              const void* conv1_w, const void* conv1_b, const void* conv2_w,
                              const void* conv2_b, const void* pos, void* y, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Bytes of workspace edda_encoder_stem needs (0 if the shape is invalid). */
size_t edda_encoder_stem_workspace_bytes(int32_t batch, int32_t n_mels, int32_t n_frames);

/* ------------------------------------------------------------------------------------
 * The decoder's verification layer. "audio.cpp PR #1223" (PR description, commit messages):
 * the target decoder verifies an anchor plus up to 15 drafted tokens in one pass over KV
 * slots indexed by position, beams share one token-tree cache whose mask rows admit only a
 * beam's ancestors, and the decoder attends to the encoder output. The layer itself follows
 * the public Whisper-large-v3 decoder: pre-norm self-attention (block K/V appended to the
 * cache first), cross-attention over projected encoder frames, GELU MLP (width 5120).
 * ------------------------------------------------------------------------------------ */

/* Weights of one decoder layer, all fp16 device pointers, Linear layout ([out, in]). */
typedef struct {
  const void* ln1_gamma;  /* [1280] */
  const void* ln1_beta;
  const void* w_qkv;      /* [3840, 1280]: q | k | v rows, as for edda_qkv_pack */
  const void* b_qkv;      /* [3840] or NULL (no key bias in Whisper: pass zeros there) */
  const void* w_o;        /* [1280, 1280] self-attention output projection */
  const void* b_o;        /* or NULL */
  const void* ln2_gamma;
  const void* ln2_beta;
  const void* w_q_cross;  /* [1280, 1280] cross-attention query projection */
  const void* b_q_cross;  /* or NULL */
  const void* w_o_cross;  /* [1280, 1280] cross-attention output projection */
  const void* b_o_cross;  /* or NULL */
  const void* ln3_gamma;
  const void* ln3_beta;
  const void* w_fc1;      /* [5120, 1280] */
  const void* b_fc1;      /* or NULL */
  const void* w_fc2;      /* [1280, 5120] */
  const void* b_fc2;      /* or NULL */
} edda_decoder_layer_weights;

/*
 * One decoder layer over the n_q block tokens:
 *   h = LN1(x); qkv = h W_qkv + b_qkv; the K and V rows of token t are written to cache slot
 *   slots[t]; o = verify attention of the Q rows over cache slots 0..n_kv-1 under mask_rows
 *   (as edda_verify_attn); x1 = x + o W_o + b_o;
 *   x2 = x1 + verify attention of (LN2(x1) W_qc + b_qc) over cross_k / cross_v (no mask),
 *        projected by W_oc + b_oc;
 *   y = x2 + GELU(LN3(x2) W1 + b1) W2 + b2.
 *  x, y        [n_q, 1280] fp16 (y may equal x); n_q in [1, 16].
 *  slots       HOST int32[n_q]: distinct cache slots in [0, n_kv) of the block tokens (the
 *              last n_q slots for a chain; a beam's fresh slots for a token tree).
 *  k_cache, v_cache  [cache_slots, 20, 64] fp16, updated in place at `slots`.
 *  n_kv        slots the self-attention reads, 1 <= n_kv <= cache_slots.
 *  mask_rows   DEVICE uint32 [n_q][ceil(n_kv/32)] or NULL, as for edda_verify_attn.
 *  cross_k, cross_v  [n_frames, 20, 64] fp16 (edda_cross_kv of the encoder output).
 *  workspace   at least edda_decoder_verify_workspace_bytes(n_q, n_kv, n_frames) bytes; its
 *              first EDDA_VERIFY_COUNTER_BYTES bytes must be zero before its first use (every
 *              call leaves them zero); the rest is scratch. Calls sharing it must not overlap.
 * Errors: EDDA_ERR_INVALID_ARGUMENT (NULL pointers, n_q, slots out of range or repeated,
 * n_kv, n_frames), EDDA_ERR_MISALIGNED, EDDA_ERR_WORKSPACE, EDDA_ERR_HIP.
 */
edda_status edda_decoder_verify_layer(const void* x, int32_t n_q, const int32_t* slots, void* k_cache,
                                      void* v_cache, int32_t cache_slots, int32_t n_kv,
                                      const uint32_t* mask_rows, const void* cross_k, const void* cross_v,
                                      int32_t n_frames, const edda_decoder_layer_weights* weights, void* y,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace edda_decoder_verify_layer needs (0 if the shape is invalid). */
size_t edda_decoder_verify_workspace_bytes(int32_t n_q, int32_t n_kv, int32_t n_frames);

/* One layer of a stack: its weights, its self-attention caches and its cross K/V. */
typedef struct {
  edda_decoder_layer_weights weights;
  void* k_cache;        /* [cache_slots, 20, 64] fp16 */
  void* v_cache;
  const void* cross_k;  /* [n_frames, 20, 64] fp16 */
  const void* cross_v;
} edda_decoder_stack_layer;

/* Largest cache edda_decoder_verify_stack serves (every Whisper self-attention cache: the
 * decoder context is 448 tokens). */
#define EDDA_DECODER_STACK_MAX_KV 512
/* Leading bytes of its workspace that must be zero before first use (each call leaves them so). */
#define EDDA_DECODER_STACK_ZERO_BYTES 40960

/*
 * n_layers consecutive decoder layers over one block (layer l's y is layer l + 1's x; y is the
 * last layer's output), each as edda_decoder_verify_layer with the same slots, n_kv, mask_rows
 * and n_frames, in ceil(n_layers / 8) launches (each layer's weights stream in while the layer
 * before it runs). Results are bit-identical to calling edda_decoder_verify_layer layer by layer
 * (for n_kv <= EDDA_DECODER_STACK_MAX_KV that entry point takes the same one-launch kernel).
 *  layers      HOST array of n_layers >= 1 layers (pointers device, 16-byte aligned).
 *  x, y        [n_q, 1280] fp16 (y may equal x).
 *  workspace   at least edda_decoder_verify_stack_workspace_bytes(n_q, n_kv, n_frames) bytes,
 *              256-byte aligned, whose first EDDA_DECODER_STACK_ZERO_BYTES bytes are zero before
 *              its first use; calls sharing it must not overlap.
 * Other arguments and errors as for edda_decoder_verify_layer; EDDA_ERR_UNSUPPORTED for n_kv
 * above EDDA_DECODER_STACK_MAX_KV or n_frames above 6144 (the kernel's work-item budget).
 */
edda_status edda_decoder_verify_stack(const void* x, int32_t n_q, const int32_t* slots, int32_t cache_slots,
                                      int32_t n_kv, const uint32_t* mask_rows, int32_t n_frames,
                                      const edda_decoder_stack_layer* layers, int32_t n_layers, void* y,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace edda_decoder_verify_stack needs (0 if the shape is invalid or unsupported). */
size_t edda_decoder_verify_stack_workspace_bytes(int32_t n_q, int32_t n_kv, int32_t n_frames);

/* ------------------------------------------------------------------------------------
 * Q8_0 decoder weights ("audio.cpp PR #1223", PR description and results table: the decoder
 * runs with Q8_0 weights beside an F16 encoder). The pages name the format only; it is read
 * as GGML's Q8_0: each weight row (an output feature's inputs, in order) is cut into blocks
 * of 32 values; a block stores d = max|x| / 127 (computed in fp32, stored as fp16) and 32
 * int8 codes q = round(x / d) (x * (1/d) in fp32, rounded half away from zero); the weight
 * is d * q. Codes are kept row-major like the fp16 weights; scales step-major:
 * scales[k / 32][n] belongs to codes[n][k .. k+31].
 * ------------------------------------------------------------------------------------ */

/* One weight matrix in Q8_0 form: codes int8 [out, in], scales fp16 [in / 32, out]. */
typedef struct {
  const void* codes;
  const void* scales;
} edda_q8_matrix;

/*
 * Q8_0 codes and scales of fp16 weights w [rows, cols] (Linear layout, one row per output
 * feature): codes int8 [rows, cols], scales fp16 [cols / 32, rows]. cols must be a
 * multiple of 32. Device pointers; w and codes 16-byte aligned, scales 2-byte aligned.
 * Errors: EDDA_ERR_INVALID_ARGUMENT, EDDA_ERR_UNSUPPORTED (cols), EDDA_ERR_MISALIGNED,
 * EDDA_ERR_HIP.
 */
edda_status edda_quantize_q8_0(const void* w, int32_t rows, int32_t cols, void* codes, void* scales, void* stream);

/*
 * edda_linear with Q8_0 weights, for block-sized inputs: rows in [1, 16]; in_features a
 * multiple of 32, out_features a multiple of 16; codes / scales as edda_quantize_q8_0
 * writes them for the [out_features, in_features] weight. Each 32-deep block's dot product
 * is taken on the codes and scaled in fp32, so the result is that of the dequantized
 * weights up to fp32 summation order. Errors as edda_linear; EDDA_ERR_UNSUPPORTED for rows
 * above 16 or the feature counts.
 */
edda_status edda_linear_q8(const void* x, int64_t rows, int32_t in_features, const void* codes, const void* scales,
                           int32_t out_features, const void* bias, int32_t activation, const void* residual,
                           int64_t residual_rows, void* y, void* stream);

/* edda_decoder_layer_weights with every projection matrix in Q8_0 form. */
typedef struct {
  const void* ln1_gamma;
  const void* ln1_beta;
  edda_q8_matrix w_qkv;
  const void* b_qkv;
  edda_q8_matrix w_o;
  const void* b_o;
  const void* ln2_gamma;
  const void* ln2_beta;
  edda_q8_matrix w_q_cross;
  const void* b_q_cross;
  edda_q8_matrix w_o_cross;
  const void* b_o_cross;
  const void* ln3_gamma;
  const void* ln3_beta;
  edda_q8_matrix w_fc1;
  const void* b_fc1;
  edda_q8_matrix w_fc2;
  const void* b_fc2;
} edda_decoder_layer_weights_q8;

/*
 * edda_decoder_verify_layer with Q8_0 projection weights (LayerNorm parameters and biases
 * fp16; codes and scales 16-byte aligned). Same arguments, workspace
 * (edda_decoder_verify_workspace_bytes) and errors.
 */
edda_status edda_decoder_verify_layer_q8(const void* x, int32_t n_q, const int32_t* slots, void* k_cache,
                                         void* v_cache, int32_t cache_slots, int32_t n_kv,
                                         const uint32_t* mask_rows, const void* cross_k, const void* cross_v,
                                         int32_t n_frames, const edda_decoder_layer_weights_q8* weights, void* y,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* One layer of a stack with Q8_0 projection weights. */
typedef struct {
  edda_decoder_layer_weights_q8 weights;
  void* k_cache;
  void* v_cache;
  const void* cross_k;
  const void* cross_v;
} edda_decoder_stack_layer_q8;

/*
 * edda_decoder_verify_stack with Q8_0 projection weights (as edda_decoder_verify_layer_q8, layer
 * by layer, bit for bit). Same workspace (edda_decoder_verify_stack_workspace_bytes) and errors;
 * EDDA_ERR_INVALID_ARGUMENT also for a matrix without scales.
 */
edda_status edda_decoder_verify_stack_q8(const void* x, int32_t n_q, const int32_t* slots, int32_t cache_slots,
                                         int32_t n_kv, const uint32_t* mask_rows, int32_t n_frames,
                                         const edda_decoder_stack_layer_q8* layers, int32_t n_layers, void* y,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Cross-attention keys and values of the encoder output, once per utterance and layer:
 * cross_k = enc W_k (no bias), cross_v = enc W_v + b_v.
 *  enc            [n_frames, 1280] fp16.
 *  w_k, w_v       [1280, 1280] fp16, Linear layout; b_v [1280] or NULL.
 *  cross_k, cross_v [n_frames, 1280] = [n_frames, 20, 64] fp16.
 * Errors: EDDA_ERR_INVALID_ARGUMENT, EDDA_ERR_MISALIGNED, EDDA_ERR_HIP.
 */
edda_status edda_cross_kv(const void* enc, int32_t n_frames, const void* w_k, const void* w_v, const void* b_v,
                          void* cross_k, void* cross_v, void* stream);

/* ------------------------------------------------------------------------------------
 * Attention variants of the drafter (llama.cpp DSpark diff: common/speculative.cpp, a flag
 * for causal block-internal attention, non-causal by default; src/models/dflash.cpp,
 * optional per-head attention sinks passed into the attention call).
 * ------------------------------------------------------------------------------------ */

typedef enum {
  EDDA_MASK_ROWS = 0,         /* mask_rows given (as for edda_verify_attn)                        */
  EDDA_MASK_NONE = 1,         /* every slot admitted (cross-attention, non-causal block)          */
  EDDA_MASK_CAUSAL_BLOCK = 2  /* the block in the last n_q slots: token t admits 0..n_kv-n_q+t    */
} edda_mask_mode;

/*
 * Verification attention with a head count, a mask mode and optional attention sinks:
 *   o[t,h] = sum_j e^(s_j - m) v[j,h] / (e^(sink_h - m) + sum_j e^(s_j - m)), s_j = q[t,h].k[j,h]/8
 * over the admitted slots j, m = max(sink_h, max_j s_j) (a sink is one extra logit, in
 * scaled-score units, with a zero value; -inf or NULL sinks = none; a query with neither an
 * admitted slot nor a sink gets 0).
 *  q          [n_q, n_heads, 64] fp16; k, v [n_kv, n_heads, 64]; o [n_q, n_heads, 64].
 *  n_heads    in [1, EDDA_MAX_VERIFY_HEADS].
 *  mask_mode  edda_mask_mode; mask_rows is required for EDDA_MASK_ROWS and ignored otherwise;
 *             EDDA_MASK_CAUSAL_BLOCK needs n_q <= n_kv.
 *  sinks      DEVICE fp32 [n_heads] or NULL.
 *  workspace  at least edda_verify_workspace_bytes_ex(n_q, n_kv, n_heads) bytes, first
 *             EDDA_VERIFY_COUNTER_BYTES zero before first use (as for edda_verify_attn).
 * Errors: EDDA_ERR_INVALID_ARGUMENT, EDDA_ERR_MISALIGNED (sinks 4-byte aligned), EDDA_ERR_WORKSPACE,
 * EDDA_ERR_HIP.
 */
edda_status edda_verify_attn_ex(const void* q, int32_t n_q, const void* k, const void* v, int32_t n_kv,
                                int32_t n_heads, int32_t mask_mode, const uint32_t* mask_rows, const float* sinks,
                                void* o, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace edda_verify_attn_ex needs (0 for caches of at most 512 keys or an invalid shape). */
size_t edda_verify_workspace_bytes_ex(int32_t n_q, int32_t n_kv, int32_t n_heads);

/* Text of the calling thread's most recent error ("" after a successful call). */
const char* edda_last_error(void);

/* Library version string. */
const char* edda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EDDA_H */
