/*
 * tte.h -- C ABI of the packed text-embedding encoder for MI355X (gfx950).
 *
 * The library computes the embedding pass described on the tensai
 * "テキスト埋め込み" page (mattn.github.io/tensai/ja/embeddings):
 *   - section 何が動くか, encoder paragraph: a ModernBERT encoder whose layers
 *     are a bias-free LayerNorm, multi-head attention with RoPE and a GeGLU
 *     feed-forward; layer 0 and every third layer after it attend over the
 *     whole text (RoPE base 160000), the others only to the 64 tokens on
 *     either side (base 10000);
 *   - same section, pooling paragraph: the last layer's output is averaged
 *     over each text and scaled to unit length;
 *   - same section, packing paragraph: several texts are processed in one
 *     pass, positions restart in every text and attention never crosses a
 *     text, so a packed call returns the same vectors as one call per text;
 *   - section 精度と量子化: the integer paths (-q8 and -q4 there) round each
 *     activation row to 7 bits with one scale per row and use the stored
 *     weight blocks as they are.
 *
 * Conventions shared by every entry point:
 *   - Every function returns a tte_status.  On failure nothing has been
 *     enqueued on the stream and tte_last_error() (per calling thread) holds
 *     a message; the model stays usable.
 *   - Pointers named d_* are device pointers (HIP device memory), h_* are
 *     host pointers.  The library never takes ownership of caller memory.
 *   - Work is stream-ordered: results in d_* outputs are valid only once the
 *     given stream (a hipStream_t passed as void*, NULL = default stream)
 *     has reached the enqueued work.
 *   - Matrices are row-major.  Activations are token-major [T, H].  Weights
 *     are [out, in], so every projection is Y = X * W^T.
 *
 * Diagnostics, read from the environment once per process (set to any value
 * but "0"):
 *   - TTE_LOG: one stderr line per tte_create, per pass of tte_embed /
 *     tte_embed_tokens / tte_embed_trace and per error, prefixed "[tte]".
 *   - TTE_DEBUG: host-side checks around every pass of those three entry
 *     points, each of which waits for the stream (for finding faults, not
 *     for timing): the token ids are read back and must lie in [0, vocab)
 *     (TTE_E_INVALID before anything is enqueued; without TTE_DEBUG they
 *     are clamped on the device); a 256-byte guard after every workspace
 *     region (tte_workspace_size grows accordingly) must keep its fill
 *     after the pass; the outputs must be finite, pooled vectors of unit
 *     length (TTE_E_DEVICE otherwise).  TTE_FLAG_GRAPH is ignored.
 */
#ifndef TTE_H
#define TTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TTE_OK = 0,
  TTE_E_INVALID = 1,     /* bad argument: nothing was enqueued */
  TTE_E_UNSUPPORTED = 2, /* valid but not implemented (e.g. head_dim != 64) */
  TTE_E_NOMEM = 3,       /* workspace too small, or host allocation failed */
  TTE_E_DEVICE = 4       /* no GPU, or a HIP runtime error */
} tte_status;

typedef enum {
  TTE_FP32 = 0, /* fp32 weights and activations, fp32 matrix cores */
  TTE_BF16 = 1, /* bf16 weights, matmul/attention operands and residual
                   stream (each update added in fp32, rounded once); fp32
                   accumulate, norms and softmax statistics */
  TTE_INT8 = 2, /* int8 weight blocks of 32 inputs with fp32 scales; every
                   weight matmul input rounded per row to 7 bits (|q| <= 63)
                   with an fp32 row scale; int8 matrix cores, int32 sums per
                   block; attention, norms and residual in fp32 */
  TTE_INT4 = 3  /* the page's -q4 (section 精度と量子化): layer matrices as
                   asymmetric 4-bit blocks of 32 inputs (codes 0..15, two per
                   byte, the even input in the low nibble), with per 128
                   inputs a 16-byte record: four 6-bit block scales sc and
                   offsets mn (a byte each), then the fp32 d and dmin of
                   their 256-input super-block; block scale es = fp32(d*sc),
                   offset eo = fp32(dmin*mn), weight es*q - eo.  The token
                   table is int8 blocks as in TTE_INT8.  Activations, MFMA
                   and the rest as TTE_INT8; hidden and intermediate must be
                   multiples of 256 */
} tte_precision;

/* Execution options (tte_config.flags). */
typedef enum {
  /* Split the two residual products (attention output H -> H and the
   * down-projection I -> H) of short packs over K into up to four partial
   * products, summed into the residual stream, in part order, by the norm
   * kernel that follows each.  An H-wide output of a ~2k-token pack makes
   * fewer tiles than the chip's compute units can hold; the parts fill
   * them (the count is chosen per product from its shape, so it is the
   * same for every call of a shape).  Costs 4 * max_tokens * H * 4 bytes
   * of workspace and the partials' memory traffic. */
  TTE_FLAG_SPLIT_K = 1,
  /* HIP-graph replay of the pass.  Prior art: the xujun.org note on 58.com's
   * multimodal (VLM) inference optimisation, section 4.3 (CUDA graphs for
   * the ViT module), records the launch sequence once and keeps a pool of
   * graphs keyed by batch size; here the key is the pack's shape.
   * tte_embed and tte_embed_tokens record, per model, the shapes
   * (n_tokens, n_texts, pool units = sum over texts of ceil(len / 32),
   * output kind) they are called with; at a shape's second call on a
   * non-null stream the kernel sequence is captured into a graph, which
   * that call and every later call of the shape replay with one launch.
   * The token ids and output pointers travel with the offsets upload and
   * are read by the kernels from device memory, so a replay takes the
   * call's own buffers.  At most 64 shapes per model are kept (the least
   * recently used is dropped).  Results are bit-identical to the eager
   * pass.  Calls on the null stream, tte_embed_trace and calls made while
   * tte_profile_start is active run eagerly.  A graph baked with a
   * model's workspace must not outlive it: tte_destroy releases them. */
  TTE_FLAG_GRAPH = 2
} tte_flag;

/* Model shape and limits.  Defaults in parentheses are the page's values. */
typedef struct {
  int32_t vocab;
  int32_t hidden;           /* H = n_heads * head_dim */
  int32_t n_heads;
  int32_t head_dim;         /* must be 64 */
  int32_t intermediate;     /* I: the GeGLU up-projection has 2*I outputs */
  int32_t n_layers;
  int32_t global_every;     /* layer l is global iff l % global_every == 0 (3) */
  int32_t window;           /* local layers: |i - j| <= window (64) */
  float rope_base_global;   /* (160000) */
  float rope_base_local;    /* (10000) */
  float ln_eps;             /* (1e-5) */
  int32_t max_tokens;       /* largest n_tokens of one tte_embed call */
  int32_t max_text_len;     /* longest text (RoPE tables are sized by it) */
  int32_t max_texts;        /* largest n_texts of one call */
  int32_t precision;        /* tte_precision */
  int32_t flags;            /* OR of tte_flag values (0) */
} tte_config;

/* Device pointers to one layer's weights, in the storage format of the
 * precision: fp32 or bf16 (raw uint16 bits) arrays, or int8 codes with fp32
 * scales [out, in/32] (the *_scale pointers are read only in TTE_INT8); in
 * TTE_INT4 each matrix is codes [out, in/2] bytes and its *_scale pointer
 * the records [out, in/128] x 16 bytes. */
typedef struct {
  const void* wqkv;  const float* wqkv_scale;  /* [3H, H]: rows Q, then K, then V; head j at rows j*64.. */
  const void* wo;    const float* wo_scale;    /* [H, H] */
  const void* wi;    const float* wi_scale;    /* [2I, H]: rows 0..I-1 pass through GELU, I..2I-1 gate */
  const void* wo2;   const float* wo2_scale;   /* [H, I] */
  const float* attn_norm;                      /* [H] fp32; NULL on layer 0 (no norm there) */
  const float* mlp_norm;                       /* [H] fp32 */
} tte_layer_weights;

typedef struct {
  const void* tok_emb; const float* tok_emb_scale; /* [vocab, H] (+ [vocab, H/32] scales in TTE_INT8) */
  const float* emb_norm;                           /* [H] fp32 */
  const float* final_norm;                         /* [H] fp32 */
  const tte_layer_weights* layers;                 /* host array of n_layers entries, copied by tte_create */
} tte_weights;

typedef struct tte_model tte_model;

/* Bytes of device workspace a model of this config needs (activations,
 * per-token text bounds, RoPE tables, pooling partials).  *bytes is set on
 * success; nothing else happens (no GPU is needed).
 * Passage: tensai "テキスト埋め込み", section 精度と量子化, speed table and
 * the sentence after it: loading the model is the slow, one-time step and
 * memory is sized then; embedding reuses it.  Errors: TTE_E_INVALID for a
 * config the library cannot run (the message names the field) or a NULL
 * bytes. */
tte_status tte_workspace_size(const tte_config* cfg, size_t* bytes);

/* Create a model over BORROWED device weights and a BORROWED device
 * workspace of at least tte_workspace_size bytes (256-byte aligned).  Both
 * must outlive the model.  Writes the RoPE tables into the workspace
 * (synchronously) and allocates a small pinned host staging area.  Several
 * models may share one set of weights; use one model per concurrent stream.
 * Passage: tensai "テキスト埋め込み", section 何が動くか, encoder
 * paragraph (the layers and the global / local schedule this config
 * describes) and section サーバー (requests are stateless and may run
 * concurrently: one model per stream over shared weights).  Errors:
 * TTE_E_INVALID for a bad config, a NULL required weight or a misaligned
 * workspace; TTE_E_NOMEM if the workspace is too small or host memory runs
 * out; TTE_E_DEVICE when no GPU is present.  *out is NULL on failure. */
tte_status tte_create(const tte_config* cfg, const tte_weights* w, void* d_workspace,
                      size_t workspace_bytes, tte_model** out);

/* Embed one pack.  Passage: tensai "テキスト埋め込み", section サーバー
 * (token ids in, one float32 vector per input text out, <s> and </s>
 * counted as tokens) and section 何が動くか, pooling paragraph (mean over
 * the text, unit length) and packing paragraph (texts packed into one pass
 * give the same vectors as one text at a time).
 * d_token_ids: int32 [n_tokens] on the device, the texts
 * concatenated.  h_offsets: host int32 [n_texts + 1], offsets[0] = 0,
 * strictly increasing (no empty text), offsets[n_texts] = n_tokens, every
 * text at most max_text_len tokens, n_tokens <= max_tokens, n_texts <=
 * max_texts.  The offsets are validated before anything is enqueued and
 * copied, so the caller may reuse h_offsets when the call returns.
 * d_out: fp32 [n_texts, H], one unit-norm vector per text (mean over every
 * token of the text, BOS/EOS included, after the final LayerNorm).  Token ids
 * outside [0, vocab) are clamped on the device.  n_texts = 0 with
 * n_tokens = 0 is a no-op.  With TTE_FLAG_GRAPH the pass may run as a
 * replayed graph (see there); the results are the same bits. */
tte_status tte_embed(tte_model* m, const int32_t* d_token_ids, int32_t n_tokens,
                     const int32_t* h_offsets, int32_t n_texts, float* d_out, void* stream);

/* Per-token output of the same pass (section 何が動くか, encoder and pooling
 * paragraphs: the encoder's states after its final LayerNorm, which pooling
 * would then average): d_out_tokens fp32 [n_tokens, H], row t for token t of
 * the pack.  Same arguments, validation and stream semantics as tte_embed. */
tte_status tte_embed_tokens(tte_model* m, const int32_t* d_token_ids, int32_t n_tokens,
                            const int32_t* h_offsets, int32_t n_texts, float* d_out_tokens, void* stream);

/* Cosine-similarity matrix of the introduction's -sim example: for unit
 * vectors (tte_embed's output) the cosine is the dot product, so
 * d_sim fp32 [n, n] = E E^T with E = d_emb fp32 [n, dim] row-major.
 * dim must be a positive multiple of 16 (else TTE_E_UNSUPPORTED), n <= 65536;
 * n = 0 is a no-op.  Device buffers, caller-owned, stream-ordered. */
tte_status tte_similarity(const float* d_emb, int32_t n, int32_t dim, float* d_sim, void* stream);

/* Like tte_embed, but also copies the residual stream after the embedding
 * LayerNorm and after each of the first n_dump layers into
 * d_states (fp32 [n_dump + 1, n_tokens, H]; in TTE_BF16 the bf16 stream's
 * values, exactly).  If n_dump < n_layers the pass
 * stops there and d_out is not written (it may be NULL). */
tte_status tte_embed_trace(tte_model* m, const int32_t* d_token_ids, int32_t n_tokens,
                           const int32_t* h_offsets, int32_t n_texts, float* d_out,
                           float* d_states, int32_t n_dump, void* stream);

/* Host-only check of a pack against a config, with the same rules and
 * messages tte_embed applies before enqueuing anything (needs no GPU). */
tte_status tte_check_pack(const tte_config* cfg, int32_t n_tokens, const int32_t* h_offsets, int32_t n_texts);

/* Free the model (not the borrowed weights or workspace).  Waits for the
 * model's pending offset upload; a model with captured graphs
 * (TTE_FLAG_GRAPH) first waits for each graph's last replay, since it may
 * still be running on a caller's stream.  Passage: the counterpart of
 * tte_create (section 精度と量子化 of the tensai page: the model is loaded
 * once and then serves many requests).  Errors: TTE_E_INVALID for NULL. */
tte_status tte_destroy(tte_model* m);

/* Message of the calling thread's last failure ("" if none). */
const char* tte_last_error(void);

/* ---------------------------------------------------------------------------
 * Single-kernel entry points (the production kernels on caller buffers),
 * used by the per-kernel parity tests.  Sizes follow the same rules as the
 * model's: row widths are multiples of 64, GEMM N and K are multiples of 128.
 * ------------------------------------------------------------------------- */

typedef enum { TTE_OUT_F32 = 0, TTE_OUT_BF16 = 1, TTE_OUT_I8 = 2 } tte_out_kind;

/* Bias-free LayerNorm of d_x fp32 [rows, width] with gain d_gamma (fp32
 * [width]; NULL = no normalisation, a plain copy/convert/quantise), written
 * as fp32, bf16, or 7-bit int8 codes plus one fp32 scale per row into
 * d_scale (section 何が動くか, encoder paragraph; section 精度と量子化). */
tte_status tte_op_layernorm(const float* d_x, const float* d_gamma, int32_t rows, int32_t width,
                            float eps, int32_t out_kind, void* d_out, float* d_scale, void* stream);

/* Per-row 7-bit quantisation of fp32 [rows, width]: amax = max|x|,
 * q = clamp(rint(x * (63/amax)), -63, 63), scale = amax/63 (zero row: 0, 0),
 * each step rounded to fp32 (section 精度と量子化). */
tte_status tte_op_quant7(const float* d_x, int32_t rows, int32_t width, int8_t* d_q, float* d_scale,
                         void* stream);

typedef enum { TTE_EPI_STORE = 0, TTE_EPI_RESIDUAL = 1, TTE_EPI_GEGLU = 2 } tte_epilogue;

/* Y = A * W^T on the matrix cores.  precision selects the operand format:
 * TTE_FP32 (A, W fp32), TTE_BF16 (A, W bf16), TTE_INT8 (A int8 codes with
 * d_a_scale fp32 [M]; W int8 with d_w_scale fp32 [N_w, K/32]; y[m,n] =
 * a_scale[m] * sum_b w_scale[n,b] * (int32 sum over block b)), TTE_INT4
 * (A as for TTE_INT8; W packed 4-bit codes, bytes [N_w, K/2], and d_w_scale
 * pointing to its 16-byte records [N_w, K/128] (see TTE_INT4); y[m,n] =
 * a_scale[m] * sum_b (es[n,b] * P[m,n,b] - eo[n,b] * S[m,b]) with P the
 * int32 block product and S the block sum of the activation codes; K a
 * multiple of 256).
 * epilogue: STORE writes d_c [M, N] (fp32, or bf16 if out_kind is BF16);
 * RESIDUAL adds into fp32 d_c [M, N], or with TTE_BF16 and out_kind BF16
 * into bf16 d_c (the sum taken in fp32 and rounded once to nearest even;
 * out_kind BF16 with another precision is TTE_E_INVALID); GEGLU takes W
 * with 2N rows and writes
 * d_c[m, n] = GELU(y[m, n]) * y[m, N + n] (erf GELU). */
tte_status tte_op_gemm(int32_t precision, int32_t epilogue, const void* d_a, const float* d_a_scale,
                       const void* d_w, const float* d_w_scale, int32_t M, int32_t N, int32_t K,
                       void* d_c, int32_t out_kind, void* stream);

/* Split-K form of the same product for the residual projections: K is cut
 * into `splits` equal parts (each a multiple of 128 bytes of an operand
 * row) and part s writes its fp32 product to d_partials + s * M * N
 * (int8: already multiplied by both scales). */
tte_status tte_op_gemm_splitk(int32_t precision, const void* d_a, const float* d_a_scale, const void* d_w,
                              const float* d_w_scale, int32_t M, int32_t N, int32_t K, int32_t splits,
                              float* d_partials, void* stream);

/* Residual update from split-K partials fused with the next norm: d_x fp32
 * [rows, width] += d_partials[0] + ... + d_partials[splits-1] (in that
 * order, each [rows, width]), written back; then, as tte_op_layernorm, the
 * updated rows are normalised (d_gamma non-null) or converted into d_out;
 * out_kind = -1 writes no output. */
tte_status tte_op_resid_ln(float* d_x, const float* d_partials, int32_t splits, const float* d_gamma, int32_t rows,
                           int32_t width, float eps, int32_t out_kind, void* d_out, float* d_scale, void* stream);

/* Attention of layer `layer` of model m over the pack described by
 * h_offsets: d_qkv [n_tokens, 3H] (fp32, or bf16 in TTE_BF16) -> d_o
 * [n_tokens, H] (same format).  RoPE with positions restarting per text,
 * text-confined mask, window on local layers (section 何が動くか). */
tte_status tte_op_attention(tte_model* m, int32_t layer, const void* d_qkv, int32_t n_tokens,
                            const int32_t* h_offsets, int32_t n_texts, void* d_o, void* stream);

/* QKV projection of layer `layer` with its fused epilogue: d_a is the
 * layer's attention input [n_tokens, H] in the model's operand format (fp32,
 * bf16, or int8 codes with d_a_scale fp32 [n_tokens] in TTE_INT8).  Writes
 * d_qk [n_tokens, 3H] with RoPE applied (positions restarting per text,
 * the layer's base) to the Q and K columns 0 .. 2H-1 (columns 2H.. are left
 * untouched), and V transposed into d_vt [H, n_tokens] (token order).
 * fp32 outputs, bf16 in TTE_BF16 (section 何が動くか, encoder and packing
 * paragraphs). */
tte_status tte_op_qkv(tte_model* m, int32_t layer, const void* d_a, const float* d_a_scale, int32_t n_tokens,
                      const int32_t* h_offsets, int32_t n_texts, void* d_qk, void* d_vt, void* stream);

/* Final LayerNorm (gain = the model's final_norm), mean over each text,
 * L2 normalisation: d_x fp32 [n_tokens, H] -> d_out fp32 [n_texts, H]
 * (section 何が動くか, pooling paragraph). */
tte_status tte_op_pool(tte_model* m, const float* d_x, int32_t n_tokens, const int32_t* h_offsets,
                       int32_t n_texts, float* d_out, void* stream);

/* tte_op_pool with no device allocation and no workspace use, for callers
 * that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, validation, kernels and
 * results (bit for bit) as tte_op_pool; the pack's offsets, pool-unit starts
 * and per-unit partial sums go to a static device scratch of 8 MiB per GPU,
 * held from the library's load until the process ends.  A pack needing more
 * -- 8 * (n_texts + 1) bytes rounded up to 256, plus
 * 4 * hidden * sum over texts of ceil(len / 32) -- is refused with
 * TTE_E_UNSUPPORTED before anything is enqueued (hidden 768: about 2700
 * partial rows, e.g. 85k tokens in long texts).  Every call on one GPU
 * shares that scratch: calls that overlap on one GPU (other streams or
 * threads) race and must be serialised by the caller; each call rewrites
 * everything it reads, so nothing carries over between calls. */
tte_status tte_op_pool_static(tte_model* m, const float* d_x, int32_t n_tokens, const int32_t* h_offsets,
                              int32_t n_texts, float* d_out, void* stream);

/* ---------------------------------------------------------------------------
 * Per-kernel timing with HIP events on the model's stream.
 * ------------------------------------------------------------------------- */

typedef enum {
  TTE_K_EMBED = 0, TTE_K_NORM = 1, TTE_K_QUANT = 2, TTE_K_GEMM_QKV = 3, TTE_K_ATTN_GLOBAL = 4,
  TTE_K_ATTN_LOCAL = 5, TTE_K_GEMM_O = 6, TTE_K_GEMM_GEGLU = 7, TTE_K_GEMM_O2 = 8, TTE_K_POOL = 9,
  TTE_K_COUNT = 10
} tte_kernel_class;

/* Start recording an event pair around every launch whose class bit is set
 * in class_mask, for up to max_launches launches in total.  Every class
 * but TTE_K_POOL is one kernel per launch and records its pair as part of
 * that kernel's dispatch (the kernel's execution alone); TTE_K_POOL (two
 * kernels) records it as marker packets on the stream around them (which
 * adds the packets' latency).  Calls on a model while recording run eagerly (no
 * TTE_FLAG_GRAPH replay). */
tte_status tte_profile_start(tte_model* m, uint32_t class_mask, int32_t max_launches);

/* Wait for the recorded events and return, per class, the summed kernel
 * time in milliseconds and the number of timed launches (arrays of
 * TTE_K_COUNT entries).  Stops recording. */
tte_status tte_profile_stop(tte_model* m, double* ms_per_class, int64_t* launches_per_class);

/* TTE_FLAG_GRAPH bookkeeping of a model (host counters, no GPU work):
 * *n_shapes = pack shapes currently recorded, *n_graphs = those with an
 * instantiated graph, *n_replays = graph launches since tte_create (the
 * call that captures a shape counts as its first replay).  All three are
 * 0 for a model without the flag.  Returns TTE_E_INVALID on NULL
 * arguments. */
tte_status tte_graph_stats(const tte_model* m, int32_t* n_shapes, int32_t* n_graphs, int64_t* n_replays);

#ifdef __cplusplus
}
#endif

#endif /* TTE_H */
