/*
 * tlp.h - C ABI of the MI355X (gfx950) transformer-layer prefill library.
 *
 * The library runs the batched prefill forward of a dense Llama/Qwen3-style
 * decoder layer over a micro-batch of prompt tokens, and a chunk driver that
 * repeats it over every layer and micro-batch and finishes with a last-token
 * LM head.  The operations are those of:
 *   - oxibonsai-kernels 0.1.1, gpu_backend/metal_prefill.rs:
 *     encode_layer_prefill steps 1-7 (the layer) and the "Tail" block of
 *     encode_full_forward_prefill (final norm + LM head of the last token);
 *   - oxibonsai-kernels 0.1.0, gpu_backend/metal_full_layer.rs: GpuKvCache
 *     (cache layout [n_layers][n_kv][max_seq][head_dim]) and the fused
 *     gate ++ up weight;
 *   - turbospark-runtime 0.3.0, families/llama/prefill.rs:
 *     prefill_chunk_real_llama_dense (micro-batches at start_position +
 *     offset, head on the last micro-batch only).
 *
 * Conventions for every entry point:
 *   - Every array argument is a DEVICE pointer unless marked "host".  The
 *     caller owns every buffer and every stream and event the calls use (a
 *     tlp_pipeline for two micro-batches in flight); the prefill calls
 *     allocate nothing and keep no state between calls.  The only resources
 *     the library creates are those of tlp_pipeline_create and
 *     tlp_profile_begin, released by tlp_pipeline_destroy and
 *     tlp_profile_end, and the static scratch of tlp_prefill_layer_noalloc.
 *   - Matrices are row-major.  Activations are token-major: row t of
 *     hidden [n_tokens][hidden] is token t, at absolute position
 *     start_position + t.  Projection weights are [out_features][in_features].
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     runs asynchronously; the caller synchronises.
 *   - Arguments are validated before anything is enqueued.  On an error the
 *     call returns a non-zero tlp_status, enqueues nothing and touches no
 *     buffer; tlp_last_error() then describes it (thread-local text).  A
 *     failed kernel launch returns TLP_ERR_HIP after earlier launches of the
 *     same call may already be enqueued.
 *   - Concurrent calls that share a workspace or a cache slot race; calls on
 *     one stream are ordered.
 */
#ifndef TLP_H
#define TLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TLP_OK = 0,
  TLP_ERR_NULL = 1,        /* a required pointer is NULL */
  TLP_ERR_SHAPE = 2,       /* a size or a shape relation is invalid */
  TLP_ERR_POSITION = 3,    /* start_position < 0 or start_position + n_tokens > max_seq */
  TLP_ERR_UNSUPPORTED = 4, /* a valid but unsupported combination (dtype, format, group size) */
  TLP_ERR_WORKSPACE = 5,   /* workspace_bytes below tlp_workspace_bytes() */
  TLP_ERR_HIP = 6          /* a HIP launch failed; tlp_last_error() has its text */
} tlp_status;

/* Activation / norm-gain / KV-cache element type. */
typedef enum { TLP_F32 = 0, TLP_BF16 = 1 } tlp_dtype;

/* Projection weight format.
 * TLP_W_DENSE: [N][K] in the config's dtype.
 * TLP_W_SIGN1_G128: 1-bit signs plus one fp16 scale per 128 consecutive
 *   weights of a row (metal_prefill.rs only names a structure-of-arrays 1-bit
 *   layout; this library fixes the format): `data` is uint32 [N][K/32] where bit b of
 *   word w is the sign of column 32w+b, least-significant bit first, 1 = +1 and
 *   0 = -1; `scales` is IEEE fp16 [N][K/128].  W[n][k] = scales[n][k/128] * sign.
 *   Requires K % 128 == 0 and dtype TLP_BF16. */
typedef enum { TLP_W_DENSE = 0, TLP_W_SIGN1_G128 = 1 } tlp_wformat;

/* KV-cache element format.
 * TLP_KV_ACT: the cache holds K and V in the config's dtype.
 * TLP_KV_F16: IEEE fp16 (the cache type of the layer page's GpuKvCache and of
 *   the chunk page's attention), rounded to nearest-even when stored; needs
 *   dtype TLP_BF16.  Values beyond the fp16 range become +-inf. */
typedef enum { TLP_KV_ACT = 0, TLP_KV_F16 = 1 } tlp_kv_format;

typedef struct {
  int32_t hidden;       /* H; multiple of 8, at most 16384 */
  int32_t intermediate; /* I; multiple of 8 */
  int32_t n_q_heads;    /* nq; multiple of n_kv_heads */
  int32_t n_kv_heads;   /* nkv; nq/nkv in {1, 2, 4} or a multiple of 4 */
  int32_t head_dim;     /* hd in {64, 128} */
  int32_t max_seq;      /* cache slots per kv head */
  int32_t n_layers;     /* layers held by the caches (and by tlp_prefill_chunk) */
  float rms_eps;        /* eps of every RMSNorm of the layer (incl. QK-norm) */
  int32_t qk_norm;      /* non-zero: per-head RMSNorm of Q and K before RoPE */
  int32_t dtype;        /* tlp_dtype */
  int32_t wformat;      /* tlp_wformat */
  int32_t kv_format;    /* tlp_kv_format (0: caches in dtype) */
} tlp_config;

/* One projection weight.  Dense: data = [N][K], scales = NULL (ignored: the
 * format is tlp_config.wformat).  1-bit: data = sign words, scales = fp16
 * group scales (see tlp_wformat). */
typedef struct {
  const void* data;
  const void* scales;
} tlp_weight;

/* Weights of one layer (metal_prefill.rs LayerWeightRefs).  Gains are [H]
 * (q_norm/k_norm: [hd], shared by all heads; ignored unless qk_norm) in the
 * config's dtype, every gain 16-byte aligned.  Shapes: w_qkv [(nq+2nkv)hd][H]
 * with Q rows, then K, then V; w_o [H][nq*hd]; w_gate_up [2I][H] with the
 * gate rows first; w_down [H][I]. */
typedef struct {
  const void* attn_norm;
  tlp_weight w_qkv;
  const void* q_norm;
  const void* k_norm;
  tlp_weight w_o;
  const void* ffn_norm;
  tlp_weight w_gate_up;
  tlp_weight w_down;
} tlp_layer_weights;

/* Workspace regions (for tlp_workspace_layout).  After tlp_prefill_layer they
 * hold that call's intermediates: RES fp32 [n][H] the residual stream, i.e.
 * the layer's output before it is rounded to dtype; XN the FFN-normed rows
 * [n][H] (dtype); QKV [n][(nq+2nkv)hd] (dtype) whose Q columns hold the normed,
 * roped queries (its K and V columns hold the projected K and V when the
 * projection writes whole rows: with fp32 activations, and with bf16 ones when
 * it runs in one pass, as for 512- and 2048-token micro-batches at the 8B
 * shapes; when a bf16 projection splits K, and on the decode path, K and V go
 * from the split-K sums straight to the cache and those columns are not
 * written); ATTN [n][nq*hd]
 * attention output (dtype); ACT [n][I]
 * SwiGLU output (dtype); HEAD fp32 [H] normed last row (chunk with a head);
 * PART fp32 split-K slices of the output and down projections (bf16 only). */
enum { TLP_WS_RES = 0, TLP_WS_XN = 1, TLP_WS_QKV = 2, TLP_WS_ATTN = 3, TLP_WS_ACT = 4,
       TLP_WS_HEAD = 5, TLP_WS_PART = 6, TLP_WS_COUNT = 7 };

/* Bytes of workspace a call with up to `max_tokens` tokens per micro-batch
 * needs (tlp_prefill_chunk: max_tokens = min(n_tokens, micro_batch); twice
 * that lets it run two micro-batches at once).  The workspace stands in for
 * metal_prefill.rs PrefillBuffers (the lazily allocated intermediate buffers
 * sized for the batch, reallocated when a larger batch comes): here the caller
 * allocates it once for its largest micro-batch.
 * Returns 0 for an invalid config or max_tokens <= 0. */
size_t tlp_workspace_bytes(const tlp_config* cfg, int32_t max_tokens);

/* Byte offsets of the TLP_WS_* regions inside such a workspace (host array
 * offsets[TLP_WS_COUNT]), i.e. where the PrefillBuffers of metal_prefill.rs
 * (normed rows, q/k/v, attention output, gate/up output, hidden) live.  Same
 * validation as tlp_workspace_bytes. */
tlp_status tlp_workspace_layout(const tlp_config* cfg, int32_t max_tokens, size_t* offsets);

/* RoPE tables on the HOST: cos_host/sin_host [n_pos][head_dim/2] fp32 with
 * entry [p][i] = cos/sin(p * theta^(-2i/head_dim)), evaluated in double and
 * rounded once (metal_prefill.rs: host-built cos_table/sin_table of half_dim
 * entries per position).  The caller uploads them for the rope_cos/rope_sin
 * arguments below (indexed by absolute position).  head_dim even, > 0. */
tlp_status tlp_rope_table(double theta, int32_t head_dim, int32_t n_pos, float* cos_host,
                          float* sin_host);

/* One decoder layer over n_tokens tokens at start_position .. +n_tokens-1
 * (metal_prefill.rs encode_layer_prefill):
 *   1 x_n = RMSNorm(x; attn_norm)           2 qkv = W_qkv x_n
 *   3 optional per-head QK-norm, rotate-half RoPE at the absolute position,
 *     K (roped) and V (raw) stored to cache[layer][j][start_position + t],
 *     causal GQA attention of every query over slots [0, its position]
 *   4 x += W_o attn                         5 x_n2 = RMSNorm(x; ffn_norm)
 *   6 a = silu(W_gate x_n2) * (W_up x_n2)   7 x += W_down a
 * hidden: [n_tokens][H] in dtype, read and overwritten in place.  The residual
 * stream inside the call is fp32.  k_cache, v_cache: [n_layers][nkv][max_seq][hd]
 * in dtype (fp16 with TLP_KV_F16); exactly the slots [start_position, start_position + n_tokens) of
 * `layer` are written, slots [0, start_position + n_tokens) of `layer` are read,
 * and every slot below start_position must already hold that position's K/V.
 * rope_cos, rope_sin: device fp32 [>= start_position + n_tokens][hd/2],
 * 16-byte aligned.
 * workspace: device, >= tlp_workspace_bytes(cfg, n_tokens) bytes, 256-aligned. */
tlp_status tlp_prefill_layer(const tlp_config* cfg, const tlp_layer_weights* weights,
                             int32_t layer, void* hidden, int32_t n_tokens,
                             int32_t start_position, void* k_cache, void* v_cache,
                             const float* rope_cos, const float* rope_sin, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Bytes of the library's static scratch array (per GPU) that
 * tlp_prefill_layer_noalloc uses as its workspace: 64 MiB. */
#define TLP_NOALLOC_SCRATCH_BYTES (64u << 20)

/* tlp_prefill_layer without a workspace argument, for callers that cannot
 * allocate device memory (work captured into HIP graphs, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, contract and result as
 * tlp_prefill_layer, bit-identical; the workspace is a static device array of
 * TLP_NOALLOC_SCRATCH_BYTES owned by the library (one per GPU, held until the
 * process ends).  The call itself allocates nothing: on its first call on a
 * GPU it looks up that array's device address (hipGetSymbolAddress, with that
 * GPU current) and keeps it.  The GPU is the one `stream` belongs to (the
 * current device for the null stream).
 * A call needing more than TLP_NOALLOC_SCRATCH_BYTES
 * (tlp_workspace_bytes(cfg, n_tokens); e.g. up to about 240 tokens of an
 * 8B-shape layer, every decode step) returns TLP_ERR_WORKSPACE before
 * anything is enqueued.  Every call on one GPU uses the same array and leaves
 * its intermediates there (layout as tlp_workspace_layout); the kernels need
 * no part of it cleared.  Calls that overlap on one GPU (different streams,
 * threads or processes sharing the library) race on it. */
tlp_status tlp_prefill_layer_noalloc(const tlp_config* cfg, const tlp_layer_weights* weights,
                                     int32_t layer, void* hidden, int32_t n_tokens,
                                     int32_t start_position, void* k_cache, void* v_cache,
                                     const float* rope_cos, const float* rope_sin, void* stream);

/* Caller-owned resources for keeping two micro-batches of tlp_prefill_chunk in
 * flight (the chunk page runs its micro-batches one after another; this
 * library can overlap consecutive ones, which only need each other's K/V):
 * a second stream (default priority, non-blocking) and 2*max_layers + 2
 * events, created on the current device.  Create once, pass to any number of
 * chunk calls with at most max_layers layers on streams of the same device,
 * destroy when done (tlp_pipeline_destroy waits for the second stream).  Two
 * calls in flight at once must not share a pipeline. */
typedef struct tlp_pipeline tlp_pipeline;
tlp_status tlp_pipeline_create(int32_t max_layers, tlp_pipeline** out);
tlp_status tlp_pipeline_destroy(tlp_pipeline* pipeline);

/* Chunked prefill of n_tokens prompt tokens through all cfg->n_layers layers
 * (turbospark llama/prefill.rs prefill_chunk_real_llama_dense): micro-batch b
 * holds tokens [b*micro_batch, min(n_tokens, (b+1)*micro_batch)) at positions
 * start_position + offset and runs layer 0, 1, ... in order; the residual
 * stream stays fp32 across layers and is rounded to dtype once per
 * micro-batch into `hidden` ([n_tokens][H], in place).  layers: host array of
 * cfg->n_layers weight structs.  If lm_head is not NULL, after the last
 * micro-batch logits[v] = sum_k lm_head[v][k] * RMSNorm(x_last; final_norm,
 * final_eps)[k] (fp32 [vocab]); lm_head is [vocab][H] in dtype, final_norm [H]
 * in dtype.  workspace >= W = tlp_workspace_bytes(cfg, min(n_tokens, micro_batch)).
 * With a pipeline (tlp_pipeline_create, NULL: none), workspace_bytes >= 2 W
 * and more than one micro-batch, micro-batch b uses the bytes
 * [(b % 2) W, (b % 2 + 1) W) of the workspace and the odd ones run on the
 * pipeline's second stream: each layer's attention of micro-batch b waits
 * for the K/V that micro-batch b-1 stored for that layer, so consecutive
 * micro-batches overlap one layer apart.  The second stream starts behind the
 * work already on `stream` and is joined back into it before the call
 * returns, so the call's work completes in `stream`'s order either way.
 * A pipeline made for fewer layers is TLP_ERR_SHAPE, one made on another
 * device than `stream`'s TLP_ERR_UNSUPPORTED.
 * While `stream` is being captured into a graph the micro-batches run one at
 * a time on it (the call then only enqueues kernels, as tlp_prefill_layer).
 * The caller tracks the cache position: a chunk must start where the previous
 * one ended (the stateless library cannot check that). */
tlp_status tlp_prefill_chunk(const tlp_config* cfg, const tlp_layer_weights* layers,
                             void* hidden, int32_t n_tokens, int32_t start_position,
                             int32_t micro_batch, void* k_cache, void* v_cache,
                             const float* rope_cos, const float* rope_sin,
                             const void* final_norm, const void* lm_head, int32_t vocab,
                             float final_eps, float* logits, void* workspace,
                             size_t workspace_bytes, tlp_pipeline* pipeline, void* stream);

/* Greedy token choice (prefill page, encode_full_forward_prefill: the greedy
 * branch of the tail runs an argmax over the logits on the GPU and returns a
 * 4-byte token id instead of the logits).  token_ids[r] = the lowest index v
 * in [0, vocab) whose logits[r * ld + v] is maximal, compared in fp32; NaN
 * entries are never chosen and a row with no entry above -inf gives 0.
 * logits: device fp32 [rows][ld] with ld >= vocab; token_ids: device int32
 * [rows].  rows > 0, vocab > 0 (TLP_ERR_SHAPE otherwise). */
tlp_status tlp_argmax_rows(const float* logits, int32_t rows, int32_t vocab, int64_t ld,
                           int32_t* token_ids, void* stream);

/* Workspace bytes tlp_verify_tail needs for up to n_rows rows (0 if the
 * config is invalid or n_rows <= 0). */
size_t tlp_verify_workspace_bytes(const tlp_config* cfg, int32_t n_rows);

/* Speculative-decode verify tail (prefill page,
 * encode_full_forward_prefill_verify, its tail: final RMSNorm and LM head on
 * every batch position, then a per-position argmax).  For each row r of
 * hidden [n_rows][H] (dtype; e.g. the rows tlp_prefill_chunk wrote):
 *   logits[r][v] = sum_k lm_head[v][k] * RMSNorm(hidden[r]; final_norm, final_eps)[k]
 *   token_ids[r] = tlp_argmax_rows of logits row r   (if token_ids is not NULL)
 * lm_head [vocab][H] and final_norm [H] in dtype, 16-byte aligned; logits
 * device fp32 [n_rows][vocab], 16-byte aligned, required (the product is
 * written there); token_ids device int32 [n_rows] or NULL.  The config's
 * layer fields other than hidden, dtype and rms limits are not used.
 * workspace >= tlp_verify_workspace_bytes(cfg, n_rows), 256-byte aligned. */
tlp_status tlp_verify_tail(const tlp_config* cfg, const void* hidden, int32_t n_rows,
                           const void* final_norm, const void* lm_head, int32_t vocab,
                           float final_eps, float* logits, int32_t* token_ids, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Kernels as timed by the profiler below. */
enum { TLP_K_ATTN_NORM = 0, TLP_K_QKV_GEMM = 1, TLP_K_QK_ROPE_KV = 2, TLP_K_ATTENTION = 3,
       TLP_K_O_GEMM = 4, TLP_K_FFN_NORM = 5, TLP_K_GATE_UP_GEMM = 6, TLP_K_DOWN_GEMM = 7,
       TLP_K_FINAL_NORM = 8, TLP_K_LM_HEAD = 9, TLP_K_OUT_ROWS = 10, TLP_K_SWIGLU = 11,
       TLP_K_ARGMAX = 12, TLP_K_COUNT = 13 };

/* Per-kernel GPU timing, the analog of the per-layer / per-command-buffer
 * profiling switches of metal_full_layer.rs (OXIBONSAI_PROFILE and
 * OXIBONSAI_PROFILE_GPU).  tlp_profile_begin creates max_launches pairs of
 * HIP events for the calling thread; until tlp_profile_end, every kernel
 * launched by this thread's tlp_* calls is bracketed by the next pair,
 * recorded on the call's stream (launches past max_launches are not timed).
 * tlp_profile_end waits for those events, writes the summed elapsed
 * milliseconds and the launch count per TLP_K_* kernel into the HOST arrays
 * total_ms[TLP_K_COUNT] and launches[TLP_K_COUNT] (and the number of launches
 * not timed into *not_timed, if not NULL), and destroys the events. */
tlp_status tlp_profile_begin(int32_t max_launches);
tlp_status tlp_profile_end(double* total_ms, int32_t* launches, int32_t* not_timed);

/* Static text of a status code.  The codes play the part of the
 * MetalGraphError results of the metal_prefill.rs entry points
 * (EncodingFailed for a buffer that is too short or a dimension that does not
 * match, ExecutionFailed for a failed command buffer). */
const char* tlp_status_string(tlp_status status);

/* Text of the calling thread's most recent error ("" if none): the message a
 * MetalGraphError carries on the pages, kept per thread because the C ABI
 * returns only the code. */
const char* tlp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TLP_H */
