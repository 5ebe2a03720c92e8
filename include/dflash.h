/*
 * dflash.h - C ABI of libdflash, the DFlash block-diffusion drafter step for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *  [FN]  "DFlash — 블록 확산 드래프터로 6배 빨라지는 투기적 디코딩" (LLM field
 *        notes appendix), sections 1, 2, 3.1, 6, 7.
 *  [INS] "한 번에 초안을 생성하는 DFlash …" (molayo insight article), paragraph on
 *        multi-layer feature fusion and Key/Value injection.
 *  [SUM] "기술 요약: DFlash – 플래시 추측적 디코딩을 위한 블록 확산" (gist.science
 *        summary of arXiv 2602.06036), sections 2.2 and 2.3.
 *  [PKR] "DFlash 소개" (discuss.pytorch.kr), ``spec_generate`` example.
 *
 * Entry points: handle and workspace (dflash_create, dflash_destroy,
 * dflash_workspace_size, dflash_workspace_init); the drafter step
 * (dflash_inject_context, dflash_draft_block, dflash_lmhead_argmax,
 * dflash_accept_len; dflash_lmhead_argmax_noalloc for callers that cannot
 * allocate); the rest of the speculative cycle (dflash_target_verify,
 * dflash_accept_len_ragged, dflash_sample_workspace_size, dflash_sample,
 * dflash_accept_sample); dflash_check_inputs; measurement
 * (dflash_set_stage_events, dflash_stream_read); dflash_status_str.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer unless stated otherwise; the
 *    library never allocates, frees or retains caller memory beyond the
 *    lifetime stated below, and the compute entry points allocate nothing.
 *  - Matrices are row-major [out, in].  The storage type of weights,
 *    features, caches and hidden states is the handle's dtype (fp32 or bf16;
 *    bf16 = raw 16-bit patterns).  Token ids are int32; logits are fp32.
 *  - ``stream`` is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued on it asynchronously; nothing synchronises.
 *  - Every call returns a dflash_status.  Validation happens on the host
 *    before anything is enqueued; a failed validation enqueues nothing.
 *    Device faults surface as HIP errors at the caller's next synchronisation.
 *    Out-of-range device data (ids >= vocab, page ids >= n_pages) is the
 *    caller's responsibility: the compute calls do not check it;
 *    dflash_check_inputs reports it when the caller enqueues that check.
 *  - A handle is not thread-safe; concurrent streams need separate
 *    workspaces.  Two calls that share a workspace must be ordered on one
 *    stream.
 *  - A workspace must be zero-filled before its first use (a zero-filled
 *    allocation, or dflash_workspace_init).  The counters in it are left at
 *    zero by every call, so it can be reused without clearing.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dflash_handle_s *dflash_handle;

typedef enum {
    DFLASH_OK = 0,
    DFLASH_ERR_NULL = -1,        /* a required pointer is NULL */
    DFLASH_ERR_SHAPE = -2,       /* a size is out of the supported range */
    DFLASH_ERR_DTYPE = -3,       /* unknown storage type */
    DFLASH_ERR_RANGE = -4,       /* a host-side value is out of range */
    DFLASH_ERR_WORKSPACE = -5,   /* workspace too small */
    DFLASH_ERR_UNSUPPORTED = -6, /* combination not implemented */
    DFLASH_ERR_HIP = -7          /* a HIP runtime call failed */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Drafter shape.  Supported: head_dim in {64, 128}; n_q_heads a multiple of
 * n_kv_heads; (n_q_heads / n_kv_heads) * block_size <= 128; 2 <= block_size
 * <= 64; hidden, n_q_heads*head_dim and ffn multiples of 64; hidden <= 16384;
 * vocab a multiple of 16; page_size 16; 1 <= n_layers <= 64.  The mask token is a row of the
 * shared embedding (mask_token_id < vocab). */
typedef struct {
    int32_t hidden;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t ffn;
    int32_t vocab;
    int32_t n_layers;
    int32_t n_feat_layers;   /* L: the context feature is [L * hidden] wide */
    int32_t block_size;      /* B: anchor + (B-1) masked positions */
    int32_t mask_token_id;
    int32_t page_size;       /* positions per KV page; must be 16 */
    int32_t dtype;           /* dflash_dtype */
    float rope_theta;
    float rms_eps;
    int32_t window;                 /* 0: attend to the whole context; > 0: a sliding
                                       window over the last `window` context positions
                                       (long-context use; the block is always attended) */
    int32_t ctx_norm;               /* 0: c = W_fc f; 1: c = RMSNorm(W_fc f) with gain
                                       dflash_weights::ctx_norm (an option: the pages name
                                       only a lightweight projection, [INS]; [SUM] §2.2) */
} dflash_config;

/* Device pointers to the drafter's weights (borrowed for the handle's
 * lifetime; the pointer arrays are copied at creation).  The embedding and the
 * LM head are the target's, shared and frozen ([FN] §3.1; [SUM] §2.3). */
typedef struct {
    const void *embed;              /* [vocab, hidden] */
    const void *lm_head;            /* [vocab, hidden] */
    const void *w_fc;               /* [hidden, n_feat_layers*hidden] fusion projection;
                                       may be NULL for a target handle (no inject) */
    const void *final_norm;         /* [hidden] */
    const void *const *attn_norm;   /* n_layers host-array entries, each [hidden] */
    const void *const *w_qkv;       /* [(nq + 2*nkv)*head_dim, hidden]: q rows, k rows, v rows */
    const void *const *w_o;         /* [hidden, nq*head_dim] */
    const void *const *mlp_norm;    /* [hidden] */
    const void *const *w_gate_up;   /* [2*ffn, hidden]: gate rows first, then up rows */
    const void *const *w_down;      /* [hidden, ffn] */
    const void *ctx_norm;           /* [hidden] gain of the optional RMSNorm after the fusion
                                       projection; required when config.ctx_norm == 1 */
} dflash_weights;

/* Paged drafter context cache (injected K/V, [FN] §2 "KV injection").
 * Position t of sequence s lives in physical page block_table[s*max_pages +
 * t/page_size], slot t % page_size.  The anchor of sequence s sits at position
 * ctx_len[s]; positions 0..ctx_len[s]-1 are the context. */
typedef struct {
    void *k;                        /* [n_layers][n_pages][page_size][n_kv_heads][head_dim],
                                       16-byte aligned (DFLASH_ERR_RANGE otherwise) */
    void *v;                        /* same layout and alignment as k */
    const int32_t *block_table;     /* device [batch][max_pages] */
    const int32_t *ctx_len;         /* device [batch] */
    int32_t batch;
    int32_t max_pages;
    int32_t n_pages;
    int32_t max_ctx;                /* HOST value: upper bound of every ctx_len[s];
                                       sizes launch grids and workspace */
    const int32_t *block_len;       /* device [batch] or NULL: per-sequence block size
                                       B_s ([SUM] §3 item 4, §4: a drafter trained with
                                       B runs smaller blocks; values clamped to 1..B);
                                       block rows j >= B_s
                                       are left out of every row's attention, so rows
                                       < B_s equal a pass with block size B_s and rows
                                       >= B_s carry no meaning */
} dflash_kv;

/* Creates a handle for one drafter (or, for dflash_target_verify, one target
 * decoder of the same layer structure).  ``cfg`` and ``w`` are host structs
 * read during the call; the weight memory they point to is borrowed until
 * dflash_destroy.  Validates shapes only; launches nothing. */
int dflash_create(const dflash_config *cfg, const dflash_weights *w, dflash_handle *out);

/* Releases the handle (host memory only). */
int dflash_destroy(dflash_handle h);

/* Workspace bytes needed for calls with at most ``max_batch`` sequences, an
 * upper bound ``max_ctx`` on context lengths, and at most ``max_new`` positions
 * per dflash_inject_context call.  ``bytes`` is a host pointer. */
int dflash_workspace_size(dflash_handle h, int32_t max_batch, int32_t max_ctx, int32_t max_new,
                          size_t *bytes);

/* Zero-fills the counter region of a workspace (enqueued on ``stream``). */
int dflash_workspace_init(dflash_handle h, void *ws, size_t ws_bytes, void *stream);

/* A1 + A2: feature fusion and KV injection ([INS]; [SUM] §2.2; [FN] §2).
 * For each of the ``n_new`` rows: c = W_fc * feats[row] (rounded to the
 * storage type), then for every drafter layer l the layer's own K and V
 * projections of c are written to the cache at (seq[row], pos[row]); K gets
 * RoPE at pos[row].
 *   feats  [n_new, n_feat_layers*hidden] storage type
 *   seq    [n_new] int32 sequence index (< kv->batch)
 *   pos    [n_new] int32 position (< kv->max_pages * page_size)
 * Rows must not write the same (seq, pos) twice in one call.  ctx_len is not
 * read or written; the caller advances it. */
int dflash_inject_context(dflash_handle h, const void *feats, const int32_t *seq, const int32_t *pos,
                          int32_t n_new, const dflash_kv *kv, void *ws, size_t ws_bytes, void *stream);

/* A3..A8: one drafter forward pass over each sequence's block
 * [anchor, mask x (B-1)] at positions ctx_len[s] .. ctx_len[s]+B-1 ([FN] §2
 * cycle and §7; [SUM] §2.2).  Attention covers the context K/V and the block's
 * own K/V without a mask ([FN] §6).  The block K/V stay in the workspace: the
 * context cache is only read.
 *   anchor_ids [kv->batch] int32
 *   hidden_out [kv->batch * (B-1), hidden] storage type: final-norm hidden
 *              states of mask rows 1..B-1 of every sequence (sequence-major). */
int dflash_draft_block(dflash_handle h, const int32_t *anchor_ids, const dflash_kv *kv, void *hidden_out,
                       void *ws, size_t ws_bytes, void *stream);

/* Target verify: one causal pass of a target decoder (a handle created from
 * its config and weights; cfg.block_size = rows per sequence) over the tokens
 * ids[s][0..B-1] at positions ctx_len[s] .. ctx_len[s]+B-1.  The target checks
 * the whole drafted block in one forward pass ([FN] §1 and the §2 cycle) and
 * its hidden states at uniformly spaced layers become the drafter's context
 * features ([SUM] §2.2; [INS]).  Each row attends to the context and to the
 * block rows up to itself; every layer's block K/V are written to the cache at
 * those positions (ctx_len is not changed: the caller advances it by the
 * accepted length, and a later call overwrites the rest).  The same call with
 * B = prompt length serves as the prefill.
 *   ids        [kv->batch, B] int32 token ids
 *   tap_layers HOST [n_taps] 0-indexed layers (< n_layers), 0 <= n_taps <= 64
 *   taps_out   [kv->batch * B, n_taps * hidden] storage type: the residual
 *              stream after layer tap_layers[i] (before the final norm) in
 *              column block i; may be NULL when n_taps == 0
 *   hidden_out [kv->batch * B, hidden] storage type: final-norm hidden states
 *              of every row; dflash_lmhead_argmax turns them into y_1..y_B.
 * Errors: NULL pointers, n_taps out of range (DFLASH_ERR_SHAPE), a tap layer
 * out of range (DFLASH_ERR_RANGE), a workspace below dflash_workspace_size. */
int dflash_target_verify(dflash_handle h, const int32_t *ids, const dflash_kv *kv, const int32_t *tap_layers,
                         int32_t n_taps, void *taps_out, void *hidden_out, void *ws, size_t ws_bytes, void *stream);

/* A9: shared LM head and greedy argmax ([FN] §3.1; [SUM] §2.3).
 * logits = hidden * lm_head^T in fp32; ids_out[r] = the lowest id among the
 * maxima of row r.  A NaN logit never wins; a row with no logit above -inf
 * (all NaN or -inf) gets id 0 and max logit -inf, so ids_out always lies in
 * [0, vocab).
 *   hidden        [rows, hidden] storage type
 *   ids_out       [rows] int32; may be NULL when logits_out is given (logits only,
 *                 the input of temperature sampling; max_logit_out is then unused)
 *   max_logit_out [rows] fp32, may be NULL
 *   logits_out    [rows, vocab] fp32, may be NULL */
int dflash_lmhead_argmax(dflash_handle h, const void *hidden, int32_t rows, int32_t *ids_out,
                         float *max_logit_out, float *logits_out, void *ws, size_t ws_bytes, void *stream);

/* dflash_lmhead_argmax without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments and results as dflash_lmhead_argmax
 * with logits_out NULL.  The argmax partials live in a scratch array inside the
 * library instead of a caller workspace: 8 MiB per device, held until the
 * process ends, its address looked up once per device on the first call made
 * with that device current.  Calls may use up to
 *   256 KiB + 2 * (rows * (vocab / 16) * 4 bytes, rounded up to 256) <= 8 MiB
 * (106 rows at vocab 151936); more rows return DFLASH_ERR_WORKSPACE.  The
 * call allocates nothing.  Every call on one device shares that device's
 * array: calls that overlap on one GPU (two streams, two threads) race, so
 * order them on one stream.  Nothing in the array needs clearing between
 * calls (each call writes every partial it reads). */
int dflash_lmhead_argmax_noalloc(dflash_handle h, const void *hidden, int32_t rows, int32_t *ids_out,
                                 float *max_logit_out, void *stream);

/* A10: greedy verify ([FN] §1 and §2 box, point (b)).  For each sequence,
 * k = the number of leading positions where draft_ids equals target_ids
 * (at most B-1), accept_len_out = k + 1 and bonus_out = target_ids[k].
 *   draft_ids  [batch, B-1] int32: d_1..d_{B-1}
 *   target_ids [batch, B]   int32: the target's greedy token y_1..y_B for the
 *              positions after anchor, d_1, .., d_{B-1}
 * Needs no handle; 2 <= block_size <= 64. */
int dflash_accept_len(const int32_t *draft_ids, const int32_t *target_ids, int32_t batch, int32_t block_size,
                      int32_t *accept_len_out, int32_t *bonus_out, void *stream);

/* A10 with a block size per sequence (dynamic block size at inference: the
 * drafter trained with B drafts B_s - 1 <= B - 1 tokens, [SUM] §3 item 4 and
 * §4 block-size ablation): as dflash_accept_len over the first B_s - 1 drafts and B_s
 * target tokens of each sequence, so accept_len_out <= B_s.
 *   block_len [batch] int32 device, B_s clamped to 1..block_size; NULL means
 *             block_size for every sequence.  Layouts as dflash_accept_len. */
int dflash_accept_len_ragged(const int32_t *draft_ids, const int32_t *target_ids, int32_t batch,
                             int32_t block_size, const int32_t *block_len, int32_t *accept_len_out,
                             int32_t *bonus_out, void *stream);

/* Range check of the device-resident indices the hot calls trust (they do not
 * test them: an id >= vocab or a page >= n_pages there is undefined).  Enqueues
 * one small kernel on `stream` that ORs into *err_out (device int32, zeroed by
 * the caller) these bits:
 *   DFLASH_BAD_CTX_LEN    ctx_len[s] outside [0, kv->max_ctx]
 *   DFLASH_BAD_CTX_PAGE   a block_table entry covering context positions
 *                         0 .. ctx_len[s]-1 outside [0, n_pages)
 *   DFLASH_BAD_BLOCK_PAGE ctx_len[s] + block_size > max_pages * page_size, or an
 *                         entry covering the block positions outside [0, n_pages)
 *                         (only dflash_target_verify writes there)
 *   DFLASH_BAD_TOKEN_ID   anchor_ids[s] (kv->batch entries) or ids[t] (n_ids
 *                         entries) outside [0, vocab)
 *   DFLASH_BAD_INJECT_SLOT an inject (seq[t], pos[t]) pair (n_new entries) with
 *                         seq outside [0, batch), pos outside [0, max_pages *
 *                         page_size) or its page entry outside [0, n_pages).
 * anchor_ids, ids and seq/pos may be NULL (not checked) when their count is 0
 * (anchor_ids: NULL skips them).  Every read is bounded by the host-side sizes,
 * so any index values are safe to check.  Host errors: NULL handle, kv or
 * err_out, invalid kv sizes, negative counts. */
enum {
    DFLASH_BAD_CTX_LEN = 1,
    DFLASH_BAD_CTX_PAGE = 2,
    DFLASH_BAD_BLOCK_PAGE = 4,
    DFLASH_BAD_TOKEN_ID = 8,
    DFLASH_BAD_INJECT_SLOT = 16
};
int dflash_check_inputs(dflash_handle h, const dflash_kv *kv, const int32_t *anchor_ids, const int32_t *ids,
                        int32_t n_ids, const int32_t *seq, const int32_t *pos, int32_t n_new, int32_t *err_out,
                        void *stream);

/* Verification at temperature T > 0 ([FN] §1: drafts that pass are kept and
 * the first failing position is drawn again from the target's distribution, so
 * the output has the target's own distribution).  The rule is the published
 * speculative-sampling one: with p_i = softmax(target logits / T) and
 * q_i = softmax(drafter logits / T) for position p+i, draft d_i (drawn from
 * q_i) is kept while u_i * q_i(d_i) < p_i(d_i), u_i uniform on (0, 1); the first
 * rejected position takes a draw from max(0, p_i - q_i) (normalised), and when
 * every draft is kept the next token is the target's draw from p_B.
 *
 * Random numbers: Philox4x32-10 (Salmon et al., SC 2011) keyed by `seed`,
 * counter (column / 4, row, offset, tag), word column mod 4, u = (w >> 9 + 1/2)
 * * 2^-23.  A categorical draw is the Gumbel-max rule argmax_v(log weight_v -
 * log(-log u_v)), lowest id on ties.  The same (seed, offset, tag, row) gives
 * the same draw; advance `offset` between cycles.
 *
 * Logits are fp32 row-major [rows, vocab] (dflash_lmhead_argmax with
 * ids_out == NULL writes them) and must be finite.  Temperature must be finite
 * and > 0 (greedy verify is dflash_accept_len).  Workspace: at least
 * dflash_sample_workspace_size(rows, vocab) bytes (rows = batch for
 * dflash_accept_sample), device memory owned by the caller. */
int dflash_sample_workspace_size(int32_t rows, int32_t vocab, size_t *bytes);

/* One draw per row from softmax(logits[r] / T), with counter row r and the
 * caller's `tag` (tags 0xFFFFFFFE and 0xFFFFFFFF are dflash_accept_sample's:
 * DFLASH_ERR_RANGE).  ids_out [rows] int32; lse_out [rows] fp32 (may be NULL):
 * the natural log of sum_v exp(logits[r][v] / T).  Drafts are drawn with it
 * from the drafter's logits, and the target's rows give p_B's draw and the
 * target lse dflash_accept_sample needs. */
int dflash_sample(const float *logits, int32_t rows, int32_t vocab, float temperature, uint64_t seed,
                  uint32_t offset, uint32_t tag, int32_t *ids_out, float *lse_out, void *ws, size_t ws_bytes,
                  void *stream);

/* The accept / resample rule above for each sequence s (counter row s):
 *   draft_logits [batch * (B-1), vocab] fp32: the drafter's rows for p+1..p+B-1
 *   draft_lse    [batch * (B-1)] fp32 and draft_ids [batch, B-1] int32: from
 *                dflash_sample over draft_logits (an id outside the vocabulary
 *                is rejected)
 *   target_logits [batch * B, vocab] fp32: verify rows 0..B-1 (positions p+1..p+B)
 *   target_lse    [batch * B] fp32 and target_ids [batch, B] int32: from
 *                dflash_sample over target_logits
 *   block_len    [batch] int32 or NULL: per-sequence block size B_s (clamped to 1..B)
 *   accept_len_out [batch]: tau in [1, B_s]; bonus_out [batch]: the token at
 *                position p + tau.  If fp32 rounding leaves no positive
 *                residual at a rejected position, the target's draw there is
 *                taken.  2 <= block_size <= 64. */
int dflash_accept_sample(const float *draft_logits, const float *draft_lse, const int32_t *draft_ids,
                         const float *target_logits, const float *target_lse, const int32_t *target_ids,
                         int32_t batch, int32_t block_size, const int32_t *block_len, int32_t vocab,
                         float temperature, uint64_t seed, uint32_t offset, int32_t *accept_len_out,
                         int32_t *bonus_out, void *ws, size_t ws_bytes, void *stream);

/* Measurement hook (not a step of the method): HIP events recorded on the
 * launch stream around each stage of every layer of dflash_draft_block and
 * dflash_target_verify, so that a caller can time each kernel of the pass in
 * place (the draft step is memory-bound, [FN] introduction and section 1, and
 * each stage is reported against its own roofline).  Stages: QKV = the
 * attention RMSNorm and QKV projection with RoPE; ATTENTION = block attention
 * (and, in a target verify over more than 16 rows, the cache append); O = the
 * output projection and residual; GATE_UP = the MLP RMSNorm, gate/up
 * projection and SwiGLU; DOWN = the down projection and residual.
 *   events   HOST array of n_events hipEvent_t handles (as void*), created by
 *            the caller, or NULL to turn the hook off (the default).  The
 *            array is copied; the events must outlive every call that records
 *            them.  For layer l and stage s the pass records
 *            events[2 * (l * DFLASH_N_STAGES + s)] before the stage's first
 *            launch and events[2 * (l * DFLASH_N_STAGES + s) + 1] after its last.
 *   n_events 2 * DFLASH_N_STAGES * n_layers when events is not NULL.
 * Errors: NULL handle or a NULL entry (DFLASH_ERR_NULL), a wrong n_events
 * (DFLASH_ERR_SHAPE). */
enum {
    DFLASH_STAGE_QKV = 0,
    DFLASH_STAGE_ATTENTION = 1,
    DFLASH_STAGE_O = 2,
    DFLASH_STAGE_GATE_UP = 3,
    DFLASH_STAGE_DOWN = 4,
    DFLASH_N_STAGES = 5
};
int dflash_set_stage_events(dflash_handle h, void *const *events, int32_t n_events);

/* Streaming read of `bytes` bytes at `src` (device, 16-byte aligned, bytes a
 * multiple of 16): every 32-bit word is XOR-folded into *sink (device, one
 * uint32 the caller zeroes first).  Not a step of the method: it measures the
 * read bandwidth that bounds the draft step, which [FN] (introduction and
 * section 1) describes as memory-bound, i.e. timed by moving weights and KV
 * through memory; a step's bytes/s are reported against it.
 * Errors: NULL pointers (DFLASH_ERR_NULL), a misaligned `src` or a size that
 * is not a multiple of 16 (DFLASH_ERR_SHAPE).  bytes == 0 enqueues nothing. */
int dflash_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* Human-readable name of a status code (static string). */
const char *dflash_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
