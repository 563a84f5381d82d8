/*
 * pcd.h -- C ABI of the parallel constrained decoding (PCD) library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (pages cited by title and section):
 *   - "Parallel Constrained Decoding from Scratch" (faritgaleev.com), sections
 *     "The piece of plumbing you need: the KV cache" and "The idea: parallel
 *     constrained decoding": prefill a shared prompt once; give every schema
 *     field one short row that ends where its labels part ways; run all rows
 *     in one batched pass over the shared prompt's KV cache; read each row's
 *     next-token distribution restricted to the tokens that start an allowed
 *     label; report the renormalised probabilities and the candidate mass.
 *   - same page, "When one token is not enough": labels whose first tokens
 *     collide are told apart by extending the row down the shared branch in
 *     the same batched pass and multiplying along the path.
 *   - "Parallel Constrained Decoding: A Technical Reference" (shivam2003.com),
 *     section 4 "The algorithm": candidate softmax with temperature, argmax.
 *   - "Parallel Constrained Decoding from Scratch", "Small models quote their
 *     booleans": a label is the set of its spellings; its probability is the
 *     sum of its spellings' path products (pcd_candidate.spell_len).
 *   - Scoring modes for multi-token labels (pcd_field.score_mode): the same
 *     page's "When one token is not enough" (scoring a label to the end of
 *     its line), the "Parallel Constrained Decoding" engine README, "The
 *     technique" (a product of per-level probabilities), and "Parallel
 *     Constrained Decoding, From First Principles", "Multi-token candidates"
 *     (length-normalised log-probabilities).
 *
 * Everything here works on token ids; tokenizing is the caller's business.
 *
 * Conventions
 *   - Every function returns an int status: PCD_OK (0) or a negative PCD_E_*
 *     code; pcd_last_error() then holds a message (thread-local).
 *   - All validation happens before any device work: a failing call leaves
 *     no partial state and writes no output.
 *   - Device memory (weights, KV buffers, workspace) is allocated by the
 *     caller and borrowed by the library; it must outlive the handles that
 *     use it.  Handles are library-owned host objects, freed with pcd_free_*.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call that
 *     takes a stream enqueues its device work there and returns after that
 *     stream has drained, except pcd_prefill, pcd_prefill_many and
 *     pcd_extend_decide_start, which return once their work is enqueued.
 *   - A model's passes share its workspace: while a call of the model is
 *     still running on the device, the model's other calls go on the same
 *     stream.  A prefill, extend or decide call on another stream fails with
 *     PCD_E_ARG (before any device work) while a started decide call or a
 *     prefill / extend pass of the same model has not left the device.
 *   - A model is used from one host thread at a time.
 */
#ifndef PCD_H
#define PCD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PCD_OK 0
#define PCD_E_ARG (-1)     /* null pointer, negative count, unsupported shape */
#define PCD_E_TOKEN (-2)   /* token id outside [0, vocab_size) */
#define PCD_E_NCAND (-3)   /* a field with fewer than 2 or more than 255 candidates, or too many spellings */
#define PCD_E_EMPTY (-4)   /* empty scaffold, empty candidate or spelling, or a label without spellings */
#define PCD_E_DUP (-5)     /* two identical candidate token sequences in one field */
#define PCD_E_PREFIX (-6)  /* a candidate is a proper prefix of another one */
#define PCD_E_CAP (-7)     /* a size exceeds max_seq, the workspace limits or a buffer */
#define PCD_E_STATE (-8)   /* state handle of another model */
#define PCD_E_DEVICE (-9)  /* HIP runtime error; the HIP message is in pcd_last_error() */
#define PCD_E_NOMEM (-10)  /* host allocation failed */

#define PCD_MAX_CANDIDATES 255
#define PCD_MAX_SPELLINGS 1024 /* spellings of all labels of one field */

/* Scoring modes.  A label's spelling c is scored on the log-probabilities of
 * its tokens c[0..u], each conditioned on prefix + scaffold + c[<i]:
 *   PATH  (0, the default): full-vocabulary log p, down to u(c), the first
 *         token at which no other spelling of the field shares c's tokens;
 *   EXACT (1): full-vocabulary log p of every token of c, to its end;
 *   LEVEL (2): down to u(c), each token's probability renormalised over the
 *         distinct tokens that the field's spellings continue with at that
 *         point (a softmax over the trie node's children);
 *   MEAN  (3): the EXACT sum divided by c's token count.
 * The candidate mass is always the full-vocabulary probability of the
 * distinct first tokens. */
#define PCD_SCORE_PATH 0
#define PCD_SCORE_EXACT 1
#define PCD_SCORE_LEVEL 2
#define PCD_SCORE_MEAN 3

#define PCD_DTYPE_F32 0
#define PCD_DTYPE_BF16 1

/* ---- model description ---------------------------------------------------- */
/* A Qwen2.5-shaped decoder: RMSNorm, rotate-half RoPE, grouped-query attention
 * without biases, SwiGLU MLP.  head_dim must be 32, 64 or 128; d_model,
 * n_heads*head_dim and ffn_dim must be multiples of 128 (64 for f32 models);
 * vocab_size a multiple of 128. */
typedef struct {
    int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab_size;
    int32_t max_seq;       /* largest position id + 1 (RoPE table size) */
    float rope_theta;      /* inverse frequency of pair j is theta^(-2j/head_dim) */
    float rms_eps;         /* x / sqrt(mean(x^2) + eps) * w */
    int32_t tied_lm_head;  /* 1: the LM head is the embedding matrix */
    int32_t dtype;         /* PCD_DTYPE_F32 or PCD_DTYPE_BF16: weights and activations */
} pcd_config;

/* Device pointers to the weights, elements of cfg.dtype (bf16 = raw 16-bit
 * patterns), every matrix [out][in] row-major.  The per-layer fields are HOST
 * arrays of n_layers DEVICE pointers; the library copies the arrays.  Norm
 * weights are fp32 vectors of d_model.  Every pointer is 16-byte aligned
 * (PCD_E_ARG otherwise), as are KV buffers; the workspace is 256-byte
 * aligned. */
typedef struct {
    const void *embed;          /* [vocab][d] */
    const void *lm_head;        /* [vocab][d]; NULL when tied_lm_head */
    const float *final_norm;    /* [d] */
    const float *const *attn_norm, *const *mlp_norm;           /* [L] -> [d] */
    const void *const *wq, *const *wk, *const *wv, *const *wo; /* [Hq*hd][d], [Hkv*hd][d] x2, [d][Hq*hd] */
    const void *const *w_gate, *const *w_up, *const *w_down;   /* [F][d] x2, [d][F] */
} pcd_weights;

/* Upper bounds a model's workspace is sized for. */
typedef struct {
    int32_t max_prefill_tokens;  /* token rows of one prefill or extend pass: pcd_prefill, pcd_extend,
                                    all sequences of one pcd_prefill_many (each sequence still at
                                    most max_seq); at most 262144 */
    int32_t max_branch_tokens;   /* scaffold + trie tokens of one decide call, all requests; at most 262144 */
    int32_t max_readouts;        /* readout rows of one decide call */
    int32_t max_gathers;         /* candidate-token logits gathered by one decide call */
    int32_t max_fields;          /* fields of one decide call, all requests */
    int32_t max_candidates;      /* candidates of one decide call, all requests */
    int32_t max_requests;        /* requests of one pcd_decide_many call */
    int32_t max_spellings;       /* spellings of one decide call, all requests; 0: max_candidates */
} pcd_limits;

/* ---- one request's schema (host memory, read during the call) ------------ */
/* A candidate is one label.  Without spellings (spell_len NULL) its token
 * ids are `tokens`.  With spellings, `tokens` holds n_spellings token
 * sequences back to back, of lengths spell_len[0..n_spellings), each >= 1 and
 * summing to n_tokens; the label's probability sums over them.  Within a
 * field, all spellings of all labels must be distinct and none a proper
 * prefix of another; a field has at most PCD_MAX_SPELLINGS spellings. */
typedef struct {
    const int32_t *tokens;
    int32_t n_tokens;
    const int32_t *spell_len;  /* NULL: one spelling */
    int32_t n_spellings;       /* ignored when spell_len is NULL */
} pcd_candidate;

typedef struct {
    const int32_t *scaffold;  /* the field's row: key tokens up to where its labels part ways */
    int32_t n_scaffold;
    int32_t cand_offset;      /* first candidate of this field in the request's candidate array */
    int32_t n_cands;          /* 2..255 */
    int32_t score_mode;       /* PCD_SCORE_*; 0 (zero-initialised) is PCD_SCORE_PATH */
} pcd_field;

typedef struct {
    const pcd_field *fields;
    int32_t n_fields;
    const pcd_candidate *candidates;
    int32_t n_candidates;
} pcd_request;

/* ---- results (caller-owned HOST arrays, written only on PCD_OK) ---------- */
typedef struct {
    float *cand_prob;        /* [n_candidates] softmax of logscore / T over each field's candidates */
    float *cand_logscore;    /* [n_candidates] nullable: the label's score under its field's mode; with
                              * spellings, log of the sum of exp(spelling score) */
    float *field_mass;       /* [n_fields] full-vocabulary probability of the distinct first tokens */
    float *field_margin;     /* [n_fields] top-1 minus top-2 logscore, nats */
    int32_t *field_argmax;   /* [n_fields] candidate index within the field; ties to the lowest index */
    float *readout_lse;      /* nullable [n_readouts]: log-sum-exp of each readout row's logits */
    float *gather_logit;     /* nullable [n_gathers]: the gathered candidate-token logits */
} pcd_outputs;

/* Counters of the last calls on a model. */
typedef struct {
    int64_t prefill_passes;   /* batched decoder passes run by prefill calls */
    int64_t branch_passes;    /* batched decoder passes run by decide calls */
    int32_t last_branch_tokens, last_readouts, last_gathers, last_requests;
    float last_prefill_ms, last_branch_ms, last_readout_ms; /* hipEvent times of the last calls */
    int64_t workspace_bytes;
} pcd_stats;

/* Plan of one decide call, as laid out for the batched pass (host only). */
typedef struct {
    int32_t n_branch, n_readouts, n_gathers, n_fields, n_candidates, n_paths, n_anc, n_spellings;
    /* Optional host arrays (NULL to skip), sized by the counts above:
     * per branch token: tok, pos, req, field; anc_off [n_branch+1] and anc
     * [n_anc]: the branch tokens each one sees (ascending, itself last);
     * per readout: ro_tok, ro_field, g_off [n_readouts+1]; per gather: g_tok;
     * per field: f_ro_root, f_cand_off [n_fields+1], f_mode (PCD_SCORE_*);
     * per candidate: c_spell_off [n_candidates+1] (its spellings); per
     * spelling: s_path_off [n_spellings+1] and s_path [n_paths] (the gather
     * indices it is scored on, in depth order). */
    int32_t *tok, *pos, *req, *field, *anc_off, *anc;
    int32_t *ro_tok, *ro_field, *g_off, *g_tok;
    int32_t *f_ro_root, *f_cand_off, *f_mode, *c_spell_off, *s_path_off, *s_path;
} pcd_plan_info;

/* ---- functions -------------------------------------------------------------- */

typedef struct pcd_model pcd_model;  /* opaque, library-owned host object */
typedef struct pcd_state pcd_state;  /* opaque: a prefilled prefix over a caller-owned KV buffer */
typedef struct pcd_pending pcd_pending;  /* opaque: a started decide call, until pcd_finish */

/* Decide calls of one model that may be in flight at once (started and not
 * yet finished). */
#define PCD_MAX_PENDING 4

/* Bytes of device workspace a model with this config and these limits needs.
 * Returns 0 on invalid arguments. */
size_t pcd_workspace_bytes(const pcd_config *cfg, const pcd_limits *lim);

/* Create a model over caller-owned device weights and a caller-owned device
 * workspace of ws_bytes >= pcd_workspace_bytes(cfg, lim).  Uploads the RoPE
 * cos/sin table (computed on the host in double precision, stored as fp32)
 * into the workspace on `stream`.  The weights are only read, never written,
 * so several models may borrow the same weights: each with its own workspace
 * and on its own stream, their calls run on the device at once (independent
 * requests overlap, and one request's kernels use the compute units another's
 * leave idle). */
int pcd_load_weights(const pcd_config *cfg, const pcd_limits *lim, const pcd_weights *w,
                     void *workspace, size_t ws_bytes, void *stream, pcd_model **out);

/* pcd_load_weights for callers that cannot allocate device memory: code
 * that must not call hipMalloc (under HIP graph capture, in tight serving
 * loops, in harnesses that forbid it).  The model's workspace is the
 * library's static device array of PCD_NOALLOC_WORKSPACE_MAX bytes (one per
 * GPU, in the library's code object, held until the process ends), so this
 * call allocates no device or pinned memory: its plan and result staging are
 * pageable host memory, and its calls run the same kernels as a model from
 * pcd_load_weights.  Weights, KV buffers and result arrays stay the
 * caller's.  Fails with PCD_E_CAP when the config and limits need a larger
 * workspace (pcd_workspace_bytes), and with PCD_E_ARG while another model
 * on the same device (the current one at this call) uses the static array:
 * one such model per GPU at a time, freed with pcd_free_model like any
 * other.  The array keeps the contents of the last call; every pass writes
 * what it reads first, as with a caller's workspace.  Its calls follow the
 * model's stream rule; calls on one GPU that overlap in time race on the
 * array.  Arguments, errors and everything else as for pcd_load_weights. */
#define PCD_NOALLOC_WORKSPACE_MAX ((size_t)128 << 20)
int pcd_load_weights_noalloc(const pcd_config *cfg, const pcd_limits *lim, const pcd_weights *w, void *stream,
                             pcd_model **out);

/* Bytes of the KV buffer a state of n_tokens needs:
 * n_tokens x n_layers x 2 (K, V) x n_kv_heads x head_dim x element size
 * ("Parallel Constrained Decoding from Scratch", "the KV cache").
 * Layout: [layer][K|V][kv head][cap][head_dim], K after RoPE, where the
 * buffer's capacity cap = min(kv_bytes / pcd_state_bytes(m, 1), max_seq)
 * tokens is fixed when the state is created (equal to the token count for a
 * buffer of exactly pcd_state_bytes(m, n) bytes).  A state may grow by
 * pcd_extend up to its capacity. */
size_t pcd_state_bytes(const pcd_model *m, int32_t n_tokens);

/* Prefill: one causal pass of the decoder over tokens[0..n_tokens) (host
 * array) at positions 0..n_tokens-1, writing every layer's K and V into the
 * caller's device buffer kv_buf (kv_bytes >= pcd_state_bytes).  No final norm
 * and no LM head are run ("The idea: parallel constrained decoding", step 1:
 * the shared prompt is read once).  On success *out is a new state handle
 * that borrows kv_buf.  The call returns once the pass is enqueued on
 * `stream` (it waits only for its small host-to-device plan upload), so the
 * host can prepare the decide call while the device runs the prefill: kv_buf
 * is complete when `stream` reaches the end of this call's work.  Decide
 * calls on the same stream are ordered after it; other streams must wait on
 * it first.  last_prefill_ms in pcd_get_stats is read when the pass has
 * finished (pcd_get_stats waits for it). */
int pcd_prefill(pcd_model *m, const int32_t *tokens, int32_t n_tokens, void *kv_buf, size_t kv_bytes,
                void *stream, pcd_state **out);

/* Prefill of a batch of prompts in one causal pass: n_seqs sequences given
 * back to back in tokens (host array; sequence r has lens[r] >= 1 tokens),
 * each at positions 0..lens[r]-1 and attending only its own tokens, so the
 * result per sequence is that of pcd_prefill on it alone (the batched form of
 * "Parallel Constrained Decoding from Scratch", "The idea: parallel
 * constrained decoding", step 1, for many requests at once).  Sequence r's K
 * and V go to kv_bufs[r] (device, kv_bytes[r] >= pcd_state_bytes(m,
 * lens[r]); buffers must not overlap), and out[r] (host array of n_seqs
 * handles) receives its state.  n_seqs <= max_requests and the total token
 * count <= max_prefill_tokens; everything is validated before any device
 * work, and on failure no state is created.  Ordering and timing as for
 * pcd_prefill. */
int pcd_prefill_many(pcd_model *m, int32_t n_seqs, const int32_t *tokens, const int32_t *lens, void *const *kv_bufs,
                     const size_t *kv_bytes, void *stream, pcd_state **out);

/* Append tokens[0..n_tokens) (host array) to a state: one causal pass of the
 * decoder at positions P..P+n_tokens-1 whose attention covers the state's P
 * cached tokens and the new ones before each token, writing the new tokens'
 * K and V into the state's buffer after the cached ones.  The result equals a
 * prefill of the concatenated tokens.  This is how a cached prompt head is
 * completed by a per-request input, and how a decided field's answer is
 * written in before the remaining fields are decided ("Parallel Constrained
 * Decoding from Scratch", "The idea: parallel constrained decoding": the
 * prompt and the first field's answer).  PCD_E_CAP if P + n_tokens exceeds
 * the buffer's capacity, max_seq or max_prefill_tokens; PCD_E_TOKEN for an id
 * outside the vocabulary; on error the state is unchanged.  Asynchronous
 * like pcd_prefill; counted as a prefill pass. */
int pcd_extend(pcd_state *s, const int32_t *tokens, int32_t n_tokens, void *stream);

/* A new state holding a copy of s's cached tokens in the caller's device
 * buffer kv_buf (kv_bytes >= pcd_state_bytes of s's token count; its
 * capacity as for pcd_prefill), so that one cached prompt head can be
 * extended by many requests.  The copy is enqueued on `stream`; s must not be
 * extended before the stream has passed it.  s is unchanged. */
int pcd_fork(const pcd_state *s, void *kv_buf, size_t kv_bytes, void *stream, pcd_state **out);

/* Tokens a state holds (P); negative (PCD_E_STATE) for an invalid handle. */
int pcd_state_tokens(const pcd_state *s);

/* Decide every field of one request against a prefilled state in ONE batched
 * decoder pass ("Parallel Constrained Decoding from Scratch", "The idea:
 * parallel constrained decoding", steps 2-3: one short row per field that
 * ends where the field's labels part ways, all rows in one batched pass over
 * the shared prompt's cache, the next-token distribution at each row's end
 * restricted to the allowed first tokens and renormalised; the same page,
 * "And you get confidence for free", for the candidate mass; the
 * "Parallel Constrained Decoding" engine README, "The technique": broadcast
 * of the cached prefix, one batched pass, softmax over the candidate tokens
 * only).  Each field's row is its scaffold, placed right after the
 * state's prefix (positions P, P+1, ...).  Candidates whose leading tokens
 * are shared by other candidates are extended by teacher-forced continuation
 * tokens in the same pass (a trie per field); a candidate's logscore sums
 * log p(token | prefix + scaffold + earlier tokens) over its tokens up to and
 * including the first one no other candidate shares.  cand_prob is
 * softmax(logscore / temperature) over the field, field_mass the
 * full-vocabulary probability of the field's distinct first tokens at the
 * scaffold's end (temperature 1).  The state's KV buffer is read, never
 * written, so any number of decide calls may share one state. */
int pcd_decide(pcd_state *s, const pcd_field *fields, int32_t n_fields, const pcd_candidate *candidates,
               int32_t n_candidates, float temperature, pcd_outputs *out, void *stream);

/* Single-pass mode: append tokens[0..n_tokens) to the state AND decide the
 * request's fields against the extended prefix, in ONE batched decoder pass
 * whose first rows are the new tokens (causal over the cached ones and each
 * other, their K/V written into the state's buffer) and whose remaining rows
 * are the fields' branch tokens ("Parallel Constrained Decoding", the Java +
 * llama.cpp engine page, "Java engine details": its optional single-pass
 * mode, prefill and field suffixes in one forward pass).  The results equal
 * pcd_extend followed by pcd_decide, with every weight matrix streamed once.
 * n_tokens may be 0 (then this is pcd_decide).  The pass needs n_tokens plus
 * the branch tokens within the workspace's rows (the larger of
 * max_prefill_tokens and max_branch_tokens).  Errors as for pcd_extend and
 * pcd_decide, all before any device work; on error the state is unchanged.
 * Counted as one branch pass. */
int pcd_extend_decide(pcd_state *s, const int32_t *tokens, int32_t n_tokens, const pcd_field *fields,
                      int32_t n_fields, const pcd_candidate *candidates, int32_t n_candidates, float temperature,
                      pcd_outputs *out, void *stream);

/* pcd_extend_decide in two halves, so that a caller can prepare its next
 * request while the device runs this one (the pages' engines keep one request
 * in flight; a server keeps the device busy across requests).
 *
 * pcd_extend_decide_start validates, plans and enqueues exactly the work of
 * pcd_extend_decide on `stream`, then returns *p without waiting for the
 * device.  The state holds the new tokens at once, so later calls on the
 * same stream may use it.  The arrays of *out (copied by value) receive the
 * results only in pcd_finish(*p); until then they must stay valid and
 * unread.  The token, field and candidate arrays are not read after the call
 * returns.  At most PCD_MAX_PENDING calls of a model are in flight: one more
 * fails with PCD_E_CAP before any device work.  Other errors as for
 * pcd_extend_decide.
 *
 * pcd_finish waits for the call's results, writes them to its output arrays,
 * updates the model's statistics and frees p (also on error).  Calls may be
 * finished in any order.  Every started call must be finished before
 * pcd_free_model. */
int pcd_extend_decide_start(pcd_state *s, const int32_t *tokens, int32_t n_tokens, const pcd_field *fields,
                            int32_t n_fields, const pcd_candidate *candidates, int32_t n_candidates,
                            float temperature, const pcd_outputs *out, void *stream, pcd_pending **p);
int pcd_finish(pcd_pending *p);

/* An empty state (0 tokens) over the caller's device buffer kv_buf (capacity
 * as for pcd_prefill), for pcd_extend / pcd_extend_decide to fill: a cold
 * request in single-pass mode is pcd_new_state + pcd_extend_decide. */
int pcd_new_state(pcd_model *m, void *kv_buf, size_t kv_bytes, pcd_state **out);

/* The first-field round: decide fields[0..n_first) in one batched pass,
 * append each of them (its scaffold followed by its argmax candidate's
 * tokens, the first spelling of a label with spellings, in field order) to
 * the state with pcd_extend, then decide the
 * remaining fields in a second batched pass against the extended prefix, so
 * that their rows see the earlier answers ("Parallel Constrained Decoding
 * from Scratch", "The idea: parallel constrained decoding": decide the first
 * field, write its answer in, decide the rest).  Outputs are indexed as for
 * pcd_decide over the whole request; readout_lse and gather_logit must be
 * NULL.  The whole request is validated first (plans at the longest possible
 * extended prefix, the buffer's capacity); the state then ends holding the
 * prefix plus the answers.  Passes: 2 branch passes and 1 extend. */
int pcd_decide_sequenced(pcd_state *s, const pcd_field *fields, int32_t n_fields, const pcd_candidate *candidates,
                         int32_t n_candidates, int32_t n_first, float temperature, pcd_outputs *out, void *stream);

/* Several requests, each on its own state, in ONE batched pass; outs[i]
 * receives request i's results (arrays indexed within that request).  Each
 * request is decided exactly as pcd_decide decides it ("Parallel Constrained
 * Decoding from Scratch", "The idea: parallel constrained decoding", steps
 * 2-3; the engine README, "The technique"): the rows of all requests share
 * one pass over the weights, and every row attends only its own request's
 * cached prefix, its own scaffold and its trie ancestors.  reqs[i] has the
 * same layout as pcd_decide's arguments; the whole call is validated (every
 * request, and the sum of their rows, readouts, gathers, fields, candidates
 * and spellings against the model's limits, n_req <= max_requests) before
 * any device work, and on error no output is written.  The states' KV
 * buffers are only read. */
int pcd_decide_many(pcd_state *const *states, const pcd_request *reqs, int32_t n_req, float temperature,
                    pcd_outputs *outs, void *stream);

/* Plan of a decide call over requests with the given prefix lengths, without
 * any device work (the branch-token layout, readouts and gathers the batched
 * pass uses).  Fills the counts; fills each non-NULL array. */
int pcd_debug_plan(int32_t vocab_size, int32_t max_seq, int32_t n_req, const int32_t *prefix_lens,
                   const pcd_request *reqs, pcd_plan_info *info);

int pcd_get_stats(const pcd_model *m, pcd_stats *out);

/* Per-kernel timing (for measurement; off by default).  With timing on, every
 * launch of the classes below is bracketed by a pair of hipEvents on the
 * call's stream, and after each call the elapsed times are added to
 * per-class totals.  Enabling resets the totals. */
#define PCD_KC_PREFILL_QKV 0     /* prefill: QKV projection + RoPE + KV write */
#define PCD_KC_PREFILL_ATTN 1    /* prefill: causal attention (its split merge counts as OTHER) */
#define PCD_KC_PREFILL_O 2       /* prefill: O projection + residual */
#define PCD_KC_PREFILL_GATEUP 3  /* prefill: gate/up projection + SwiGLU */
#define PCD_KC_PREFILL_DOWN 4    /* prefill: down projection + residual */
#define PCD_KC_BRANCH_QKV 5
#define PCD_KC_BRANCH_ATTN 6     /* branch: shared-prefix attention over the prefix */
#define PCD_KC_BRANCH_TAIL 7     /* branch: split merge + scaffold/trie-ancestor keys */
#define PCD_KC_BRANCH_O 8
#define PCD_KC_BRANCH_GATEUP 9
#define PCD_KC_BRANCH_DOWN 10
#define PCD_KC_READOUT_LMHEAD 11 /* LM head with online log-sum-exp and candidate gather */
#define PCD_KC_OTHER 12          /* embedding, RMSNorm, log-sum-exp merge, combine, split merges outside the branch pass */
#define PCD_KC_FUSED_QKV 13      /* single-pass mode (pcd_extend_decide): new and branch rows together */
#define PCD_KC_FUSED_ATTN 14     /* single-pass mode: causal and shared-prefix attention (split merge: OTHER) */
#define PCD_KC_FUSED_O 15
#define PCD_KC_FUSED_GATEUP 16
#define PCD_KC_FUSED_DOWN 17
#define PCD_KC_COUNT 18

int pcd_set_kernel_timing(pcd_model *m, int32_t enable);
/* total_ms[PCD_KC_COUNT] and launches[PCD_KC_COUNT], host arrays. */
int pcd_get_kernel_times(const pcd_model *m, float *total_ms, int64_t *launches);

/* NULL-safe.  A state must be freed before its model. */
void pcd_free_state(pcd_state *s);
void pcd_free_model(pcd_model *m);

/* Message of the last failing call on this thread ("" if none). */
const char *pcd_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
