// Launch interface of the gfx950 kernels (internal header, host side).
//
// Element type `dt` is PCD_DTYPE_F32 or PCD_DTYPE_BF16 for weights and
// activations; the residual stream, softmax statistics and all reductions are
// fp32.  Every launch goes on the given stream; none allocates or syncs.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace pcd {

// Rows of B (a weight matrix [N][K], row-major) may come from up to three
// concatenated matrices: rows [begin[s], begin[s+1]) of the virtual matrix
// are rows [0, ...) of ptr[s].
struct BSegs {
    const void *ptr[3];
    int32_t begin[3];
    int32_t nseg;
};

enum class Epi : int {
    Qkv,      // RoPE on q and k, q -> q buffer, k and v -> a KV cache
    Resid,    // x[m][n] += c (fp32 residual stream), then h = rmsnorm(x) * norm_w for the next GEMM
    Partial,  // split-K partial sums -> part[split][m][n] (chosen inside gemm() for Resid)
    SwiGlu,   // two B operands: out[m][n] = silu(c_gate) * c_up
    Readout,  // per-row (max, sum exp) of the tile + gathered candidate logits
};

struct GemmCall {
    int dt;
    const void *A;   // [M][K] activations, element type dt
    int32_t M, N, K;
    BSegs B[2];      // B[1] used by SwiGlu only
    Epi epi;
    // epilogue arguments
    float *x;        // Resid: residual [M][N]
    float *part;     // Resid: scratch for the (split-K) partial sums
    size_t part_cap; // floats available at part (at least M*N)
    const float *norm_w;  // Resid: weight of the RMSNorm that follows (NULL: none)
    float eps;
    void *h_out;     // Resid: [M][N] normalised rows (dt)
    void *out;       // SwiGlu: [M][N] of dt;  Qkv: q buffer [M][Hq][hd]
    void *kc, *vc;   // Qkv: K and V cache of this layer, [Hkv][cap][hd] each
    int32_t cap;     // Qkv: tokens per KV head in the cache
    void *kc2, *vc2; // Qkv (optional): rows m >= kv_split go to row m - kv_split of this cache instead
    int32_t cap2, kv_split;
    // Qkv (optional, replaces kc/vc): rows spread over several KV buffers.
    // Row m goes to buffer kv_req[m] at token slot kv_row[m]; buffer r
    // starts at kv_base[r], is laid out [layer][K|V][Hkv][kv_cap[r]][hd],
    // and this call writes layer kv_layer.
    const int32_t *kv_req, *kv_row, *kv_cap;
    const uint64_t *kv_base;
    int32_t kv_layer;
    const int32_t *pos;  // Qkv: position of each row (NULL: row index)
    const float2 *rope;  // Qkv: [max_seq][hd/2] (cos, sin)
    int32_t n_q, n_k, hd;    // Qkv: columns of q and of k; head dim
    float2 *ro_part;         // Readout: [N/128][M] (max, sum exp) per vocab tile
    const int32_t *g_tok, *g_ro;  // Readout: gathered token ids and their readout rows
    int32_t n_gather;
    float *g_logit;          // Readout: [n_gather]
    int32_t stagger;         // k-stage rotation per row tile (0: every tile in k order)
};

// Returns false (and does nothing) on a shape the kernels do not support.
bool gemm(const GemmCall &c, hipStream_t st);
int gemm_k_tile(int dt);  // elements of K per pipeline stage

// x[t] = E[tok[t]]; h[t] = rmsnorm(x[t]) * w as dt
void embed(int dt, const int32_t *tok, int32_t T, const void *E, int32_t d, float *x, const float *w, float eps,
           void *h, hipStream_t st);
// out[i] = x[rows ? rows[i] : i] / sqrt(mean(x^2) + eps) * w, as dt
void rmsnorm(int dt, const float *x, const int32_t *rows, int32_t n, int32_t d, const float *w, float eps, void *out,
             hipStream_t st);
// x[m][n] += sum over s of part[s][m][n] (s increasing); then, if w, h[m] = rmsnorm(x[m]) * w
void resid_norm(int dt, const float *part, int32_t splits, int32_t M, int32_t N, float *x, const float *w, float eps,
                void *h, hipStream_t st);

// Attention over KV caches, flash style.  Query rows of a block are (token,
// head within the KV group) pairs, token-major.  A block covers prefix keys
// [key0, key1) of its request's state and, for branch tokens, the branch keys
// [sfx_lo, sfx_hi) (masked to each row's scaffold up to itself and its trie
// ancestors).  nsplit == 1: the block writes the final output; otherwise
// partials for attention_merge.
struct AttnBlock {
    int32_t req, g, row0, nrows, key0, key1, split, nsplit, sfx_lo, sfx_hi;
    int32_t causal;  // rows see keys up to their own position; else the whole key range
    int32_t qoff;    // causal blocks: row token t is at position t + qoff and sees keys <= t + qoff
                     // (rows with t + qoff < key0 are skipped)
};
struct AttnCall {
    int dt;
    int32_t hd, n_heads, n_kv_heads, layer;
    const void *q;          // [tokens][Hq][hd]
    const uint64_t *req_kv; // per request: device address of its KV buffer ([L][2][Hkv][P][hd])
    const int32_t *req_stride; // per request: tokens per (layer, K|V, KV head) slab of its KV buffer
    const AttnBlock *blocks;
    int32_t n_blocks;
    int32_t branch0;        // first row token of the branch tokens (their plan index is token - branch0)
    const int32_t *tok_splits;  // per row token: key splits covering it (<= 1: written directly)
    void *out;              // [tokens][Hq][hd] (dt)
    float *part_o;          // [split][tokens][Hq][hd] unnormalised
    float2 *part_ml;        // [split][tokens][Hq] (max in log2 units, sum)
    int32_t n_tokens;       // tokens of this pass (row stride of the partials)
    const void *kb, *vb;    // branch K/V of this layer, [Hkv][cap][hd] (branch pass only)
    int32_t cap;
    const int32_t *fs, *nsc, *par;  // per branch token: field start, scaffold length, trie parent
    const int4 *chain;              // per branch token: 8 links of its trie chain (itself, parent, ...; -1 past the root)
    int32_t wide;  // nonzero: blocks of up to 128 query rows, causal prefix keys only (bf16); else up to 64 rows
    int32_t halves;  // nonzero (64-row bf16 blocks): 8-wave blocks walking two key chains each, whatever the block
                     // count (else only launches of at most 256 blocks)
};
bool attention(const AttnCall &c, hipStream_t st);  // false: unsupported head_dim/dtype

// 64-row bf16 launches of at most this many blocks take the two-chain form
// (8-wave blocks, one per compute unit) without being asked.
constexpr int ATT_HALVES_MAX_BLOCKS = 256;

// Key splits of one attention row block at most (the merge kernel holds
// every split of a (token, head) in registers).
constexpr int ATT_MAX_SPLITS = 8;

// Merge the split partials of each (token, head) whose request used more
// than one split.
struct TailCall {
    int dt;
    int32_t hd, n_heads, n_kv_heads, n_tokens;
    int32_t tok0;               // tokens [tok0, n_tokens) are merged
    const float *part_o;
    const float2 *part_ml;
    const int32_t *tok_splits;  // per token: its splits are 0..tok_splits[t]-1 (<= 1: nothing to merge)
    void *out;                  // [tokens][Hq][hd]
};
void attention_merge(const TailCall &c, hipStream_t st);

// Row i of dst_a / dst_b = row rows[i] of src_a / src_b, for i < n (rows of
// bytes_a / bytes_b bytes, multiples of 16).
void gather_rows2(const void *src_a, size_t bytes_a, void *dst_a, const void *src_b, size_t bytes_b, void *dst_b,
                  const int32_t *rows, int32_t n, hipStream_t st);

// lse[r] from the per-tile partials of the readout GEMM.
void readout_lse(const float2 *part, int32_t n_tiles, int32_t R, float *lse, hipStream_t st);

// Scoring modes of a field in CombineCall::f_mode (the public PCD_SCORE_* values).
constexpr int SCORE_PATH = 0, SCORE_EXACT = 1, SCORE_LEVEL = 2, SCORE_MEAN = 3;

// Per field: logscore, softmax(logscore / T), mass, argmax, margin.
struct CombineCall {
    int32_t n_fields;
    const int32_t *f_cand_off, *f_ro_root, *f_mode, *c_spell_off, *s_path_off, *s_path, *g_off, *g_ro;
    const float *z, *lse;
    float temperature;
    float *prob, *logscore, *mass, *margin;
    int32_t *argmax;
};
void combine(const CombineCall &c, hipStream_t st);

}  // namespace pcd
