// C ABI of the PCD library: validation, workspace layout, plan upload and the
// launch sequences of prefill and of the batched branch pass + readout.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/pcd.h"
#include "pcd_kernels.h"
#include "pcd_plan.h"

using namespace pcd;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string &msg) {
    g_err = msg;
    return code;
}

#define HIP_TRY(expr)                                                                        \
    do {                                                                                     \
        hipError_t e_ = (expr);                                                              \
        if (e_ != hipSuccess) return fail(PCD_E_DEVICE, std::string(#expr ": ") + hipGetErrorString(e_)); \
    } while (0)

constexpr int MAX_SPLITS = ATT_MAX_SPLITS;  // key splits of one attention row block
constexpr int ATT_ROWS = 64;          // query rows per attention workgroup
// Causal prefill launches (no branch keys) in bf16 use blocks of 128 query
// rows, two 16-row groups per wave, when those alone give at least
// ATT_WIDE_MIN_BLOCKS workgroups (two per compute unit): each K and V
// fragment read from LDS then feeds twice the matrix work.
constexpr int ATT_WIDE_ROWS = 128;
#ifndef ATT_WIDE_MIN_BLOCKS
#define ATT_WIDE_MIN_BLOCKS 512
#endif
constexpr int SPLITK_MAX = 8;
constexpr int SPLITK_ROWS = 1024;     // split-K is only used below this many rows
constexpr uint64_t STATE_MAGIC = 0x70636473746174ull;
constexpr uint64_t PENDING_MAGIC = 0x70636470656e64ull;

size_t align_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }
// device buffers are read and written in 16-byte vectors
bool misaligned(const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 != 0; }

// Attention workgroups per launch below which keys are split over
// workgroups, and the shortest key range worth a workgroup of its own.  Key
// splits cost partial writes and a merge kernel; they pay when few row
// blocks would leave most compute units idle on a long prefix.  On the 1.5B
// shape's 799-row single pass (150 row blocks), a target of 64 (no splits)
// and one of 256 (2 splits, then the merge) give the same time for one
// request at a time, and 64 is 2% faster with three requests running
// concurrently (less total work); 512 and 1024 were slower.
constexpr int ATT_TARGET_BLOCKS = 64;
constexpr int ATT_MIN_SPLIT_TILES = 2;  // 64-key tiles
constexpr int MAX_PASS_ROWS = 1 << 18;  // token rows of one decoder pass
// Long key ranges (branch rows over a long prefix, whose chains are all
// equally long): the split count s that minimises the launch's critical path,
// the rounds of blocks over ATT_SLOTS (two blocks per compute unit) times the
// tiles of one chain, ceil(row_blocks * s / ATT_SLOTS) * ceil(key_tiles / s);
// no split shorter than ATT_LONG_MIN_TILES.  (The 7B shape's 668 branch rows
// over a 16,384-token prefix: 296 row blocks of 256 tiles.)
constexpr int ATT_SLOTS = 2 * 256;
constexpr int ATT_LONG_MIN_TILES = 16;
static int64_t long_chain_splits(int64_t row_blocks, int key_tiles) {
    int64_t best_s = 1, best = -1;
    for (int s = 1; s <= MAX_SPLITS; ++s) {
        const int64_t chain = (key_tiles + s - 1) / s;
        if (s > 1 && chain < ATT_LONG_MIN_TILES) break;
        const int64_t cost = (std::max<int64_t>(1, row_blocks) * s + ATT_SLOTS - 1) / ATT_SLOTS * chain;
        if (best < 0 || cost < best) {
            best = cost;
            best_s = s;
        }
    }
    return best_s;
}
// Key splits of a row block: enough for `row_blocks` blocks to reach the
// target count, no split shorter than the minimum, at most MAX_SPLITS; or,
// in a launch of branch rows only (`equal_chains`: causal rows' lengths vary,
// and their long chains start first), the long-chain count above if larger.
// In a pass that also runs new tokens' causal rows, those fill the slots and
// splitting the branch rows only adds blocks and partials (the 7B single
// pass with 5 splits: 283.1 -> 284.9 ms per request).
static int att_splits(int64_t row_blocks, int key_tiles, bool equal_chains) {
    const int64_t want = (ATT_TARGET_BLOCKS + row_blocks - 1) / std::max<int64_t>(1, row_blocks);
    const int by_len = std::max(1, key_tiles / ATT_MIN_SPLIT_TILES);
    const int64_t want_long = equal_chains ? long_chain_splits(row_blocks, key_tiles) : 1;
    return (int)std::max<int64_t>(1, std::min<int64_t>({std::max(want, want_long), (int64_t)MAX_SPLITS, (int64_t)by_len}));
}

// Causal launches with few blocks per compute unit: a block's keys end at
// its last row, so the longest chains set the launch time (the 2,048-token
// prompt at the 1.5B widths: 384 blocks of 1 to 32 key tiles in 42.7 us,
// about the longest chain's time).  Where the longest chain reaches
// ATT_CHAIN_MODEL_TILES, the split count and block form are the ones of
// least estimated time: the larger of the longest chain and the total work
// over the slots, each workgroup costing ATT_BLOCK_FIXED plus its key tiles.
// 4-wave blocks take two slots per compute unit; 8-wave blocks walking two
// key chains (the form launches of at most ATT_HALVES_MAX_BLOCKS take anyway)
// one slot per compute unit, their chains halved.  Split keys add the merge kernel:
// ATT_MERGE_FIXED plus its fp32 partials (each token's splits x query heads
// x head_dim x 4 bytes) at ATT_MERGE_MB_PER_TILE.  Times are in key tiles
// (about 1.2 us per 64-key tile of a 64-row block).
constexpr int ATT_CHAIN_MODEL_TILES = 16;
constexpr double ATT_BLOCK_FIXED = 2.4;  // entry to first DMA, output write: about 2.8 us
constexpr double ATT_MERGE_FIXED = 1.7;  // the merge kernel's launch and ramp: about 2 us
constexpr double ATT_MERGE_MB_PER_TILE = 3.6;  // partials it reads per key-tile time (about 3 TB/s)
struct ChainSpec {
    int kend;   // keys the block reaches (its last row's causal bound, or the whole prefix)
    int extra;  // key tiles its last split adds (branch keys)
};
struct TokRange {
    int kend0, count;  // count row tokens reaching kend0, kend0 + 1, ... (step) or all kend0
    bool step;
};
struct SplitCost {
    double chain, work;  // longest workgroup and total work over the slots, in key tiles
};
static SplitCost split_cost(const std::vector<ChainSpec> &blocks, int slen, int ns, bool halves) {
    int64_t n = 0, sum = 0, sum_half = 0;
    int longest = 0;
    for (const ChainSpec &b : blocks)
        for (int k = 0; k < ns && k * slen < b.kend; ++k) {
            const bool last = k == ns - 1 || (k + 1) * slen >= b.kend;
            const int t = (std::min(b.kend, (k + 1) * slen) - k * slen + 63) / 64 + (last ? b.extra : 0);
            ++n;
            sum += t;
            sum_half += (t + 1) / 2;
            longest = std::max(longest, t);
        }
    if (halves || n <= ATT_HALVES_MAX_BLOCKS)
        return {ATT_BLOCK_FIXED + (longest + 1) / 2, (sum_half + ATT_BLOCK_FIXED * n) / ATT_HALVES_MAX_BLOCKS};
    return {ATT_BLOCK_FIXED + longest, (sum + ATT_BLOCK_FIXED * n) / ATT_SLOTS};
}
static double merge_cost(const std::vector<TokRange> &toks, int slen, int ns, double tok_bytes) {
    double mb = 0;  // partial bytes of the tokens with more than one split
    for (const TokRange &r : toks) {
        if (!r.step) {
            const int t = std::min(ns, (r.kend0 + slen - 1) / slen);
            if (t > 1) mb += (double)t * r.count * tok_bytes;
            continue;
        }
        const int lo = r.kend0, hi = r.kend0 + r.count - 1;
        for (int j = 2; j <= ns; ++j) {  // tokens with j splits reach keys in ((j-1) slen, j slen]
            const int a = std::max(lo, (j - 1) * slen + 1), b = j == ns ? hi : std::min(hi, j * slen);
            if (b >= a) mb += (double)j * (b - a + 1) * tok_bytes;
        }
    }
    return ATT_MERGE_FIXED + mb / 1e6 / ATT_MERGE_MB_PER_TILE;
}
// The split count and block form of least estimated time (a larger count or
// the two-chain form must gain 3%); s = 0 when the longest chain is below
// ATT_CHAIN_MODEL_TILES.  toks: the row tokens and the keys they reach;
// tok_bytes: one split's partials of one token; two_chains: the launch may
// take the two-chain form (64-row bf16 blocks; the fp32 kernel has one form).
struct SplitPlan {
    int s;
    bool halves;
};
static SplitPlan model_splits(const std::vector<ChainSpec> &blocks, int keys, const std::vector<TokRange> &toks,
                              double tok_bytes, bool two_chains) {
    int longest = 0;
    for (const ChainSpec &b : blocks) longest = std::max(longest, (b.kend + 63) / 64 + b.extra);
    if (longest < ATT_CHAIN_MODEL_TILES) return {0, false};
    SplitPlan best_p{1, false};
    double best = 0;
    for (int h = 0; h < (two_chains ? 2 : 1); ++h)
        for (int s = 1; s <= MAX_SPLITS; ++s) {
            const int slen = s == 1 ? keys : ((keys + s - 1) / s + 63) / 64 * 64;
            if (s > 1 && slen / 64 < ATT_MIN_SPLIT_TILES) break;
            const int ns = s == 1 ? 1 : (keys + slen - 1) / slen;
            if (ns != s) continue;  // the same split as a smaller count
            const SplitCost c = split_cost(blocks, slen, ns, h == 1);
            const double t = std::max(c.chain, c.work) + (ns > 1 ? merge_cost(toks, slen, ns, tok_bytes) : 0.0);
            if ((h == 0 && s == 1) || t < 0.97 * best) {
                best = t;
                best_p = {s, h == 1};
            }
            if (s == 1 && c.work >= c.chain) break;  // the slots are full: splitting only adds work
        }
    return best_p;
}

// Key tiles a block walks (prefix part up to its last row's causal bound,
// plus its branch keys).
static int block_tiles(const AttnBlock &b, int grp) {
    int kmax = b.key1;
    if (b.causal) kmax = std::min(kmax, b.qoff + (b.row0 + b.nrows - 1) / grp + 1);
    int n = kmax > b.key0 ? (kmax - b.key0 + 63) / 64 : 0;
    if (b.sfx_hi > b.sfx_lo) n += (b.sfx_hi - b.sfx_lo + 63) / 64;
    return n;
}

// Blocks with the longest key chains first.  Workgroups are handed out in
// index order, so the longest chains start first and the short ones fill
// the compute units behind them; in row order the longest causal rows
// would start last and run alone at the end of the launch.
static void longest_first(std::vector<AttnBlock> &v, size_t from, size_t to, int grp) {
    std::stable_sort(v.begin() + from, v.begin() + to,
                     [grp](const AttnBlock &a, const AttnBlock &b) { return block_tiles(a, grp) > block_tiles(b, grp); });
}

// XCD-aware block order.  Workgroup b of a launch runs on XCD b % 8, and
// each XCD has its own L2.  The blocks that read the same keys (one
// request's KV head and key range) are given to the same XCD(s): G such
// groups share the 8 XCDs (group i gets XCDs i, i + G, ... when G < 8, XCD
// i % 8 otherwise), so an XCD streams one group's keys through its L2
// instead of every group's.  Each XCD keeps the blocks' current order
// (longest chain first); a slot whose XCD has no block left takes one from
// the XCD with the most left, so no slot is wasted.
static void xcd_order(std::vector<AttnBlock> &v, size_t from, size_t to) {
    constexpr int NX = 8;
    if (to - from <= (size_t)NX) return;
    std::vector<std::array<int32_t, 3>> keys;
    for (size_t i = from; i < to; ++i) keys.push_back({v[i].req, v[i].g, v[i].split});
    std::vector<std::array<int32_t, 3>> groups = keys;
    std::sort(groups.begin(), groups.end());
    groups.erase(std::unique(groups.begin(), groups.end()), groups.end());
    const int G = (int)groups.size();
    std::vector<int> seen(G, 0);
    std::vector<AttnBlock> q[NX];
    for (size_t i = from; i < to; ++i) {
        const int gi = (int)(std::lower_bound(groups.begin(), groups.end(), keys[i - from]) - groups.begin());
        int x;
        if (G >= NX) {
            x = gi % NX;
        } else {
            const int per = (NX - gi + G - 1) / G;  // XCDs gi, gi + G, ... below NX
            x = gi + G * (seen[gi]++ % per);
        }
        q[x].push_back(v[i]);
    }
    size_t head[NX] = {};
    for (size_t p = from; p < to; ++p) {
        int x = (int)((p - from) % NX);
        if (head[x] == q[x].size()) {
            int best = -1;
            for (int y = 0; y < NX; ++y)
                if (head[y] < q[y].size() && (best < 0 || q[y].size() - head[y] > q[best].size() - head[best])) best = y;
            x = best;
        }
        v[p] = q[x][head[x]++];
    }
}

struct Layout {
    size_t rope, x, h, q, ao, act, splitk, kvb, part_o, part_ml, hr, xr, aor, ro_part, lse, z, outs, plan;
    size_t plan_bytes, outs_bytes, total;
};

int64_t plan_block_cap(const pcd_config &c, const pcd_limits &l) {
    const int grp = c.n_heads / c.n_kv_heads;
    const int64_t pre =
        (int64_t)c.n_kv_heads * (((int64_t)l.max_prefill_tokens * grp + ATT_ROWS - 1) / ATT_ROWS) * MAX_SPLITS;
    const int64_t br = (int64_t)c.n_kv_heads *
                       (((int64_t)l.max_branch_tokens * grp + ATT_ROWS - 1) / ATT_ROWS + l.max_requests) * MAX_SPLITS;
    return pre + br;  // a fused pass has both kinds of blocks
}

// spellings of one decide call: the limit, or one per candidate when unset
static_assert(SCORE_PATH == PCD_SCORE_PATH && SCORE_EXACT == PCD_SCORE_EXACT && SCORE_LEVEL == PCD_SCORE_LEVEL &&
                  SCORE_MEAN == PCD_SCORE_MEAN,
              "kernel scoring-mode values");

int64_t spell_cap(const pcd_limits &l) { return l.max_spellings > 0 ? l.max_spellings : l.max_candidates; }
int64_t path_cap(const pcd_limits &l) { return 8 * spell_cap(l) + l.max_gathers; }

// partial sums of the residual GEMMs: up to SPLITK_MAX splits below
// SPLITK_ROWS rows, 4 below 4 * SPLITK_ROWS (the long-K down projection at a
// few thousand rows), one above
size_t splitk_floats(const pcd_config &c, const pcd_limits &l) {
    const size_t rows = (size_t)std::max(l.max_prefill_tokens, l.max_branch_tokens);
    return std::max({(size_t)SPLITK_MAX * std::min(rows, (size_t)SPLITK_ROWS),
                     (size_t)4 * std::min(rows, (size_t)4 * SPLITK_ROWS), rows}) *
           c.d_model;
}

Layout layout(const pcd_config &c, const pcd_limits &l) {
    Layout L{};
    const size_t esz = c.dtype == PCD_DTYPE_F32 ? 4 : 2;
    const size_t rows = (size_t)std::max(l.max_prefill_tokens, l.max_branch_tokens);
    const size_t d = c.d_model, hq = (size_t)c.n_heads * c.head_dim;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    L.rope = take((size_t)c.max_seq * (c.head_dim / 2) * sizeof(float2));
    L.x = take(rows * d * 4);
    L.h = take(rows * d * esz);
    L.q = take(rows * hq * esz);
    L.ao = take(rows * hq * esz);
    L.act = take(rows * c.ffn_dim * esz);
    L.splitk = take(splitk_floats(c, l) * 4);
    L.kvb = take((size_t)c.n_layers * 2 * c.n_kv_heads * l.max_branch_tokens * c.head_dim * esz);
    L.part_o = take((size_t)MAX_SPLITS * rows * hq * 4);
    L.part_ml = take((size_t)MAX_SPLITS * rows * c.n_heads * sizeof(float2));
    L.hr = take((size_t)l.max_readouts * d * esz);
    L.xr = take((size_t)l.max_readouts * d * 4);     // the last layer's readout rows: residual stream
    L.aor = take((size_t)l.max_readouts * hq * esz);  // and attention output
    L.ro_part = take((size_t)(c.vocab_size / 128) * l.max_readouts * sizeof(float2));
    L.lse = take((size_t)l.max_readouts * 4);
    L.z = take((size_t)l.max_gathers * 4);
    L.outs_bytes = align_up((size_t)(2 * l.max_candidates + 3 * l.max_fields + l.max_readouts + l.max_gathers) * 4 + 8 * 256);
    L.outs = take(L.outs_bytes);
    const int64_t ints = 8 * (int64_t)rows + 8 * (int64_t)l.max_branch_tokens + 2 * (int64_t)l.max_readouts + 2 + 2 * (int64_t)l.max_gathers +
                         3 * (int64_t)l.max_fields + 1 + (int64_t)l.max_candidates + 1 + spell_cap(l) + 1 + path_cap(l) +
                         2 * (int64_t)l.max_requests;
    L.plan_bytes = align_up((size_t)ints * 4 + 32 * 256) + align_up((size_t)l.max_requests * 8) +
                   align_up((size_t)plan_block_cap(c, l) * sizeof(AttnBlock));
    L.plan = take(L.plan_bytes);
    L.total = off;
    return L;
}

int check_config(const pcd_config *c, const pcd_limits *l) {
    if (!c || !l) return fail(PCD_E_ARG, "null config or limits");
    if (c->dtype != PCD_DTYPE_F32 && c->dtype != PCD_DTYPE_BF16) return fail(PCD_E_ARG, "dtype must be f32 or bf16");
    if (c->n_layers <= 0 || c->d_model <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
        c->ffn_dim <= 0 || c->vocab_size <= 0 || c->max_seq <= 0)
        return fail(PCD_E_ARG, "non-positive model dimension");
    if (c->n_heads % c->n_kv_heads) return fail(PCD_E_ARG, "n_heads must be a multiple of n_kv_heads");
    if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return fail(PCD_E_ARG, "head_dim must be 32, 64 or 128");
    if (c->dtype == PCD_DTYPE_F32 && c->head_dim == 128) return fail(PCD_E_ARG, "f32 models support head_dim 32 or 64");
    const int kt = gemm_k_tile(c->dtype);
    if (c->d_model % 128 || c->ffn_dim % 128 || (c->n_heads * c->head_dim) % 128 || c->vocab_size % 128 ||
        c->d_model % kt || c->ffn_dim % kt)
        return fail(PCD_E_ARG, "d_model, ffn_dim, n_heads*head_dim and vocab_size must be multiples of 128");
    if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.f)) return fail(PCD_E_ARG, "rms_eps and rope_theta must be positive");
    if (l->max_prefill_tokens <= 0 || l->max_branch_tokens <= 0 || l->max_readouts <= 0 || l->max_gathers <= 0 ||
        l->max_fields <= 0 || l->max_candidates <= 0 || l->max_requests <= 0 || l->max_spellings < 0)
        return fail(PCD_E_ARG, "limits must be positive");
    // rows of one pass (pcd_prefill_many puts every sequence in one); each
    // sequence is bounded by max_seq on its own
    if (l->max_prefill_tokens > MAX_PASS_ROWS || l->max_branch_tokens > MAX_PASS_ROWS)
        return fail(PCD_E_ARG, "max_prefill_tokens and max_branch_tokens must be at most " +
                                   std::to_string(MAX_PASS_ROWS));
    return PCD_OK;
}

}  // namespace

struct pcd_model {
    pcd_config cfg;
    pcd_limits lim;
    Layout L;
    char *ws = nullptr;
    size_t ws_bytes = 0;
    const void *embed = nullptr, *head = nullptr;
    const float *final_norm = nullptr;
    std::vector<const void *> wq, wk, wv, wo, wg, wu, wd;
    std::vector<const float *> an, mn;
    // The workspace is the library's static scratch of this device
    // (pcd_load_weights_noalloc); its host staging is then pageable memory
    // from new[] instead of pinned memory.
    bool static_ws = false;
    int ws_device = -1;
    char *plan_host = nullptr;  // staging for a prefill's plan upload (pinned unless static_ws)
    // Decide calls in flight: each holds one slot, with its own pinned plan
    // and result staging and its events, from its start to its finish.
    struct Slot {
        char *plan_host = nullptr, *outs_host = nullptr;
        hipEvent_t ev[4] = {};  // pass start (plan uploaded), pass end, readout end, results on the host
        hipStream_t st = nullptr;  // stream of the call holding the slot
        bool busy = false;
    };
    Slot slots[PCD_MAX_PENDING];
    hipEvent_t ev[6] = {};  // branch start/end, readout end, prefill start/end, plan upload done
    pcd_stats stats{};
    bool prefill_pending = false;  // last_prefill_ms not yet read from ev[3], ev[4]
    hipStream_t prefill_st = nullptr;  // stream of the last prefill or extend pass
    // Every pass reads and writes the one workspace (plan, activations,
    // branch K/V, partials, results), so a call may go on another stream only
    // once the model's earlier calls have left the device: a started decide
    // call until its results are on the host (slot event 3), a prefill or
    // extend until its pass has ended (ev[4]).  Refuses, before any device
    // work, a call on a stream other than that of a call still running.
    int check_stream(hipStream_t st) {
        for (int k = 0; k < PCD_MAX_PENDING; ++k) {
            const Slot &sl = slots[k];
            if (sl.busy && sl.st != st && hipEventQuery(sl.ev[3]) == hipErrorNotReady)
                return fail(PCD_E_ARG, "a started decide call of this model is still running on another stream; "
                                       "use that stream or finish the call first");
        }
        if (prefill_pending && prefill_st != st && hipEventQuery(ev[4]) == hipErrorNotReady)
            return fail(PCD_E_ARG, "a prefill or extend pass of this model is still running on another stream; "
                                   "use that stream or wait for it first");
        return PCD_OK;
    }
    // fold a finished prefill's event time into the stats (waits for it)
    void settle_prefill() {
        if (!prefill_pending) return;
        prefill_pending = false;
        float ms = 0.f;
        if (hipEventSynchronize(ev[4]) == hipSuccess && hipEventElapsedTime(&ms, ev[3], ev[4]) == hipSuccess)
            stats.last_prefill_ms = ms;
    }
    int n_states = 0;
    // per-kernel-class timing
    bool timing = false;
    std::vector<hipEvent_t> tev;         // pool, used in (start, end) pairs
    std::vector<int> tcls;               // class of each used pair
    size_t tused = 0;
    float kc_ms[PCD_KC_COUNT] = {};
    int64_t kc_n[PCD_KC_COUNT] = {};
    void tbegin(int cls, hipStream_t st) {
        if (!timing) return;
        if (2 * tused + 2 > tev.size()) {
            for (int i = 0; i < 256; ++i) {
                hipEvent_t e;
                if (hipEventCreate(&e) != hipSuccess) return;
                tev.push_back(e);
            }
        }
        (void)hipEventRecord(tev[2 * tused], st);
        if (tcls.size() <= tused) tcls.resize(tused + 1);
        tcls[tused] = cls;
    }
    void tend(hipStream_t st) {
        if (!timing || 2 * tused + 2 > tev.size()) return;
        (void)hipEventRecord(tev[2 * tused + 1], st);
        ++tused;
    }
    // after the stream has drained
    void tcollect() {
        for (size_t i = 0; i < tused; ++i) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, tev[2 * i], tev[2 * i + 1]) == hipSuccess) {
                kc_ms[tcls[i]] += ms;
                kc_n[tcls[i]] += 1;
            }
        }
        tused = 0;
    }
};

struct pcd_state {
    uint64_t magic;
    pcd_model *m;
    void *kv;
    int32_t P;    // tokens held
    int32_t cap;  // tokens per (layer, K|V, KV head) slab of the buffer: its layout stride
};

// A decide call between its start and its finish: its slot, where the
// results go and how they are laid out in the slot's staging.
struct pcd_pending {
    uint64_t magic;
    pcd_model *m;
    int slot;
    hipStream_t st;
    int n_req, Tb, R, G;
    std::vector<pcd_outputs> outs;
    std::vector<int32_t> r_cand, r_field, r_ro, r_g;
    size_t o_prob, o_ls, o_mass, o_marg, o_arg, o_lse, o_z;
};

namespace {

size_t esize(const pcd_model *m) { return m->cfg.dtype == PCD_DTYPE_F32 ? 4 : 2; }

// O projection or down projection into the residual stream (split-K inside
// gemm() when the tile count is too small for the chip), followed by the
// RMSNorm with weight `norm_w` whose output is the next GEMM's input
bool gemm_resid(pcd_model *m, const void *A, int M, int N, int K, const void *W, const float *norm_w, hipStream_t st,
                float *x = nullptr, void *h_out = nullptr) {
    GemmCall c{};
    c.dt = m->cfg.dtype;
    c.A = A;
    c.M = M;
    c.N = N;
    c.K = K;
    c.B[0].ptr[0] = W;
    c.B[0].nseg = 1;
    c.epi = Epi::Resid;
    c.x = x ? x : reinterpret_cast<float *>(m->ws + m->L.x);
    c.part = reinterpret_cast<float *>(m->ws + m->L.splitk);
    c.part_cap = splitk_floats(m->cfg, m->lim);
    c.norm_w = norm_w;
    c.eps = m->cfg.rms_eps;
    c.h_out = h_out ? h_out : m->ws + m->L.h;
    return gemm(c, st);
}

// one decoder layer over M rows whose K/V go to (kc, vc) with `cap` tokens per
// KV head, and whose attention is run by `attn` (prefill or branch)
enum class Pass { Prefill, Branch, Fused };  // which timing classes a layer's kernels count under

// K/V destinations of rows spread over several state buffers (batched prefill)
struct KvRows {
    const int32_t *req, *row, *cap;  // per row: buffer, token slot; per buffer: tokens per slab
    const uint64_t *base;            // per buffer: device address
};

// The last layer of a pass computes only what later work reads: every row's
// K and V (the state keeps the new tokens', the branch attention reads the
// branch tokens'), then either nothing more (n_keep == 0: a prefill or
// extend) or the residual stream of the readout rows keep[0..n_keep), which
// after the attention are gathered into rows 0..n_keep-1 of the compact
// buffers L.aor / L.xr.  n_keep < 0: the whole layer over all M rows.
template <class Attn>
int layer(pcd_model *m, int l, int M, const int32_t *pos, void *kc, void *vc, int cap, Pass kind, Attn attn,
          hipStream_t st, void *kc2 = nullptr, void *vc2 = nullptr, int cap2 = 0, int kv_split = 0,
          const KvRows *kr = nullptr, const int32_t *keep = nullptr, int n_keep = -1) {
    const bool br = kind == Pass::Branch, fu = kind == Pass::Fused;
    // the readout rows' kernels of a trimmed last layer count as "other", so
    // every launch of a class has the class's row count
    const bool few = n_keep > 0;
    const int K_QKV = fu ? PCD_KC_FUSED_QKV : br ? PCD_KC_BRANCH_QKV : PCD_KC_PREFILL_QKV;
    const int K_O = few ? PCD_KC_OTHER : fu ? PCD_KC_FUSED_O : br ? PCD_KC_BRANCH_O : PCD_KC_PREFILL_O;
    const int K_GU = few ? PCD_KC_OTHER : fu ? PCD_KC_FUSED_GATEUP : br ? PCD_KC_BRANCH_GATEUP : PCD_KC_PREFILL_GATEUP;
    const int K_DN = few ? PCD_KC_OTHER : fu ? PCD_KC_FUSED_DOWN : br ? PCD_KC_BRANCH_DOWN : PCD_KC_PREFILL_DOWN;
    const pcd_config &c = m->cfg;
    const int d = c.d_model, hd = c.head_dim, nq = c.n_heads * hd, nk = c.n_kv_heads * hd;
    float *x = reinterpret_cast<float *>(m->ws + m->L.x);
    void *h = m->ws + m->L.h, *q = m->ws + m->L.q, *ao = m->ws + m->L.ao, *act = m->ws + m->L.act;
    // h holds rmsnorm(x) * attn_norm[l] on entry (embedding or previous layer)
    GemmCall g{};
    g.dt = c.dtype;
    g.A = h;
    g.M = M;
    g.N = nq + 2 * nk;
    g.K = d;
    g.B[0].ptr[0] = m->wq[l];
    g.B[0].ptr[1] = m->wk[l];
    g.B[0].ptr[2] = m->wv[l];
    g.B[0].begin[0] = 0;
    g.B[0].begin[1] = nq;
    g.B[0].begin[2] = nq + nk;
    g.B[0].nseg = 3;
    g.epi = Epi::Qkv;
    g.out = q;
    g.kc = kc;
    g.vc = vc;
    g.cap = cap;
    g.kc2 = kc2;  // rows from kv_split on (the branch tokens of a fused pass)
    g.vc2 = vc2;
    g.cap2 = cap2;
    g.kv_split = kv_split;
    if (kr) {
        g.kv_req = kr->req;
        g.kv_row = kr->row;
        g.kv_cap = kr->cap;
        g.kv_base = kr->base;
        g.kv_layer = l;
    }
    g.pos = pos;
    g.rope = reinterpret_cast<const float2 *>(m->ws + m->L.rope);
    g.n_q = nq;
    g.n_k = nk;
    g.hd = hd;
    m->tbegin(K_QKV, st);
    if (!gemm(g, st)) return fail(PCD_E_ARG, "QKV projection: unsupported shape");
    m->tend(st);
    if (n_keep == 0) return PCD_OK;
    int rc = attn(q, ao, n_keep > 0);
    if (rc != PCD_OK) return rc;
    float *xo = nullptr;  // residual stream of the rows that go on (NULL: the full buffer)
    if (n_keep > 0) {
        xo = reinterpret_cast<float *>(m->ws + m->L.xr);
        void *aor = m->ws + m->L.aor;
        m->tbegin(K_O, st);
        gather_rows2(ao, (size_t)nq * esize(m), aor, x, (size_t)d * 4, xo, keep, n_keep, st);
        m->tend(st);
        ao = aor;
        M = n_keep;
    }
    m->tbegin(K_O, st);
    if (!gemm_resid(m, ao, M, d, nq, m->wo[l], m->mn[l], st, xo))
        return fail(PCD_E_ARG, "O projection: unsupported shape");
    m->tend(st);
    GemmCall f{};
    f.dt = c.dtype;
    f.A = h;
    f.M = M;
    f.N = c.ffn_dim;
    f.K = d;
    f.B[0].ptr[0] = m->wg[l];
    f.B[0].nseg = 1;
    f.B[1].ptr[0] = m->wu[l];
    f.B[1].nseg = 1;
    f.epi = Epi::SwiGlu;
    f.out = act;
    m->tbegin(K_GU, st);
    if (!gemm(f, st)) return fail(PCD_E_ARG, "gate/up projection: unsupported shape");
    m->tend(st);
    m->tbegin(K_DN, st);
    const float *next_norm = l + 1 < c.n_layers ? m->an[l + 1] : nullptr;
    if (!gemm_resid(m, act, M, d, c.ffn_dim, m->wd[l], next_norm, st, xo))
        return fail(PCD_E_ARG, "down projection: unsupported shape");
    m->tend(st);
    return PCD_OK;
}

// bump-allocator over the pinned plan staging buffer, mirrored on the device
struct Packer {
    char *host;
    char *dev;
    size_t cap, off = 0;
    bool overflow = false;
    template <class T> T *put(const T *src, size_t n) {
        const size_t o = off;
        off = align_up(off + n * sizeof(T));
        if (off > cap) {
            overflow = true;
            return nullptr;
        }
        if (n) std::memcpy(host + o, src, n * sizeof(T));
        return reinterpret_cast<T *>(dev + o);
    }
};

}  // namespace

// Workspace of the no-allocation models (pcd_load_weights_noalloc): one
// static array per device, in the library's code object, so that creating
// such a model allocates no device memory.  Host code never passes `scratch`
// itself (in host code it names a host-side stand-in): once per device, with
// that device current, its device address is read with hipGetSymbolAddress
// and kept here; models use that address like a caller's workspace.
static __device__ __align__(256) char scratch[PCD_NOALLOC_WORKSPACE_MAX];

namespace {

constexpr int MAX_DEVICES = 64;
struct ScratchDev {
    void *ptr = nullptr;             // device address of `scratch` on this device
    const pcd_model *owner = nullptr;  // the live model using it
};
std::mutex g_scratch_mu;
ScratchDev g_scratch[MAX_DEVICES];

// Claims the current device's scratch for model m (one model per device at
// a time): its device address in *ptr.
int claim_scratch(const pcd_model *m, int *dev_out, void **ptr) {
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= MAX_DEVICES) return fail(PCD_E_DEVICE, "device index out of range");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    ScratchDev &sd = g_scratch[dev];
    if (sd.owner) return fail(PCD_E_ARG, "another model on this device already uses the static workspace; free it first");
    if (!sd.ptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(PCD_E_DEVICE, std::string("address of the static workspace: ") + hipGetErrorString(e));
        sd.ptr = p;
    }
    sd.owner = m;
    *dev_out = dev;
    *ptr = sd.ptr;
    return PCD_OK;
}

void release_scratch(const pcd_model *m) {
    if (!m->static_ws || m->ws_device < 0) return;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch[m->ws_device].owner == m) g_scratch[m->ws_device].owner = nullptr;
}

// pinned (hipHostMalloc) or, for a static-workspace model, pageable staging
bool host_alloc(const pcd_model *m, char **p, size_t bytes) {
    if (m->static_ws) {
        *p = new (std::nothrow) char[bytes];
        return *p != nullptr;
    }
    return hipHostMalloc((void **)p, bytes, hipHostMallocDefault) == hipSuccess;
}

void host_free(const pcd_model *m, char *p) {
    if (!p) return;
    if (m->static_ws) delete[] p;
    else (void)hipHostFree(p);
}

int load_model(const pcd_config *cfg, const pcd_limits *lim, const pcd_weights *w, void *workspace, size_t ws_bytes,
               void *stream, pcd_model **out, bool noalloc);

}  // namespace

extern "C" {

const char *pcd_last_error(void) { return g_err.c_str(); }

size_t pcd_workspace_bytes(const pcd_config *cfg, const pcd_limits *lim) {
    if (check_config(cfg, lim) != PCD_OK) return 0;
    return layout(*cfg, *lim).total;
}

int pcd_load_weights(const pcd_config *cfg, const pcd_limits *lim, const pcd_weights *w, void *workspace,
                     size_t ws_bytes, void *stream, pcd_model **out) {
    return load_model(cfg, lim, w, workspace, ws_bytes, stream, out, false);
}

int pcd_load_weights_noalloc(const pcd_config *cfg, const pcd_limits *lim, const pcd_weights *w, void *stream,
                             pcd_model **out) {
    return load_model(cfg, lim, w, nullptr, PCD_NOALLOC_WORKSPACE_MAX, stream, out, true);
}

}  // extern "C"

namespace {

int load_model(const pcd_config *cfg, const pcd_limits *lim, const pcd_weights *w, void *workspace, size_t ws_bytes,
               void *stream, pcd_model **out, bool noalloc) {
    int rc = check_config(cfg, lim);
    if (rc != PCD_OK) return rc;
    if (!w || (!workspace && !noalloc) || !out) return fail(PCD_E_ARG, "null weights, workspace or out");
    const int L = cfg->n_layers;
    if (!w->embed || !w->final_norm || !w->attn_norm || !w->mlp_norm || !w->wq || !w->wk || !w->wv || !w->wo ||
        !w->w_gate || !w->w_up || !w->w_down || (!cfg->tied_lm_head && !w->lm_head))
        return fail(PCD_E_ARG, "null weight pointer");
    for (int l = 0; l < L; ++l)
        if (!w->attn_norm[l] || !w->mlp_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->w_gate[l] ||
            !w->w_up[l] || !w->w_down[l])
            return fail(PCD_E_ARG, "null per-layer weight pointer");
    bool mis = misaligned(w->embed) || misaligned(w->lm_head) || misaligned(w->final_norm) ||
               (!noalloc && reinterpret_cast<uintptr_t>(workspace) % 256 != 0);
    for (int l = 0; l < L; ++l)
        mis = mis || misaligned(w->attn_norm[l]) || misaligned(w->mlp_norm[l]) || misaligned(w->wq[l]) ||
              misaligned(w->wk[l]) || misaligned(w->wv[l]) || misaligned(w->wo[l]) || misaligned(w->w_gate[l]) ||
              misaligned(w->w_up[l]) || misaligned(w->w_down[l]);
    if (mis) return fail(PCD_E_ARG, "weights must be 16-byte aligned and the workspace 256-byte aligned");
    Layout lay = layout(*cfg, *lim);
    if (ws_bytes < lay.total)
        return fail(PCD_E_CAP, (noalloc ? "the static workspace holds " : "workspace of ") + std::to_string(ws_bytes) +
                                   " bytes, these limits need " + std::to_string(lay.total));
    pcd_model *m = new (std::nothrow) pcd_model();
    if (!m) return fail(PCD_E_NOMEM, "model allocation");
    if (noalloc) {
        rc = claim_scratch(m, &m->ws_device, &workspace);
        if (rc != PCD_OK) {
            delete m;
            return rc;
        }
        m->static_ws = true;
    }
    m->cfg = *cfg;
    m->lim = *lim;
    m->L = lay;
    m->ws = static_cast<char *>(workspace);
    m->ws_bytes = ws_bytes;
    m->embed = w->embed;
    m->head = cfg->tied_lm_head ? w->embed : w->lm_head;
    m->final_norm = w->final_norm;
    m->wq.assign(w->wq, w->wq + L);
    m->wk.assign(w->wk, w->wk + L);
    m->wv.assign(w->wv, w->wv + L);
    m->wo.assign(w->wo, w->wo + L);
    m->wg.assign(w->w_gate, w->w_gate + L);
    m->wu.assign(w->w_up, w->w_up + L);
    m->wd.assign(w->w_down, w->w_down + L);
    m->an.assign(w->attn_norm, w->attn_norm + L);
    m->mn.assign(w->mlp_norm, w->mlp_norm + L);
    m->stats.workspace_bytes = (int64_t)lay.total;
    auto cleanup = [&](int code, const std::string &msg) {
        pcd_free_model(m);
        return fail(code, msg);
    };
    if (!host_alloc(m, &m->plan_host, lay.plan_bytes)) return cleanup(PCD_E_NOMEM, "staging allocation failed");
    for (auto &sl : m->slots) {
        if (!host_alloc(m, &sl.plan_host, lay.plan_bytes) || !host_alloc(m, &sl.outs_host, lay.outs_bytes))
            return cleanup(PCD_E_NOMEM, "staging allocation failed");
        for (auto &e : sl.ev)
            if (hipEventCreate(&e) != hipSuccess) return cleanup(PCD_E_DEVICE, "event creation failed");
    }
    for (auto &e : m->ev)
        if (hipEventCreate(&e) != hipSuccess) return cleanup(PCD_E_DEVICE, "event creation failed");
    // RoPE table: (cos, sin) of pos * theta^(-2j/hd), computed in double
    const int half = cfg->head_dim / 2;
    std::vector<float2> rope((size_t)cfg->max_seq * half);
    for (int p = 0; p < cfg->max_seq; ++p)
        for (int j = 0; j < half; ++j) {
            const double inv = std::pow((double)cfg->rope_theta, -2.0 * j / cfg->head_dim);
            const double a = p * inv;
            rope[(size_t)p * half + j] = make_float2((float)std::cos(a), (float)std::sin(a));
        }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(m->ws + lay.rope, rope.data(), rope.size() * sizeof(float2), hipMemcpyHostToDevice, st) !=
            hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return cleanup(PCD_E_DEVICE, std::string("RoPE upload: ") + hipGetErrorString(hipGetLastError()));
    *out = m;
    return PCD_OK;
}

}  // namespace

extern "C" {

size_t pcd_state_bytes(const pcd_model *m, int32_t n) {
    if (!m || n < 0) return 0;
    return (size_t)n * m->cfg.n_layers * 2 * m->cfg.n_kv_heads * m->cfg.head_dim * esize(m);
}

namespace {

size_t per_token_bytes(const pcd_model *m) {
    return (size_t)m->cfg.n_layers * 2 * m->cfg.n_kv_heads * m->cfg.head_dim * esize(m);
}

// One causal pass over tokens[0..n) at positions P0..P0+n-1, appending their
// K and V to a KV buffer with `cap` tokens per slab that holds P0 tokens
// already: prefill (P0 = 0) and extend.  Attention of each new token covers
// keys 0..P0+t, split over workgroups when the row blocks alone do not fill
// the chip (split k covers [k*slen, (k+1)*slen); only row blocks that reach
// key k*slen get a workgroup for it), then merged.
int causal_pass(pcd_model *m, void *kv_buf, int32_t cap, int32_t P0, const int32_t *tokens, int32_t n,
                hipStream_t st) {
    const pcd_config &c = m->cfg;
    const int grp = c.n_heads / c.n_kv_heads, hd = c.head_dim;
    const int keys = P0 + n;
    std::vector<AttnBlock> blocks;
    const int rows = n * grp;
    const bool wide = c.dtype == PCD_DTYPE_BF16 &&
                      (int64_t)c.n_kv_heads * ((rows + ATT_WIDE_ROWS - 1) / ATT_WIDE_ROWS) >= ATT_WIDE_MIN_BLOCKS;
    const int arows = wide ? ATT_WIDE_ROWS : ATT_ROWS;
    const int64_t row_blocks = (int64_t)c.n_kv_heads * ((rows + arows - 1) / arows);
    int ns = att_splits(row_blocks, (keys + 63) / 64, false);
    bool halves = false;  // two key chains per 8-wave block whatever the block count
    {
        std::vector<ChainSpec> chains;
        for (int g = 0; g < c.n_kv_heads; ++g)
            for (int r0 = 0; r0 < rows; r0 += arows)
                chains.push_back({P0 + (r0 + std::min(arows, rows - r0) - 1) / grp + 1, 0});
        const SplitPlan sp = model_splits(chains, keys, {{P0 + 1, n, true}}, 4.0 * c.n_heads * hd,
                                           !wide && c.dtype == PCD_DTYPE_BF16);
        if (sp.s) ns = sp.s;
        halves = sp.halves;
    }
    const int slen = ((keys + ns - 1) / ns + 63) / 64 * 64;
    ns = (keys + slen - 1) / slen;
    for (int g = 0; g < c.n_kv_heads; ++g)
        for (int r0 = 0; r0 < rows; r0 += arows) {
            const int nr = std::min(arows, rows - r0), t_last = P0 + (r0 + nr - 1) / grp;
            for (int k = 0; k < ns && k * slen <= t_last; ++k)
                blocks.push_back(AttnBlock{0, g, r0, nr, k * slen, std::min(keys, (k + 1) * slen), k, ns, 0, 0, 1, P0});
        }
    longest_first(blocks, 0, blocks.size(), grp);
    xcd_order(blocks, 0, blocks.size());
    if ((int64_t)blocks.size() > plan_block_cap(c, m->lim)) return fail(PCD_E_CAP, "too many attention blocks");
    std::vector<int32_t> tok_splits(n);
    for (int t = 0; t < n; ++t) tok_splits[t] = (P0 + t) / slen + 1;
    std::vector<int32_t> pos;
    if (P0 > 0) {
        pos.resize(n);
        for (int i = 0; i < n; ++i) pos[i] = P0 + i;
    }
    Packer pk{m->plan_host, m->ws + m->L.plan, m->L.plan_bytes};
    const int32_t *d_tok = pk.put(tokens, n);
    const int32_t *d_pos = P0 > 0 ? pk.put(pos.data(), n) : nullptr;
    const uint64_t kvaddr = reinterpret_cast<uint64_t>(kv_buf);
    const uint64_t *d_kv = pk.put(&kvaddr, 1);
    const int32_t *d_stride = pk.put(&cap, 1);
    const int32_t *d_tsp = pk.put(tok_splits.data(), n);
    const AttnBlock *d_blk = pk.put(blocks.data(), blocks.size());
    if (pk.overflow) return fail(PCD_E_CAP, "plan staging overflow");
    if (int rc = m->check_stream(st)) return rc;
    m->settle_prefill();
    HIP_TRY(hipMemcpyAsync(m->ws + m->L.plan, m->plan_host, pk.off, hipMemcpyHostToDevice, st));
    HIP_TRY(hipEventRecord(m->ev[5], st));
    HIP_TRY(hipEventRecord(m->ev[3], st));
    float *x = reinterpret_cast<float *>(m->ws + m->L.x);
    m->tbegin(PCD_KC_OTHER, st);
    embed(c.dtype, d_tok, n, m->embed, c.d_model, x, m->an[0], c.rms_eps, m->ws + m->L.h, st);
    m->tend(st);
    const size_t es = esize(m);
    const size_t slab = (size_t)cap * hd;  // elements of one (layer, K|V, KV head) slab
    float *part_o = reinterpret_cast<float *>(m->ws + m->L.part_o);
    float2 *part_ml = reinterpret_cast<float2 *>(m->ws + m->L.part_ml);
    for (int l = 0; l < c.n_layers; ++l) {
        // this layer's K and V slabs, at the first new token's row
        char *kc = static_cast<char *>(kv_buf) + ((size_t)l * 2 * c.n_kv_heads * slab + (size_t)P0 * hd) * es;
        char *vc = kc + (size_t)c.n_kv_heads * slab * es;
        auto attn = [&](void *q, void *ao, bool) {
            AttnCall a{};
            a.dt = c.dtype;
            a.hd = hd;
            a.n_heads = c.n_heads;
            a.n_kv_heads = c.n_kv_heads;
            a.layer = l;
            a.q = q;
            a.req_kv = d_kv;
            a.req_stride = d_stride;
            a.blocks = d_blk;
            a.n_blocks = (int)blocks.size();
            a.tok_splits = d_tsp;
            a.out = ao;
            a.part_o = part_o;
            a.part_ml = part_ml;
            a.n_tokens = n;
            a.wide = wide;
            a.halves = halves;
            m->tbegin(PCD_KC_PREFILL_ATTN, st);
            const bool ok = attention(a, st);
            m->tend(st);
            if (!ok) return fail(PCD_E_ARG, "attention: unsupported head_dim/dtype");
            if (ns > 1) {
                TailCall t{};
                t.dt = c.dtype;
                t.hd = hd;
                t.n_heads = c.n_heads;
                t.n_kv_heads = c.n_kv_heads;
                t.n_tokens = n;
                t.tok0 = std::max(0, std::min(n, slen - P0));  // earlier tokens have one split
                t.part_o = part_o;
                t.part_ml = part_ml;
                t.tok_splits = d_tsp;
                t.out = ao;
                m->tbegin(PCD_KC_OTHER, st);
                attention_merge(t, st);
                m->tend(st);
            }
            return PCD_OK;
        };
        int rc = layer(m, l, n, d_pos, kc, vc, cap, Pass::Prefill, attn, st, nullptr, nullptr, 0, 0, nullptr, nullptr,
                       l + 1 == c.n_layers ? 0 : -1);
        if (rc != PCD_OK) return rc;
    }
    HIP_TRY(hipEventRecord(m->ev[4], st));
    HIP_TRY(hipGetLastError());
    // The pass stays in flight: only the plan upload must have left the
    // pinned staging buffer before the next call refills it.
    HIP_TRY(hipEventSynchronize(m->ev[5]));
    m->prefill_pending = true;
    m->prefill_st = st;
    if (m->timing) {
        HIP_TRY(hipStreamSynchronize(st));
        m->tcollect();
    }
    m->stats.prefill_passes += 1;
    return PCD_OK;
}

// One causal pass over n_seqs sequences laid back to back (prefill of a batch
// of prompts): token t of sequence r sits at position t - t0[r] and attends
// the keys of its own sequence up to itself; each sequence's K and V go to
// its own buffer (bufs[r], caps[r] tokens per slab).  Attention is split over
// workgroups as in causal_pass, with one split length for all sequences.
int causal_many(pcd_model *m, int n_seqs, void *const *bufs, const int32_t *caps, const int32_t *tokens,
                const int32_t *lens, hipStream_t st) {
    const pcd_config &c = m->cfg;
    const int grp = c.n_heads / c.n_kv_heads, hd = c.head_dim;
    std::vector<int32_t> t0(n_seqs + 1, 0);
    int max_len = 0;
    int64_t wide_blocks = 0;
    for (int r = 0; r < n_seqs; ++r) {
        t0[r + 1] = t0[r] + lens[r];
        max_len = std::max(max_len, lens[r]);
        wide_blocks += (int64_t)c.n_kv_heads * (((int64_t)lens[r] * grp + ATT_WIDE_ROWS - 1) / ATT_WIDE_ROWS);
    }
    const bool wide = c.dtype == PCD_DTYPE_BF16 && wide_blocks >= ATT_WIDE_MIN_BLOCKS;
    const int arows = wide ? ATT_WIDE_ROWS : ATT_ROWS;
    int64_t row_blocks = 0;
    for (int r = 0; r < n_seqs; ++r)
        row_blocks += (int64_t)c.n_kv_heads * (((int64_t)lens[r] * grp + arows - 1) / arows);
    const int n = t0[n_seqs];
    int ns = att_splits(row_blocks, (max_len + 63) / 64, false);
    bool halves = false;  // two key chains per 8-wave block whatever the block count
    {
        std::vector<ChainSpec> chains;
        std::vector<TokRange> toks;
        for (int r = 0; r < n_seqs; ++r) {
            toks.push_back({1, lens[r], true});
            for (int g = 0; g < c.n_kv_heads; ++g)
                for (int r0 = t0[r] * grp; r0 < t0[r + 1] * grp; r0 += arows)
                    chains.push_back({(r0 + std::min(arows, t0[r + 1] * grp - r0) - 1) / grp - t0[r] + 1, 0});
        }
        const SplitPlan sp = model_splits(chains, max_len, toks, 4.0 * c.n_heads * hd,
                                           !wide && c.dtype == PCD_DTYPE_BF16);
        if (sp.s) ns = sp.s;
        halves = sp.halves;
    }
    const int slen = ((max_len + ns - 1) / ns + 63) / 64 * 64;
    ns = (max_len + slen - 1) / slen;
    std::vector<AttnBlock> blocks;
    for (int r = 0; r < n_seqs; ++r)
        for (int g = 0; g < c.n_kv_heads; ++g)
            for (int r0 = t0[r] * grp; r0 < t0[r + 1] * grp; r0 += arows) {
                const int nr = std::min(arows, t0[r + 1] * grp - r0);
                const int p_last = (r0 + nr - 1) / grp - t0[r];  // position of the block's last token
                for (int k = 0; k < ns && k * slen <= p_last; ++k)
                    blocks.push_back(AttnBlock{r, g, r0, nr, k * slen, std::min(lens[r], (k + 1) * slen), k, ns, 0, 0,
                                               1, -t0[r]});
            }
    longest_first(blocks, 0, blocks.size(), grp);
    xcd_order(blocks, 0, blocks.size());
    if ((int64_t)blocks.size() > plan_block_cap(c, m->lim)) return fail(PCD_E_CAP, "too many attention blocks");
    std::vector<int32_t> tok_splits(n), pos(n), req(n);
    std::vector<uint64_t> base(n_seqs);
    for (int r = 0; r < n_seqs; ++r) {
        base[r] = reinterpret_cast<uint64_t>(bufs[r]);
        for (int t = t0[r]; t < t0[r + 1]; ++t) {
            pos[t] = t - t0[r];
            req[t] = r;
            tok_splits[t] = pos[t] / slen + 1;
        }
    }
    Packer pk{m->plan_host, m->ws + m->L.plan, m->L.plan_bytes};
    const int32_t *d_tok = pk.put(tokens, n);
    const int32_t *d_pos = pk.put(pos.data(), n);
    const int32_t *d_req = pk.put(req.data(), n);
    const uint64_t *d_kv = pk.put(base.data(), n_seqs);
    const int32_t *d_stride = pk.put(caps, n_seqs);
    const int32_t *d_tsp = pk.put(tok_splits.data(), n);
    const AttnBlock *d_blk = pk.put(blocks.data(), blocks.size());
    if (pk.overflow) return fail(PCD_E_CAP, "plan staging overflow");
    const KvRows kr{d_req, d_pos, d_stride, d_kv};  // a token's slot in its buffer is its position
    if (int rc = m->check_stream(st)) return rc;
    m->settle_prefill();
    HIP_TRY(hipMemcpyAsync(m->ws + m->L.plan, m->plan_host, pk.off, hipMemcpyHostToDevice, st));
    HIP_TRY(hipEventRecord(m->ev[5], st));
    HIP_TRY(hipEventRecord(m->ev[3], st));
    float *x = reinterpret_cast<float *>(m->ws + m->L.x);
    m->tbegin(PCD_KC_OTHER, st);
    embed(c.dtype, d_tok, n, m->embed, c.d_model, x, m->an[0], c.rms_eps, m->ws + m->L.h, st);
    m->tend(st);
    float *part_o = reinterpret_cast<float *>(m->ws + m->L.part_o);
    float2 *part_ml = reinterpret_cast<float2 *>(m->ws + m->L.part_ml);
    for (int l = 0; l < c.n_layers; ++l) {
        auto attn = [&](void *q, void *ao, bool) {
            AttnCall a{};
            a.dt = c.dtype;
            a.hd = hd;
            a.n_heads = c.n_heads;
            a.n_kv_heads = c.n_kv_heads;
            a.layer = l;
            a.q = q;
            a.req_kv = d_kv;
            a.req_stride = d_stride;
            a.blocks = d_blk;
            a.n_blocks = (int)blocks.size();
            a.tok_splits = d_tsp;
            a.out = ao;
            a.part_o = part_o;
            a.part_ml = part_ml;
            a.n_tokens = n;
            a.wide = wide;
            a.halves = halves;
            m->tbegin(PCD_KC_PREFILL_ATTN, st);
            const bool ok = attention(a, st);
            m->tend(st);
            if (!ok) return fail(PCD_E_ARG, "attention: unsupported head_dim/dtype");
            if (ns > 1) {
                TailCall t{};
                t.dt = c.dtype;
                t.hd = hd;
                t.n_heads = c.n_heads;
                t.n_kv_heads = c.n_kv_heads;
                t.n_tokens = n;
                t.part_o = part_o;
                t.part_ml = part_ml;
                t.tok_splits = d_tsp;
                t.out = ao;
                m->tbegin(PCD_KC_OTHER, st);
                attention_merge(t, st);
                m->tend(st);
            }
            return PCD_OK;
        };
        int rc = layer(m, l, n, d_pos, nullptr, nullptr, 0, Pass::Prefill, attn, st, nullptr, nullptr, 0, 0, &kr,
                       nullptr, l + 1 == c.n_layers ? 0 : -1);
        if (rc != PCD_OK) return rc;
    }
    HIP_TRY(hipEventRecord(m->ev[4], st));
    HIP_TRY(hipGetLastError());
    HIP_TRY(hipEventSynchronize(m->ev[5]));
    m->prefill_pending = true;
    m->prefill_st = st;
    if (m->timing) {
        HIP_TRY(hipStreamSynchronize(st));
        m->tcollect();
    }
    m->stats.prefill_passes += 1;
    return PCD_OK;
}

int check_tokens(const pcd_model *m, const int32_t *tokens, int32_t n) {
    for (int i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= m->cfg.vocab_size)
            return fail(PCD_E_TOKEN, "token id " + std::to_string(tokens[i]) + " outside the vocabulary");
    return PCD_OK;
}

}  // namespace

int pcd_prefill_many(pcd_model *m, int32_t n_seqs, const int32_t *tokens, const int32_t *lens, void *const *kv_bufs,
                     const size_t *kv_bytes, void *stream, pcd_state **out) {
    if (!m || !tokens || !lens || !kv_bufs || !kv_bytes || !out) return fail(PCD_E_ARG, "null argument");
    const pcd_config &c = m->cfg;
    if (n_seqs <= 0 || n_seqs > m->lim.max_requests)
        return fail(PCD_E_ARG, std::to_string(n_seqs) + " sequences (allowed 1.." +
                                   std::to_string(m->lim.max_requests) + ")");
    int64_t total = 0;
    std::vector<int32_t> caps(n_seqs);
    std::vector<std::pair<uint64_t, uint64_t>> spans(n_seqs);
    for (int r = 0; r < n_seqs; ++r) {
        if (lens[r] <= 0) return fail(PCD_E_ARG, "sequence " + std::to_string(r) + " is empty");
        if (!kv_bufs[r] || misaligned(kv_bufs[r]))
            return fail(PCD_E_ARG, "null or misaligned KV buffer for sequence " + std::to_string(r));
        if (lens[r] > c.max_seq) return fail(PCD_E_CAP, "sequence " + std::to_string(r) + " exceeds max_seq");
        if (kv_bytes[r] < pcd_state_bytes(m, lens[r]))
            return fail(PCD_E_CAP, "KV buffer of sequence " + std::to_string(r) + " too small");
        total += lens[r];
        caps[r] = (int32_t)std::min<size_t>(kv_bytes[r] / per_token_bytes(m), (size_t)c.max_seq);
        const uint64_t b = reinterpret_cast<uint64_t>(kv_bufs[r]);
        spans[r] = {b, b + (uint64_t)caps[r] * per_token_bytes(m)};
    }
    if (total > m->lim.max_prefill_tokens)
        return fail(PCD_E_CAP, std::to_string(total) + " tokens exceed the model's max_prefill_tokens");
    std::sort(spans.begin(), spans.end());
    for (int r = 1; r < n_seqs; ++r)
        if (spans[r].first < spans[r - 1].second) return fail(PCD_E_ARG, "two sequences share KV buffer memory");
    int rc = check_tokens(m, tokens, (int32_t)total);
    if (rc != PCD_OK) return rc;
    std::vector<pcd_state *> made(n_seqs, nullptr);
    for (int r = 0; r < n_seqs; ++r) {
        made[r] = new (std::nothrow) pcd_state{STATE_MAGIC, m, kv_bufs[r], 0, caps[r]};
        if (!made[r]) {
            for (pcd_state *p : made) delete p;
            return fail(PCD_E_NOMEM, "state allocation");
        }
    }
    rc = causal_many(m, n_seqs, kv_bufs, caps.data(), tokens, lens, static_cast<hipStream_t>(stream));
    if (rc != PCD_OK) {
        for (pcd_state *p : made) delete p;
        return rc;
    }
    for (int r = 0; r < n_seqs; ++r) {
        made[r]->P = lens[r];
        out[r] = made[r];
    }
    m->n_states += n_seqs;
    return PCD_OK;
}

int pcd_prefill(pcd_model *m, const int32_t *tokens, int32_t n, void *kv_buf, size_t kv_bytes, void *stream,
                pcd_state **out) {
    if (!m || !tokens || !kv_buf || !out) return fail(PCD_E_ARG, "null argument");
    if (misaligned(kv_buf)) return fail(PCD_E_ARG, "the KV buffer must be 16-byte aligned");
    const pcd_config &c = m->cfg;
    if (n <= 0) return fail(PCD_E_ARG, "empty prefix");
    if (n > m->lim.max_prefill_tokens || n > c.max_seq)
        return fail(PCD_E_CAP, "prefix of " + std::to_string(n) + " tokens exceeds the model's limits");
    if (kv_bytes < pcd_state_bytes(m, n)) return fail(PCD_E_CAP, "KV buffer too small");
    const size_t cap_tokens = kv_bytes / per_token_bytes(m);
    const int32_t cap = (int32_t)std::min<size_t>(cap_tokens, (size_t)c.max_seq);
    int rc = check_tokens(m, tokens, n);
    if (rc != PCD_OK) return rc;
    pcd_state *s = new (std::nothrow) pcd_state{STATE_MAGIC, m, kv_buf, 0, cap};
    if (!s) return fail(PCD_E_NOMEM, "state allocation");
    rc = causal_pass(m, kv_buf, cap, 0, tokens, n, static_cast<hipStream_t>(stream));
    if (rc != PCD_OK) {
        delete s;
        return rc;
    }
    s->P = n;
    m->n_states++;
    *out = s;
    return PCD_OK;
}

int pcd_extend(pcd_state *s, const int32_t *tokens, int32_t n, void *stream) {
    if (!s || s->magic != STATE_MAGIC) return fail(PCD_E_STATE, "invalid state handle");
    if (!tokens) return fail(PCD_E_ARG, "null argument");
    if (n <= 0) return fail(PCD_E_ARG, "nothing to append");
    pcd_model *m = s->m;
    if (n > m->lim.max_prefill_tokens || s->P + n > m->cfg.max_seq)
        return fail(PCD_E_CAP, "appending " + std::to_string(n) + " tokens exceeds the model's limits");
    if (s->P + n > s->cap)
        return fail(PCD_E_CAP, "the state's KV buffer holds " + std::to_string(s->cap) + " tokens, " +
                                   std::to_string(s->P + n) + " needed");
    int rc = check_tokens(m, tokens, n);
    if (rc != PCD_OK) return rc;
    rc = causal_pass(m, s->kv, s->cap, s->P, tokens, n, static_cast<hipStream_t>(stream));
    if (rc != PCD_OK) return rc;
    s->P += n;
    return PCD_OK;
}

int pcd_fork(const pcd_state *s, void *kv_buf, size_t kv_bytes, void *stream, pcd_state **out) {
    if (!s || s->magic != STATE_MAGIC) return fail(PCD_E_STATE, "invalid state handle");
    if (!kv_buf || !out) return fail(PCD_E_ARG, "null argument");
    if (misaligned(kv_buf)) return fail(PCD_E_ARG, "the KV buffer must be 16-byte aligned");
    pcd_model *m = s->m;
    if (kv_bytes < pcd_state_bytes(m, s->P)) return fail(PCD_E_CAP, "KV buffer too small");
    const int32_t cap = (int32_t)std::min<size_t>(kv_bytes / per_token_bytes(m), (size_t)m->cfg.max_seq);
    const size_t row = (size_t)m->cfg.head_dim * esize(m);
    // every (layer, K|V, KV head) slab: the first P rows, from stride s->cap to stride cap
    HIP_TRY(hipMemcpy2DAsync(kv_buf, (size_t)cap * row, s->kv, (size_t)s->cap * row, (size_t)s->P * row,
                             (size_t)m->cfg.n_layers * 2 * m->cfg.n_kv_heads, hipMemcpyDeviceToDevice,
                             static_cast<hipStream_t>(stream)));
    pcd_state *f = new (std::nothrow) pcd_state{STATE_MAGIC, m, kv_buf, s->P, cap};
    if (!f) return fail(PCD_E_NOMEM, "state allocation");
    m->n_states++;
    *out = f;
    return PCD_OK;
}

int pcd_state_tokens(const pcd_state *s) {
    if (!s || s->magic != STATE_MAGIC) return fail(PCD_E_STATE, "invalid state handle");
    return s->P;
}

int pcd_debug_plan(int32_t V, int32_t max_seq, int32_t n_req, const int32_t *prefix_lens, const pcd_request *reqs,
                   pcd_plan_info *info) {
    if (!info) return fail(PCD_E_ARG, "null info");
    Plan p;
    std::string err;
    int rc = build_plan(V, max_seq, n_req, prefix_lens, reqs, p, err, true);
    if (rc != PCD_OK) return fail(rc, err);
    info->n_branch = (int32_t)p.tok.size();
    info->n_readouts = (int32_t)p.ro_tok.size();
    info->n_gathers = (int32_t)p.g_tok.size();
    info->n_fields = (int32_t)p.f_ro_root.size();
    info->n_candidates = (int32_t)p.c_spell_off.size() - 1;
    info->n_spellings = (int32_t)p.s_path_off.size() - 1;
    info->n_paths = (int32_t)p.s_path.size();
    info->n_anc = (int32_t)p.anc.size();
    auto cp = [](int32_t *dst, const std::vector<int32_t> &v) {
        if (dst && !v.empty()) std::memcpy(dst, v.data(), v.size() * 4);
    };
    cp(info->tok, p.tok);
    cp(info->pos, p.pos);
    cp(info->req, p.req);
    cp(info->field, p.field);
    cp(info->anc_off, p.anc_off);
    cp(info->anc, p.anc);
    cp(info->ro_tok, p.ro_tok);
    cp(info->ro_field, p.ro_field);
    cp(info->g_off, p.g_off);
    cp(info->g_tok, p.g_tok);
    cp(info->f_ro_root, p.f_ro_root);
    cp(info->f_cand_off, p.f_cand_off);
    cp(info->f_mode, p.f_mode);
    cp(info->c_spell_off, p.c_spell_off);
    cp(info->s_path_off, p.s_path_off);
    cp(info->s_path, p.s_path);
    return PCD_OK;
}

namespace {

// One batched branch pass over the fields of n_req requests, each on its own
// state.  With n_new > 0 (one request) the pass also carries new_tok, which
// are appended to the state: its first rows are those tokens, causal over the
// state's cached tokens and each other, their K/V written into the state's
// buffer; the branch rows then see the whole extended prefix.  One pass thus
// does the work of pcd_extend followed by pcd_decide, streaming every weight
// matrix once.
// The pass is enqueued on `stream` and the call returns with a pending
// handle; decide_finish waits for it and writes the outputs.
int decide_start(pcd_state *const *states, const pcd_request *reqs, int32_t n_req, float T, const pcd_outputs *outs,
                 void *stream, const int32_t *new_tok, int32_t n_new, pcd_pending **pend) {
    if (!states || !reqs || !outs || n_req <= 0) return fail(PCD_E_ARG, "null argument or no requests");
    if (!(T > 0.f) || !std::isfinite(T)) return fail(PCD_E_ARG, "temperature must be positive and finite");
    for (int r = 0; r < n_req; ++r)
        if (!states[r] || states[r]->magic != STATE_MAGIC) return fail(PCD_E_STATE, "invalid state handle");
    pcd_model *m = states[0]->m;
    for (int r = 1; r < n_req; ++r)
        if (states[r]->m != m) return fail(PCD_E_STATE, "states of different models in one call");
    for (int r = 0; r < n_req; ++r)
        if (!outs[r].cand_prob || !outs[r].field_mass || !outs[r].field_margin || !outs[r].field_argmax)
            return fail(PCD_E_ARG, "null output array");
    const pcd_config &c = m->cfg;
    const pcd_limits &lim = m->lim;
    if (n_req > lim.max_requests) return fail(PCD_E_CAP, "more requests than max_requests");
    if (n_new > 0) {
        if (n_req != 1) return fail(PCD_E_ARG, "new tokens go with exactly one request");
        if (!new_tok) return fail(PCD_E_ARG, "null argument");
        const pcd_state *s0 = states[0];
        if (s0->P + n_new > s0->cap)
            return fail(PCD_E_CAP, "the state's KV buffer holds " + std::to_string(s0->cap) + " tokens, " +
                                       std::to_string(s0->P + n_new) + " needed");
        for (int i = 0; i < n_new; ++i)
            if (new_tok[i] < 0 || new_tok[i] >= c.vocab_size)
                return fail(PCD_E_TOKEN, "token id " + std::to_string(new_tok[i]) + " outside the vocabulary");
    }
    const int P0 = n_new > 0 ? states[0]->P : 0;  // cached tokens before the new ones
    std::vector<int32_t> lens(n_req);
    for (int r = 0; r < n_req; ++r) lens[r] = states[r]->P + (r == 0 ? n_new : 0);
    Plan p;
    std::string err;
    int rc = build_plan(c.vocab_size, c.max_seq, n_req, lens.data(), reqs, p, err);
    if (rc != PCD_OK) return fail(rc, err);
    const int Tb = (int)p.tok.size(), R = (int)p.ro_tok.size(), G = (int)p.g_tok.size();
    const int F = (int)p.f_ro_root.size(), C = (int)p.c_spell_off.size() - 1, S = (int)p.s_path_off.size() - 1;
    const int NP = (int)p.s_path.size();
    if (Tb > lim.max_branch_tokens || R > lim.max_readouts || G > lim.max_gathers || F > lim.max_fields ||
        C > lim.max_candidates || S > spell_cap(lim) || NP > path_cap(lim))
        return fail(PCD_E_CAP, "decide call of " + std::to_string(Tb) + " branch tokens, " + std::to_string(R) +
                                   " readouts, " + std::to_string(G) + " gathers exceeds the model's limits");
    const int grp = c.n_heads / c.n_kv_heads, hd = c.head_dim, d = c.d_model;
    const int M = n_new + Tb;  // rows of the pass: new tokens, then branch tokens
    const int64_t ws_rows = std::max(lim.max_prefill_tokens, lim.max_branch_tokens);
    if (M > ws_rows)
        return fail(PCD_E_CAP, std::to_string(n_new) + " new tokens and " + std::to_string(Tb) +
                                   " branch tokens exceed the workspace's " + std::to_string(ws_rows) + " rows");

    // attention blocks, per KV head and 64-row block; with too few row blocks
    // for the chip the keys are split over workgroups (the partials are then
    // merged by a second kernel).  New tokens: causal over the extended
    // prefix.  Branch tokens: the prefix of their request, split; the last
    // split also covers the branch keys of the fields its rows belong to.
    //
    // With enough new tokens (bf16) their causal rows take 128-row blocks
    // (as a prefill pass does) in a launch of their own after the branch
    // blocks' launch; the branch rows then split their keys as in a pass of
    // branch rows only.
    std::vector<int32_t> tok_splits(M, 1);
    std::vector<uint64_t> req_kv(n_req);
    std::vector<AttnBlock> blocks;
    bool any_split = false;
    const int64_t new_wide_blocks = (int64_t)c.n_kv_heads * (((int64_t)n_new * grp + ATT_WIDE_ROWS - 1) / ATT_WIDE_ROWS);
    const bool wide_new = n_new > 0 && c.dtype == PCD_DTYPE_BF16 && new_wide_blocks >= ATT_WIDE_MIN_BLOCKS;
    int64_t branch_row_blocks = 0;
    for (int r = 0; r < n_req; ++r)
        branch_row_blocks +=
            (int64_t)c.n_kv_heads * (((int64_t)(p.r_tok[r + 1] - p.r_tok[r]) * grp + ATT_ROWS - 1) / ATT_ROWS);
    const int64_t row_blocks =
        wide_new ? 0 : branch_row_blocks + (int64_t)c.n_kv_heads * (((int64_t)n_new * grp + ATT_ROWS - 1) / ATT_ROWS);
    // A pass with new tokens serves one request, whose branch rows see the
    // same extended prefix: where the longest chains bind, one split count
    // for both groups of the launch (and for the causal launch of its own).
    int model_s = 0;
    bool halves = false;  // two key chains per 8-wave block (the one launch of a pass that is not wide)
    if (n_new > 0) {
        std::vector<ChainSpec> chains;
        std::vector<TokRange> toks{{P0 + 1, n_new, true}};
        const int keys = P0 + n_new;
        const int rows = n_new * grp, arows = wide_new ? ATT_WIDE_ROWS : ATT_ROWS;
        for (int g = 0; g < c.n_kv_heads; ++g)
            for (int r0 = 0; r0 < rows; r0 += arows)
                chains.push_back({P0 + (r0 + std::min(arows, rows - r0) - 1) / grp + 1, 0});
        if (!wide_new) {  // the branch blocks share the launch; their tokens reach every key
            toks.push_back({keys, p.r_tok[1], false});
            const int row_beg = n_new * grp, row_end = (n_new + p.r_tok[1]) * grp;
            for (int g = 0; g < c.n_kv_heads; ++g)
                for (int r0 = row_beg; r0 < row_end; r0 += ATT_ROWS) {
                    const int nr = std::min(ATT_ROWS, row_end - r0);
                    const int b_first = r0 / grp - n_new, b_last = (r0 + nr - 1) / grp - n_new;
                    chains.push_back({lens[0], (b_last + 1 - p.fs[b_first] + 63) / 64});
                }
        }
        if (n_req == 1 && lens[0] == keys) {
            const SplitPlan sp = model_splits(chains, keys, toks, 4.0 * c.n_heads * hd,
                                               !wide_new && c.dtype == PCD_DTYPE_BF16);
            model_s = sp.s;
            halves = sp.halves;
        }
    }
    auto split_keys = [&](int keys, bool causal, int &s, int &slen) {
        if (wide_new)  // two launches: each group of blocks on its own
            s = causal ? (model_s ? model_s : att_splits(new_wide_blocks, (keys + 63) / 64, false))
                       : att_splits(branch_row_blocks, (keys + 63) / 64, true);
        else
            s = model_s ? model_s : att_splits(row_blocks, (keys + 63) / 64, !causal && n_new == 0);
        if (keys == 0) {
            s = 1;
            slen = 0;
            return;
        }
        slen = ((keys + s - 1) / s + 63) / 64 * 64;
        s = (keys + slen - 1) / slen;
    };
    // The branch tokens' blocks come first (the last layer runs only them),
    // then the new tokens' causal blocks; each group longest chain first.
    for (int r = 0; r < n_req; ++r) {
        const int P = lens[r];
        int s, slen;
        split_keys(P, false, s, slen);
        any_split |= s > 1;
        for (int t = p.r_tok[r]; t < p.r_tok[r + 1]; ++t) tok_splits[n_new + t] = s;
        req_kv[r] = reinterpret_cast<uint64_t>(states[r]->kv);
        const int row_beg = (n_new + p.r_tok[r]) * grp, row_end = (n_new + p.r_tok[r + 1]) * grp;
        for (int g = 0; g < c.n_kv_heads; ++g)
            for (int r0 = row_beg; r0 < row_end; r0 += ATT_ROWS) {
                const int nr = std::min(ATT_ROWS, row_end - r0);
                const int b_first = r0 / grp - n_new, b_last = (r0 + nr - 1) / grp - n_new;  // plan indices
                for (int k = 0; k < s; ++k)
                    blocks.push_back(AttnBlock{r, g, r0, nr, k * slen, std::min(P, (k + 1) * slen), k, s,
                                               k == s - 1 ? p.fs[b_first] : 0, k == s - 1 ? b_last + 1 : 0, 0, 0});
            }
    }
    const int n_branch_blocks = (int)blocks.size();
    longest_first(blocks, 0, blocks.size(), grp);
    xcd_order(blocks, 0, blocks.size());
    int merge_tok0 = n_new;  // the merge starts at the first token with more than one split
    if (n_new > 0) {
        int s, slen;
        split_keys(P0 + n_new, true, s, slen);
        any_split |= s > 1;
        if (s > 1) merge_tok0 = std::max(0, std::min(n_new, slen - P0));
        for (int t = 0; t < n_new; ++t) tok_splits[t] = (P0 + t) / slen + 1;
        const int rows = n_new * grp, arows = wide_new ? ATT_WIDE_ROWS : ATT_ROWS;
        for (int g = 0; g < c.n_kv_heads; ++g)
            for (int r0 = 0; r0 < rows; r0 += arows) {
                const int nr = std::min(arows, rows - r0), t_last = P0 + (r0 + nr - 1) / grp;
                for (int k = 0; k < s && k * slen <= t_last; ++k)
                    blocks.push_back(
                        AttnBlock{0, g, r0, nr, k * slen, std::min(P0 + n_new, (k + 1) * slen), k, s, 0, 0, 1, P0});
            }
        longest_first(blocks, n_branch_blocks, blocks.size(), grp);
        xcd_order(blocks, n_branch_blocks, blocks.size());
    }
    if ((int64_t)blocks.size() > plan_block_cap(c, lim)) return fail(PCD_E_CAP, "too many attention blocks");

    hipStream_t st = static_cast<hipStream_t>(stream);
    if (int rc = m->check_stream(st)) return rc;
    int si = -1;
    for (int k = 0; k < PCD_MAX_PENDING && si < 0; ++k)
        if (!m->slots[k].busy) si = k;
    if (si < 0)
        return fail(PCD_E_CAP, std::to_string(PCD_MAX_PENDING) + " decide calls of this model are already in flight");
    auto &slot = m->slots[si];
    Packer pk{slot.plan_host, m->ws + m->L.plan, m->L.plan_bytes};
    std::vector<int32_t> toks(M), poss(M);
    for (int i = 0; i < n_new; ++i) {
        toks[i] = new_tok[i];
        poss[i] = P0 + i;
    }
    std::copy(p.tok.begin(), p.tok.end(), toks.begin() + n_new);
    std::copy(p.pos.begin(), p.pos.end(), poss.begin() + n_new);
    std::vector<int32_t> ro_rows(p.ro_tok);
    for (auto &v : ro_rows) v += n_new;
    const int32_t *d_tok = pk.put(toks.data(), M);
    const int32_t *d_pos = pk.put(poss.data(), M);
    const int32_t *d_tsp = pk.put(tok_splits.data(), M);
    const int32_t *d_fs = pk.put(p.fs.data(), Tb);
    const int32_t *d_nsc = pk.put(p.nsc.data(), Tb);
    const int32_t *d_par = pk.put(p.par.data(), Tb);
    // the first 8 links of every trie token's chain (itself, parent, ...), so
    // the attention kernel reads them with two independent loads
    std::vector<int32_t> chain((size_t)8 * Tb, -1);
    for (int t = 0; t < Tb; ++t) {
        if (t < p.fs[t] + p.nsc[t]) continue;  // scaffold token: no chain
        int a = t;
        for (int i = 0; i < 8 && a >= 0; ++i) {
            chain[(size_t)8 * t + i] = a;
            a = p.par[a];
        }
    }
    const int4 *d_chain = reinterpret_cast<const int4 *>(pk.put(chain.data(), chain.size()));
    const int32_t *d_ro = pk.put(ro_rows.data(), R);
    const int32_t *d_goff = pk.put(p.g_off.data(), R + 1);
    const int32_t *d_gtok = pk.put(p.g_tok.data(), G);
    const int32_t *d_gro = pk.put(p.g_ro.data(), G);
    const int32_t *d_froot = pk.put(p.f_ro_root.data(), F);
    const int32_t *d_fcand = pk.put(p.f_cand_off.data(), F + 1);
    const int32_t *d_fmode = pk.put(p.f_mode.data(), F);
    const int32_t *d_cso = pk.put(p.c_spell_off.data(), C + 1);
    const int32_t *d_spo = pk.put(p.s_path_off.data(), S + 1);
    const int32_t *d_sp = pk.put(p.s_path.data(), NP);
    std::vector<int32_t> strides(n_req);
    for (int r = 0; r < n_req; ++r) strides[r] = states[r]->cap;
    const int32_t *d_stride = pk.put(strides.data(), n_req);
    const uint64_t *d_kv = pk.put(req_kv.data(), n_req);
    const AttnBlock *d_blk = pk.put(blocks.data(), blocks.size());
    if (pk.overflow) return fail(PCD_E_CAP, "plan staging overflow");

    // result block on the device, packed by this call's sizes
    char *ob = m->ws + m->L.outs;
    size_t oo = 0;
    auto oslot = [&](size_t bytes) {
        const size_t o = oo;
        oo = align_up(oo + bytes);
        return o;
    };
    const size_t o_prob = oslot((size_t)C * 4), o_ls = oslot((size_t)C * 4), o_mass = oslot((size_t)F * 4),
                 o_marg = oslot((size_t)F * 4), o_arg = oslot((size_t)F * 4), o_lse = oslot((size_t)R * 4),
                 o_z = oslot((size_t)G * 4);
    if (oo > m->L.outs_bytes) return fail(PCD_E_CAP, "output staging overflow");

    HIP_TRY(hipMemcpyAsync(m->ws + m->L.plan, slot.plan_host, pk.off, hipMemcpyHostToDevice, st));
    HIP_TRY(hipEventRecord(slot.ev[0], st));
    float *x = reinterpret_cast<float *>(m->ws + m->L.x);
    m->tbegin(PCD_KC_OTHER, st);
    embed(c.dtype, d_tok, M, m->embed, d, x, m->an[0], c.rms_eps, m->ws + m->L.h, st);
    m->tend(st);
    const size_t layer_elems = (size_t)2 * c.n_kv_heads * Tb * hd;
    const size_t es = esize(m), sslab = n_new > 0 ? (size_t)states[0]->cap * hd : 0;
    float *part_o = reinterpret_cast<float *>(m->ws + m->L.part_o);
    float2 *part_ml = reinterpret_cast<float2 *>(m->ws + m->L.part_ml);
    for (int l = 0; l < c.n_layers; ++l) {
        char *kc = m->ws + m->L.kvb + (size_t)l * layer_elems * es;
        char *vc = kc + layer_elems / 2 * es;
        // new tokens' K/V: the state's slabs of this layer, at row P0
        char *skc = n_new > 0 ? static_cast<char *>(states[0]->kv) +
                                    ((size_t)l * 2 * c.n_kv_heads * sslab + (size_t)P0 * hd) * es
                              : nullptr;
        char *svc = n_new > 0 ? skc + (size_t)c.n_kv_heads * sslab * es : nullptr;
        auto attn = [&](void *q, void *ao, bool last) {
            AttnCall a{};
            a.dt = c.dtype;
            a.hd = hd;
            a.n_heads = c.n_heads;
            a.n_kv_heads = c.n_kv_heads;
            a.layer = l;
            a.q = q;
            a.req_kv = d_kv;
            a.req_stride = d_stride;
            // the last layer needs no attention output for the new tokens
            a.blocks = d_blk;
            a.n_blocks = last ? n_branch_blocks : (int)blocks.size();
            a.branch0 = n_new;
            a.tok_splits = d_tsp;
            a.out = ao;
            a.part_o = part_o;
            a.part_ml = part_ml;
            a.n_tokens = M;
            a.kb = kc;
            a.vb = vc;
            a.cap = Tb;
            a.fs = d_fs;
            a.nsc = d_nsc;
            a.par = d_par;
            a.chain = d_chain;
            a.halves = halves;
            m->tbegin(last ? PCD_KC_OTHER : n_new > 0 ? PCD_KC_FUSED_ATTN : PCD_KC_BRANCH_ATTN, st);
            bool ok;
            if (wide_new && !last) {
                a.n_blocks = n_branch_blocks;
                ok = attention(a, st);
                AttnCall b = a;  // the new tokens' 128-row causal blocks
                b.blocks = d_blk + n_branch_blocks;
                b.n_blocks = (int)blocks.size() - n_branch_blocks;
                b.wide = 1;
                ok = ok && attention(b, st);
            } else {
                ok = attention(a, st);
            }
            m->tend(st);
            if (!ok) return fail(PCD_E_ARG, "attention: unsupported head_dim/dtype");
            if (any_split) {
                TailCall t{};
                t.dt = c.dtype;
                t.hd = hd;
                t.n_heads = c.n_heads;
                t.n_kv_heads = c.n_kv_heads;
                t.n_tokens = M;
                t.tok0 = last ? n_new : merge_tok0;
                t.part_o = part_o;
                t.part_ml = part_ml;
                t.tok_splits = d_tsp;
                t.out = ao;
                m->tbegin(last || n_new > 0 ? PCD_KC_OTHER : PCD_KC_BRANCH_TAIL, st);
                attention_merge(t, st);
                m->tend(st);
            }
            return PCD_OK;
        };
        // the last layer carries on only the readout rows
        const bool last = l + 1 == c.n_layers;
        const int32_t *keep = last ? d_ro : nullptr;
        const int n_keep = last ? R : -1;
        rc = n_new > 0 ? layer(m, l, M, d_pos, skc, svc, states[0]->cap, Pass::Fused, attn, st, kc, vc, Tb, n_new,
                               nullptr, keep, n_keep)
                       : layer(m, l, M, d_pos, kc, vc, Tb, Pass::Branch, attn, st, nullptr, nullptr, 0, 0, nullptr, keep,
                               n_keep);
        if (rc != PCD_OK) return rc;
    }
    HIP_TRY(hipEventRecord(slot.ev[1], st));
    // readout: final norm of the readout rows, LM head with online log-sum-exp, combine
    void *hr = m->ws + m->L.hr;
    m->tbegin(PCD_KC_OTHER, st);
    // the readout rows' residual stream, gathered in the last layer
    rmsnorm(c.dtype, reinterpret_cast<const float *>(m->ws + m->L.xr), nullptr, R, d, m->final_norm, c.rms_eps, hr,
            st);
    m->tend(st);
    float2 *ro_part = reinterpret_cast<float2 *>(m->ws + m->L.ro_part);
    float *z = reinterpret_cast<float *>(ob + o_z), *lse = reinterpret_cast<float *>(ob + o_lse);
    GemmCall g{};
    g.dt = c.dtype;
    g.A = hr;
    g.M = R;
    g.N = c.vocab_size;
    g.K = d;
    g.B[0].ptr[0] = m->head;
    g.B[0].nseg = 1;
    g.epi = Epi::Readout;
    g.ro_part = ro_part;
    g.g_tok = d_gtok;
    g.g_ro = d_gro;
    g.n_gather = G;
    g.g_logit = z;
    m->tbegin(PCD_KC_READOUT_LMHEAD, st);
    if (!gemm(g, st)) return fail(PCD_E_ARG, "LM head: unsupported shape");
    m->tend(st);
    m->tbegin(PCD_KC_OTHER, st);
    readout_lse(ro_part, c.vocab_size / 128, R, lse, st);
    CombineCall cc{};
    cc.n_fields = F;
    cc.f_cand_off = d_fcand;
    cc.f_ro_root = d_froot;
    cc.f_mode = d_fmode;
    cc.c_spell_off = d_cso;
    cc.s_path_off = d_spo;
    cc.s_path = d_sp;
    cc.g_off = d_goff;
    cc.g_ro = d_gro;
    cc.z = z;
    cc.lse = lse;
    cc.temperature = T;
    cc.prob = reinterpret_cast<float *>(ob + o_prob);
    cc.logscore = reinterpret_cast<float *>(ob + o_ls);
    cc.mass = reinterpret_cast<float *>(ob + o_mass);
    cc.margin = reinterpret_cast<float *>(ob + o_marg);
    cc.argmax = reinterpret_cast<int32_t *>(ob + o_arg);
    combine(cc, st);
    m->tend(st);
    HIP_TRY(hipEventRecord(slot.ev[2], st));
    HIP_TRY(hipGetLastError());
    HIP_TRY(hipMemcpyAsync(slot.outs_host, ob, oo, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipEventRecord(slot.ev[3], st));

    auto *pd = new (std::nothrow) pcd_pending{};
    if (!pd) {
        (void)hipEventSynchronize(slot.ev[3]);
        return fail(PCD_E_NOMEM, "pending call allocation");
    }
    pd->magic = PENDING_MAGIC;
    pd->m = m;
    pd->slot = si;
    pd->st = st;
    pd->n_req = n_req;
    pd->Tb = Tb;
    pd->R = R;
    pd->G = G;
    pd->outs.assign(outs, outs + n_req);
    pd->r_cand = p.r_cand;
    pd->r_field = p.r_field;
    pd->r_ro = p.r_ro;
    pd->r_g = p.r_g;
    pd->o_prob = o_prob;
    pd->o_ls = o_ls;
    pd->o_mass = o_mass;
    pd->o_marg = o_marg;
    pd->o_arg = o_arg;
    pd->o_lse = o_lse;
    pd->o_z = o_z;
    slot.busy = true;
    slot.st = st;
    // the new tokens are the state's from now on: later calls on the stream see them
    if (n_new > 0) states[0]->P += n_new;
    m->stats.branch_passes += 1;
    *pend = pd;
    return PCD_OK;
}

// Wait for a started call, copy its results out of its slot, free the slot.
int decide_finish(pcd_pending *pd) {
    if (!pd || pd->magic != PENDING_MAGIC) return fail(PCD_E_ARG, "invalid pending call");
    pcd_model *m = pd->m;
    auto &slot = m->slots[pd->slot];
    pd->magic = 0;
    const hipError_t e = hipEventSynchronize(slot.ev[3]);
    if (m->timing && e == hipSuccess) {
        (void)hipStreamSynchronize(pd->st);  // every timed kernel of the stream has run
        m->tcollect();
    }
    m->settle_prefill();
    const char *oh = slot.outs_host;
    if (e == hipSuccess)
        for (int r = 0; r < pd->n_req; ++r) {
            const pcd_outputs &o = pd->outs[r];
            const int c0 = pd->r_cand[r], nc = pd->r_cand[r + 1] - c0;
            const int f0 = pd->r_field[r], nf = pd->r_field[r + 1] - f0;
            const int r0 = pd->r_ro[r], nr = pd->r_ro[r + 1] - r0;
            const int g0 = pd->r_g[r], ng = pd->r_g[r + 1] - g0;
            std::memcpy(o.cand_prob, oh + pd->o_prob + (size_t)c0 * 4, (size_t)nc * 4);
            if (o.cand_logscore) std::memcpy(o.cand_logscore, oh + pd->o_ls + (size_t)c0 * 4, (size_t)nc * 4);
            std::memcpy(o.field_mass, oh + pd->o_mass + (size_t)f0 * 4, (size_t)nf * 4);
            std::memcpy(o.field_margin, oh + pd->o_marg + (size_t)f0 * 4, (size_t)nf * 4);
            std::memcpy(o.field_argmax, oh + pd->o_arg + (size_t)f0 * 4, (size_t)nf * 4);
            if (o.readout_lse) std::memcpy(o.readout_lse, oh + pd->o_lse + (size_t)r0 * 4, (size_t)nr * 4);
            if (o.gather_logit) std::memcpy(o.gather_logit, oh + pd->o_z + (size_t)g0 * 4, (size_t)ng * 4);
        }
    float ms_b = 0.f, ms_r = 0.f;
    (void)hipEventElapsedTime(&ms_b, slot.ev[0], slot.ev[1]);
    (void)hipEventElapsedTime(&ms_r, slot.ev[1], slot.ev[2]);
    m->stats.last_branch_ms = ms_b;
    m->stats.last_readout_ms = ms_r;
    m->stats.last_branch_tokens = pd->Tb;
    m->stats.last_readouts = pd->R;
    m->stats.last_gathers = pd->G;
    m->stats.last_requests = pd->n_req;
    slot.busy = false;
    delete pd;
    if (e != hipSuccess) return fail(PCD_E_DEVICE, std::string("decide pass: ") + hipGetErrorString(e));
    return PCD_OK;
}

int decide_impl(pcd_state *const *states, const pcd_request *reqs, int32_t n_req, float T, const pcd_outputs *outs,
                void *stream, const int32_t *new_tok, int32_t n_new) {
    pcd_pending *pd = nullptr;
    const int rc = decide_start(states, reqs, n_req, T, outs, stream, new_tok, n_new, &pd);
    if (rc != PCD_OK) return rc;
    return decide_finish(pd);
}

}  // namespace

int pcd_decide_many(pcd_state *const *states, const pcd_request *reqs, int32_t n_req, float T, pcd_outputs *outs,
                    void *stream) {
    return decide_impl(states, reqs, n_req, T, outs, stream, nullptr, 0);
}

int pcd_extend_decide(pcd_state *s, const int32_t *tokens, int32_t n_tokens, const pcd_field *fields,
                      int32_t n_fields, const pcd_candidate *candidates, int32_t n_candidates, float temperature,
                      pcd_outputs *out, void *stream) {
    if (n_tokens < 0) return fail(PCD_E_ARG, "negative token count");
    pcd_request r{fields, n_fields, candidates, n_candidates};
    return decide_impl(&s, &r, 1, temperature, out, stream, tokens, n_tokens);
}

int pcd_extend_decide_start(pcd_state *s, const int32_t *tokens, int32_t n_tokens, const pcd_field *fields,
                            int32_t n_fields, const pcd_candidate *candidates, int32_t n_candidates,
                            float temperature, const pcd_outputs *out, void *stream, pcd_pending **p) {
    if (!p) return fail(PCD_E_ARG, "null argument");
    if (n_tokens < 0) return fail(PCD_E_ARG, "negative token count");
    pcd_request r{fields, n_fields, candidates, n_candidates};
    return decide_start(&s, &r, 1, temperature, out, stream, tokens, n_tokens, p);
}

int pcd_finish(pcd_pending *p) { return decide_finish(p); }

int pcd_new_state(pcd_model *m, void *kv_buf, size_t kv_bytes, pcd_state **out) {
    if (!m || !kv_buf || !out) return fail(PCD_E_ARG, "null argument");
    if (misaligned(kv_buf)) return fail(PCD_E_ARG, "the KV buffer must be 16-byte aligned");
    if (kv_bytes < per_token_bytes(m)) return fail(PCD_E_CAP, "KV buffer smaller than one token");
    const int32_t cap = (int32_t)std::min<size_t>(kv_bytes / per_token_bytes(m), (size_t)m->cfg.max_seq);
    pcd_state *s = new (std::nothrow) pcd_state{STATE_MAGIC, m, kv_buf, 0, cap};
    if (!s) return fail(PCD_E_NOMEM, "state allocation");
    m->n_states++;
    *out = s;
    return PCD_OK;
}

int pcd_decide(pcd_state *s, const pcd_field *fields, int32_t n_fields, const pcd_candidate *candidates,
               int32_t n_candidates, float temperature, pcd_outputs *out, void *stream) {
    pcd_request r{fields, n_fields, candidates, n_candidates};
    return pcd_decide_many(&s, &r, 1, temperature, out, stream);
}

int pcd_decide_sequenced(pcd_state *s, const pcd_field *fields, int32_t n_fields, const pcd_candidate *candidates,
                         int32_t n_candidates, int32_t n_first, float temperature, pcd_outputs *out, void *stream) {
    if (!s || s->magic != STATE_MAGIC) return fail(PCD_E_STATE, "invalid state handle");
    if (!fields || !out) return fail(PCD_E_ARG, "null argument");
    if (n_first < 1 || n_first >= n_fields) return fail(PCD_E_ARG, "n_first must be in [1, n_fields)");
    if (out->readout_lse || out->gather_logit) return fail(PCD_E_ARG, "readout_lse / gather_logit must be NULL here");
    if (!out->cand_prob || !out->field_mass || !out->field_margin || !out->field_argmax)
        return fail(PCD_E_ARG, "null output array");
    pcd_model *m = s->m;
    // the tokens written for a label: its first spelling (the whole candidate without spellings)
    auto answer_len = [](const pcd_candidate &cd) {
        const int n = (cd.spell_len && cd.n_spellings > 0) ? cd.spell_len[0] : cd.n_tokens;
        return std::max(0, std::min(n, cd.n_tokens));
    };
    // Longest possible answer of the first fields: each scaffold plus its longest candidate.
    int64_t ans_max = 0, c1 = 0;
    for (int f = 0; f < n_first; ++f) {
        const pcd_field &fd = fields[f];
        if (fd.cand_offset < 0 || fd.n_cands < 0 || (int64_t)fd.cand_offset + fd.n_cands > n_candidates || !candidates)
            return fail(PCD_E_ARG, "field " + std::to_string(f) + ": candidates outside the candidate array");
        int lmax = 0;
        for (int k = 0; k < fd.n_cands; ++k) lmax = std::max(lmax, answer_len(candidates[fd.cand_offset + k]));
        ans_max += std::max(0, fd.n_scaffold) + lmax;
        c1 += fd.n_cands;
    }
    // Validate the whole request before any device work: the plan at the
    // longest extended prefix, the buffer's capacity and the pass size.
    const int64_t P_max = (int64_t)s->P + ans_max;
    if (P_max > s->cap || P_max > m->cfg.max_seq || ans_max > m->lim.max_prefill_tokens)
        return fail(PCD_E_CAP, "the first fields' answers may need " + std::to_string(ans_max) +
                                   " more tokens than the state's buffer or the model's limits allow");
    {
        const int32_t Pc = (int32_t)P_max;
        pcd_request all{fields, n_fields, candidates, n_candidates};
        Plan p;
        std::string err;
        const int rc = build_plan(m->cfg.vocab_size, m->cfg.max_seq, 1, &Pc, &all, p, err);
        if (rc != PCD_OK) return fail(rc, err);
    }
    pcd_request r1{fields, n_first, candidates, n_candidates};
    pcd_outputs o1 = *out;
    int rc = pcd_decide_many(&s, &r1, 1, temperature, &o1, stream);
    if (rc != PCD_OK) return rc;
    // write the answers in: each first field's scaffold, then its chosen candidate
    std::vector<int32_t> ans;
    ans.reserve((size_t)ans_max);
    for (int f = 0; f < n_first; ++f) {
        const pcd_field &fd = fields[f];
        ans.insert(ans.end(), fd.scaffold, fd.scaffold + fd.n_scaffold);
        const pcd_candidate &cd = candidates[fd.cand_offset + out->field_argmax[f]];
        ans.insert(ans.end(), cd.tokens, cd.tokens + answer_len(cd));
    }
    rc = pcd_extend(s, ans.data(), (int32_t)ans.size(), stream);
    if (rc != PCD_OK) return rc;
    pcd_request r2{fields + n_first, n_fields - n_first, candidates, n_candidates};
    pcd_outputs o2 = *out;
    o2.cand_prob += c1;
    if (o2.cand_logscore) o2.cand_logscore += c1;
    o2.field_mass += n_first;
    o2.field_margin += n_first;
    o2.field_argmax += n_first;
    return pcd_decide_many(&s, &r2, 1, temperature, &o2, stream);
}

int pcd_get_stats(const pcd_model *m, pcd_stats *out) {
    if (!m || !out) return fail(PCD_E_ARG, "null argument");
    const_cast<pcd_model *>(m)->settle_prefill();
    *out = m->stats;
    return PCD_OK;
}

int pcd_set_kernel_timing(pcd_model *m, int32_t enable) {
    if (!m) return fail(PCD_E_ARG, "null model");
    m->timing = enable != 0;
    m->tused = 0;
    for (int i = 0; i < PCD_KC_COUNT; ++i) {
        m->kc_ms[i] = 0.f;
        m->kc_n[i] = 0;
    }
    return PCD_OK;
}

int pcd_get_kernel_times(const pcd_model *m, float *total_ms, int64_t *launches) {
    if (!m || !total_ms || !launches) return fail(PCD_E_ARG, "null argument");
    for (int i = 0; i < PCD_KC_COUNT; ++i) {
        total_ms[i] = m->kc_ms[i];
        launches[i] = m->kc_n[i];
    }
    return PCD_OK;
}

void pcd_free_state(pcd_state *s) {
    if (!s || s->magic != STATE_MAGIC) return;
    s->magic = 0;
    s->m->n_states--;
    delete s;
}

void pcd_free_model(pcd_model *m) {
    if (!m) return;
    m->settle_prefill();
    for (auto &sl : m->slots)
        if (sl.busy && sl.ev[3]) (void)hipEventSynchronize(sl.ev[3]);  // an unfinished call's copies end first
    host_free(m, m->plan_host);
    release_scratch(m);
    for (auto &sl : m->slots) {
        host_free(m, sl.plan_host);
        host_free(m, sl.outs_host);
        for (auto &e : sl.ev)
            if (e) (void)hipEventDestroy(e);
    }
    for (auto &e : m->ev)
        if (e) (void)hipEventDestroy(e);
    for (auto &e : m->tev) (void)hipEventDestroy(e);
    delete m;
}

}  // extern "C"
