// Host-side plan of one batched branch pass (internal header).
//
// The plan lays out every branch token of a decide call: per request, per
// field, the field's scaffold tokens, then its trie continuation tokens.  A
// trie continuation token exists for every non-root trie node that has two
// or more candidates below it: the labels still agree up to that node, so
// the row is extended one token down the shared branch, teacher-forced,
// in the same pass ("Parallel Constrained Decoding from Scratch", "When one
// token is not enough").  Readout rows are the scaffold's last token (the
// trie root) and every continuation token.
//
// Spellings ("Parallel Constrained Decoding from Scratch", "Small models
// quote their booleans"): a label may be a set of token paths; the trie is
// built over every spelling of every label of the field, and a spelling is
// followed until no other spelling shares its tokens.  Scoring modes that
// score a label to its end (EXACT, MEAN) make every node some spelling
// continues from a continuation token and a readout.
//
// Canonical numbering: spellings are inserted in declaration order (label by
// label, then in the order given), so a node's children are ordered by the
// first spelling that reaches them; nodes are numbered breadth-first.  The
// test suite checks these arrays against an independent CPU implementation
// element by element.
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/pcd.h"

namespace pcd {

struct Plan {
    int32_t n_req = 0;
    // per branch token
    std::vector<int32_t> tok, pos, req, field;
    std::vector<int32_t> fs;   // index of the first scaffold token of its field
    std::vector<int32_t> nsc;  // scaffold length of its field
    std::vector<int32_t> par;  // branch index of its trie parent; -1 for scaffold tokens and depth-1 nodes
    std::vector<int32_t> anc_off, anc;  // visible branch tokens (debug view; the device walks fs/nsc/par)
    // per readout row
    std::vector<int32_t> ro_tok, ro_field, g_off;
    // per gather
    std::vector<int32_t> g_tok, g_ro;
    // per field
    std::vector<int32_t> f_ro_root, f_cand_off, f_mode;
    // per candidate: its spellings
    std::vector<int32_t> c_spell_off;
    // per spelling: the gathers it is scored on, in depth order
    std::vector<int32_t> s_path_off, s_path;
    // per request: first branch token / readout / gather / field / candidate (size n_req + 1)
    std::vector<int32_t> r_tok, r_ro, r_g, r_field, r_cand;
    std::vector<int32_t> prefix_len;  // per request
    int32_t max_depth = 0;           // deepest trie continuation token
};

// Validates and lays out the requests.  Returns PCD_OK or a PCD_E_* code with
// a message in err.  The visibility lists anc_off/anc (a debug view) are
// filled only when with_anc is set.
int build_plan(int32_t vocab_size, int32_t max_seq, int32_t n_req, const int32_t *prefix_lens,
               const pcd_request *reqs, Plan &out, std::string &err, bool with_anc = false);

}  // namespace pcd
