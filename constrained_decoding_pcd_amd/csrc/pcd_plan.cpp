// Host-side plan builder: validation, canonical trie per field, branch-token
// layout, readouts, gathers and candidate paths.  Pure C++, no device code.
#include "pcd_plan.h"

#include <algorithm>
#include <cstdio>

namespace pcd {

namespace {

struct Node {
    int32_t token = -1, parent = -1, depth = 0, n_cands = 0;
    std::vector<int32_t> kids;  // in the order the first candidate reached them
};

std::string fmt(const char *f, long a = 0, long b = 0, long c = 0) {
    char buf[256];
    std::snprintf(buf, sizeof buf, f, a, b, c);
    return buf;
}

// One spelling of a label, as a view into the candidate's token array.
struct Spell {
    const int32_t *tok;
    int32_t n;
};

// Field validation in a fixed order: scoring mode, empty scaffold, candidate
// count, spelling layout, spelling count, token range, empty spelling,
// duplicate, proper prefix.  The limits follow the pages' schema rules
// ("Parallel Constrained Decoding: A Technical Reference", "At a glance" and
// the schema checklist: 2..255 choices).  On success `sp` holds the field's
// spellings, label by label.
int validate(const pcd_field &f, const pcd_candidate *cands, int32_t V, std::vector<Spell> &sp,
             std::vector<int32_t> &n_spell, std::string &err) {
    if (f.score_mode < PCD_SCORE_PATH || f.score_mode > PCD_SCORE_MEAN) {
        err = fmt("unknown scoring mode %ld", f.score_mode);
        return PCD_E_ARG;
    }
    if (f.n_scaffold <= 0 || !f.scaffold) { err = "empty scaffold"; return PCD_E_EMPTY; }
    if (f.n_cands < 2 || f.n_cands > PCD_MAX_CANDIDATES) {
        err = fmt("%ld candidates (allowed 2..%ld)", f.n_cands, PCD_MAX_CANDIDATES);
        return PCD_E_NCAND;
    }
    sp.clear();
    n_spell.clear();
    sp.reserve(f.n_cands);
    n_spell.reserve(f.n_cands);
    for (int c = 0; c < f.n_cands; ++c) {
        const pcd_candidate &k = cands[c];
        if (k.n_tokens < 0 || (k.n_tokens > 0 && !k.tokens)) { err = "null candidate tokens"; return PCD_E_ARG; }
        if (!k.spell_len) {
            sp.push_back({k.tokens, k.n_tokens});
            n_spell.push_back(1);
            continue;
        }
        if (k.n_spellings <= 0) { err = fmt("candidate %ld: a label without spellings", c); return PCD_E_EMPTY; }
        if (k.n_spellings > PCD_MAX_SPELLINGS) {
            err = fmt("%ld spellings (allowed up to %ld)", k.n_spellings, PCD_MAX_SPELLINGS);
            return PCD_E_NCAND;
        }
        int64_t off = 0;
        for (int j = 0; j < k.n_spellings; ++j) {
            if (k.spell_len[j] < 0 || off + k.spell_len[j] > k.n_tokens) {
                err = fmt("candidate %ld: spelling lengths do not add up to its %ld tokens", c, k.n_tokens);
                return PCD_E_ARG;
            }
            sp.push_back({k.tokens + off, k.spell_len[j]});
            off += k.spell_len[j];
        }
        if (off != k.n_tokens) {
            err = fmt("candidate %ld: spelling lengths do not add up to its %ld tokens", c, k.n_tokens);
            return PCD_E_ARG;
        }
        n_spell.push_back(k.n_spellings);
    }
    if ((int64_t)sp.size() > PCD_MAX_SPELLINGS) {
        err = fmt("%ld spellings (allowed up to %ld)", (long)sp.size(), PCD_MAX_SPELLINGS);
        return PCD_E_NCAND;
    }
    for (int i = 0; i < f.n_scaffold; ++i)
        if (f.scaffold[i] < 0 || f.scaffold[i] >= V) {
            err = fmt("token id %ld outside [0, %ld)", f.scaffold[i], V);
            return PCD_E_TOKEN;
        }
    for (const Spell &s : sp)
        for (int i = 0; i < s.n; ++i)
            if (s.tok[i] < 0 || s.tok[i] >= V) {
                err = fmt("token id %ld outside [0, %ld)", s.tok[i], V);
                return PCD_E_TOKEN;
            }
    for (const Spell &s : sp)
        if (s.n <= 0) { err = "empty candidate"; return PCD_E_EMPTY; }
    // spellings in lexicographic order: a duplicate sits next to its twin, and a
    // proper prefix right before some extension of it
    std::vector<int32_t> ord(sp.size());
    for (size_t i = 0; i < ord.size(); ++i) ord[i] = (int32_t)i;
    auto less = [&](int32_t x, int32_t y) {
        return std::lexicographical_compare(sp[x].tok, sp[x].tok + sp[x].n, sp[y].tok, sp[y].tok + sp[y].n);
    };
    std::sort(ord.begin(), ord.end(), less);
    for (size_t i = 1; i < ord.size(); ++i) {
        const Spell &a = sp[ord[i - 1]], &b = sp[ord[i]];
        if (a.n == b.n && std::equal(a.tok, a.tok + a.n, b.tok)) {
            err = fmt("duplicate candidate (%ld tokens)", (long)a.n);
            return PCD_E_DUP;
        }
    }
    for (size_t i = 1; i < ord.size(); ++i) {
        const Spell &a = sp[ord[i - 1]], &b = sp[ord[i]];
        if (a.n < b.n && std::equal(a.tok, a.tok + a.n, b.tok)) {
            err = fmt("a candidate of %ld tokens is a proper prefix of one of %ld", (long)a.n, (long)b.n);
            return PCD_E_PREFIX;
        }
    }
    return PCD_OK;
}

// Trie over the spellings with nodes renumbered breadth-first (node 0 = root).
std::vector<Node> make_trie(const std::vector<Spell> &sp) {
    std::vector<Node> t(1);
    for (const Spell &s : sp) {
        int cur = 0;
        t[0].n_cands++;
        for (int i = 0; i < s.n; ++i) {
            int32_t tk = s.tok[i];
            int nxt = -1;
            for (int k : t[cur].kids)
                if (t[k].token == tk) { nxt = k; break; }
            if (nxt < 0) {
                Node nd;
                nd.token = tk;
                nd.parent = cur;
                nd.depth = t[cur].depth + 1;
                t.push_back(nd);
                nxt = (int)t.size() - 1;
                t[cur].kids.push_back(nxt);
            }
            cur = nxt;
            t[cur].n_cands++;
        }
    }
    std::vector<int> order{0};
    for (size_t i = 0; i < order.size(); ++i)
        for (int k : t[order[i]].kids) order.push_back(k);
    std::vector<int> newid(t.size());
    for (size_t i = 0; i < order.size(); ++i) newid[order[i]] = (int)i;
    std::vector<Node> out(t.size());
    for (size_t i = 0; i < order.size(); ++i) {
        Node nd = t[order[i]];
        nd.parent = nd.parent < 0 ? -1 : newid[nd.parent];
        for (int &k : nd.kids) k = newid[k];
        out[i] = nd;
    }
    return out;
}

}  // namespace

int build_plan(int32_t V, int32_t max_seq, int32_t n_req, const int32_t *prefix_lens, const pcd_request *reqs,
               Plan &p, std::string &err, bool with_anc) {
    p = Plan();
    if (n_req <= 0 || !prefix_lens || !reqs) { err = "no requests"; return PCD_E_ARG; }
    p.n_req = n_req;
    p.anc_off.push_back(0);
    p.g_off.push_back(0);
    p.f_cand_off.push_back(0);
    p.c_spell_off.push_back(0);
    p.s_path_off.push_back(0);
    int32_t gf = 0;
    for (int r = 0; r < n_req; ++r) {
        const pcd_request &rq = reqs[r];
        const int32_t P = prefix_lens[r];
        if (P <= 0) { err = fmt("request %ld has an empty prefix", r); return PCD_E_ARG; }
        if (rq.n_fields <= 0 || !rq.fields || rq.n_candidates < 0 || (rq.n_candidates > 0 && !rq.candidates)) {
            err = fmt("request %ld: no fields or null arrays", r);
            return PCD_E_ARG;
        }
        p.prefix_len.push_back(P);
        p.r_tok.push_back((int32_t)p.tok.size());
        p.r_ro.push_back((int32_t)p.ro_tok.size());
        p.r_g.push_back((int32_t)p.g_tok.size());
        p.r_field.push_back(gf);
        p.r_cand.push_back(p.f_cand_off.back());
        for (int fi = 0; fi < rq.n_fields; ++fi, ++gf) {
            const pcd_field &f = rq.fields[fi];
            if (f.cand_offset < 0 || f.n_cands < 0 || (int64_t)f.cand_offset + f.n_cands > rq.n_candidates) {
                err = fmt("request %ld field %ld: candidate range outside the candidate array", r, fi);
                return PCD_E_ARG;
            }
            const pcd_candidate *cands = rq.candidates + f.cand_offset;
            std::vector<Spell> sp;
            std::vector<int32_t> n_spell;
            int rc = validate(f, cands, V, sp, n_spell, err);
            if (rc != PCD_OK) {
                err = fmt("request %ld field %ld: ", r, fi) + err;
                return rc;
            }
            // scoring to the end: every node a spelling continues from is read out
            const bool to_end = f.score_mode == PCD_SCORE_EXACT || f.score_mode == PCD_SCORE_MEAN;
            std::vector<Node> t = make_trie(sp);
            auto is_ro = [&](size_t v) { return v == 0 || (to_end ? !t[v].kids.empty() : t[v].n_cands >= 2); };
            const int32_t ns = f.n_scaffold;
            if (P + ns - 1 >= max_seq) {
                err = fmt("position %ld reaches max_seq %ld", P + ns - 1, max_seq);
                return PCD_E_CAP;
            }
            const int32_t base = (int32_t)p.tok.size();
            // scaffold tokens
            for (int j = 0; j < ns; ++j) {
                p.tok.push_back(f.scaffold[j]);
                p.pos.push_back(P + j);
                p.req.push_back(r);
                p.field.push_back(gf);
                p.fs.push_back(base);
                p.nsc.push_back(ns);
                p.par.push_back(-1);
                if (with_anc) {
                    for (int a = base; a <= base + j; ++a) p.anc.push_back(a);
                    p.anc_off.push_back((int32_t)p.anc.size());
                }
            }
            // continuation tokens: non-root readout nodes, BFS order
            std::vector<int32_t> branch_of(t.size(), -1), ro_of(t.size(), -1);
            branch_of[0] = base + ns - 1;
            for (size_t v = 1; v < t.size(); ++v) {
                if (!is_ro(v)) continue;
                const int32_t bi = (int32_t)p.tok.size();
                branch_of[v] = bi;
                const int32_t posv = P + ns + t[v].depth - 1;
                if (posv >= max_seq) {
                    err = fmt("position %ld reaches max_seq %ld", posv, max_seq);
                    return PCD_E_CAP;
                }
                p.max_depth = std::max(p.max_depth, t[v].depth);
                p.tok.push_back(t[v].token);
                p.pos.push_back(posv);
                p.req.push_back(r);
                p.field.push_back(gf);
                p.fs.push_back(base);
                p.nsc.push_back(ns);
                p.par.push_back(t[v].parent == 0 ? -1 : branch_of[t[v].parent]);
                if (with_anc) {
                    std::vector<int32_t> chain;
                    for (int a = (int)v; a != 0; a = t[a].parent) chain.push_back(branch_of[a]);
                    for (int a = base; a < base + ns; ++a) p.anc.push_back(a);
                    std::sort(chain.begin(), chain.end());
                    p.anc.insert(p.anc.end(), chain.begin(), chain.end());
                    p.anc_off.push_back((int32_t)p.anc.size());
                }
            }
            // readouts (root first, then BFS) and the child tokens gathered at each
            std::vector<int32_t> g_first(t.size(), -1);
            for (size_t v = 0; v < t.size(); ++v) {
                if (!is_ro(v)) continue;
                const int32_t ri = (int32_t)p.ro_tok.size();
                if (v == 0) p.f_ro_root.push_back(ri);
                ro_of[v] = ri;
                p.ro_tok.push_back(branch_of[v]);
                p.ro_field.push_back(gf);
                g_first[v] = (int32_t)p.g_tok.size();
                for (int k : t[v].kids) {
                    p.g_tok.push_back(t[k].token);
                    p.g_ro.push_back(ri);
                }
                p.g_off.push_back((int32_t)p.g_tok.size());
            }
            // each spelling is scored on its edges down to the first node no other
            // spelling reaches, or on all of them when scoring to the end
            for (const Spell &s : sp) {
                int cur = 0;
                for (int i = 0; i < s.n; ++i) {
                    const int32_t tk = s.tok[i];
                    int slot = 0, nxt = -1;
                    for (; slot < (int)t[cur].kids.size(); ++slot)
                        if (t[t[cur].kids[slot]].token == tk) { nxt = t[cur].kids[slot]; break; }
                    p.s_path.push_back(g_first[cur] + slot);
                    if (t[nxt].n_cands == 1 && !to_end) break;
                    cur = nxt;
                }
                p.s_path_off.push_back((int32_t)p.s_path.size());
            }
            for (int c = 0; c < f.n_cands; ++c) p.c_spell_off.push_back(p.c_spell_off.back() + n_spell[c]);
            p.f_cand_off.push_back(p.f_cand_off.back() + f.n_cands);
            p.f_mode.push_back(f.score_mode);
        }
    }
    p.r_tok.push_back((int32_t)p.tok.size());
    p.r_ro.push_back((int32_t)p.ro_tok.size());
    p.r_g.push_back((int32_t)p.g_tok.size());
    p.r_field.push_back(gf);
    p.r_cand.push_back(p.f_cand_off.back());
    return PCD_OK;
}

}  // namespace pcd
