/*
 * drafter.c - plain CPU reference of the context-mixing drafter.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h). It shares no code with the HIP
 * implementation.
 *
 * Source: [P1] "GPU-Resident Speculative Decoding for In-Browser LLM
 * Inference with WebGPU", Design, Draft-Free Drafting From Web Context: find
 * earlier occurrences of the current suffix at every order up to 8, blend the
 * continuations of the best positions into a weighted trie, using a fixed
 * function of the match length as the weight, and emit the most probable
 * prefix-closed set of nodes as the next tree.
 *
 * Readings where the page leaves a step open (all integer, so the result is
 * exact):
 *  - The stream is s[0..n): the committed tokens followed by the pending root
 *    s[n-1]. The current suffix ends at the root.
 *  - Position p in [0, n-2] matches with length l(p), the largest l in
 *    [0, min(max_order, p + 1)] with s[p - i] == s[n - 1 - i] for all i < l.
 *  - The candidates are the `cands` positions with l(p) >= 1 that are largest
 *    by (l(p), p): longer matches first, then the most recent.
 *  - The continuation of candidate p is s[p+1 .. min(p + depth, n - 1)].
 *  - The trie hangs under the root. Candidates are inserted in candidate
 *    order; a node is created when a path first reaches it, and its weight is
 *    the sum of weight[l(p)] over the candidates whose continuation passes
 *    through it.
 *  - The tree keeps the width - 1 trie nodes that are largest by (weight,
 *    then smaller depth, then earlier creation). A child never outweighs its
 *    parent, and on equal weight the parent is shallower, so the kept set is
 *    prefix-closed.
 *  - Node 0 is the root (parent -1). The kept nodes follow in order of depth,
 *    then of their rank in the selection, so every parent precedes its
 *    children.
 *  - The best match of the step is l of the first candidate (0 if none).
 */
#include "oracle.h"

#include <stdlib.h>

#define ORC_MAX_CANDS 32
#define ORC_MAX_DEPTH 8
#define ORC_MAX_NODES (ORC_MAX_CANDS * ORC_MAX_DEPTH)

typedef struct {
    int parent;      /* trie node id, -1 for children of the root */
    int32_t token;
    int depth;       /* 0 for a child of the root */
    uint32_t weight;
} trie_node;

int orc_cm_draft(const int32_t* s, int n, int max_order, int cands, int depth, const uint32_t* weight,
                 int width, int32_t* parent, int32_t* token, int32_t* best_match) {
    if (!s || n < 1 || max_order < 1 || max_order > 8 || cands < 1 || cands > ORC_MAX_CANDS || depth < 1 ||
        depth > ORC_MAX_DEPTH || !weight || width < 1 || width > 16 || !parent || !token || !best_match)
        return -1;
    for (int l = 1; l <= 8; l++)
        if (weight[l] < 1u || weight[l] > (1u << 24)) return -1;

    /* match lengths and candidate selection (a plain selection sort) */
    int* len = (int*)calloc((size_t)n, sizeof(int));
    if (!len) return -1;
    for (int p = 0; p + 1 < n; p++) {
        int l = 0;
        while (l < max_order && l <= p && s[p - l] == s[n - 1 - l]) l++;
        len[p] = l;
    }
    int cand[ORC_MAX_CANDS];
    int nc = 0;
    char* taken = (char*)calloc((size_t)n, 1);
    if (!taken) {
        free(len);
        return -1;
    }
    while (nc < cands) {
        int best = -1;
        for (int p = 0; p + 1 < n; p++) {
            if (taken[p] || len[p] < 1) continue;
            if (best < 0 || len[p] > len[best] || (len[p] == len[best] && p > best)) best = p;
        }
        if (best < 0) break;
        taken[best] = 1;
        cand[nc++] = best;
    }
    free(taken);
    *best_match = nc ? len[cand[0]] : 0;

    /* weighted trie, nodes numbered in creation order */
    trie_node node[ORC_MAX_NODES];
    int nn = 0;
    for (int c = 0; c < nc; c++) {
        const int p = cand[c];
        const uint32_t w = weight[len[p]];
        int at = -1; /* current trie node, -1 = root */
        for (int d = 0; d < depth && p + 1 + d <= n - 1; d++) {
            const int32_t tok = s[p + 1 + d];
            int child = -1;
            for (int i = 0; i < nn; i++)
                if (node[i].parent == at && node[i].token == tok) {
                    child = i;
                    break;
                }
            if (child < 0) {
                child = nn++;
                node[child].parent = at;
                node[child].token = tok;
                node[child].depth = d;
                node[child].weight = 0;
            }
            node[child].weight += w;
            at = child;
        }
    }
    free(len);

    /* keep the width - 1 largest by (weight, smaller depth, earlier creation) */
    int keep[16];
    int nk = 0;
    char chosen[ORC_MAX_NODES] = {0};
    while (nk < width - 1) {
        int best = -1;
        for (int i = 0; i < nn; i++) {
            if (chosen[i]) continue;
            if (best < 0 || node[i].weight > node[best].weight ||
                (node[i].weight == node[best].weight && node[i].depth < node[best].depth))
                best = i; /* equal weight and depth: the earlier node stays */
        }
        if (best < 0) break;
        chosen[best] = 1;
        keep[nk++] = best;
    }

    /* output: root, then the kept nodes by depth, then by selection rank */
    int out_of[ORC_MAX_NODES];
    for (int i = 0; i < nn; i++) out_of[i] = -1;
    parent[0] = -1;
    token[0] = s[n - 1];
    int no = 1;
    for (int d = 0; d < depth; d++)
        for (int r = 0; r < nk; r++) {
            const trie_node* t = &node[keep[r]];
            if (t->depth != d) continue;
            out_of[keep[r]] = no;
            parent[no] = t->parent < 0 ? 0 : out_of[t->parent];
            token[no] = t->token;
            if (parent[no] < 0) return -1; /* unreachable: the kept set is prefix-closed */
            no++;
        }
    return no;
}
