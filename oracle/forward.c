/*
 * forward.c - plain CPU reference of the tree-masked verification forward,
 * the greedy step and the synthetic drafter of the speculation window.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.c). Every fp32 operation is one IEEE
 * binary32 operation rounded to nearest-even, in the order written; no FMA.
 *
 * Sources, cited by page title and section:
 *  [P1] "GPU-Resident Speculative Decoding for In-Browser LLM Inference with
 *       WebGPU": Small-Batch Verification Kernels (chunked attention with a
 *       merge pass, GQA heads sharing K/V); GPU-Resident Speculation Loop
 *       (node 0 is the last step's token, ancestors visible through a mask,
 *       acceptance, compaction, at most 8 drafted tokens); Implementation
 *       (fixed reduction order in matmuls and attention).
 * The model is Qwen2.5-shaped (RMSNorm, rotary positions, grouped-query
 * attention, SiLU-gated MLP); the pages do not print its equations, so the
 * readings below are the standard ones of that architecture, stated at each
 * function. Attention scores are scaled by 1/sqrt(head_dim).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* ---------------------------------------------------------------- exp */

/*
 * A deterministic exp, so that both implementations produce the same bits
 * (the pages require attention to reduce in a fixed order; a vendor exp would
 * not be reproducible). Method: Cody and Waite's additive range reduction
 * x = n ln2 + r with ln2 split into C1 (9 significant bits, so n*C1 is exact
 * for |n| <= 128) and C2 = fl(ln2 - C1); a degree-7 Taylor polynomial in r
 * evaluated by Horner's rule with separate multiplies and adds; scaling by
 * 2^n built from the exponent bits.
 */
float orc_det_exp(float x) {
    if (x > 88.0f) return INFINITY;
    if (x < -87.0f) return 0.0f;
    const float inv_ln2 = (float)(1.0 / 0.69314718055994530942);
    const float C1 = 355.0f / 512.0f;                                   /* 0.693359375 */
    const float C2 = (float)(0.69314718055994530942 - 355.0 / 512.0);  /* fl(ln2 - C1) */
    float n = nearbyintf(x * inv_ln2);
    float r = (x - n * C1) - n * C2;
    const float c[8] = {1.0f, 1.0f, (float)(1.0 / 2), (float)(1.0 / 6), (float)(1.0 / 24),
                        (float)(1.0 / 120), (float)(1.0 / 720), (float)(1.0 / 5040)};
    float p = c[7];
    for (int k = 6; k >= 0; k--) p = p * r + c[k];
    int ni = (int)n;
    uint32_t bits = (uint32_t)(ni + 127) << 23;
    float scale;
    memcpy(&scale, &bits, 4);
    return p * scale;
}

/* silu(g) = g / (1 + exp(-g)), with the exp above. */
float orc_silu(float g) { return g / (1.0f + orc_det_exp(-g)); }

/*
 * RMSNorm: ss = R16(x_k * x_k), ms = ss / H, rs = 1 / sqrt(ms + eps),
 * y_k = (x_k * rs) * w_k; sqrt and division correctly rounded.
 */
void orc_rmsnorm(const float* x, const float* w, int H, float eps, float* y) {
    float* sq = (float*)malloc(sizeof(float) * (size_t)H);
    for (int k = 0; k < H; k++) sq[k] = x[k] * x[k];
    float ss = orc_r16(sq, H);
    free(sq);
    float ms = ss / (float)H;
    float rs = 1.0f / sqrtf(ms + eps);
    for (int k = 0; k < H; k++) y[k] = (x[k] * rs) * w[k];
}

/*
 * Rotary table: for position p and pair i < hd/2, angle p * theta^(-2i/hd)
 * evaluated in double and rounded to fp32 (cos and sin).
 */
int orc_rope_table(float* cos_t, float* sin_t, int max_pos, int head_dim, double theta) {
    if (max_pos < 1 || head_dim < 2 || head_dim % 2) return -1;
    int half = head_dim / 2;
    for (int p = 0; p < max_pos; p++)
        for (int i = 0; i < half; i++) {
            double inv = pow(theta, -2.0 * i / head_dim);
            double a = (double)p * inv;
            cos_t[(size_t)p * half + i] = (float)cos(a);
            sin_t[(size_t)p * half + i] = (float)sin(a);
        }
    return 0;
}

/* Rotate-half RoPE on one head vector at position p. */
static void rope(float* x, int hd, const float* cos_t, const float* sin_t, int p) {
    int half = hd / 2;
    for (int i = 0; i < half; i++) {
        float c = cos_t[(size_t)p * half + i], s = sin_t[(size_t)p * half + i];
        float a = x[i], b = x[i + half];
        x[i] = a * c - b * s;
        x[i + half] = b * c + a * s;
    }
}

/* ---------------------------------------------------------------- blocks */

/* quantize rows then W4A8 linear: y [T][N]. A non-finite activation is
 * outside the quantiser's domain; the outputs are then NaN, so no comparison
 * can pass on them. */
static void qlinear(const float* x, int T, int K, const uint8_t* w, const uint16_t* s, int N, float* y) {
    int8_t* xq = (int8_t*)malloc((size_t)T * K);
    float* xs = (float*)malloc(sizeof(float) * (size_t)T);
    if (orc_quantize_act(x, T, K, xq, xs) != 0)
        for (int64_t i = 0; i < (int64_t)T * N; i++) y[i] = NAN;
    else
        orc_w4a8_linear(w, s, xq, xs, y, T, N, K);
    free(xq);
    free(xs);
}

/*
 * Attention of one query head over the visible sequence of a node, chunked on
 * logical positions ([P1, Small-Batch Verification Kernels]: chunks processed
 * separately, then merged). Reading: chunks of 256 logical positions; scores
 * s_j = R16_d(q_d * K_jd) * scale (scale = 1/sqrt(head_dim), exact for head
 * dims that are powers of 4, e.g. 0.125 for 64); per chunk the max
 * m_c, weights e_j = E(s_j - m_c), l_c = R16_j(e_j), o_cd = R16_j(e_j * V_jd);
 * merge: m = max m_c, w_c = E(m_c - m), l = R16_c(w_c * l_c),
 * o_d = R16_c(w_c * o_cd), out_d = o_d / l. The sums over j run over the
 * chunk's positions in logical order; over c in chunk order.
 */
#define ORC_CHUNK 256
static void attend(const float* q, const uint16_t* kc, const uint16_t* vc, int hd, const int* rows,
                   int len, float scale, float* out) {
    int nch = (len + ORC_CHUNK - 1) / ORC_CHUNK;
    float* mc = (float*)malloc(sizeof(float) * (size_t)nch);
    float* lc = (float*)malloc(sizeof(float) * (size_t)nch);
    float* oc = (float*)malloc(sizeof(float) * (size_t)nch * hd);
    float s[ORC_CHUNK], e[ORC_CHUNK], tmp[ORC_CHUNK];
    float* prod = (float*)malloc(sizeof(float) * (size_t)hd);
    for (int c = 0; c < nch; c++) {
        int j0 = c * ORC_CHUNK, cnt = len - j0 < ORC_CHUNK ? len - j0 : ORC_CHUNK;
        float m = -INFINITY;
        for (int jj = 0; jj < cnt; jj++) {
            const uint16_t* krow = kc + (size_t)rows[j0 + jj] * hd;
            for (int d = 0; d < hd; d++) prod[d] = q[d] * orc_f16_to_f32(krow[d]);
            s[jj] = orc_r16(prod, hd) * scale;
            if (s[jj] > m) m = s[jj];
        }
        for (int jj = 0; jj < cnt; jj++) e[jj] = orc_det_exp(s[jj] - m);
        mc[c] = m;
        lc[c] = orc_r16(e, cnt);
        for (int d = 0; d < hd; d++) {
            for (int jj = 0; jj < cnt; jj++) tmp[jj] = e[jj] * orc_f16_to_f32(vc[(size_t)rows[j0 + jj] * hd + d]);
            oc[(size_t)c * hd + d] = orc_r16(tmp, cnt);
        }
    }
    float m = -INFINITY;
    for (int c = 0; c < nch; c++)
        if (mc[c] > m) m = mc[c];
    float* wc = (float*)malloc(sizeof(float) * (size_t)nch);
    float* t2 = (float*)malloc(sizeof(float) * (size_t)nch);
    for (int c = 0; c < nch; c++) wc[c] = orc_det_exp(mc[c] - m);
    for (int c = 0; c < nch; c++) t2[c] = wc[c] * lc[c];
    float l = orc_r16(t2, nch);
    for (int d = 0; d < hd; d++) {
        for (int c = 0; c < nch; c++) t2[c] = wc[c] * oc[(size_t)c * hd + d];
        out[d] = orc_r16(t2, nch) / l;
    }
    free(mc); free(lc); free(oc); free(prod); free(wc); free(t2);
}

int orc_attention(const float* q, const uint16_t* kc, const uint16_t* vc, int hd, const int* rows,
                  int len, float* out) {
    if (hd < 1 || len < 1) return -1;
    attend(q, kc, vc, hd, rows, len, (float)(1.0 / sqrt((double)hd)), out);
    return 0;
}

static int tree_depths(const int32_t* parent, int N, int* depth) {
    if (N < 1 || parent[0] != -1) return -1;
    depth[0] = 0;
    for (int i = 1; i < N; i++) {
        if (parent[i] < 0 || parent[i] >= i) return -1;
        depth[i] = depth[parent[i]] + 1;
    }
    return 0;
}

/*
 * One forward pass over the tree ([P1, GPU-Resident Speculation Loop]): node
 * i sits at logical position L + depth(i) and physical KV row L + i; it
 * attends to the committed rows 0..L-1 and to the rows of its ancestors and
 * itself, in increasing depth, which is the sequence a single-token step at
 * that position would see after committing the path. Layer order:
 *   r = RMSNorm(h); q,k,v = W4A8(r); RoPE(q,k); K,V rows -> fp16 cache;
 *   a = attention; h = h + W4A8_o(a);
 *   r = RMSNorm(h); z = silu(W4A8_g(r)) * W4A8_u(r); h = h + W4A8_d(z);
 * final: logits = W4A8_lm(RMSNorm(h)). Embedding: the dequantised lm_head
 * row of the token (tied), exact: f32(scale) * code.
 */
int orc_forward(const orc_model* m, uint16_t* kc, uint16_t* vc, int cap, int L, int N,
                const int32_t* parent, const int32_t* token, float* logits) {
    const int H = m->hidden, nh = m->n_heads, nkv = m->n_kv_heads, hd = m->head_dim, I = m->inter;
    if (N < 1 || N > 64 || L < 0 || L + N > cap || nh % nkv || H % 32 || I % 32) return -1;
    int depth[64];
    if (tree_depths(parent, N, depth)) return -1;
    for (int i = 0; i < N; i++)
        if (L + depth[i] >= m->max_pos || token[i] < 0 || token[i] >= m->vocab) return -1;
    const int qd = nh * hd, kd = nkv * hd, G = H / 32;
    float* h = (float*)malloc(sizeof(float) * (size_t)N * H);
    float* r = (float*)malloc(sizeof(float) * (size_t)N * H);
    float* q = (float*)malloc(sizeof(float) * (size_t)N * qd);
    float* k = (float*)malloc(sizeof(float) * (size_t)N * kd);
    float* v = (float*)malloc(sizeof(float) * (size_t)N * kd);
    float* a = (float*)malloc(sizeof(float) * (size_t)N * qd);
    float* o = (float*)malloc(sizeof(float) * (size_t)N * H);
    float* g = (float*)malloc(sizeof(float) * (size_t)N * I);
    float* u = (float*)malloc(sizeof(float) * (size_t)N * I);
    int* rows = (int*)malloc(sizeof(int) * (size_t)(L + 64));

    for (int i = 0; i < N; i++) {
        const uint8_t* wrow = m->wlm + (size_t)token[i] * (H / 2);
        for (int kk = 0; kk < H; kk++) {
            uint8_t b = wrow[kk / 2];
            int code = ((kk & 1) ? (b >> 4) : (b & 15)) - 8;
            h[(size_t)i * H + kk] = orc_f16_to_f32(m->slm[(size_t)token[i] * G + kk / 32]) * (float)code;
        }
    }
    const size_t plane = (size_t)cap * hd;
    /* 1/sqrt(head_dim), exact when head_dim is a power of 4 (64 -> 0.125) */
    const float score_scale = (float)(1.0 / sqrt((double)hd));
    for (int l = 0; l < m->n_layers; l++) {
        for (int i = 0; i < N; i++) orc_rmsnorm(h + (size_t)i * H, m->norm_attn[l], H, m->eps, r + (size_t)i * H);
        qlinear(r, N, H, m->wq[l], m->sq[l], qd, q);
        qlinear(r, N, H, m->wk[l], m->sk[l], kd, k);
        qlinear(r, N, H, m->wv[l], m->sv[l], kd, v);
        for (int i = 0; i < N; i++) {
            int p = L + depth[i];
            for (int hh = 0; hh < nh; hh++) rope(q + (size_t)i * qd + hh * hd, hd, m->rope_cos, m->rope_sin, p);
            for (int hh = 0; hh < nkv; hh++) {
                rope(k + (size_t)i * kd + hh * hd, hd, m->rope_cos, m->rope_sin, p);
                uint16_t* krow = kc + ((size_t)l * nkv + hh) * plane + (size_t)(L + i) * hd;
                uint16_t* vrow = vc + ((size_t)l * nkv + hh) * plane + (size_t)(L + i) * hd;
                for (int d = 0; d < hd; d++) {
                    krow[d] = orc_f32_to_f16(k[(size_t)i * kd + hh * hd + d]);
                    vrow[d] = orc_f32_to_f16(v[(size_t)i * kd + hh * hd + d]);
                }
            }
        }
        for (int i = 0; i < N; i++) {
            int len = 0;
            for (int j = 0; j < L; j++) rows[len++] = j;
            int chain[64], c = 0;
            for (int x = i; x != -1; x = parent[x]) chain[c++] = x;
            while (c > 0) rows[len++] = L + chain[--c];
            for (int hh = 0; hh < nh; hh++) {
                int g_kv = hh / (nh / nkv);
                attend(q + (size_t)i * qd + hh * hd, kc + ((size_t)l * nkv + g_kv) * plane,
                       vc + ((size_t)l * nkv + g_kv) * plane, hd, rows, len, score_scale,
                       a + (size_t)i * qd + hh * hd);
            }
        }
        qlinear(a, N, qd, m->wo[l], m->so[l], H, o);
        for (size_t x = 0; x < (size_t)N * H; x++) h[x] = h[x] + o[x];
        for (int i = 0; i < N; i++) orc_rmsnorm(h + (size_t)i * H, m->norm_mlp[l], H, m->eps, r + (size_t)i * H);
        qlinear(r, N, H, m->wg[l], m->sg[l], I, g);
        qlinear(r, N, H, m->wu[l], m->su[l], I, u);
        for (size_t x = 0; x < (size_t)N * I; x++) g[x] = orc_silu(g[x]) * u[x];
        qlinear(g, N, I, m->wd[l], m->sd[l], H, o);
        for (size_t x = 0; x < (size_t)N * H; x++) h[x] = h[x] + o[x];
    }
    for (int i = 0; i < N; i++) orc_rmsnorm(h + (size_t)i * H, m->norm_final, H, m->eps, r + (size_t)i * H);
    qlinear(r, N, H, m->wlm, m->slm, m->vocab, logits);
    free(h); free(r); free(q); free(k); free(v); free(a); free(o); free(g); free(u); free(rows);
    return 0;
}

int orc_tree_step(const orc_model* m, uint16_t* kc, uint16_t* vc, int cap, int* L, int N,
                  const int32_t* parent, const int32_t* token, float* logits, int32_t* amax,
                  int32_t* path, int32_t* bonus) {
    float* lg = logits ? logits : (float*)malloc(sizeof(float) * (size_t)N * m->vocab);
    int rc = orc_forward(m, kc, vc, cap, *L, N, parent, token, lg);
    if (rc == 0) rc = orc_argmax(lg, N, m->vocab, amax);
    int mm = rc == 0 ? orc_tree_accept(parent, token, amax, N, path, bonus) : -1;
    if (mm >= 0) {
        orc_kv_compact(kc, m->n_layers, m->n_kv_heads, cap, m->head_dim, *L, path, mm);
        orc_kv_compact(vc, m->n_layers, m->n_kv_heads, cap, m->head_dim, *L, path, mm);
        *L += mm + 1;
    }
    if (!logits) free(lg);
    return mm;
}

/*
 * Synthetic drafter standing in for the context-mixing drafter
 * ([P1, GPU-Resident Speculation Loop]: the drafter extends a candidate by
 * at most 8 tokens). Reading: for a tree of `width` nodes, node 0 is the root
 * carrying root_token; nodes 1..D, D = min(width-1, 8), form a chain (parent
 * k-1); the remaining nodes attach round-robin to nodes 0..D-1. Chain node k
 * (logical position L+k) copies the reference token greedy[L+k] when its
 * draw is below `threshold`, otherwise takes a different token; extra nodes
 * take draw mod vocab. best_match = D.
 */
int orc_draft_tree(int width, int L, int32_t root_token, const int32_t* greedy, int stream_len,
                   const uint32_t* draws, uint32_t threshold, int vocab, int32_t* parent,
                   int32_t* token, int* best_match) {
    if (width < 1 || width > 16 || vocab < 2) return -1;
    int D = width - 1 < 8 ? width - 1 : 8;
    parent[0] = -1;
    token[0] = root_token;
    for (int k = 1; k <= D; k++) {
        parent[k] = k - 1;
        uint32_t d = draws[k];
        if (L + k < stream_len) {
            int32_t ref = greedy[L + k];
            token[k] = d < threshold ? ref : (int32_t)(((uint32_t)ref + 1u + d % (uint32_t)(vocab - 1)) % (uint32_t)vocab);
        } else {
            token[k] = (int32_t)(d % (uint32_t)vocab);
        }
    }
    for (int e = D + 1; e < width; e++) {
        parent[e] = (e - D - 1) % D;
        token[e] = (int32_t)(draws[e] % (uint32_t)vocab);
    }
    *best_match = D;
    return 0;
}
