/*
 * Plain CPU float64 oracle for the TwoTower block-attention step and the
 * confidence-unmask SampleStep.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file or the library built from it; only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg do. It shares no code
 * with the HIP library.
 *
 * Source: "Nemotron-TwoTower: Diffusion Language Modeling with Pretrained
 * Autoregressive Context" (arXiv 2606.26493), section 2.1 "Bidirectional
 * attention", Eq. (1), and section 2.2 "Sampling", Algorithm 2; the
 * commit-time cache append follows Algorithm 1 of section 2.1, and the
 * masked negative log-likelihood is Eq. (4) of section 2.2.
 *
 * Every function is the plain definition, written out in double precision
 * over the exactly decoded inputs (a bf16 value widened to double is exact).
 * No blocking, no online softmax, no reordering beyond the definition.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F32 0
#define OR_BF16 1

/* Widen element i of a float32 or bf16 array to double. bf16 is the upper
 * half of an IEEE binary32, so widening is a 16-bit shift. */
static double ld(const void* base, size_t i, int dtype) {
    if (dtype == OR_F32) return (double)((const float*)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the parallel loops from now on (timing at one thread and at all of them). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Eq. (1): Attn(Q_b, [K_ctx(<b); K_den(b)], [V_ctx(<b); V_den(b)]).
 *
 * Attn is read as scaled-dot-product softmax attention with no mask: every
 * prefix key and every in-block key is visible to every query of the block
 * (bidirectional inside the block; the prefix precedes the block, so the
 * causal relation to past blocks needs no mask at this step).
 *
 * Layouts (dense, row-major):
 *   Q          [B][S][Hq][D]
 *   Kc, Vc     [num_pages][Hkv][page_size][D]; prefix token j of sequence b
 *              lives in page page_table[b*max_pages + j/page_size], slot
 *              j%page_size
 *   ctx_len    [B] prefix lengths
 *   Kd, Vd     [B][S][Hkv][D] in-block keys/values, or NULL (prefix only)
 *   rows       n_rows triples (b, h, s) selecting which outputs to compute
 *   O          [n_rows][D] double, LSE [n_rows] double (natural log)
 * Query head h reads KV head h / (Hq/Hkv). An empty key set gives O=0 and
 * LSE=-inf. Returns 0, or -1 on bad arguments.
 *
 * Out-of-range device data (not the paper's; the library's contract, so that
 * corrupt data never makes it read outside its arrays): a prefix length is
 * taken clamped into [0, len_cap] (len_cap = min(max_ctx_len, max_pages *
 * page_size)), and a page id clamped into [0, num_pages).
 */
int oracle_block_attn(int dtype, int B, int S, int Hq, int Hkv, int D, double scale,
                      const void* Q, const void* Kc, const void* Vc, int page_size, int num_pages,
                      const int32_t* page_table, int max_pages, const int32_t* ctx_len, int len_cap,
                      const void* Kd, const void* Vd, int n_rows, const int32_t* rows,
                      double* O, double* LSE) {
    if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || page_size <= 0 || num_pages <= 0 || len_cap < 0) return -1;
    if ((long long)len_cap > (long long)max_pages * page_size) return -1;
    const int G = Hq / Hkv;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int r = 0; r < n_rows; ++r) {
        const int b = rows[3 * r], h = rows[3 * r + 1], s = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= Hq || s < 0 || s >= S) { bad = 1; continue; }
        const int g = h / G;
        int L = ctx_len[b];
        if (L < 0) L = 0;
        if (L > len_cap) L = len_cap;
        const int n = L + (Kd ? S : 0);
        double* o = O + (size_t)r * D;
        for (int k = 0; k < D; ++k) o[k] = 0.0;
        if (n == 0) { LSE[r] = -INFINITY; continue; }
        double* sc = (double*)malloc(sizeof(double) * (size_t)n);
        size_t* off = (size_t*)malloc(sizeof(size_t) * (size_t)n);
        const void* ks[2] = {Kc, Kd};
        const void* vs[2] = {Vc, Vd};
        const size_t qoff = (((size_t)b * S + s) * Hq + h) * D;
        /* the concatenated key list: prefix tokens 0..L-1, then block tokens 0..S-1 */
        for (int j = 0; j < n; ++j) {
            int src;
            if (j < L) {
                int page = page_table[(size_t)b * max_pages + j / page_size];
                if (page < 0) page = 0;
                if (page >= num_pages) page = num_pages - 1;
                off[j] = (((size_t)page * Hkv + g) * page_size + j % page_size) * D;
                src = 0;
            } else {
                off[j] = (((size_t)b * S + (j - L)) * Hkv + g) * D;
                src = 1;
            }
            double dot = 0.0;
            for (int k = 0; k < D; ++k) dot += ld(Q, qoff + k, dtype) * ld(ks[src], off[j] + k, dtype);
            sc[j] = scale * dot;
        }
        double m = -INFINITY;
        for (int j = 0; j < n; ++j) if (sc[j] > m) m = sc[j];
        double Z = 0.0;
        for (int j = 0; j < n; ++j) Z += exp(sc[j] - m);
        for (int j = 0; j < n; ++j) {
            const double w = exp(sc[j] - m) / Z;
            const void* vsrc = vs[j < L ? 0 : 1];
            for (int k = 0; k < D; ++k) o[k] += w * ld(vsrc, off[j] + k, dtype);
        }
        LSE[r] = m + log(Z);
        free(sc);
        free(off);
    }
    return bad ? -1 : 0;
}

/*
 * Merge of P partial attentions over disjoint key sets into the attention
 * over their union. Attention over a concatenation (Eq. 1) is the
 * softmax-weighted combination of the parts:
 *   M = max_p lse_p,  w_p = exp(lse_p - M),
 *   O = sum_p w_p O_p / sum_p w_p,  lse = M + ln(sum_p w_p).
 * Parts with lse = -inf carry no keys and weigh 0; if every part is empty the
 * result is O=0, lse=-inf.
 * O_parts [P][n][D], lse_parts [P][n] -> O [n][D], lse [n].
 */
int oracle_lse_merge(int P, int n, int D, const double* O_parts, const double* lse_parts,
                     double* O, double* lse) {
    if (P < 1 || n < 0 || D < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < n; ++i) {
        double M = -INFINITY;
        for (int p = 0; p < P; ++p) if (lse_parts[(size_t)p * n + i] > M) M = lse_parts[(size_t)p * n + i];
        double* o = O + (size_t)i * D;
        for (int k = 0; k < D; ++k) o[k] = 0.0;
        if (M == -INFINITY) { lse[i] = -INFINITY; continue; }
        double W = 0.0;
        for (int p = 0; p < P; ++p) {
            const double l = lse_parts[(size_t)p * n + i];
            if (l == -INFINITY) continue;
            const double w = exp(l - M);
            W += w;
            for (int k = 0; k < D; ++k) o[k] += w * O_parts[((size_t)p * n + i) * D + k];
        }
        for (int k = 0; k < D; ++k) o[k] /= W;
        lse[i] = M + log(W);
    }
    return 0;
}

/* Categorical draw from softmax(x / temperature) over one row of V logits
 * starting at element base, by inverse transform sampling with uniform u:
 * the cumulative sum C_v = e_0 + ... + e_v of e_v = exp((x_v - max x)/temperature)
 * is compared with u * C_{V-1}. */
static void draw_token(int dtype, const void* logits, size_t base, int V, double temperature, float uf,
                       int32_t* tok, double* conf, double* margin) {
    double u = (double)uf;
    if (!(u > 0.0)) u = 0.0;
    if (u > 1.0) u = 1.0;
    double m = -INFINITY;
    for (int v = 0; v < V; ++v) {
        const double x = ld(logits, base + v, dtype);
        if (x > m) m = x;
    }
    if (m == -INFINITY) { *tok = 0; *conf = NAN; if (margin) *margin = 0.0; return; }
    double* e = (double*)malloc(sizeof(double) * (size_t)V);
    double Z = 0.0;
    for (int v = 0; v < V; ++v) {
        e[v] = exp((ld(logits, base + v, dtype) - m) / temperature);
        Z += e[v];
    }
    const double t = u * Z;
    double C = 0.0, lo = 0.0, hi = 0.0, e_a = 0.0, C_last = 0.0;
    int a = -1, last = -1;
    for (int v = 0; v < V; ++v) {
        const double Cn = C + e[v];
        if (e[v] > 0.0) { last = v; C_last = C; }
        if (a < 0 && Cn > t) { a = v; lo = C; hi = Cn; e_a = e[v]; }
        C = Cn;
    }
    if (a < 0) { a = last; lo = C_last; e_a = e[last]; hi = C_last + e_a; }
    free(e);
    *tok = a;
    *conf = e_a / Z;
    if (margin) *margin = fmin(t - lo, hi - t) / Z;
}

/*
 * One ConfidenceSample step of Algorithm 2 (single-block confidence
 * unmasking), for B independent blocks of S positions.
 *
 * For every masked position l (mask[b][l] != 0), over its V logits x:
 *   m = max_v x_v, a = the smallest v with x_v = m (the greedy prediction),
 *   conf = max_v softmax(x / temperature)_v = 1 / sum_v exp((x_v - m)/temperature).
 * Predictions with conf > gamma are committed. So that the block completes
 * within the steps left (steps_left = T - r + 1), at least
 * k_min = ceil(M / steps_left) positions are committed, M = number masked:
 * when fewer than k_min pass, the k_min masked positions of highest
 * confidence are committed instead (ties go to the lower position).
 * Committed positions take token a and leave the mask; all other positions,
 * and every already-unmasked position, are left untouched.
 *
 * Stochastic variant (the sampler's temperature argument, section 2.2
 * "Sampling"): when uniforms is not NULL, each masked row draws its token
 * from p = softmax(x / temperature) by inverting the cumulative distribution
 * in vocabulary order with the row's uniform u (clamped to [0, 1], NaN as 0):
 * a = the smallest v with p_0 + ... + p_v > u, or, when no v qualifies
 * (u = 1), the largest v with p_v > 0; its confidence is p_a. The commit rule
 * is unchanged. margin_out (may be NULL) receives, per masked row, the
 * distance of u from the nearer of the two cumulative values that bracket a,
 * so that a caller can tell draws that rounding could move to a neighbour.
 *
 * logits [B][S][V] (float32 or bf16, rows row_stride elements apart),
 * mask_in [B][S] (1 = masked), tokens_in [B][S] -> tokens_out, mask_out,
 * conf_out [B][S] (NaN where not masked), argmax_out [B][S] (the predicted
 * token: greedy or drawn; -1 where not masked), num_masked_out [B] (count
 * after the step).
 */
int oracle_conf_unmask(int dtype, int B, int S, int V, long long row_stride, const void* logits,
                       const uint8_t* mask_in, const int32_t* tokens_in, double gamma,
                       double temperature, int steps_left, const float* uniforms, int32_t* tokens_out,
                       uint8_t* mask_out, double* conf_out, int32_t* argmax_out, double* margin_out,
                       int32_t* num_masked_out) {
    if (B < 0 || S < 1 || V < 1 || steps_left < 1 || !(temperature > 0.0) || gamma != gamma) return -1;
    /* step 1: per masked row, the predicted token and its confidence */
#pragma omp parallel for schedule(dynamic, 1)
    for (int row = 0; row < B * S; ++row) {
        if (!mask_in[row]) { conf_out[row] = NAN; argmax_out[row] = -1; continue; }
        if (uniforms) {
            draw_token(dtype, logits, (size_t)row * (size_t)row_stride, V, temperature, uniforms[row],
                       &argmax_out[row], &conf_out[row], margin_out ? &margin_out[row] : NULL);
            continue;
        }
        const size_t base = (size_t)row * (size_t)row_stride;
        double m = -INFINITY;
        int a = 0;
        for (int v = 0; v < V; ++v) {
            const double x = ld(logits, base + v, dtype);
            if (x > m) { m = x; a = v; }
        }
        double Z = 0.0;
        for (int v = 0; v < V; ++v) Z += exp((ld(logits, base + v, dtype) - m) / temperature);
        conf_out[row] = 1.0 / Z;
        argmax_out[row] = a;
    }
    /* step 2: per block, the commit set */
    for (int b = 0; b < B; ++b) {
        const uint8_t* mk = mask_in + (size_t)b * S;
        const double* cf = conf_out + (size_t)b * S;
        int M = 0, n_pass = 0;
        for (int l = 0; l < S; ++l) {
            tokens_out[(size_t)b * S + l] = tokens_in[(size_t)b * S + l];
            mask_out[(size_t)b * S + l] = mk[l];
            if (mk[l]) { ++M; if (cf[l] > gamma) ++n_pass; }
        }
        const int k_min = (M + steps_left - 1) / steps_left;
        int committed = 0;
        if (n_pass >= k_min) {
            for (int l = 0; l < S; ++l)
                if (mk[l] && cf[l] > gamma) {
                    tokens_out[(size_t)b * S + l] = argmax_out[(size_t)b * S + l];
                    mask_out[(size_t)b * S + l] = 0;
                    ++committed;
                }
        } else {
            /* order the masked positions by (conf descending, position ascending) */
            int* ord = (int*)malloc(sizeof(int) * (size_t)S);
            int n = 0;
            for (int l = 0; l < S; ++l) if (mk[l]) ord[n++] = l;
            for (int i = 1; i < n; ++i) {
                const int cur = ord[i];
                int j = i - 1;
                while (j >= 0 && (cf[ord[j]] < cf[cur] || (cf[ord[j]] == cf[cur] && ord[j] > cur))) {
                    ord[j + 1] = ord[j];
                    --j;
                }
                ord[j + 1] = cur;
            }
            for (int i = 0; i < k_min; ++i) {
                const int l = ord[i];
                tokens_out[(size_t)b * S + l] = argmax_out[(size_t)b * S + l];
                mask_out[(size_t)b * S + l] = 0;
                ++committed;
            }
            free(ord);
        }
        num_masked_out[b] = M - committed;
    }
    return 0;
}

/* Commit-time KV append (Algorithm 1, section 2.1: after block b is committed
 * the context tower extends its KV cache, so the next block sees a prefix
 * longer by S). For every sequence b with L = max(ctx_len[b], 0), new row s
 * goes to prefix position L + s, which is slot (L + s) % page_size of page
 * page_table[b][(L + s) / page_size], and ctx_len[b] becomes L + S. A table
 * entry below 0 that a new position needs takes a page from the top of the
 * pool, in the order sequence first, then position. Elements are copied as
 * raw bytes (esz bytes each); Kn and Vn are dense [B][S][Hkv][D].
 * All or nothing: returns 1 if a sequence would pass max_pages * page_size
 * positions, 2 if the pool holds too few pages, 3 if a page id it would write
 * to is outside [0, num_pages), and then changes nothing; else 0. */
int oracle_kv_append(int esz, int B, int S, int Hkv, int D, int page_size, int num_pages, int max_pages,
                     unsigned char* Kc, unsigned char* Vc, int* page_table, int* ctx_len,
                     const unsigned char* Kn, const unsigned char* Vn, const int* pool, int* pool_count) {
    const long long cap = (long long)max_pages * page_size;
    for (int b = 0; b < B; ++b) {
        const int L = ctx_len[b] < 0 ? 0 : ctx_len[b];
        if ((long long)L + S > cap) return 1;
    }
    int needed = 0, bad = 0;
    for (int b = 0; b < B; ++b) {
        const int L = ctx_len[b] < 0 ? 0 : ctx_len[b];
        for (int p = L / page_size; p <= (L + S - 1) / page_size; ++p) {
            const int e = page_table[(size_t)b * max_pages + p];
            if (e < 0) ++needed;
            else if (e >= num_pages) bad = 1;
        }
    }
    const int count = pool_count && *pool_count > 0 ? *pool_count : 0;
    if (needed > count) return 2;
    for (int k = 0; k < needed; ++k) {
        const int pg = pool[count - 1 - k];
        if (pg < 0 || pg >= num_pages) bad = 1;
    }
    if (bad) return 3;
    int k = 0;
    for (int b = 0; b < B; ++b) {
        const int L = ctx_len[b] < 0 ? 0 : ctx_len[b];
        for (int p = L / page_size; p <= (L + S - 1) / page_size; ++p) {
            int* e = &page_table[(size_t)b * max_pages + p];
            if (*e < 0) *e = pool[count - 1 - k++];
        }
    }
    const size_t row = (size_t)D * esz;
    for (int b = 0; b < B; ++b) {
        const int L = ctx_len[b] < 0 ? 0 : ctx_len[b];
        for (int s = 0; s < S; ++s) {
            const int j = L + s;
            const int pidx = j / page_size;
            const int page = page_table[(size_t)b * max_pages + pidx];
            const int slot = j % page_size;
            for (int g = 0; g < Hkv; ++g) {
                const size_t dst = (((size_t)page * Hkv + g) * page_size + slot) * row;
                const size_t src = (((size_t)b * S + s) * Hkv + g) * row;
                memcpy(Kc + dst, Kn + src, row);
                memcpy(Vc + dst, Vn + src, row);
            }
        }
        ctx_len[b] = L + S;
    }
    if (needed > 0) *pool_count = count - needed;
    return 0;
}

/* L_MD, Eq. (4) of section 2.2: for each masked position (mask != 0) with
 * clean token y, -log p(y) = ln sum_v exp(x_v) - x_y (softmax at temperature
 * 1, written with the row max m as m + ln sum_v exp(x_v - m)); loss is their
 * mean over the masked positions, 0 when there are none. A target outside
 * [0, V) gives NaN. nll_out is written for masked rows only. Returns 0. */
int oracle_masked_nll(int dtype, int B, int S, int V, long long row_stride, const void* logits,
                      const int* targets, const unsigned char* mask, double* nll_out, double* loss_out,
                      int* count_out) {
    double sum = 0.0;
    int count = 0;
    for (long long row = 0; row < (long long)B * S; ++row) {
        if (!mask[row]) continue;
        const size_t base = (size_t)row * (size_t)row_stride;
        double m = -INFINITY;
        for (int v = 0; v < V; ++v) {
            const double x = ld(logits, base + v, dtype);
            if (x > m) m = x;
        }
        double Z = 0.0;
        for (int v = 0; v < V; ++v) Z += exp(ld(logits, base + v, dtype) - m);
        const int y = targets[row];
        const double nll = (y >= 0 && y < V) ? m + log(Z) - ld(logits, base + y, dtype) : NAN;
        nll_out[row] = nll;
        sum += nll;
        ++count;
    }
    *loss_out = count > 0 ? sum / count : 0.0;
    *count_out = count;
    return 0;
}
