/*
 * CPU oracle for the fused top-k Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes (all arithmetic in float64 unless stated):
 *  - Routing: the router yields a weight distribution over the experts, the
 *    k highest are kept and the experts' outputs are summed with those
 *    weights (FusedMoE vs MegaMoE post, section 2 and the "Top-k Gating" row
 *    of the comparison table in section 5).  Selection is on the float32
 *    logits (softmax is monotone), repeatedly taking the largest unselected
 *    logit with the lowest index winning ties; weights are the softmax
 *    restricted to the selected logits (renormalise=1), or the full softmax
 *    entries of the selected experts (renormalise=0).
 *  - Alignment: each (token, slot) pair p = t*k + j is sorted by expert,
 *    stably in p, every expert's run padded to a multiple of block_m with the
 *    sentinel P, giving the index system that maps every position to its
 *    expert (same post, section 3.1, steps 1-2).
 *  - Expert FFN per pair (same post, section 3.1 step 3; the routed-row
 *    product A[M,K] x B[K,N] of the MoE kernel engineering post, Eq. 1):
 *    g = W1[e][0:I] x, u = W1[e][I:2I] x, a = silu(g) * u, y = W2[e] a.
 *  - Combine: out[t] = sum_j w[t,j] * y[t*k+j], j ascending (section 3.1,
 *    step 4).
 *  - FP8 (MoE kernel engineering post, "FP8 backend routing" section: one
 *    scale per tensor): x and the weights are e4m3 codes times their float32
 *    scale; the intermediate a is quantised with one dynamic per-tensor
 *    scale, then dequantised before the down projection: s = amax/448 with
 *    amax the largest |a| of this float64 intermediate over every pair, and
 *    code = e4m3(f32(a) / s) with a float32 division.  The pages leave the
 *    intermediate's precision open; the oracle keeps its own float64 value
 *    up to that one decision.
 *
 * Codecs are written from the formats' definitions: bfloat16 is the upper
 * half of an IEEE binary32; OCP OFP8 E4M3 has 1 sign, 4 exponent (bias 7)
 * and 3 mantissa bits, subnormals at exponent field 0, no infinities, NaN at
 * S.1111.111, largest finite 448.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8 = 2, OR_W4A16 = 3 };
enum { OR_OK = 0, OR_EARG = 1, OR_ENONFINITE = 2, OR_ENOMEM = 3 };

/* ---------------------------------------------------------------- codecs */

double oracle_bf16_decode(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_e4m3_decode(uint8_t b) {
    int sign = (b >> 7) & 1;
    int ef = (b >> 3) & 0xF;
    int m = b & 7;
    double v;
    if (ef == 0xF && m == 7) return NAN;
    if (ef == 0)
        v = ldexp((double)m, -9); /* m/8 * 2^-6 */
    else
        v = ldexp(8.0 + m, ef - 7 - 3); /* (1 + m/8) * 2^(ef-7) */
    return sign ? -v : v;
}

/* Round to nearest, ties to even, saturating to +-448. */
uint8_t oracle_e4m3_encode(double v) {
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a >= 448.0) return sign | 0x7E;
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1; /* a in [2^e, 2^(e+1)) */
    if (e < -6) e = -6; /* subnormal range shares the quantum 2^-9 */
    double q = ldexp(1.0, e - 3);
    double r = a / q; /* exact: q is a power of two */
    double fl = floor(r);
    double fr = r - fl;
    double n = fl;
    if (fr > 0.5 || (fr == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;
    if (n >= 16.0) { /* carried into the next binade */
        e += 1;
        n = 8.0;
    }
    if (n < 8.0) /* only reachable at e == -6: subnormal */
        return sign | (uint8_t)n;
    int ef = e + 7;
    if (ef > 15 || (ef == 15 && n - 8.0 > 6.0)) return sign | 0x7E;
    return sign | (uint8_t)(ef << 3) | (uint8_t)(n - 8.0);
}

/* oracle_e4m3_decode of every code, filled once when the library is loaded
 * (the same function, looked up instead of recomputed per element). */
static double e4m3_value[256];

__attribute__((constructor)) static void fill_e4m3_table(void) {
    for (int c = 0; c < 256; ++c) e4m3_value[c] = oracle_e4m3_decode((uint8_t)c);
}

static double elem(int dtype, const void* base, int64_t i) {
    switch (dtype) {
        case OR_F32: return (double)((const float*)base)[i];
        case OR_BF16: return oracle_bf16_decode(((const uint16_t*)base)[i]);
        default: return e4m3_value[((const uint8_t*)base)[i]];
    }
}

/* Bytes of an activation element (the W4A16 layer's activations are bfloat16). */
static size_t elem_bytes(int dtype) { return dtype == OR_F32 ? 4 : (dtype == OR_BF16 || dtype == OR_W4A16) ? 2 : 1; }

/* Storage dtype of the activations. */
static int x_dtype_of(int dtype) { return dtype == OR_W4A16 ? OR_BF16 : dtype; }

/* ---------------------------------------------------- int4 weights (W4A16)
 *
 * Weight-only 4-bit storage of a weight matrix W[N][K] (K contiguous), the
 * "INT4 weight quantisation" of the FusedMoE vs MegaMoE post, section 6.2
 * (the pages fix no format; this one is symmetric round-to-nearest with one
 * float32 scale per 128 consecutive k of a row):
 *  - value W[n][k] = (u - 8) * scale[k / 128][n], u in [0, 15] (u = 8 + q,
 *    q in [-7, 7] for a round-to-nearest code with scale = amax / 7);
 *  - the codes of 8 consecutive k (k0 = a multiple of 8) fill one 32-bit
 *    little-endian word: k0 + 2i at bits 4i..4i+3, k0 + 2i + 1 at bits
 *    16 + 4i..16 + 4i + 3 (i = 0..3); rows are K/2 bytes, one after another;
 *  - scales are group-major: scale[g][n] for the 128-wide group g.
 * One expert's matrix is N*K/2 bytes of codes and (K/128)*N scales. */
double oracle_int4_weight(const uint8_t* codes, const float* gscale, int64_t N, int64_t K, int64_t n, int64_t k) {
    const uint8_t* p = codes + ((size_t)n * K + (size_t)(k & ~(int64_t)7)) / 2;
    const uint32_t word = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
    const int i = (int)((k & 7) >> 1);
    const int shift = (k & 1) ? 16 + 4 * i : 4 * i;
    const int u = (int)((word >> shift) & 15u);
    return (double)(u - 8) * (double)gscale[(size_t)(k / 128) * N + n];
}

/* Expert e's weight matrix (rows x K) and its scales: a byte pointer and
 * either one scalar scale (fp8) or the group scales (W4A16). */
static const void* wexp(int dtype, const void* w, int e, int64_t rows, int64_t K) {
    const size_t bytes = dtype == OR_W4A16 ? (size_t)rows * K / 2 : (size_t)rows * K * elem_bytes(dtype);
    return (const char*)w + (size_t)e * bytes;
}

static const float* wgscale(int dtype, const float* s, int e, int64_t rows, int64_t K) {
    return dtype == OR_W4A16 ? s + (size_t)e * (K / 128) * rows : NULL;
}

/* W[n][k] of an expert matrix widened (times its scale). */
static double wval(int dtype, const void* w_e, double w_scale, const float* gs_e, int64_t N, int64_t K, int64_t n,
                   int64_t k);

static double wval(int dtype, const void* w_e, double w_scale, const float* gs_e, int64_t N, int64_t K, int64_t n,
                   int64_t k) {
    if (dtype == OR_W4A16) return oracle_int4_weight((const uint8_t*)w_e, gs_e, N, K, n, k);
    return elem(dtype, w_e, n * K + k) * w_scale;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* --------------------------------------------------------------- routing */

static int route_one(const float* l, int E, int k, int renorm, int32_t* ids, double* w) {
    char sel[256];
    if (E > 256) return OR_EARG;
    for (int e = 0; e < E; ++e) {
        if (!isfinite(l[e])) return OR_ENONFINITE;
        sel[e] = 0;
    }
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (sel[e]) continue;
            if (best < 0 || l[e] > l[best]) best = e; /* strict: lowest index wins ties */
        }
        sel[best] = 1;
        ids[j] = best;
    }
    double lmax = (double)l[ids[0]];
    double den = 0.0;
    if (renorm) {
        for (int j = 0; j < k; ++j) den += exp((double)l[ids[j]] - lmax);
    } else {
        for (int e = 0; e < E; ++e) den += exp((double)l[e] - lmax);
    }
    for (int j = 0; j < k; ++j) w[j] = exp((double)l[ids[j]] - lmax) / den;
    return OR_OK;
}

int oracle_route(const float* logits, int64_t M, int E, int k, int renorm, int32_t* ids, double* w) {
    if (M < 0 || E < 1 || E > 256 || k < 1 || k > E) return OR_EARG;
    for (int64_t t = 0; t < M; ++t) {
        int rc = route_one(logits + t * E, E, k, renorm, ids + t * k, w + t * k);
        if (rc) return rc;
    }
    return OR_OK;
}

/* The router (FusedMoE vs MegaMoE post, section 2: the router yields one
 * score per expert for each token): logits[t][e] = sum_h x[t][h] * wg[e][h],
 * x widened from its storage (times its scale), wg float32 [E][H]. */
int oracle_router_logits(int dtype, const void* x, const float* x_scale, const float* wg, int64_t M, int E,
                         int64_t H, double* logits) {
    if (M < 0 || E < 1 || H < 1) return OR_EARG;
    size_t eb = dtype == OR_F32 ? 4 : dtype == OR_BF16 ? 2 : 1;
    double xs = x_scale ? (double)x_scale[0] : 1.0;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < M; ++t) {
        const char* row = (const char*)x + (size_t)t * H * eb;
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                double xv = dtype == OR_F32   ? (double)((const float*)row)[h]
                            : dtype == OR_BF16 ? oracle_bf16_decode(((const uint16_t*)row)[h])
                                               : oracle_e4m3_decode(((const uint8_t*)row)[h]);
                s += xv * xs * (double)wg[(size_t)e * H + h];
            }
            logits[t * E + e] = s;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------- alignment */

int64_t oracle_align_capacity(int64_t M, int k, int E, int bm) {
    int64_t P = M * k;
    int64_t a = P < E ? P : E;
    int64_t rows = P + a * (bm - 1);
    return (rows + bm - 1) / bm * bm;
}

int oracle_align(const int32_t* ids, int64_t M, int k, int E, int bm, int64_t cap, int32_t* counts,
                 int32_t* offsets, int32_t* sorted, int32_t* tile_expert, int32_t* active,
                 int32_t* num_active) {
    int64_t P = M * k;
    if (M < 0 || E < 1 || k < 1 || bm < 1 || cap < oracle_align_capacity(M, k, E, bm)) return OR_EARG;
    for (int64_t p = 0; p < P; ++p)
        if (ids[p] < 0 || ids[p] >= E) return OR_EARG;
    for (int e = 0; e < E; ++e) {
        counts[e] = 0;
        for (int64_t p = 0; p < P; ++p) counts[e] += (ids[p] == e);
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
        int32_t padded = (counts[e] + bm - 1) / bm * bm;
        offsets[e + 1] = offsets[e] + padded;
    }
    for (int64_t r = 0; r < cap; ++r) sorted[r] = (int32_t)P;
    for (int e = 0; e < E; ++e) {
        int32_t r = offsets[e];
        for (int64_t p = 0; p < P; ++p)
            if (ids[p] == e) sorted[r++] = (int32_t)p;
    }
    int64_t tiles = cap / bm;
    for (int64_t t = 0; t < tiles; ++t) {
        tile_expert[t] = -1;
        for (int e = 0; e < E; ++e)
            if (t * bm >= offsets[e] && t * bm < offsets[e + 1]) tile_expert[t] = e;
    }
    int64_t na = 0, amax = P < E ? P : E;
    for (int e = 0; e < E; ++e)
        if (counts[e] > 0) active[na++] = e;
    for (int64_t i = na; i < amax; ++i) active[i] = -1;
    *num_active = (int32_t)na;
    return OR_OK;
}

/* ------------------------------------------------------------ expert FFN */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* a[n] = silu(W1[n].x) * W1[I+n].x for one pair, x and W1 widened (times
 * scales; gs1_e: the group scales of int4 weights, else NULL). */
void oracle_gate_up(int dtype, const void* x_row, double x_scale, const void* w1_e, double w1_scale,
                    const float* gs1_e, int64_t H, int64_t I, double* a) {
    const int xd = x_dtype_of(dtype);
    for (int64_t n = 0; n < I; ++n) {
        double g = 0.0, u = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            double xv = elem(xd, x_row, h) * x_scale;
            g += wval(dtype, w1_e, w1_scale, gs1_e, 2 * I, H, n, h) * xv;
            u += wval(dtype, w1_e, w1_scale, gs1_e, 2 * I, H, I + n, h) * xv;
        }
        a[n] = silu(g) * u;
    }
}

/* y[h] = W2[h].a for one pair. */
void oracle_down(int dtype, const double* a, const void* w2_e, double w2_scale, const float* gs2_e, int64_t H,
                 int64_t I, double* y) {
    for (int64_t h = 0; h < H; ++h) {
        double s = 0.0;
        for (int64_t i = 0; i < I; ++i) s += wval(dtype, w2_e, w2_scale, gs2_e, H, I, h, i) * a[i];
        y[h] = s;
    }
}

/* The fp8 intermediate: s = f32(amax)/448 in float32 (1 if amax is 0),
 * code = e4m3(f32(a)/s) with float32 division, value = decode(code)*s. */
void oracle_quant_act(double* a, int64_t I, double amax) {
    float s = (float)amax / 448.0f;
    if (!(amax > 0.0)) s = 1.0f;
    for (int64_t i = 0; i < I; ++i) {
        float v = (float)a[i] / s;
        a[i] = oracle_e4m3_decode(oracle_e4m3_encode((double)v)) * (double)s;
    }
}

static double sc(const float* p, int64_t i) { return p ? (double)p[i] : 1.0; }

/* The scalar scale of expert e's matrix: fp8's per-expert scale, 1 otherwise
 * (int4 weights carry group scales instead). */
static double wsc(int dtype, const float* p, int e) { return dtype == OR_W4A16 ? 1.0 : sc(p, e); }

/* Largest |a| over every (token, slot) pair of the batch: the dynamic
 * per-tensor statistic of the fp8 intermediate. */
int oracle_act_amax(int dtype, const void* x, const float* x_scale, const float* logits, const void* w1,
                    const float* w1_scale, int64_t M, int E, int k, int64_t H, int64_t I, int renorm,
                    double* amax_out) {
    if (M < 0 || E < 1 || k < 1 || k > E || H < 1 || I < 1) return OR_EARG;
    size_t eb = elem_bytes(dtype);
    double amax = 0.0;
    int err = 0;
#pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * I);
        int32_t ids[256];
        double w[256];
        double local = 0.0;
        if (!a) err = OR_ENOMEM;
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < M; ++t) {
            if (!a) continue;
            int rc = route_one(logits + t * E, E, k, renorm, ids, w);
            if (rc) {
                err = rc;
                continue;
            }
            for (int j = 0; j < k; ++j) {
                int e = ids[j];
                oracle_gate_up(dtype, (const char*)x + (size_t)t * H * eb, sc(x_scale, 0), wexp(dtype, w1, e, 2 * I, H),
                               wsc(dtype, w1_scale, e), wgscale(dtype, w1_scale, e, 2 * I, H), H, I, a);
                for (int64_t n = 0; n < I; ++n)
                    if (fabs(a[n]) > local) local = fabs(a[n]);
            }
        }
#pragma omp critical
        {
            if (local > amax) amax = local;
        }
        free(a);
    }
    *amax_out = amax;
    return err;
}

/* Per-token version of oracle_act_amax: amax_out[t] = largest |a| over the
 * token's k pairs, so the batch statistic of any prefix of tokens is the max
 * of a prefix of this array. */
int oracle_act_amax_per_token(int dtype, const void* x, const float* x_scale, const float* logits,
                              const void* w1, const float* w1_scale, int64_t M, int E, int k, int64_t H,
                              int64_t I, int renorm, double* amax_out) {
    if (M < 0 || E < 1 || k < 1 || k > E || H < 1 || I < 1) return OR_EARG;
    size_t eb = elem_bytes(dtype);
    int err = 0;
#pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * I);
        int32_t ids[256];
        double w[256];
        if (!a) err = OR_ENOMEM;
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < M; ++t) {
            if (!a) continue;
            double local = 0.0;
            int rc = route_one(logits + t * E, E, k, renorm, ids, w);
            if (rc) {
                err = rc;
                continue;
            }
            for (int j = 0; j < k; ++j) {
                int e = ids[j];
                oracle_gate_up(dtype, (const char*)x + (size_t)t * H * eb, sc(x_scale, 0), wexp(dtype, w1, e, 2 * I, H),
                               wsc(dtype, w1_scale, e), wgscale(dtype, w1_scale, e, 2 * I, H), H, I, a);
                for (int64_t n = 0; n < I; ++n)
                    if (fabs(a[n]) > local) local = fabs(a[n]);
            }
            amax_out[t] = local;
        }
        free(a);
    }
    return err;
}

/* The whole layer for the tokens listed in `tokens` (n_tok entries):
 * out[i][h] for token tokens[i].  For fp8, act_amax is the batch-wide
 * statistic from oracle_act_amax. */
int oracle_moe(int dtype, const void* x, const float* x_scale, const float* logits, const void* w1,
               const float* w1_scale, const void* w2, const float* w2_scale, int64_t M, int E, int k,
               int64_t H, int64_t I, int renorm, double act_amax, const int64_t* tokens, int64_t n_tok,
               double* out) {
    if (M < 0 || E < 1 || E > 256 || k < 1 || k > E || H < 1 || I < 1) return OR_EARG;
    for (int64_t i = 0; i < n_tok; ++i)
        if (tokens[i] < 0 || tokens[i] >= M) return OR_EARG;
    size_t eb = elem_bytes(dtype);
    int err = 0;
#pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * I);
        double* y = (double*)malloc(sizeof(double) * H);
        int32_t ids[256];
        double w[256];
        if (!a || !y) err = OR_ENOMEM;
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_tok; ++i) {
            if (!a || !y) continue;
            int64_t t = tokens[i];
            double* o = out + i * H;
            for (int64_t h = 0; h < H; ++h) o[h] = 0.0;
            int rc = route_one(logits + t * E, E, k, renorm, ids, w);
            if (rc) {
                err = rc;
                continue;
            }
            for (int j = 0; j < k; ++j) {
                int e = ids[j];
                oracle_gate_up(dtype, (const char*)x + (size_t)t * H * eb, sc(x_scale, 0), wexp(dtype, w1, e, 2 * I, H),
                               wsc(dtype, w1_scale, e), wgscale(dtype, w1_scale, e, 2 * I, H), H, I, a);
                if (dtype == OR_FP8) oracle_quant_act(a, I, act_amax);
                oracle_down(dtype, a, wexp(dtype, w2, e, H, I), wsc(dtype, w2_scale, e), wgscale(dtype, w2_scale, e, H, I), H,
                            I, y);
                for (int64_t h = 0; h < H; ++h) o[h] += w[j] * y[h];
            }
        }
        free(a);
        free(y);
    }
    return err;
}

/* Step-level references over a list of pairs p (token p/k, expert ids[p]). */
int oracle_pairs_gate_up(int dtype, const void* x, const float* x_scale, const int32_t* ids, int64_t M,
                         int k, const void* w1, const float* w1_scale, int E, int64_t H, int64_t I,
                         const int64_t* pairs, int64_t n_pairs, double* act) {
    size_t eb = elem_bytes(dtype);
    for (int64_t i = 0; i < n_pairs; ++i)
        if (pairs[i] < 0 || pairs[i] >= M * k || ids[pairs[i]] < 0 || ids[pairs[i]] >= E) return OR_EARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_pairs; ++i) {
        int64_t p = pairs[i];
        int e = ids[p];
        oracle_gate_up(dtype, (const char*)x + (size_t)(p / k) * H * eb, sc(x_scale, 0), wexp(dtype, w1, e, 2 * I, H),
                       wsc(dtype, w1_scale, e), wgscale(dtype, w1_scale, e, 2 * I, H), H, I, act + i * I);
    }
    return OR_OK;
}

/* act_dtype: storage of the act rows (OR_F32 or OR_BF16); for fp8 weights the
 * rows are quantised with act_amax first, as in the layer. */
int oracle_pairs_down(int dtype, int act_dtype, const void* act, double act_amax, const int32_t* ids,
                      int64_t P, const void* w2, const float* w2_scale, int E, int64_t H, int64_t I,
                      const int64_t* pairs, int64_t n_pairs, double* y) {
    size_t ab = elem_bytes(act_dtype);
    for (int64_t i = 0; i < n_pairs; ++i)
        if (pairs[i] < 0 || pairs[i] >= P || ids[pairs[i]] < 0 || ids[pairs[i]] >= E) return OR_EARG;
    int err = 0;
#pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * I);
        if (!a) err = OR_ENOMEM;
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_pairs; ++i) {
            if (!a) continue;
            int64_t p = pairs[i];
            int e = ids[p];
            for (int64_t n = 0; n < I; ++n) a[n] = elem(act_dtype, (const char*)act + (size_t)p * I * ab, n);
            if (dtype == OR_FP8) oracle_quant_act(a, I, act_amax);
            oracle_down(dtype, a, wexp(dtype, w2, e, H, I), wsc(dtype, w2_scale, e), wgscale(dtype, w2_scale, e, H, I),
                        H, I, y + i * H);
        }
        free(a);
    }
    return err;
}

/* out[t][h] = sum_j w[t*k+j] * y[t*k+j][h], j ascending; y stored as y_dtype. */
int oracle_combine(int y_dtype, const void* y, const float* w, int64_t M, int k, int64_t H, double* out) {
    size_t yb = elem_bytes(y_dtype);
    for (int64_t t = 0; t < M; ++t)
        for (int64_t h = 0; h < H; ++h) {
            double s = 0.0;
            for (int j = 0; j < k; ++j)
                s += (double)w[t * k + j] * elem(y_dtype, (const char*)y + (size_t)(t * k + j) * H * yb, h);
            out[t * H + h] = s;
        }
    return OR_OK;
}
