/*
 * moe_oracle.c -- plain, slow, single-threaded CPU oracle for the routed-expert
 * MoE layer and the expert-pruning statistic.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may link,
 * load or call this file; only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code with the HIP path.
 *
 * Sources (the pages, cited by title and section):
 *   [P1] "Strata Coder 编程模型深度剖析：RCO 专家剪枝砍掉一半专家却保留 91% 编程能力"
 *        §1 "先搞懂 Strata" (48 layers x 512 experts, 10 routed per token),
 *        §3 "RCO 专家剪枝是怎么砍一半而不伤脑的" (gate/up/down per expert; routing
 *        counted on calibration data; the 256 most-selected kept per layer; the
 *        keep decision shared by the three projections; kept experts listed in
 *        their original order).
 *   [P2] Coder benchmark write-up (kwkr.cn), "测试环境与运行配置" (still 10 active
 *        experts per token after pruning) and "专家配置文件：48 x 256 的全量排名"
 *        (per-(layer, expert) ranking, -1 for unranked).
 *   The workload definition this library is built to fills in what the pages do
 *   not print: SwiGLU experts down(silu(gate x) * up x), top-K softmax
 *   renormalised over the selected experts, fp32 router, ties toward the lower
 *   expert index, bf16 activations/weights and int4 blocks of 32 with an fp16
 *   scale.
 *
 * Readings taken where the pages are silent:
 *   R1  logits: l[t][e] = fp32(S) with S the fp64 sum of the exact products
 *       x[t][h]*Wr[e][h] in "wave-64 order": 64 partial sums P_j = sum over i of
 *       prod[j + 64 i] (i ascending), then P_j += P_{j+32}, +16, +8, +4, +2, +1;
 *       the bias, if any, is then added in fp32.  Products of a bf16 or fp32 x
 *       with an fp32 weight are exact in fp64, so only the summation order
 *       needs fixing; it is fixed so that exact top-K parity is well defined.
 *   R2  selection is on the fp32 logits; descending, ties to the lower index;
 *       IEEE comparison (-0 == +0); NaN is rejected.
 *   R3  w[t][k] = exp(l_k - l_0) / sum_j exp(l_j - l_0) over the K selected,
 *       computed in fp64 and rounded to fp32.
 *   R4  permutation: stable counting sort of flat slots s = t*K + k by expert.
 *   R5  expert FFN: y = Wd (silu(Wg x) .* (Wu x)), no biases, weights stored
 *       out x in; silu(z) = z / (1 + exp(-z)); fp64 accumulation; for bf16
 *       activations the product a = silu(g) * u is rounded to bf16 (RNE).
 *   R6  combine: out[t] = cast(sum_k w[t][k] * y_k + residual[t]) with the sum
 *       in fp64 in k order and one final rounding (fp32, or bf16 RNE).
 *   R7  int4: w = d * (nibble - 8), d the fp16 scale of the 32-element block
 *       along the input dimension; byte j holds element 2j low, 2j+1 high.
 *   R16 int2 / int3 (a lower-bit expert variant): w = d * (u - 2) or d * (u - 4),
 *       u the element's stored level, d the fp16 scale of its 32-element block.
 *       A row holds the low two bits of every level as 32-bit little-endian
 *       words of 16 elements (element 4k + j of a word in byte j, bits 2k and
 *       2k + 1); int3 rows then hold the third bit as words of 32 elements
 *       (element 16g + 4k + j of a word in byte j, bit 4g + k).
 *   R8  counts[l][e] = number of rows whose top-K holds e; rank by (count
 *       descending, index ascending); keep_map[l] = the ids of rank < keep,
 *       in ascending id order.
 *
 * Build: gcc -std=c11 -O3 -ffp-contract=off -fno-fast-math -fPIC -shared.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_INT4 = 2, OR_INT2 = 3, OR_INT3 = 4 };
enum { OR_OK = 0, OR_EINVAL = 1, OR_ENAN = 2, OR_ENOMEM = 3 };

int oracle_rank_keep(const int64_t* counts, int L, int E, int keep, int32_t* rank_of, int32_t* keep_map);

/* ------------------------------------------------------------------ number formats */

/* bfloat16 bits -> value (the top half of an IEEE binary32). */
double oracle_bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a double directly to bfloat16, nearest-even (one rounding, no detour
 * through fp32).  bfloat16: 8 significant bits, fp32's exponent range,
 * subnormal quantum 2^-133, largest finite (2 - 2^-7) * 2^127. */
uint16_t oracle_round_bf16(double v) {
    float f;
    uint32_t u;
    if (isnan(v)) return 0x7FC0;
    if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
    int e;
    double m = frexp(v, &e);                /* v = m * 2^e, 0.5 <= |m| < 1 */
    double r;
    if (e - 1 >= -126) {
        r = ldexp(nearbyint(ldexp(m, 8)), e - 8);   /* 8 significant bits */
    } else {
        r = ldexp(nearbyint(ldexp(v, 133)), -133);  /* fixed subnormal quantum */
    }
    const double maxf = ldexp(255.0, 120);          /* (2 - 2^-7) * 2^127 */
    if (fabs(r) > maxf) r = copysign(INFINITY, v);
    f = (float)r;                                   /* exact: r has <= 8 bits */
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* IEEE binary16 bits -> value: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_fp16_value(uint16_t h) {
    int s = (h >> 15) & 1, ex = (h >> 10) & 31, fr = h & 1023;
    double v;
    if (ex == 0) v = ldexp((double)fr, -24);                 /* subnormal */
    else if (ex == 31) v = fr ? NAN : INFINITY;
    else v = ldexp(1024.0 + fr, ex - 25);
    return s ? -v : v;
}

static double act_value(const void* x, int dt, int64_t i) {
    return dt == OR_F32 ? (double)((const float*)x)[i] : oracle_bf16_value(((const uint16_t*)x)[i]);
}

/* The stored level u of element c of one int2 or int3 row of `cols`
 * elements (R16). */
static int lowbit_level(const uint8_t* row, int64_t cols, int bits, int64_t c) {
    const int64_t word = c / 16;
    const int i = (int)(c % 16), k = i / 4, j = i % 4;
    int u = (row[word * 4 + j] >> (2 * k)) & 3;
    if (bits == 3) {
        const uint8_t* third = row + cols / 4;
        const int64_t word3 = c / 32;
        const int i3 = (int)(c % 32), g = i3 / 16, k3 = (i3 % 16) / 4, j3 = i3 % 4;
        u |= ((third[word3 * 4 + j3] >> (4 * g + k3)) & 1) << 2;
    }
    return u;
}

/* One weight element of matrix `mat` (shape [E][rows][cols], out x in) at
 * (e, r, c), as an exact double.  R7 for int4, R16 for int2 / int3. */
static double weight_value(const void* mat, const uint16_t* scales, int dt,
                           int64_t e, int64_t rows, int64_t cols, int64_t r, int64_t c) {
    int64_t flat = (e * rows + r) * cols + c;
    if (dt == OR_F32) return (double)((const float*)mat)[flat];
    if (dt == OR_BF16) return oracle_bf16_value(((const uint16_t*)mat)[flat]);
    double d = oracle_fp16_value(scales[(e * rows + r) * (cols / 32) + c / 32]);
    int q;
    if (dt == OR_INT4) {
        uint8_t byte = ((const uint8_t*)mat)[flat / 2];
        q = ((c & 1) ? (byte >> 4) : (byte & 15)) - 8;
    } else {
        const int bits = dt == OR_INT2 ? 2 : 3;
        const int64_t row_bytes = cols * bits / 8;
        q = lowbit_level((const uint8_t*)mat + (e * rows + r) * row_bytes, cols, bits, c) - (1 << (bits - 1));
    }
    return d * (double)q;
}

/* Dequantise an int2 (bits = 2) or int3 (bits = 3) matrix [rows][cols] to
 * doubles (used by the format pins). */
int oracle_lowbit_dequant(const uint8_t* packed, const uint16_t* scales, int64_t rows, int64_t cols, int bits,
                          double* out) {
    if (cols % 32 || (bits != 2 && bits != 3)) return OR_EINVAL;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            out[r * cols + c] = weight_value(packed, scales, bits == 2 ? OR_INT2 : OR_INT3, 0, rows, cols, r, c);
    return OR_OK;
}

/* Dequantise one int4 matrix row range to doubles (used by the format pin). */
int oracle_int4_dequant(const uint8_t* packed, const uint16_t* scales, int64_t rows, int64_t cols,
                        double* out) {
    if (cols % 32) return OR_EINVAL;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            out[r * cols + c] = weight_value(packed, scales, OR_INT4, 0, rows, cols, r, c);
    return OR_OK;
}

/* ------------------------------------------------------------------ a1: router logits (R1) */

/* The fp64 dot product of two rows (already widened to double) in wave-64 order. */
static double dot_wave64(const double* a, const double* b, int H) {
    double P[64];
    for (int j = 0; j < 64; j++) P[j] = 0.0;
    for (int base = 0; base < H; base += 64)
        for (int j = 0; j < 64 && base + j < H; j++)
            P[j] += a[base + j] * b[base + j];          /* exact product; one rounding per add */
    for (int step = 32; step >= 1; step >>= 1)
        for (int j = 0; j < step; j++) P[j] += P[j + step];
    return P[0];
}

/* logits[t][e] for all t < T, e < E.  x: [T][H] f32 or bf16 bits; Wr: [E][H]
 * fp32; bias: [E] or NULL. */
int oracle_router_logits(const void* x, int x_dt, const float* Wr, const float* bias,
                         int64_t T, int H, int E, float* logits) {
    if (!x || !Wr || !logits || T < 0 || H <= 0 || E <= 0) return OR_EINVAL;
    double* w = (double*)malloc(sizeof(double) * (size_t)E * (size_t)H);
    double* xr = (double*)malloc(sizeof(double) * (size_t)H);
    if (!w || !xr) { free(w); free(xr); return OR_ENOMEM; }
    for (int64_t i = 0; i < (int64_t)E * H; i++) w[i] = (double)Wr[i];
    for (int64_t t = 0; t < T; t++) {
        for (int h = 0; h < H; h++) xr[h] = act_value(x, x_dt, t * (int64_t)H + h);
        for (int e = 0; e < E; e++) {
            float l = (float)dot_wave64(xr, w + (int64_t)e * H, H);
            if (bias) l = l + bias[e];          /* fp32 add, no contraction */
            logits[t * E + e] = l;
        }
    }
    free(w);
    free(xr);
    return OR_OK;
}

/* ------------------------------------------------------------------ a2: selection + weights (R2, R3) */

static int select_row(const float* l, int E, int K, int32_t* idx, unsigned char* taken) {
    for (int e = 0; e < E; e++) {
        if (isnan(l[e])) return OR_ENAN;
        taken[e] = 0;
    }
    for (int k = 0; k < K; k++) {
        int best = -1;
        for (int e = 0; e < E; e++)
            if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;   /* strict: lower id wins ties */
        taken[best] = 1;
        idx[k] = best;
    }
    return OR_OK;
}

/* idx[t][k] and (if w != NULL) w[t][k] from given logits [T][E]. */
int oracle_topk(const float* logits, int64_t T, int E, int K, int32_t* idx, float* w) {
    if (!logits || !idx || T < 0 || E <= 0 || K <= 0 || K > E) return OR_EINVAL;
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    if (!taken) return OR_ENOMEM;
    for (int64_t t = 0; t < T; t++) {
        const float* l = logits + t * E;
        int32_t* id = idx + t * K;
        int rc = select_row(l, E, K, id, taken);
        if (rc) { free(taken); return rc; }
        if (w) {
            double m = (double)l[id[0]], s = 0.0;
            for (int k = 0; k < K; k++) s += exp((double)l[id[k]] - m);
            for (int k = 0; k < K; k++) w[t * K + k] = (float)(exp((double)l[id[k]] - m) / s);
        }
    }
    free(taken);
    return OR_OK;
}

/* ------------------------------------------------------------------ a3: grouping (R4) */

int oracle_permute(const int32_t* idx, int64_t T, int K, int E,
                   int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv) {
    if (!idx || !counts || !offsets || !perm || !inv || T < 0 || K <= 0 || E <= 0) return OR_EINVAL;
    int64_t n = T * K;
    for (int e = 0; e < E; e++) counts[e] = 0;
    for (int64_t s = 0; s < n; s++) {
        if (idx[s] < 0 || idx[s] >= E) return OR_EINVAL;
        counts[idx[s]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!fill) return OR_ENOMEM;
    for (int e = 0; e < E; e++) fill[e] = offsets[e];
    for (int64_t s = 0; s < n; s++) {           /* ascending slot order => stable */
        int32_t p = fill[idx[s]]++;
        perm[p] = (int32_t)s;
        inv[s] = p;
    }
    free(fill);
    return OR_OK;
}

/* ------------------------------------------------------------------ a4: one expert on one row (R5) */

/* y[H] = Wd[e] (silu(Wg[e] x) .* (Wu[e] x)) for the activation row x (offset xoff). */
int oracle_expert_ffn(const void* x, int x_dt, int64_t xoff,
                      const void* wg, const void* wu, const void* wd,
                      const uint16_t* sg, const uint16_t* su, const uint16_t* sd, int w_dt,
                      int e, int H, int F, int round_a_bf16, double* y) {
    double* a = (double*)malloc(sizeof(double) * (size_t)F);
    if (!a) return OR_ENOMEM;
    double* xr = (double*)malloc(sizeof(double) * (size_t)H);
    if (!xr) { free(a); return OR_ENOMEM; }
    for (int h = 0; h < H; h++) xr[h] = act_value(x, x_dt, xoff + h);
    for (int f = 0; f < F; f++) {
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; h++) {
            double xv = xr[h];
            g += xv * weight_value(wg, sg, w_dt, e, F, H, f, h);
            u += xv * weight_value(wu, su, w_dt, e, F, H, f, h);
        }
        double silu = g / (1.0 + exp(-g));
        a[f] = silu * u;
        if (round_a_bf16) a[f] = oracle_bf16_value(oracle_round_bf16(a[f]));
    }
    for (int h = 0; h < H; h++) {
        double acc = 0.0;
        for (int f = 0; f < F; f++) acc += a[f] * weight_value(wd, sd, w_dt, e, H, F, h, f);
        y[h] = acc;
    }
    free(a);
    free(xr);
    return OR_OK;
}

/* ------------------------------------------------------------------ a4 + a5: layer rows (R6) */

/* For each listed token t = rows[i]: out_rows[i][:] = cast(sum_k w[t][k] * FFN_{idx[t][k]}(x[t]) + res[t]).
 * idx/w: the routing [T][K]; res: [T][H] in x's dtype or NULL; out_dt: OR_F32 or OR_BF16
 * (out_rows then holds fp32 values or bf16 bits).  y_rows, if non-NULL, receives the
 * unweighted per-slot expert outputs [n_rows][K][H] in fp64. */
int oracle_layer_rows(const void* x, int x_dt, const int32_t* idx, const float* w, int K,
                      const void* wg, const void* wu, const void* wd,
                      const uint16_t* sg, const uint16_t* su, const uint16_t* sd, int w_dt,
                      int H, int F, const void* res, const int64_t* rows, int64_t n_rows,
                      int out_dt, void* out_rows, double* y_rows) {
    if (!x || !idx || !w || !wg || !wu || !wd || !rows || !out_rows || H <= 0 || F <= 0) return OR_EINVAL;
    if (w_dt >= OR_INT4 && (!sg || !su || !sd || H % 32 || F % 32)) return OR_EINVAL;
    if (w_dt < OR_F32 || w_dt > OR_INT3) return OR_EINVAL;
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    if (!y || !acc) { free(y); free(acc); return OR_ENOMEM; }
    int round_a = (x_dt == OR_BF16);
    for (int64_t i = 0; i < n_rows; i++) {
        int64_t t = rows[i];
        for (int h = 0; h < H; h++) acc[h] = 0.0;
        for (int k = 0; k < K; k++) {
            int rc = oracle_expert_ffn(x, x_dt, t * H, wg, wu, wd, sg, su, sd, w_dt,
                                       idx[t * K + k], H, F, round_a, y);
            if (rc) { free(y); free(acc); return rc; }
            double wk = (double)w[t * K + k];
            for (int h = 0; h < H; h++) acc[h] += wk * y[h];
            if (y_rows) memcpy(y_rows + (i * K + k) * (int64_t)H, y, sizeof(double) * (size_t)H);
        }
        for (int h = 0; h < H; h++) {
            double v = acc[h] + (res ? act_value(res, x_dt, t * H + h) : 0.0);
            if (out_dt == OR_F32) ((float*)out_rows)[i * H + h] = (float)v;
            else ((uint16_t*)out_rows)[i * H + h] = oracle_round_bf16(v);
        }
    }
    free(y);
    free(acc);
    return OR_OK;
}

/* ------------------------------------------------------------------ a6: pruning statistic (R8) */

/* counts[l][e] (+=) over given logits [L][T][E]; then, if keep > 0, rank_of[l][e]
 * and keep_map[l][0..keep).  accumulate != 0 adds to counts instead of overwriting. */
int oracle_expert_freq(const float* logits, int L, int64_t T, int E, int K, int64_t* counts,
                       int accumulate, int keep, int32_t* rank_of, int32_t* keep_map) {
    if (!logits || !counts || L <= 0 || T < 0 || E <= 0 || K <= 0 || K > E || keep < 0 || keep > E)
        return OR_EINVAL;
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    if (!idx || !taken) { free(idx); free(taken); return OR_ENOMEM; }
    for (int l = 0; l < L; l++) {
        int64_t* c = counts + (int64_t)l * E;
        if (!accumulate) for (int e = 0; e < E; e++) c[e] = 0;
        for (int64_t t = 0; t < T; t++) {
            int rc = select_row(logits + ((int64_t)l * T + t) * E, E, K, idx, taken);
            if (rc) { free(idx); free(taken); return rc; }
            for (int k = 0; k < K; k++) c[idx[k]]++;
        }
    }
    free(idx);
    free(taken);
    if (keep > 0) return oracle_rank_keep(counts, L, E, keep, rank_of, keep_map);
    return OR_OK;
}

/* rank_of[l][e] = number of experts ahead of e in (count desc, id asc) order;
 * keep_map[l] = ids with rank_of < keep, ascending. */
int oracle_rank_keep(const int64_t* counts, int L, int E, int keep, int32_t* rank_of, int32_t* keep_map) {
    if (!counts || !rank_of || !keep_map || keep <= 0 || keep > E) return OR_EINVAL;
    for (int l = 0; l < L; l++) {
        const int64_t* c = counts + (int64_t)l * E;
        int32_t* r = rank_of + (int64_t)l * E;
        for (int e = 0; e < E; e++) {
            int ahead = 0;
            for (int f = 0; f < E; f++)
                if (c[f] > c[e] || (c[f] == c[e] && f < e)) ahead++;
            r[e] = ahead;
        }
        int n = 0;
        for (int e = 0; e < E; e++)
            if (r[e] < keep) keep_map[(int64_t)l * keep + n++] = e;
    }
    return OR_OK;
}
