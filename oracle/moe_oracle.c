/*
 * moe_oracle.c -- plain, slow, sequential CPU oracle for MoE expert-parallel
 * token dispatch and combine (router softmax/top-k, count, prefix sums,
 * stable permute-and-pack with a combine handle, all-to-all-v exchange,
 * expert stub, reverse exchange, routing-weighted top-k reduction).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP library; both sides implement the formats below from
 * their definitions.
 *
 * Sources (the four web pages on expert-parallel all-to-all):
 *  [EP]   "Expert Parallel: MoE Token 为什么要两次穿过 GPU 网络" (charlestar.github.io)
 *         sections "一个 Top-2 路由例子", "Dispatch 前为什么必须 count 和 permute",
 *         "All-to-All-v 才接近真实通信形状", "Combine 不是简单把结果发回来",
 *         "正确性检查比性能调优更早".
 *  [A2A]  "[Infra-10] All-to-All Optimization" (xutianle.me), sections 1, 2,
 *         3.5, 4.1, 5.1, 5.2.
 *  [PPLX] "高效且便携的专家混合通信" (Perplexity, pplx-kernels), router paragraph
 *         and the dispatch / combine kernel sections.
 *
 * Notation: P logical ranks, T tokens (T/P per rank, blocked: token t lives on
 * rank s = t / (T/P) with local index i = t - s*(T/P)), E experts (E/P per
 * rank, contiguous: owner(e) = e / (E/P)), top-k, hidden size H, N_a = T*k.
 *
 * Every floating-point step is either done in double (the router) or in the
 * precision the method fixes for it (fp32 scale division and e4m3 rounding of
 * the FP8 payload, fp32 stub arithmetic, fp32 fused-multiply-add accumulation
 * of the combine in slot order, bfloat16 storage).  Build with
 * -ffp-contract=off so the compiler adds no fused operations of its own.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats, from their definitions.                                   */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 stored significand bits. */
float oracle_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* Nearest bfloat16 to the finite double v, ties to the even significand.
 * |v| = m * 2^e with m in [0.5, 1); a bfloat16 has 8 significant bits, so the
 * spacing of representable values around v is 2^(e-8), never finer than the
 * subnormal spacing 2^-133.  Values that round beyond the largest finite
 * bfloat16 become infinity. */
uint16_t oracle_bf16_from_double(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    if (e < -125) e = -125;
    double q = ldexp(1.0, e - 8);          /* spacing of bf16 values near a */
    double r = rint(a / q) * q;            /* rint: nearest, ties to even (default mode) */
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
    uint32_t bits = f32_bits((float)r);    /* r has <= 8 significant bits: exact in float */
    return (uint16_t)(sign | (bits >> 16));
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 significand bits,
 * no infinities, NaN = S.1111.111, largest finite 448 = 1.75 * 2^8, subnormal
 * spacing 2^-9.  Conversion: nearest value, ties to even code, saturating to
 * +-448 (values the rounding would carry past 448 are clamped). */
float oracle_e4m3_to_f32(uint8_t c)
{
    int s = c >> 7, ex = (c >> 3) & 15, m = c & 7;
    double v;
    if (ex == 15 && m == 7) return NAN;
    if (ex == 0) v = ldexp((double)m, -9);
    else v = ldexp(8.0 + m, ex - 10);      /* (1 + m/8) * 2^(ex-7) */
    return (float)(s ? -v : v);
}

uint8_t oracle_e4m3_from_double(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (isnan(v)) return 0x7F;
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    if (e < -5) e = -5;                    /* below 2^-6 the spacing stays 2^-9 */
    double q = ldexp(1.0, e - 4);          /* 4 significant bits */
    double r = rint(a / q) * q;
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -6))                /* subnormal: r = m * 2^-9 */
        return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -9)));
    int re;
    double rm = frexp(r, &re);             /* r = rm * 2^re, rm in [0.5, 1) */
    int ex = re - 1 + 7;                   /* r = (2 rm) * 2^(re-1) */
    int m = (int)((2.0 * rm - 1.0) * 8.0);
    return (uint8_t)(sign | (ex << 3) | m);
}

/* ------------------------------------------------------------------------ */
/* Shape.                                                                     */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t P, T, E, k, H;
    int64_t fp8;       /* 0: bfloat16 dispatch rows; 1: e4m3 rows + fp32 scales */
} oracle_shape;

#define FP8_BLOCK 128  /* channels per scale, per token */

/* The combine handle that travels with each assignment ([EP] "dispatch
 * payload" and "combine handle" lists; [PPLX] dispatch-receive stores source
 * rank, expert and token index): 16 bytes, little endian. */
typedef struct {
    int32_t src_rank;      /* s */
    int32_t src_token;     /* i, index local to the source rank */
    int16_t slot;          /* j, top-k slot */
    int16_t local_expert;  /* e mod (E/P) */
    float weight;          /* routing weight w[t, j] */
} oracle_meta;

int64_t oracle_meta_bytes(void) { return (int64_t)sizeof(oracle_meta); }

/* ------------------------------------------------------------------------ */
/* a1. Router: softmax over the E logits, top-k, renormalise ([PPLX] router   */
/* paragraph: the router yields a probability distribution, the k best       */
/* experts are taken and the output is their weighted average; [EP] router   */
/* output is [num_tokens, top_k] ids and weights).                            */
/* ------------------------------------------------------------------------ */

/* Slot order: slot 0 is the most probable expert.  Because softmax is strictly
 * increasing, ordering by probability is ordering by logit; equal logits are
 * broken towards the lower expert id.  A NaN logit has no place in that order
 * and ranks below every number, -inf included (NaN against NaN is a tie, so
 * the lower id again comes first); the weights of a row that holds a NaN are
 * all NaN, because the softmax normaliser of that row is NaN. */
static int ranks_before(float a, float b) { return !isnan(a) && (isnan(b) || a > b); }

void oracle_route(const oracle_shape* s, const float* logits, int32_t* ids, float* w)
{
    int64_t E = s->E, k = s->k;
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    for (int64_t t = 0; t < s->T; ++t) {
        const float* l = logits + t * E;
        double m = l[0];
        for (int64_t e = 1; e < E; ++e) if (l[e] > m) m = l[e];
        double z = 0.0;
        for (int64_t e = 0; e < E; ++e) { p[e] = exp((double)l[e] - m); z += p[e]; }
        for (int64_t e = 0; e < E; ++e) p[e] /= z;
        memset(taken, 0, (size_t)E);
        double sel = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(l[e], l[best])) best = e;   /* strict: ties keep the lower id */
            }
            taken[best] = 1;
            ids[t * k + j] = (int32_t)best;
            sel += p[best];
        }
        for (int64_t j = 0; j < k; ++j) w[t * k + j] = (float)(p[ids[t * k + j]] / sel);
    }
    free(p);
    free(taken);
}

/* ------------------------------------------------------------------------ */
/* a2..a5. Dispatch.                                                           */
/* ------------------------------------------------------------------------ */

typedef struct {
    /* counts and offsets (int32) */
    int32_t* n;              /* [P][E]  assignments from rank s to expert e */
    int32_t* N;              /* [E]     assignments received by expert e     */
    int32_t* C;              /* [P][P]  count matrix, row = source, col = destination */
    int32_t* expert_off;     /* [E+1]   start of expert e in the receive buffer */
    int32_t* rank_recv_off;  /* [P+1]   start of rank r's receive region */
    int32_t* send_off;       /* [P][E]  start of bucket (s -> e) in the send buffer */
    int32_t* recv_off;       /* [E][P]  start of bucket (s -> e) in the receive buffer */
    /* permutation */
    int32_t* send_pos;       /* [T*k]   send row of assignment (t, j) */
    int32_t* recv_pos;       /* [T*k]   receive row of assignment (t, j) */
    /* payload (may be NULL to skip the row copies) */
    uint8_t* send_rows;      /* [N_a][row_bytes] */
    float* send_scales;      /* [N_a][H/128] (FP8 only) */
    oracle_meta* send_meta;  /* [N_a] */
    uint8_t* recv_rows;
    float* recv_scales;
    oracle_meta* recv_meta;
} oracle_dispatch_out;

int64_t oracle_row_bytes(const oracle_shape* s) { return s->fp8 ? s->H : 2 * s->H; }

/* FP8 quantisation of one token row ([A2A] 4.1: quantise before the
 * exchange; [PPLX] dispatch sends FP8 tokens with block scales).  Per block of
 * 128 channels: amax = max |x| (exact), scale = amax / 448 rounded to fp32,
 * q = e4m3(x / scale) with the quotient rounded to fp32 first.  A block of
 * zeros gets scale 0 and codes that keep the sign of each zero. */
void oracle_quantize_row(int64_t H, const uint16_t* x, uint8_t* q, float* scales)
{
    for (int64_t b = 0; b < H / FP8_BLOCK; ++b) {
        float amax = 0.0f;
        for (int64_t h = b * FP8_BLOCK; h < (b + 1) * FP8_BLOCK; ++h) {
            float a = fabsf(oracle_bf16_to_f32(x[h]));
            if (a > amax) amax = a;
        }
        float scale = amax / 448.0f;
        scales[b] = scale;
        for (int64_t h = b * FP8_BLOCK; h < (b + 1) * FP8_BLOCK; ++h) {
            float xv = oracle_bf16_to_f32(x[h]);
            if (amax == 0.0f) { q[h] = signbit(xv) ? 0x80 : 0x00; continue; }
            float r = xv / scale;
            q[h] = oracle_e4m3_from_double((double)r);
        }
    }
}

/* Count ([EP] "统计目的 rank", count matrix C_ij), prefix sums ([EP] "Prefix
 * sum 计算偏移"), stable permute-and-pack with the handle ([EP] "按目的地写入连续
 * buffer"; [A2A] 5.2 send layout [to rank 0]...[to rank P-1], each bucketed by
 * local expert), then the all-to-all-v exchange ([A2A] 1: rank j receives the
 * j-th piece of every rank; [EP] worked example: each rank's receive region
 * is grouped by local expert, and within an expert by source rank and token).
 */
void oracle_dispatch(const oracle_shape* s, const uint16_t* x, const int32_t* ids,
                     const float* w, oracle_dispatch_out* o)
{
    const int64_t P = s->P, T = s->T, E = s->E, k = s->k, H = s->H;
    const int64_t Tp = T / P, Ep = E / P, Na = T * k;
    const int64_t rb = oracle_row_bytes(s), nb = H / FP8_BLOCK;

    /* count: a direct loop over every assignment */
    memset(o->n, 0, sizeof(int32_t) * (size_t)(P * E));
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < k; ++j)
            o->n[(t / Tp) * E + ids[t * k + j]] += 1;
    for (int64_t e = 0; e < E; ++e) {
        o->N[e] = 0;
        for (int64_t r = 0; r < P; ++r) o->N[e] += o->n[r * E + e];
    }
    for (int64_t src = 0; src < P; ++src)
        for (int64_t dst = 0; dst < P; ++dst) {
            int32_t c = 0;
            for (int64_t e = dst * Ep; e < (dst + 1) * Ep; ++e) c += o->n[src * E + e];
            o->C[src * P + dst] = c;
        }

    /* exclusive prefix sums */
    o->expert_off[0] = 0;
    for (int64_t e = 0; e < E; ++e) o->expert_off[e + 1] = o->expert_off[e] + o->N[e];
    for (int64_t r = 0; r <= P; ++r) o->rank_recv_off[r] = o->expert_off[r * Ep];
    for (int64_t src = 0; src < P; ++src) {
        int32_t acc = (int32_t)(src * Tp * k);    /* rank src owns send rows [src*Tp*k, (src+1)*Tp*k) */
        for (int64_t e = 0; e < E; ++e) { o->send_off[src * E + e] = acc; acc += o->n[src * E + e]; }
    }
    for (int64_t e = 0; e < E; ++e) {
        int32_t acc = o->expert_off[e];
        for (int64_t src = 0; src < P; ++src) { o->recv_off[e * P + src] = acc; acc += o->n[src * E + e]; }
    }

    /* stable permutation: walk the assignments in token order with one cursor
     * per (source, expert) bucket */
    int32_t* cur = (int32_t*)calloc((size_t)(P * E), sizeof(int32_t));
    for (int64_t t = 0; t < T; ++t) {
        int64_t src = t / Tp;
        for (int64_t j = 0; j < k; ++j) {
            int64_t e = ids[t * k + j];
            int32_t c = cur[src * E + e]++;
            o->send_pos[t * k + j] = o->send_off[src * E + e] + c;
            o->recv_pos[t * k + j] = o->recv_off[e * P + src] + c;
        }
    }
    free(cur);

    /* pack the rows and the handle into the send buffer */
    uint8_t* qrow = (uint8_t*)malloc((size_t)rb);
    float* qsc = (float*)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
    for (int64_t t = 0; t < T; ++t) {
        int64_t src = t / Tp;
        if (o->send_rows) {
            if (s->fp8) oracle_quantize_row(H, x + t * H, qrow, qsc);
            else memcpy(qrow, x + t * H, (size_t)rb);
        }
        for (int64_t j = 0; j < k; ++j) {
            int64_t e = ids[t * k + j];
            int64_t p = o->send_pos[t * k + j];
            if (o->send_rows) {
                memcpy(o->send_rows + p * rb, qrow, (size_t)rb);
                if (s->fp8) memcpy(o->send_scales + p * nb, qsc, sizeof(float) * (size_t)nb);
            }
            if (o->send_meta) {
                oracle_meta m;
                m.src_rank = (int32_t)src;
                m.src_token = (int32_t)(t - src * Tp);
                m.slot = (int16_t)j;
                m.local_expert = (int16_t)(e % Ep);
                m.weight = w[t * k + j];
                o->send_meta[p] = m;
            }
        }
    }
    free(qrow);
    free(qsc);

    /* exchange: every assignment's send row lands on its receive row */
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < k; ++j) {
            int64_t p = o->send_pos[t * k + j], q = o->recv_pos[t * k + j];
            if (o->send_rows && o->recv_rows) {
                memcpy(o->recv_rows + q * rb, o->send_rows + p * rb, (size_t)rb);
                if (s->fp8) memcpy(o->recv_scales + q * nb, o->send_scales + p * nb, sizeof(float) * (size_t)nb);
            }
            if (o->send_meta && o->recv_meta) o->recv_meta[q] = o->send_meta[p];
        }
    (void)Na;
}

/* ------------------------------------------------------------------------ */
/* a6. Expert stub: stands in for the grouped GEMM that consumes the          */
/* expert-contiguous receive rows.  out = bf16(deq(row) * m_e) with           */
/* m_e = (E + e) / E in fp32 (that is 1 + e/E) and e the global expert of the */
/* receive segment holding the row; deq is the fp32 product code * scale for  */
/* FP8 rows.  Each product is one fp32 rounding, then one bf16 rounding.      */
/* ------------------------------------------------------------------------ */

static float stub_multiplier(int64_t e, int64_t E) { return (float)(E + e) / (float)E; }

void oracle_stub_row(const oracle_shape* s, int64_t e, const uint8_t* row, const float* scales,
                     uint16_t* out)
{
    float m = stub_multiplier(e, s->E);
    for (int64_t h = 0; h < s->H; ++h) {
        float d;
        if (s->fp8) {
            float qv = oracle_e4m3_to_f32(row[h]);
            d = qv * scales[h / FP8_BLOCK];
        } else {
            uint16_t b;
            memcpy(&b, row + 2 * h, 2);
            d = oracle_bf16_to_f32(b);
        }
        float y = d * m;
        out[h] = oracle_bf16_from_double((double)y);
    }
}

void oracle_stub(const oracle_shape* s, const int32_t* expert_off, const uint8_t* recv_rows,
                 const float* recv_scales, uint16_t* expert_out)
{
    const int64_t rb = oracle_row_bytes(s), nb = s->H / FP8_BLOCK;
    for (int64_t e = 0; e < s->E; ++e)
        for (int64_t q = expert_off[e]; q < expert_off[e + 1]; ++q)
            oracle_stub_row(s, e, recv_rows + q * rb, s->fp8 ? recv_scales + q * nb : NULL,
                            expert_out + q * s->H);
}

/* ------------------------------------------------------------------------ */
/* a7..a8. Combine ([EP] "Combine 不是简单把结果发回来": put every expert     */
/* output back at its (token, slot) using the handle, never in arrival order, */
/* then sum with the router weights; [PPLX] combine sends 16-bit activations */
/* back and the receiver forms the weighted sum).                             */
/* ------------------------------------------------------------------------ */

/* Reverse exchange: receive row q goes to combine row (s*T/P + i)*k + j of its
 * source token, found from the handle (s, i, j) that travelled with it. */
void oracle_reverse_exchange(const oracle_shape* s, const oracle_meta* recv_meta,
                             const uint16_t* expert_out, uint16_t* comb)
{
    const int64_t Tp = s->T / s->P, Na = s->T * s->k;
    for (int64_t q = 0; q < Na; ++q) {
        const oracle_meta* m = &recv_meta[q];
        int64_t t = (int64_t)m->src_rank * Tp + m->src_token;
        memcpy(comb + (t * s->k + m->slot) * s->H, expert_out + q * s->H, sizeof(uint16_t) * (size_t)s->H);
    }
}

/* Weighted reduction of one token: y32 = fma(w_j, out_j, acc) for j = 0..k-1
 * starting from 0 (fp32 accumulation in slot order), y = bf16(y32); y64 is the
 * same sum in double, for checking the fp32 result against the exact sum. */
void oracle_reduce_token(const oracle_shape* s, int64_t t, const uint16_t* comb, const float* w,
                         float* y32, uint16_t* y, double* y64)
{
    const int64_t H = s->H, k = s->k;
    for (int64_t h = 0; h < H; ++h) {
        float acc = 0.0f;
        double acc64 = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            float v = oracle_bf16_to_f32(comb[(t * k + j) * H + h]);
            acc = fmaf(w[t * k + j], v, acc);
            acc64 += (double)w[t * k + j] * (double)v;
        }
        if (y32) y32[t * H + h] = acc;
        if (y) y[t * H + h] = oracle_bf16_from_double((double)acc);
        if (y64) y64[t * H + h] = acc64;
    }
}

void oracle_combine(const oracle_shape* s, const oracle_meta* recv_meta, const uint16_t* expert_out,
                    const float* w, uint16_t* comb, float* y32, uint16_t* y, double* y64)
{
    oracle_reverse_exchange(s, recv_meta, expert_out, comb);
    for (int64_t t = 0; t < s->T; ++t) oracle_reduce_token(s, t, comb, w, y32, y, y64);
}

/* ------------------------------------------------------------------------ */
/* Array forms of the format conversions, for the tests.                      */
/* ------------------------------------------------------------------------ */

void oracle_bf16_from_double_array(int64_t n, const double* v, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_double(v[i]);
}

void oracle_e4m3_from_double_array(int64_t n, const double* v, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_from_double(v[i]);
}

void oracle_e4m3_to_f32_array(int64_t n, const uint8_t* c, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_to_f32(c[i]);
}
