/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for the single-GPU
 * MoE expert-parallel dispatch/combine data path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, helper or table with
 * the HIP library.
 *
 * Sources (page = web page of the reference set, by site):
 *  [ThunderEP]  bjdmk.com.cn ThunderEP write-up: s1.3 problem statement,
 *               s2.1 aggregation by destination into one contiguous block,
 *               s2.3 per-token dynamic int8, s3.3 layer pseudo-code.
 *  [CommWall]   juhe.plus "communication wall" explainer: router example
 *               (token -> two experts), EP=8 placement example (GPU g owns
 *               experts 8g..8g+7), the 2*T*k*H*b traffic formula.
 *  [NCCL-EP]    hotelren.com NCCL EP article, s3.3: one flat send buffer cut
 *               into per-rank segments at prefix sums of sendcounts.
 *  [Sparse]     intelliparadigm.com sparse-communication article, s2.1:
 *               softmax + top-k router, capacity factor 1.0-1.25.
 *
 * Precision.  Gate weights and the combine sum are computed in double.  The
 * int8 code of an element and the expert stand-in output are integer/bf16
 * decisions; they are taken in fp32, the precision the GPU kernels use, so
 * both sides decide identically (IEEE fp32 divide/multiply, RNE).
 *
 * Every function returns 0 on success and a negative value when a
 * precondition fails (the oracle never guesses).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* bf16 <-> fp32, from the IEEE-754 definition                         */
/* ------------------------------------------------------------------ */

/* bf16 is the upper 16 bits of a binary32: exact widening. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static float bf16_to_float(uint16_t b)
{
    return (float)oracle_bf16_to_double(b);
}

static double magnitude_bits_to_double(uint32_t mag)
{
    float f;
    memcpy(&f, &mag, sizeof f);
    return (double)f;
}

/* Round a finite value to the nearest bf16, ties to the candidate whose
 * last mantissa bit is zero (round-half-to-even).  The two candidates are
 * the bf16 magnitudes just below and just above |v|; distances are taken
 * in double, where they are exact for any binary32 input. */
uint16_t oracle_float_to_bf16(float v)
{
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    uint32_t sign = u & 0x80000000u;
    uint32_t mag = u & 0x7fffffffu;
    if (mag > 0x7f800000u) /* NaN: keep it a quiet NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    if (mag == 0x7f800000u)
        return (uint16_t)(u >> 16);
    uint32_t lo = mag & 0xffff0000u;
    if (lo == mag)
        return (uint16_t)((sign | mag) >> 16);
    uint32_t hi = lo + 0x00010000u;
    double m = magnitude_bits_to_double(mag);
    double dlo = m - magnitude_bits_to_double(lo);
    /* the candidate above the largest finite bf16 is 2^128 (overflow) */
    double vhi = (hi == 0x7f800000u) ? ldexp(1.0, 128) : magnitude_bits_to_double(hi);
    double dhi = vhi - m;
    uint32_t pick;
    if (dlo < dhi)
        pick = lo;
    else if (dhi < dlo)
        pick = hi;
    else
        pick = ((lo >> 16) & 1u) ? hi : lo;
    return (uint16_t)((sign | pick) >> 16);
}

/* ------------------------------------------------------------------ */
/* O1  route: top-k experts per token, renormalised gate weights        */
/* ------------------------------------------------------------------ */
/* [Sparse] s2.1: the router scores every expert and keeps the top-k.
 * [CommWall] router example: each token goes to its k best experts.
 * Selection is on the fp32 logits (softmax is monotone, so the set and the
 * order are the same as on probabilities).  Order of the k outputs: by
 * descending logit; equal logits go to the lower expert id.
 * Weights: softmax over the selected k logits, which equals the full softmax
 * renormalised over the selected experts:
 *     w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max)   (double).
 * Returns -1 when a logit is not finite or a shape is invalid. */
int oracle_route_topk(const float *logits, int64_t T, int E, int k,
                      int32_t *idx, float *w)
{
    if (T < 0 || E < 1 || k < 1 || k > E)
        return -1;
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    double *a = (double *)malloc(sizeof(double) * (size_t)k);
    if (!taken || !a) {
        free(taken);
        free(a);
        return -2;
    }
    int rc = 0;
    for (int64_t t = 0; t < T && rc == 0; ++t) {
        const float *l = logits + t * (int64_t)E;
        for (int e = 0; e < E; ++e) {
            if (!isfinite(l[e])) {
                rc = -1;
                break;
            }
        }
        if (rc)
            break;
        memset(taken, 0, (size_t)E);
        /* k rounds of "largest remaining logit, lowest id on ties" */
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || l[e] > l[best])
                    best = e;
            }
            taken[best] = 1;
            idx[t * k + j] = best;
        }
        double m = (double)l[idx[t * k]];
        double s = 0.0;
        for (int j = 0; j < k; ++j) {
            a[j] = exp((double)l[idx[t * k + j]] - m);
            s += a[j];
        }
        for (int j = 0; j < k; ++j)
            w[t * k + j] = (float)(a[j] / s);
    }
    free(taken);
    free(a);
    return rc;
}

/* ------------------------------------------------------------------ */
/* O2  dispatch layout for one chunk                                    */
/* ------------------------------------------------------------------ */
/* Slot s = t_local*k + j carries token t_local's j-th expert.
 * [ThunderEP] s2.1: rows for one destination are gathered into one
 * contiguous block, so at most R blocks leave the GPU.
 * [CommWall] EP placement: experts are split into R contiguous blocks of
 * E/R; expert e lives on rank e / (E/R).
 * [NCCL-EP] s3.3: rank r's segment of the flat send buffer starts at the sum
 * of the earlier ranks' counts.
 * [Sparse] s2.1: a capacity limits how many rows an expert takes; rows past
 * it are dropped (the lowest token ids are kept).  capacity <= 0: no limit.
 * Rows are ordered by (rank, expert, token id); since rank blocks are
 * contiguous ranges of experts this is the (expert, token id) order.
 * Outputs (all int32):
 *   expert_counts[E]    raw histogram (sums to Tc*k)
 *   expert_offsets[E+1] exclusive scan of kept rows; [E] = N
 *   rank_counts[R], rank_offsets[R+1]
 *   pos[Tc*k]           row of each slot, -1 when dropped
 *   row_src[Tc*k]       slot of each row, -1 for rows >= N */
int oracle_dispatch_layout(const int32_t *idx, int64_t Tc, int E, int k, int R,
                           int64_t capacity, int32_t *expert_counts,
                           int32_t *expert_offsets, int32_t *rank_counts,
                           int32_t *rank_offsets, int32_t *pos, int32_t *row_src)
{
    if (Tc < 0 || E < 1 || k < 1 || k > E || R < 1 || E % R != 0)
        return -1;
    int64_t S = Tc * (int64_t)k;
    int64_t *kept = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    int64_t *fill = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    int64_t *cnt = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    if (!kept || !fill || !cnt) {
        free(kept);
        free(fill);
        free(cnt);
        return -2;
    }
    for (int64_t s = 0; s < S; ++s) {
        int32_t e = idx[s];
        if (e < 0 || e >= E) {
            free(kept);
            free(fill);
            free(cnt);
            return -1;
        }
        cnt[e] += 1;
    }
    for (int e = 0; e < E; ++e) {
        expert_counts[e] = (int32_t)cnt[e];
        kept[e] = (capacity > 0 && cnt[e] > capacity) ? capacity : cnt[e];
    }
    int64_t run = 0;
    for (int e = 0; e < E; ++e) {
        expert_offsets[e] = (int32_t)run;
        run += kept[e];
    }
    expert_offsets[E] = (int32_t)run;
    int64_t N = run;
    int per_rank = E / R;
    for (int r = 0; r < R; ++r) {
        int64_t c = 0;
        for (int e = r * per_rank; e < (r + 1) * per_rank; ++e)
            c += kept[e];
        rank_counts[r] = (int32_t)c;
        rank_offsets[r] = expert_offsets[r * per_rank];
    }
    rank_offsets[R] = (int32_t)N;

    /* the defining sequential loop: token order, then slot order */
    for (int64_t s = 0; s < S; ++s)
        row_src[s] = -1;
    for (int64_t t = 0; t < Tc; ++t) {
        for (int j = 0; j < k; ++j) {
            int64_t s = t * k + j;
            int32_t e = idx[s];
            if (fill[e] < kept[e]) {
                int64_t p = expert_offsets[e] + fill[e];
                pos[s] = (int32_t)p;
                row_src[p] = (int32_t)s;
                fill[e] += 1;
            } else {
                pos[s] = -1;
            }
        }
    }
    free(kept);
    free(fill);
    free(cnt);
    return 0;
}

/* ------------------------------------------------------------------ */
/* int8 row record: H codes, the fp32 scale, 12 zero bytes (H+16 bytes) */
/* ------------------------------------------------------------------ */
/* [ThunderEP] s2.3: per-token dynamic quantisation, one scale per token,
 * computed at run time: scale = max|x| / 127.  A code is x / scale rounded
 * to nearest (ties to even) and clamped to [-127, 127]; an all-zero row has
 * scale 0 and zero codes.  Both divisions are single IEEE fp32 divisions. */
static void quantise_row_int8(const float *v, int H, uint8_t *rec)
{
    float a = 0.0f;
    for (int h = 0; h < H; ++h) {
        float m = fabsf(v[h]);
        if (m > a)
            a = m;
    }
    float scale = a / 127.0f;
    int8_t *codes = (int8_t *)rec;
    for (int h = 0; h < H; ++h) {
        if (a == 0.0f) {
            codes[h] = 0;
            continue;
        }
        float r = nearbyintf(v[h] / scale);
        if (r > 127.0f)
            r = 127.0f;
        if (r < -127.0f)
            r = -127.0f;
        codes[h] = (int8_t)r;
    }
    if (a == 0.0f)
        scale = 0.0f;
    memcpy(rec + H, &scale, sizeof scale);
    memset(rec + H + 4, 0, 12);
}

/* ------------------------------------------------------------------ */
/* int4 row record: H/2 bytes of codes, two per byte (element 2i in the  */
/* low nibble, 2i+1 in the high nibble, 4-bit two's complement), the     */
/* fp32 scale, 12 zero bytes (H/2 + 16 bytes)                            */
/* ------------------------------------------------------------------ */
/* [ThunderEP] s5.2 names 4-bit payloads as the next, more aggressive
 * compression step (with an accuracy caveat).  Read here as the int8 rule
 * with 4-bit codes: scale = max|x| / 7 and code = x / scale rounded to
 * nearest (ties to even), clamped to [-7, 7] (-8 unused, as -128 is for
 * int8); an all-zero row has scale 0 and zero codes.  Single IEEE fp32
 * divisions. */
static void quantise_row_int4(const float *v, int H, uint8_t *rec)
{
    float a = 0.0f;
    for (int h = 0; h < H; ++h) {
        float m = fabsf(v[h]);
        if (m > a)
            a = m;
    }
    float scale = a / 7.0f;
    memset(rec, 0, (size_t)H / 2);
    for (int h = 0; h < H; ++h) {
        int code = 0;
        if (a != 0.0f) {
            float r = nearbyintf(v[h] / scale);
            if (r > 7.0f)
                r = 7.0f;
            if (r < -7.0f)
                r = -7.0f;
            code = (int)r;
        }
        uint8_t nib = (uint8_t)(code & 0xF);
        rec[h / 2] |= (h % 2 == 0) ? nib : (uint8_t)(nib << 4);
    }
    if (a == 0.0f)
        scale = 0.0f;
    memcpy(rec + H / 2, &scale, sizeof scale);
    memset(rec + H / 2 + 4, 0, 12);
}

/* ------------------------------------------------------------------ */
/* fp8 row record: H OCP E4M3 codes, the fp32 scale, 12 zero bytes       */
/* (H + 16 bytes)                                                        */
/* ------------------------------------------------------------------ */
/* The NCCL EP article (s6.3) sends expert traffic as FP8 (e4m3) and keeps
 * the routing scores in higher precision.  Read here as the int8 rule with
 * an FP8 code: per-token scale = max|x| / 448 (448 = the largest finite
 * E4M3 value), code = E4M3(x / scale) rounded to nearest, ties to even
 * (fp32 division); an all-zero row has scale 0 and zero codes.
 *
 * OCP E4M3 (from the format's definition): 1 sign, 4 exponent (bias 7),
 * 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; no
 * infinities; S.1111.111 is NaN; the largest finite magnitude is
 * S.1111.110 = 1.75 * 2^8 = 448. */
/* 2^n as a binary32, from the encoding: biased exponent n + 127, zero
 * mantissa (-126 <= n <= 127). */
static float pow2f(int n)
{
    uint32_t u = (uint32_t)(n + 127) << 23;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float e4m3_decode(uint8_t c)
{
    int sgn = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    float mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ((float)m / 8.0f) * pow2f(-6);          /* subnormal: m/8 * 2^-6 */
    else
        mag = (1.0f + (float)m / 8.0f) * pow2f(e - 7);  /* normal: 1.m * 2^(e-7) */
    return sgn ? -mag : mag;
}

/* Nearest E4M3 code of a finite v with |v| <= 464 (beyond 448 + half a step
 * the value would not round to 448), ties to the even mantissa.  The finite
 * non-negative codes 0x00..0x7E increase with their value: binary search
 * for the last code whose value is <= |v|, then take the nearer of it and
 * the next code. */
static uint8_t e4m3_encode(float v)
{
    uint8_t sgn = (v < 0.0f || (v == 0.0f && signbit(v))) ? 0x80 : 0x00;
    double a = fabs((double)v);
    int lo = 0, hi = 0x7E;  /* value(lo) <= a; find the last such code */
    if (a >= (double)e4m3_decode(0x7E))
        return (uint8_t)(sgn | 0x7E);
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if ((double)e4m3_decode((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    /* value(lo) <= a < value(lo + 1) */
    double below = (double)e4m3_decode((uint8_t)lo);
    double above = (double)e4m3_decode((uint8_t)(lo + 1));
    double mid = 0.5 * (below + above);
    int c = lo;
    if (a > mid || (a == mid && ((lo + 1) & 1) == 0))
        c = lo + 1;
    return (uint8_t)(sgn | c);
}

float oracle_e4m3_decode(uint8_t c) { return e4m3_decode(c); }
uint8_t oracle_e4m3_encode(float v) { return e4m3_encode(v); }

static void quantise_row_fp8(const float *v, int H, uint8_t *rec)
{
    float a = 0.0f;
    for (int h = 0; h < H; ++h) {
        float m = fabsf(v[h]);
        if (m > a)
            a = m;
    }
    float scale = a / 448.0f;
    for (int h = 0; h < H; ++h)
        rec[h] = (a == 0.0f) ? 0 : e4m3_encode(v[h] / scale);
    if (a == 0.0f)
        scale = 0.0f;
    memcpy(rec + H, &scale, sizeof scale);
    memset(rec + H + 4, 0, 12);
}

static void quantise_row(const float *v, int H, int quant, uint8_t *rec)
{
    if (quant == 1)
        quantise_row_int8(v, H, rec);
    else if (quant == 2)
        quantise_row_int4(v, H, rec);
    else
        quantise_row_fp8(v, H, rec);
}

/* value of element h of a row record, in fp32 */
static float dequant_element(const uint8_t *rec, int quant, int H, int h)
{
    if (quant == 0) {
        uint16_t b;
        memcpy(&b, rec + 2 * (size_t)h, 2);
        return bf16_to_float(b);
    }
    float scale;
    if (quant == 1) {
        memcpy(&scale, rec + H, sizeof scale);
        float q = (float)((const int8_t *)rec)[h];
        return q * scale;
    }
    if (quant == 3) {
        memcpy(&scale, rec + H, sizeof scale);
        return e4m3_decode(rec[h]) * scale;
    }
    memcpy(&scale, rec + H / 2, sizeof scale);
    int nib = (h % 2 == 0) ? (rec[h / 2] & 0xF) : (rec[h / 2] >> 4);
    int code = nib >= 8 ? nib - 16 : nib;
    return (float)code * scale;
}

int64_t oracle_record_bytes(int H, int quant)
{
    if (quant == 0)
        return 2 * (int64_t)H;
    if (quant == 1)
        return (int64_t)H + 16;
    if (quant == 2)
        return (int64_t)H / 2 + 16;
    if (quant == 3)
        return (int64_t)H + 16;
    return -1;
}

static int quant_ok(int quant, int H)
{
    return quant == 0 || quant == 1 || quant == 3 || (quant == 2 && H % 2 == 0);
}

/* ------------------------------------------------------------------ */
/* O3  dispatch pack for one chunk                                      */
/* ------------------------------------------------------------------ */
/* Row pos[s] of the send buffer receives token s/k's hidden row: a plain
 * copy of the bf16 bits, or its int8 record.  Rows with no slot are left
 * untouched. */
int oracle_dispatch_pack(const uint16_t *x, int64_t Tc, int H, int k,
                         const int32_t *pos, int quant, uint8_t *send)
{
    if (Tc < 0 || H < 1 || k < 1 || !quant_ok(quant, H))
        return -1;
    int64_t stride = oracle_record_bytes(H, quant);
    float *v = (float *)malloc(sizeof(float) * (size_t)H);
    if (!v)
        return -2;
    for (int64_t s = 0; s < Tc * k; ++s) {
        int32_t p = pos[s];
        if (p < 0)
            continue;
        const uint16_t *row = x + (s / k) * (int64_t)H;
        uint8_t *rec = send + (int64_t)p * stride;
        if (quant == 0) {
            memcpy(rec, row, 2 * (size_t)H);
        } else {
            for (int h = 0; h < H; ++h)
                v[h] = bf16_to_float(row[h]);
            quantise_row(v, H, quant, rec);
        }
    }
    free(v);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O5  expert stand-in (test harness; replaces the expert FFN)          */
/* ------------------------------------------------------------------ */
/* Row p (p < N = expert_offsets[E]) belongs to the expert e whose bucket
 * [expert_offsets[e], expert_offsets[e+1]) holds it.  Output row:
 *     y = bf16_rne( v * (1 + e/8) )   (fp32 multiply; 1 + e/8 is exact)
 * where v is the dequantised input row.  With quant_out = 1 (2) the bf16 row y
 * is re-quantised to an int8 (int4) record with the dispatch rule. */
int oracle_expert_standin(const uint8_t *recv, int quant_in,
                          const int32_t *expert_offsets, int E, int H,
                          int quant_out, uint8_t *ret)
{
    if (E < 1 || H < 1 || !quant_ok(quant_in, H) || !quant_ok(quant_out, H))
        return -1;
    int64_t sin = oracle_record_bytes(H, quant_in);
    int64_t sout = oracle_record_bytes(H, quant_out);
    int64_t N = expert_offsets[E];
    float *y = (float *)malloc(sizeof(float) * (size_t)H);
    if (!y)
        return -2;
    for (int64_t p = 0; p < N; ++p) {
        int e = 0;
        while (!(expert_offsets[e] <= p && p < expert_offsets[e + 1]))
            ++e;
        float f = 1.0f + (float)e / 8.0f;
        const uint8_t *rin = recv + p * sin;
        uint8_t *rout = ret + p * sout;
        for (int h = 0; h < H; ++h) {
            float v = dequant_element(rin, quant_in, H, h);
            uint16_t b = oracle_float_to_bf16(v * f);
            if (quant_out == 0)
                memcpy(rout + 2 * (size_t)h, &b, 2);
            else
                y[h] = bf16_to_float(b);
        }
        if (quant_out)
            quantise_row(y, H, quant_out, rout);
    }
    free(y);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O6  combine for one chunk                                            */
/* ------------------------------------------------------------------ */
/* [ThunderEP] s1.3: the results come back to the token's own GPU, which
 * forms the gate-weighted sum over the token's k experts:
 *     out[t,h] = bf16( sum_{j : pos[t,j] >= 0} w[t,j] * deq(ret[pos[t,j]])[h] )
 * summed in double in slot order.  The sum of the kept terms starts from
 * -0.0, the IEEE identity of addition, so a single kept term is returned
 * unchanged (sign of zero included: permute-then-unpermute is the identity);
 * a token whose slots were all dropped gets +0. */
int oracle_combine(const uint8_t *ret, int quant, const int32_t *pos,
                   const float *w, int64_t Tc, int H, int k, uint16_t *out)
{
    if (Tc < 0 || H < 1 || k < 1 || !quant_ok(quant, H))
        return -1;
    int64_t stride = oracle_record_bytes(H, quant);
    for (int64_t t = 0; t < Tc; ++t) {
        for (int h = 0; h < H; ++h) {
            double acc = -0.0;
            int kept = 0;
            for (int j = 0; j < k; ++j) {
                int32_t p = pos[t * k + j];
                if (p < 0)
                    continue;
                float d = dequant_element(ret + (int64_t)p * stride, quant, H, h);
                acc += (double)w[t * k + j] * (double)d;
                kept += 1;
            }
            if (kept == 0)
                acc = 0.0;
            out[t * (int64_t)H + h] = oracle_float_to_bf16((float)acc);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Per-token reference for sampled checks at full size                  */
/* ------------------------------------------------------------------ */
/* With the exchange an identity and no expert between dispatch and combine,
 * each kept row of token t is token t's own record, so out[t] depends on
 * x[t], w[t,:] and which slots were kept only.  This evaluates O3 then O6 for
 * one token without building the whole send buffer. */
int oracle_roundtrip_token(const uint16_t *xrow, int H, int k,
                           const int32_t *pos_t, const float *w_t, int quant,
                           uint16_t *out_row)
{
    if (H < 1 || k < 1 || !quant_ok(quant, H))
        return -1;
    int64_t stride = oracle_record_bytes(H, quant);
    uint8_t *rec = (uint8_t *)malloc((size_t)stride);
    float *v = (float *)malloc(sizeof(float) * (size_t)H);
    if (!rec || !v) {
        free(rec);
        free(v);
        return -2;
    }
    if (quant == 0) {
        memcpy(rec, xrow, 2 * (size_t)H);
    } else {
        for (int h = 0; h < H; ++h)
            v[h] = bf16_to_float(xrow[h]);
        quantise_row(v, H, quant, rec);
    }
    for (int h = 0; h < H; ++h) {
        double acc = -0.0;
        int kept = 0;
        for (int j = 0; j < k; ++j) {
            if (pos_t[j] < 0)
                continue;
            acc += (double)w_t[j] * (double)dequant_element(rec, quant, H, h);
            kept += 1;
        }
        if (kept == 0)
            acc = 0.0;
        out_row[h] = oracle_float_to_bf16((float)acc);
    }
    free(rec);
    free(v);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Receiver side of the exchange (R ranks, every rank a source and a   */
/* receiver)                                                           */
/* ------------------------------------------------------------------ */
/* [NCCL-EP] s3.3: a rank's send buffer is one flat block cut into R
 * segments at the prefix sums of its per-rank counts, segment r going to
 * rank r; the receive buffer is laid out the same way, the segment from
 * source s starting at the sum of the counts received from sources < s.
 * [CommWall] EP=8 placement: rank r owns the contiguous experts
 * [r*E/R, (r+1)*E/R).  [Perseus] s1.1: the experts then run on the tokens
 * a rank received, so the receiver gathers each expert's rows together.
 *
 * Input of all three functions: src_offsets[s*(E+1) + e], the kept expert
 * offsets of source s's dispatch layout (oracle_dispatch_layout's
 * expert_offsets), as the count exchange hands them to every rank.  Source
 * s's segment for rank r is its rows [src_offsets[s][r*E/R],
 * src_offsets[s][(r+1)*E/R]).
 *
 * All receivers' buffers are laid end to end in rank order (one flat
 * buffer, as when every rank is simulated on one device).  Order of the
 * grouped buffer: expert ascending, then source ascending, then arrival
 * order inside the source's segment. */

static int32_t kept_rows(const int32_t *src_offsets, int E, int s, int e)
{
    const int32_t *o = src_offsets + (int64_t)s * (E + 1);
    return o[e + 1] - o[e];
}

/* recv_offsets[r*(R+1) + s]: first row (flat) of source s's segment in
 *                             receiver r's region; [r*(R+1) + R] = its end.
 * group_offsets[E+1]:         first row (flat) of expert e in the grouped
 *                             buffer; [E] = total rows N.
 * group_seg[e*R + s]:         first row (flat) of source s's rows of expert
 *                             e in the grouped buffer.
 * group_pos[max_rows]:        grouped row of receive row q (q < N), -1 for
 *                             q >= N.
 * group_src[max_rows]:        receive row held by grouped row p (p < N), -1
 *                             for p >= N.  Requires N <= max_rows. */
int oracle_recv_layout(const int32_t *src_offsets, int R, int E, int64_t max_rows,
                       int32_t *recv_offsets, int32_t *group_offsets, int32_t *group_seg,
                       int32_t *group_pos, int32_t *group_src)
{
    if (R < 1 || E < 1 || E % R != 0 || max_rows < 0)
        return -1;
    const int per_rank = E / R;
    for (int s = 0; s < R; ++s)
        for (int e = 0; e < E; ++e)
            if (kept_rows(src_offsets, E, s, e) < 0)
                return -1;
    /* receive buffers: rank by rank, source by source */
    int64_t row = 0;
    for (int r = 0; r < R; ++r) {
        for (int s = 0; s < R; ++s) {
            recv_offsets[r * (R + 1) + s] = (int32_t)row;
            for (int e = r * per_rank; e < (r + 1) * per_rank; ++e)
                row += kept_rows(src_offsets, E, s, e);
        }
        recv_offsets[r * (R + 1) + R] = (int32_t)row;
    }
    /* grouped buffer: expert by expert, source by source */
    row = 0;
    for (int e = 0; e < E; ++e) {
        group_offsets[e] = (int32_t)row;
        for (int s = 0; s < R; ++s) {
            group_seg[e * R + s] = (int32_t)row;
            row += kept_rows(src_offsets, E, s, e);
        }
    }
    group_offsets[E] = (int32_t)row;
    if (row > max_rows)
        return -1;
    /* row maps: walk the receive order, each run placed by its segment start */
    for (int64_t i = 0; i < max_rows; ++i) {
        group_pos[i] = -1;
        group_src[i] = -1;
    }
    int64_t q = 0;
    for (int r = 0; r < R; ++r)
        for (int s = 0; s < R; ++s)
            for (int e = r * per_rank; e < (r + 1) * per_rank; ++e) {
                const int64_t n = kept_rows(src_offsets, E, s, e);
                for (int64_t i = 0; i < n; ++i, ++q) {
                    const int64_t p = group_seg[e * R + s] + i;
                    group_pos[q] = (int32_t)p;
                    group_src[p] = (int32_t)q;
                }
            }
    return 0;
}

/* The payload all-to-all as a block transpose.  Source s's send buffer
 * starts at row s*source_rows of `send`; its segment for rank r is copied to
 * the next free rows of receiver r's region (regions and segments in rank
 * order).  reverse != 0 copies the other way (the return exchange of the
 * combine direction): recv -> send. */
int oracle_exchange(uint8_t *send, int64_t source_rows, const int32_t *src_offsets, int R, int E,
                    int64_t row_bytes, uint8_t *recv, int reverse)
{
    if (R < 1 || E < 1 || E % R != 0 || source_rows < 0 || row_bytes < 1)
        return -1;
    const int per_rank = E / R;
    int64_t q = 0;  /* next row of the flat receive buffer */
    for (int r = 0; r < R; ++r) {
        for (int s = 0; s < R; ++s) {
            const int32_t *o = src_offsets + (int64_t)s * (E + 1);
            const int64_t first = o[r * per_rank];
            const int64_t n = (int64_t)o[(r + 1) * per_rank] - first;
            if (n < 0 || first + n > source_rows)
                return -1;
            for (int64_t i = 0; i < n; ++i, ++q) {
                uint8_t *a = send + (s * source_rows + first + i) * row_bytes;
                uint8_t *b = recv + q * row_bytes;
                if (reverse)
                    memcpy(a, b, (size_t)row_bytes);
                else
                    memcpy(b, a, (size_t)row_bytes);
            }
        }
    }
    return 0;
}

/* Regroup the flat receive buffer (rank, source, expert order) into the
 * grouped buffer (expert, source order), by walking both orders with
 * running row counters.  reverse != 0 copies grouped -> recv (after the
 * experts, before the return exchange). */
int oracle_regroup(uint8_t *recv, const int32_t *src_offsets, int R, int E, int64_t row_bytes,
                   uint8_t *grouped, int reverse)
{
    if (R < 1 || E < 1 || E % R != 0 || row_bytes < 1)
        return -1;
    const int per_rank = E / R;
    /* where each (expert, source) run starts in the grouped buffer */
    int64_t *gstart = (int64_t *)malloc(sizeof(int64_t) * (size_t)E * (size_t)R);
    if (!gstart)
        return -2;
    int64_t row = 0;
    for (int e = 0; e < E; ++e)
        for (int s = 0; s < R; ++s) {
            gstart[(int64_t)e * R + s] = row;
            row += kept_rows(src_offsets, E, s, e);
        }
    int64_t q = 0;  /* arrival order in the receive buffer */
    for (int r = 0; r < R; ++r)
        for (int s = 0; s < R; ++s)
            for (int e = r * per_rank; e < (r + 1) * per_rank; ++e) {
                const int64_t n = kept_rows(src_offsets, E, s, e);
                for (int64_t i = 0; i < n; ++i, ++q) {
                    uint8_t *a = recv + q * row_bytes;
                    uint8_t *b = grouped + (gstart[(int64_t)e * R + s] + i) * row_bytes;
                    if (reverse)
                        memcpy(a, b, (size_t)row_bytes);
                    else
                        memcpy(b, a, (size_t)row_bytes);
                }
            }
    free(gstart);
    return 0;
}
