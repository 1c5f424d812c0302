/*
 * CPU oracle for compact (DMS-style) decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * includes this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header, table or helper with the HIP
 * path: the FP8 codec, the compaction and the attention below are written
 * out again, from their definitions, in plain C.
 *
 * What it computes, and where that comes from:
 *   - FastDMS page ("FastDMS: 6.4X KV-cache compression running faster than
 *     vLLM BF16/FP8"), DMS paragraph: every (layer, KV head) keeps only the
 *     tokens its learned eviction decision retains.  Here that decision is an
 *     input: one keep byte per (sequence, KV head, position), nonzero = keep.
 *   - Same page, release paragraph: a compact KV store that physically
 *     reclaims evicted slots.  Read as an order-preserving stream compaction
 *     of the kept rows into one packed segment per (sequence, KV head).
 *   - Same page, memory-table paragraph: "KV/stage memory is cache or cache +
 *     staging".  Read as an always-kept window of the W most recent tokens
 *     (including the current one) held in a ring in front of each segment.
 *   - Same page, summary bullets: FastDMS runs in BF16 and FP8.  FP8 is OCP
 *     E4M3FN (OCP 8-bit Floating Point specification, E4M3 encoding table),
 *     with one absmax scale per (sequence, KV head) for K and one for V.
 *   - A 4-bit store (same page, memory table, the 4-bit vLLM row; PackKV
 *     page, abstract: compressed KV decoded inside the products): the page
 *     does not define its format.  Reading: the OCP Microscaling FP4 element
 *     type E2M1 with the same per-(sequence, KV head) absmax scales as FP8,
 *     two elements per byte (element d in the low nibble of byte d/2 when d
 *     is even, the high nibble when odd).
 *   - Attention: plain scaled-dot-product softmax attention of one query
 *     token over the stored set, in fp64, in position order; no blocking,
 *     no split, no reordering.
 *
 * Readings where the pages are silent are listed with each function.
 * Build: gcc -O2 -fPIC -shared -fopenmp -ffp-contract=off -fno-fast-math
 * (x86-64 SSE arithmetic, so every float operation below is a single IEEE
 * rounding).  Independent (sequence, head) units are spread over OpenMP
 * threads; the arithmetic of each unit is sequential, so the results do not
 * depend on the number of threads.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BF16 0
#define ORC_FP8 1
#define ORC_FP4 2

/* Threads the loops over independent units use (n < 1: all cores). */
void orc_set_threads(int n)
{
    omp_set_num_threads(n > 0 ? n : omp_get_num_procs());
}

int orc_max_threads(void)
{
    return omp_get_max_threads();
}

/* Bytes of one stored row of D elements. */
static int64_t row_bytes(int D, int kv_dtype)
{
    return kv_dtype == ORC_BF16 ? 2 * (int64_t)D : kv_dtype == ORC_FP8 ? D : D / 2;
}

/* ------------------------------------------------------------------ */
/* Scalars                                                             */
/* ------------------------------------------------------------------ */

/* bfloat16 bit pattern -> float: the upper half of an IEEE binary32. */
static float bf16_to_f32(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * OCP OFP8 E4M3FN encode, round-to-nearest-even, saturating to the largest
 * finite magnitude.  Written from the value definition: the codes are
 * sign | E(4 bits, bias 7) | M(3 bits); normal values 2^(E-7) * (1 + M/8)
 * for E = 1..15 (E = 15, M = 7 is NaN, so the largest finite is 448);
 * subnormal values 2^-6 * M/8 for E = 0.
 * Readings: magnitudes >= 448 (including infinity) encode as +-448; NaN
 * encodes as the NaN code with the input's sign; the sign of zero and of
 * values that round to zero is kept.
 */
uint8_t orc_e4m3_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    if (isnan(y))
        return sign | 0x7F;
    double a = fabs((double)y);
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: a multiple of 2^-9, rounded half to even.  A
         * result of 8 is the smallest normal, whose code is also 8. */
        double m = rint(a * 512.0);
        return sign | (uint8_t)m;
    }
    int k;
    double f = frexp(a, &k);          /* a = f * 2^k, f in [0.5, 1) */
    int e = k - 1;                    /* a = (2f) * 2^e, 2f in [1, 2) */
    double m = rint((2.0 * f - 1.0) * 8.0);
    if (m == 8.0) {                   /* rounded up to the next binade */
        m = 0.0;
        e += 1;
    }
    int code = ((e + 7) << 3) | (int)m;
    if (code > 0x7E)
        code = 0x7E;
    return sign | (uint8_t)code;
}

/* OCP OFP8 E4M3FN decode (exact). */
double orc_e4m3_decode(uint8_t c)
{
    int s = c >> 7, E = (c >> 3) & 15, M = c & 7;
    if (E == 15 && M == 7)
        return NAN;
    double v = (E == 0) ? ldexp((double)M, -9) : ldexp((double)(8 + M), E - 10);
    return s ? -v : v;
}

/*
 * OCP MX FP4 E2M1 encode, round-to-nearest-even, saturating.  Codes are
 * sign | E(2 bits, bias 1) | M(1 bit); E = 1..3 stands for 2^(E-1) * (1 + M/2)
 * (1, 1.5, 2, 3, 4, 6), E = 0 for M * 0.5 (0, 0.5).  The format has no
 * infinity and no NaN.  Readings: magnitudes that round past 6 (and
 * infinity) give +-6; NaN gives +-6 with the input's sign; the sign of zero
 * and of values that round to zero is kept.  Returns the 4-bit code.
 */
uint8_t orc_e2m1_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x8 : 0x0;
    if (isnan(y))
        return sign | 0x7;
    double a = fabs((double)y);
    if (a >= 6.0)                     /* 6 and above (infinity too): +-6 */
        return sign | 0x7;
    if (a < 1.0) {
        /* multiples of 0.5, rounded half to even: 2 is the code of 1.0 */
        return sign | (uint8_t)rint(a * 2.0);
    }
    int k;
    double f = frexp(a, &k);          /* a = f * 2^k, f in [0.5, 1) */
    int e = k - 1;                    /* a = (2f) * 2^e, 2f in [1, 2) */
    double m = rint((2.0 * f - 1.0) * 2.0);
    if (m == 2.0) {                   /* rounded up to the next binade */
        m = 0.0;
        e += 1;
    }
    int code = ((e + 1) << 1) | (int)m;
    if (code > 0x7)
        code = 0x7;
    return sign | (uint8_t)code;
}

/* OCP MX FP4 E2M1 decode of a 4-bit code (exact). */
double orc_e2m1_decode(uint8_t c)
{
    int s = (c >> 3) & 1, E = (c >> 1) & 3, M = c & 1;
    double v = (E == 0) ? 0.5 * M : ldexp(1.0 + 0.5 * M, E - 1);
    return s ? -v : v;
}

/*
 * Per-head FP8 scales from an absmax a.  s dequantises (x ~ s * code), inv
 * quantises (code = enc(x * inv)).  Reading: both are single f32 divisions of
 * a and the format's largest finite value 448; a head whose absmax is zero
 * or not finite gets s = inv = 1.
 */
void orc_scales_from_amax(float amax, float *s, float *inv)
{
    if (amax > 0.0f && isfinite(amax)) {
        *s = amax / 448.0f;
        *inv = 448.0f / amax;
    } else {
        *s = 1.0f;
        *inv = 1.0f;
    }
}

/* The same for the 4-bit store, whose largest magnitude is 6. */
void orc_fp4_scales_from_amax(float amax, float *s, float *inv)
{
    if (amax > 0.0f && isfinite(amax)) {
        *s = amax / 6.0f;
        *inv = 6.0f / amax;
    } else {
        *s = 1.0f;
        *inv = 1.0f;
    }
}

/* Scales of a head for a quantised store (FP8 or FP4); 1 for BF16. */
static void head_scales(int kv_dtype, float amax, float *s, float *inv)
{
    *s = 1.0f;
    *inv = 1.0f;
    if (kv_dtype == ORC_FP8)
        orc_scales_from_amax(amax, s, inv);
    else if (kv_dtype == ORC_FP4)
        orc_fp4_scales_from_amax(amax, s, inv);
}

/*
 * Is position p in the stored set after the token at position P was
 * appended?  Stored = the W most recent positions P-W+1..P (the staging
 * window) plus every earlier position whose keep byte is nonzero.
 */
static int is_stored(const uint8_t *keep_row, int P, int W, int p)
{
    if (p < 0 || p > P)
        return 0;
    if (p > P - W)
        return 1;
    return keep_row[p] != 0;
}

int64_t orc_stored_count(const uint8_t *keep_row, int P, int W)
{
    int64_t n = 0;
    for (int p = 0; p <= P; ++p)
        n += is_stored(keep_row, P, W, p);
    return n;
}

/* ------------------------------------------------------------------ */
/* Prefill compaction                                                  */
/* ------------------------------------------------------------------ */

/*
 * Layout of the compact store after a prefill of T tokens (FastDMS page,
 * release paragraph, "physically reclaims evicted slots"; readings below).
 * For head i = b*Hkv + h:
 *   comp_len[i]  = number of kept positions p <= T-1-W
 *   seg_cap[i]   = comp_len[i] + reserve          (room for decode growth)
 *   seg_base[i]  = sum over j < i of roundup(W + seg_cap[j], align);
 *                  seg_base[B*Hkv] = total rows.  align >= 1 is a storage
 *                  granularity of the store (1 = no padding).
 *   segment rows = W ring rows, then seg_cap compact rows
 *   dst[i*T + p] = ring row p mod W for the W most recent positions,
 *                  W + (rank of p among the kept older positions) for a kept
 *                  older position (ascending position order), -1 if evicted.
 * keep is [B*Hkv] rows of keep_ld bytes.
 */
void orc_prefill_layout(int B, int Hkv, int T, int W, int reserve, int align,
                        const uint8_t *keep, int64_t keep_ld,
                        int32_t *comp_len, int32_t *seg_cap, int64_t *seg_base,
                        int32_t *dst)
{
    int64_t base = 0;
    for (int i = 0; i < B * Hkv; ++i) {
        const uint8_t *row = keep + (int64_t)i * keep_ld;
        int32_t n = 0;
        for (int p = 0; p < T; ++p) {
            int32_t d = -1;
            if (p > T - 1 - W)
                d = p % W;
            else if (row[p] != 0)
                d = W + n++;
            if (dst)
                dst[(int64_t)i * T + p] = d;
        }
        comp_len[i] = n;
        seg_cap[i] = n + reserve;
        seg_base[i] = base;
        int64_t size = (int64_t)W + n + reserve;
        base += (size + align - 1) / align * align;
    }
    seg_base[B * Hkv] = base;
}

/*
 * Absmax of K and of V per head over the stored prefill tokens S(T-1)
 * (reading: the scale covers exactly what is stored, and is then frozen for
 * the decode steps).  |bf16| is exact in f32.  A NaN anywhere makes the
 * absmax NaN (and so the scale falls back to 1).
 * k, v: bf16 bit patterns, element (b, t, h, d) at b*sb + t*st + h*sh + d.
 */
void orc_prefill_amax(int B, int Hkv, int D, int T, int W,
                      const uint16_t *k, const uint16_t *v,
                      int64_t sb, int64_t st, int64_t sh,
                      const uint8_t *keep, int64_t keep_ld,
                      float *k_amax, float *v_amax)
{
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hkv; ++h) {
            int i = b * Hkv + h;
            const uint8_t *row = keep + (int64_t)i * keep_ld;
            float mk = 0.0f, mv = 0.0f;
            for (int p = 0; p < T; ++p) {
                if (!is_stored(row, T - 1, W, p))
                    continue;
                for (int d = 0; d < D; ++d) {
                    int64_t off = b * sb + p * st + h * sh + d;
                    float ak = fabsf(bf16_to_f32(k[off]));
                    float av = fabsf(bf16_to_f32(v[off]));
                    if (isnan(ak) || ak > mk)
                        mk = ak;
                    if (isnan(av) || av > mv)
                        mv = av;
                }
            }
            k_amax[i] = mk;
            v_amax[i] = mv;
        }
}

/* Store one D-element row: BF16 bits verbatim, or FP8 / FP4 codes of
 * x * inv (FP4: two codes per byte, even element in the low nibble). */
static int64_t store_row(int D, int kv_dtype, const uint16_t *src, float inv,
                         uint8_t *dst_row)
{
    int64_t sat = 0;
    for (int d = 0; d < D; ++d) {
        if (kv_dtype == ORC_BF16) {
            dst_row[2 * d] = (uint8_t)(src[d] & 0xFF);
            dst_row[2 * d + 1] = (uint8_t)(src[d] >> 8);
        } else if (kv_dtype == ORC_FP8) {
            float y = bf16_to_f32(src[d]) * inv;
            if (fabsf(y) > 448.0f)
                ++sat;
            dst_row[d] = orc_e4m3_encode(y);
        } else {
            float y = bf16_to_f32(src[d]) * inv;
            if (fabsf(y) > 6.0f)
                ++sat;
            uint8_t c = orc_e2m1_encode(y);
            if (d % 2 == 0)
                dst_row[d / 2] = c;
            else
                dst_row[d / 2] |= (uint8_t)(c << 4);
        }
    }
    return sat;
}

/*
 * Prefill compaction of one layer: layout (orc_prefill_layout), scales
 * (scale_mode 0: computed by orc_prefill_amax; 1: k_amax/v_amax given), and
 * every stored row written to its pool row seg_base[i] + dst.  Rows the
 * layout leaves unused are not touched.  ring_keep[i*W + r] = keep bit (0/1)
 * of the position held in ring row r, 0 for a ring row not yet filled.
 * pos[b] = T.  Pools are [rows, D] elements of 2 (BF16) or 1 (FP8) bytes,
 * or half a byte (FP4, two per byte).
 * The caller passes pools of at least seg_base[B*Hkv] rows, obtained from
 * orc_prefill_layout with the same arguments.
 */
void orc_prefill_pack(int B, int Hkv, int D, int T, int W, int reserve,
                      int align, int kv_dtype, const uint16_t *k, const uint16_t *v,
                      int64_t sb, int64_t st, int64_t sh,
                      const uint8_t *keep, int64_t keep_ld, int scale_mode,
                      float *k_amax, float *v_amax, uint8_t *k_pool,
                      uint8_t *v_pool, uint8_t *ring_keep, int32_t *comp_len,
                      int32_t *seg_cap, int64_t *seg_base, int32_t *pos)
{
    int nh = B * Hkv;
    int32_t *dst = (int32_t *)malloc(sizeof(int32_t) * (size_t)nh * (size_t)(T > 0 ? T : 1));
    orc_prefill_layout(B, Hkv, T, W, reserve, align, keep, keep_ld, comp_len,
                       seg_cap, seg_base, dst);
    if (kv_dtype != ORC_BF16 && scale_mode == 0)
        orc_prefill_amax(B, Hkv, D, T, W, k, v, sb, st, sh, keep, keep_ld,
                         k_amax, v_amax);
    int64_t rowb = row_bytes(D, kv_dtype);
    for (int b = 0; b < B; ++b)
        pos[b] = T;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int i = b * Hkv + h;
            float ks, kinv, vs, vinv;
            head_scales(kv_dtype, kv_dtype == ORC_BF16 ? 0.0f : k_amax[i], &ks, &kinv);
            head_scales(kv_dtype, kv_dtype == ORC_BF16 ? 0.0f : v_amax[i], &vs, &vinv);
            for (int r = 0; r < W; ++r)
                ring_keep[(int64_t)i * W + r] = 0;
            const uint8_t *krow = keep + (int64_t)i * keep_ld;
            for (int p = 0; p < T; ++p) {
                int32_t d = dst[(int64_t)i * T + p];
                if (d < 0)
                    continue;
                if (d < W)
                    ring_keep[(int64_t)i * W + d] = krow[p] != 0;
                int64_t row = seg_base[i] + d;
                int64_t off = b * sb + p * st + h * sh;
                store_row(D, kv_dtype, k + off, kinv, k_pool + row * rowb);
                store_row(D, kv_dtype, v + off, vinv, v_pool + row * rowb);
            }
        }
    }
    free(dst);
}

/* ------------------------------------------------------------------ */
/* Decode-time append                                                  */
/* ------------------------------------------------------------------ */

/*
 * One decode step of one layer ("per-step compaction of new evictions").
 * For every sequence b (next position P = pos[b]) and head i:
 *   - W > 0: the token at P-W leaves the window.  If it exists and its keep
 *     bit is set, its ring row (P-W) mod W is copied, bytes unchanged, to the
 *     compact row W + comp_len[i] and comp_len[i] grows by one.  Then the new
 *     token is stored in ring row P mod W and its keep bit in ring_keep.
 *   - W = 0: the new token goes straight to the compact tail if kept.
 *   - A compact row beyond seg_cap[i] is not written; *err gets bit 0 and
 *     the token is lost.
 *   - pos[b] = P + 1.
 * New tokens use the frozen prefill scales and saturate.  k_new/v_new:
 * element (b, h, d) at b*sb + h*sh + d.  Returns the number of saturated FP8
 * elements.
 */
int64_t orc_append(int B, int Hkv, int D, int W, int kv_dtype,
                   const uint16_t *k_new, const uint16_t *v_new, int64_t sb,
                   int64_t sh, const uint8_t *keep_new,
                   const float *k_amax, const float *v_amax,
                   const int64_t *seg_base, const int32_t *seg_cap,
                   int32_t *comp_len, int32_t *pos, uint8_t *ring_keep,
                   uint8_t *k_pool, uint8_t *v_pool, int32_t *err)
{
    int64_t rowb = row_bytes(D, kv_dtype);
    int64_t sat = 0;
    int32_t errbits = 0;
#pragma omp parallel for collapse(2) reduction(+ : sat) reduction(| : errbits)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int P = pos[b];
            int i = b * Hkv + h;
            float ks, kinv, vs, vinv;
            head_scales(kv_dtype, kv_dtype == ORC_BF16 ? 0.0f : k_amax[i], &ks, &kinv);
            head_scales(kv_dtype, kv_dtype == ORC_BF16 ? 0.0f : v_amax[i], &vs, &vinv);
            int kept = keep_new[i] != 0;
            const uint16_t *kn = k_new + b * sb + h * sh;
            const uint16_t *vn = v_new + b * sb + h * sh;
            if (W > 0) {
                int pout = P - W;
                if (pout >= 0 && ring_keep[(int64_t)i * W + pout % W]) {
                    if (comp_len[i] < seg_cap[i]) {
                        int64_t from = seg_base[i] + pout % W;
                        int64_t to = seg_base[i] + W + comp_len[i];
                        memcpy(k_pool + to * rowb, k_pool + from * rowb, (size_t)rowb);
                        memcpy(v_pool + to * rowb, v_pool + from * rowb, (size_t)rowb);
                        comp_len[i] += 1;
                    } else {
                        errbits |= 1;
                    }
                }
                int64_t slot = seg_base[i] + P % W;
                sat += store_row(D, kv_dtype, kn, kinv, k_pool + slot * rowb);
                sat += store_row(D, kv_dtype, vn, vinv, v_pool + slot * rowb);
                ring_keep[(int64_t)i * W + P % W] = (uint8_t)kept;
            } else if (kept) {
                if (comp_len[i] < seg_cap[i]) {
                    int64_t to = seg_base[i] + comp_len[i];
                    sat += store_row(D, kv_dtype, kn, kinv, k_pool + to * rowb);
                    sat += store_row(D, kv_dtype, vn, vinv, v_pool + to * rowb);
                    comp_len[i] += 1;
                } else {
                    errbits |= 1;
                }
            }
        }
    }
    for (int b = 0; b < B; ++b)
        pos[b] += 1;
    *err |= errbits;
    return sat;
}

/* ------------------------------------------------------------------ */
/* Attention                                                           */
/* ------------------------------------------------------------------ */

/* The value a stored element stands for: the BF16 input itself, or the FP8
 * or FP4 code of x * inv decoded and multiplied by s (in fp64). */
static double stored_value(int kv_dtype, uint16_t x, float s, float inv)
{
    if (kv_dtype == ORC_BF16)
        return (double)bf16_to_f32(x);
    if (kv_dtype == ORC_FP8)
        return orc_e4m3_decode(orc_e4m3_encode(bf16_to_f32(x) * inv)) * (double)s;
    return orc_e2m1_decode(orc_e2m1_encode(bf16_to_f32(x) * inv)) * (double)s;
}

/*
 * Single-token decode attention of one query head over one KV head's stored
 * set S(P), computed from its definition on the dense history:
 *   z_p = sm_scale * sum_d q[d] * k^_p[d]           for p in S(P)
 *   out = sum_p exp(z_p - m) v^_p / sum_p exp(z_p - m),  m = max_p z_p
 *   lse = m + log(sum_p exp(z_p - m))
 * in fp64, positions in ascending order.  An empty set gives out = 0 and
 * lse = -inf (reading: a head with nothing stored contributes nothing).
 * kh, vh point at (b, t=0, h, d=0) of the dense history; rows step by st.
 */
void orc_attention_head(int D, int W, int kv_dtype, int P,
                        const uint16_t *kh, const uint16_t *vh, int64_t st,
                        const uint8_t *keep_row, float k_amax, float v_amax,
                        const uint16_t *q, double sm_scale, double *out,
                        double *lse)
{
    float ks, kinv, vs, vinv;
    head_scales(kv_dtype, k_amax, &ks, &kinv);
    head_scales(kv_dtype, v_amax, &vs, &vinv);
    if (sm_scale <= 0.0)
        sm_scale = 1.0 / sqrt((double)D);
    double *z = (double *)malloc(sizeof(double) * (size_t)(P + 1 > 0 ? P + 1 : 1));
    double m = -INFINITY;
    for (int p = 0; p <= P; ++p) {
        if (!is_stored(keep_row, P, W, p))
            continue;
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += (double)bf16_to_f32(q[d]) *
                   stored_value(kv_dtype, kh[p * st + d], ks, kinv);
        z[p] = sm_scale * acc;
        if (z[p] > m)
            m = z[p];
    }
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    if (m == -INFINITY) {
        *lse = -INFINITY;
        free(z);
        return;
    }
    double l = 0.0;
    for (int p = 0; p <= P; ++p) {
        if (!is_stored(keep_row, P, W, p))
            continue;
        double w = exp(z[p] - m);
        l += w;
        for (int d = 0; d < D; ++d)
            out[d] += w * stored_value(kv_dtype, vh[p * st + d], vs, vinv);
    }
    for (int d = 0; d < D; ++d)
        out[d] /= l;
    *lse = m + log(l);
    free(z);
}

/*
 * GQA decode attention of a whole layer: query head j of sequence b reads KV
 * head h = j / (Hq / Hkv) (reading: consecutive query heads share a KV head).
 * P[b] is the position of sequence b's newest token.  q: [B, Hq, D]
 * contiguous bf16 bits; out: [B, Hq, D]; lse: [B, Hq].
 */
void orc_attention(int B, int Hq, int Hkv, int D, int W, int kv_dtype,
                   const int32_t *P, const uint16_t *k, const uint16_t *v,
                   int64_t sb, int64_t st, int64_t sh, const uint8_t *keep,
                   int64_t keep_ld, const float *k_amax, const float *v_amax,
                   const uint16_t *q, double sm_scale, double *out, double *lse)
{
    int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < Hq; ++j) {
            int h = j / G, i = b * Hkv + h;
            orc_attention_head(D, W, kv_dtype, P[b], k + b * sb + h * sh,
                               v + b * sb + h * sh, st,
                               keep + (int64_t)i * keep_ld,
                               kv_dtype != ORC_BF16 ? k_amax[i] : 0.0f,
                               kv_dtype != ORC_BF16 ? v_amax[i] : 0.0f,
                               q + ((int64_t)b * Hq + j) * D, sm_scale,
                               out + ((int64_t)b * Hq + j) * D,
                               lse + (int64_t)b * Hq + j);
        }
}
