/*
 * BitDelta CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the GPU smoke check and the benchmark's CPU baseline
 * may load this library.  The product path (the HIP library and its Python
 * binding) never calls it and shares no code with it.
 *
 * Source of every definition: the post "BitDelta : servir 14 modèles Zen
 * depuis un seul cluster GPU" (hanzo-blog, 2026-02-28; the same post also
 * exists in th, zh-Hant and ja-JP).  Section names below are English glosses
 * of the post's headings:
 *   "Mathematical foundation"  (fr: "Le fondement mathématique")
 *   "Serving architecture"     (fr: "Architecture de service"), which holds
 *                               the serving diagram, the five-step pipeline
 *                               and the conceptual fused_bitdelta_linear
 *                               listing
 *   "Infrastructure details"   (fr: "Détails d'infrastructure")
 *
 * Readings taken where the post leaves a step open (each is listed with its
 * reason in the design notes):
 *   - Δ from a (fine-tuned, base) pair is the fp32 difference of the two
 *     bf16 weights widened to fp32 (round to nearest, ties to even).
 *   - sign(Δ) is one bit; bit = 1 encodes +1, bit = 0 encodes -1; Δ = +0 and
 *     Δ = -0 (and NaN) encode +1, i.e. bit = !(Δ < 0).
 *   - 8 signs per byte, least significant bit first along d_in; packed
 *     shape [d_out, d_in/8].
 *   - α is fp32: either one per matrix or one per output row.
 *   - The reconstructed weight is formed as an fp32 sum of the bf16 base
 *     weight and ±α, rounded once to bf16 (round to nearest, ties to even),
 *     and that bf16 value enters the product.
 *   - The product is accumulated here in fp64 and returned in fp64.
 *
 * Plain scalar loops, fp64 where the post fixes no precision, OpenMP only to
 * split independent output rows.  Compile without -ffast-math and with
 * -ffp-contract=off.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_OK = 0, ORC_ERR_ARG = 1 };

/* Threads the parallel loops below use (for reporting timings). */
int orc_num_threads(void) { return omp_get_max_threads(); }

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static double bf16_to_f64(uint16_t h) { return (double)bits_to_f32((uint32_t)h << 16); }

/*
 * One sign bit, "Mathematical foundation": sign(Δ) keeps only whether an
 * element is positive or negative.  Reading: zero counts as positive.
 */
static int sign_bit(float d) { return !(d < 0.0f); }

/*
 * Pack sign(Δ) 8 per byte ("Infrastructure details": packed int8, 8 bits per
 * byte, a 4096x4096 matrix becomes 4096x512).  Bit b of byte j of row n holds
 * the sign of Δ[n, 8j + b].
 */
int orc_pack_signs(const float* delta, int64_t d_out, int64_t d_in, uint8_t* signs)
{
    if (!delta || !signs || d_out < 0 || d_in < 0 || d_in % 8 != 0) return ORC_ERR_ARG;
    int64_t nbytes = d_in / 8;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < d_out; ++n) {
        for (int64_t j = 0; j < nbytes; ++j) {
            unsigned byte = 0;
            for (int b = 0; b < 8; ++b)
                byte |= (unsigned)sign_bit(delta[n * d_in + 8 * j + b]) << b;
            signs[n * nbytes + j] = (uint8_t)byte;
        }
    }
    return ORC_OK;
}

/*
 * Δ from a fine-tuned / base pair, "Mathematical foundation": the delta is
 * the elementwise difference W_ft − W_base.  Reading: both bf16 weights are
 * widened to fp32 (exact) and subtracted in fp32 (round to nearest, ties to
 * even); that fp32 Δ is what sign packing and α read.  For bf16 operands
 * whose exponents differ by at most 15 the fp32 difference is exact.
 */
int orc_delta_from_pair(const uint16_t* w_ft, const uint16_t* w_base, int64_t count, float* delta)
{
    if (!w_ft || !w_base || !delta || count < 0) return ORC_ERR_ARG;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        float ft = bits_to_f32((uint32_t)w_ft[i] << 16);
        float base = bits_to_f32((uint32_t)w_base[i] << 16);
        delta[i] = ft - base;
    }
    return ORC_OK;
}

/* The inverse of the packing: ±1 for every element, as fp32. */
int orc_unpack_signs(const uint8_t* signs, int64_t d_out, int64_t d_in, float* pm1)
{
    if (!signs || !pm1 || d_out < 0 || d_in < 0 || d_in % 8 != 0) return ORC_ERR_ARG;
    int64_t nbytes = d_in / 8;
    for (int64_t n = 0; n < d_out; ++n)
        for (int64_t k = 0; k < d_in; ++k) {
            int bit = (signs[n * nbytes + k / 8] >> (k % 8)) & 1;
            pm1[n * d_in + k] = bit ? 1.0f : -1.0f;
        }
    return ORC_OK;
}

/* Σ|v| over count values, fp64 with Neumaier's compensation. */
static double abs_sum(const float* v, int64_t count)
{
    double s = 0.0, c = 0.0;
    for (int64_t i = 0; i < count; ++i) {
        double a = fabs((double)v[i]);
        double t = s + a;
        if (fabs(s) >= a) c += (s - t) + a;
        else              c += (a - t) + s;
        s = t;
    }
    return s + c;
}

/*
 * Scale factor, "Mathematical foundation": α = (1/n)·||Δ||_1, the mean
 * absolute delta.  per_row = 0: one α over the whole matrix
 * (n = d_out·d_in).  per_row = 1: one α per output row ("Infrastructure
 * details": fp32, one per output dimension), n = d_in.  The fp64 mean is
 * rounded once to fp32.
 */
int orc_alpha(const float* delta, int64_t d_out, int64_t d_in, int per_row, float* alpha)
{
    if (!delta || !alpha || d_out <= 0 || d_in <= 0) return ORC_ERR_ARG;
    if (per_row) {
        #pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < d_out; ++n)
            alpha[n] = (float)(abs_sum(delta + n * d_in, d_in) / (double)d_in);
    } else {
        double total = abs_sum(delta, d_out * d_in);
        alpha[0] = (float)(total / ((double)d_out * (double)d_in));
    }
    return ORC_OK;
}

/* fp32 bit pattern -> bf16 bit pattern, round to nearest, ties to even.
 * NaN stays a (quiet) NaN of the same sign. */
uint16_t orc_bf16_rne(uint32_t u)
{
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

int orc_bf16_rne_array(const uint32_t* in, int64_t count, uint16_t* out)
{
    if (!in || !out || count < 0) return ORC_ERR_ARG;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) out[i] = orc_bf16_rne(in[i]);
    return ORC_OK;
}

/*
 * fp64 value -> bf16 bit pattern in one rounding: to nearest, ties to even,
 * with no intermediate fp32.  For the bf16 output of the fused linear: the
 * conceptual listing ends in F.linear on bf16 operands, whose result is bf16.
 * bf16 keeps 8 significant bits and fp32's exponent range, so the values
 * between 2^e and 2^(e+1) (e >= -126) are spaced 2^(e-7) apart, and below
 * 2^-126 (subnormals) 2^-133 apart.  |v| / spacing is an exact power-of-two
 * scaling; rounding it to an integer (ties to even) and scaling back gives
 * the bf16 value; at or beyond 2^128 it is infinity.  NaN -> a quiet NaN of
 * the same sign.
 */
uint16_t orc_bf16_rne_f64(double v)
{
    if (isnan(v)) return signbit(v) ? 0xFFC0u : 0x7FC0u;
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    int e;
    frexp(a, &e);                       /* a in [2^(e-1), 2^e) */
    int ex = e - 1;
    if (ex < -126) ex = -126;
    double q = ldexp(1.0, ex - 7);      /* spacing of bf16 values at a */
    double r = nearbyint(a / q) * q;    /* default rounding mode: ties to even */
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;                 /* exact: r is a bf16 value */
    return (uint16_t)(sign | (f32_to_bits(f) >> 16));
}

int orc_bf16_rne_f64_array(const double* in, int64_t count, uint16_t* out)
{
    if (!in || !out || count < 0) return ORC_ERR_ARG;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) out[i] = orc_bf16_rne_f64(in[i]);
    return ORC_OK;
}

/*
 * One reconstructed weight, "Serving architecture" step 3:
 * W_eff = W_base + α·sign(Δ).  fp32 addition (IEEE, round to nearest even),
 * then one rounding to bf16.
 */
static uint16_t weff_elem(uint16_t wbase, int bit, float a)
{
    float w = bits_to_f32((uint32_t)wbase << 16);
    float s = bit ? a : -a;
    float t = w + s;
    return orc_bf16_rne(f32_to_bits(t));
}

static void weff_row(const uint16_t* w_base, const uint8_t* signs, const float* alpha,
                     int per_row, int64_t n, int64_t d_in, uint16_t* out)
{
    int64_t nbytes = d_in / 8;
    float a = per_row ? alpha[n] : alpha[0];
    for (int64_t k = 0; k < d_in; ++k) {
        int bit = (signs[n * nbytes + k / 8] >> (k % 8)) & 1;
        out[k] = weff_elem(w_base[n * d_in + k], bit, a);
    }
}

int orc_weff(const uint16_t* w_base, const uint8_t* signs, const float* alpha, int per_row,
             int64_t d_out, int64_t d_in, uint16_t* w_eff)
{
    if (!w_base || !signs || !alpha || !w_eff || d_out < 0 || d_in < 0 || d_in % 8 != 0)
        return ORC_ERR_ARG;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < d_out; ++n)
        weff_row(w_base, signs, alpha, per_row, n, d_in, w_eff + n * d_in);
    return ORC_OK;
}

static double dot_f64(const uint16_t* x, const uint16_t* w, int64_t d_in)
{
    double acc = 0.0;
    for (int64_t k = 0; k < d_in; ++k) acc += bf16_to_f64(x[k]) * bf16_to_f64(w[k]);
    return acc;
}

/*
 * The fused linear's result, "Serving architecture" listing:
 * y = x · W_effᵀ with x [M, d_in] bf16, W_eff [d_out, d_in] bf16, y [M, d_out].
 */
int orc_linear(const uint16_t* x, const uint16_t* w_base, const uint8_t* signs,
               const float* alpha, int per_row, int64_t M, int64_t d_out, int64_t d_in,
               double* y)
{
    if (!x || !w_base || !signs || !alpha || !y || M < 0 || d_out < 0 || d_in < 0 ||
        d_in % 8 != 0)
        return ORC_ERR_ARG;
    int err = 0;
    #pragma omp parallel
    {
        uint16_t* row = (uint16_t*)malloc((size_t)(d_in > 0 ? d_in : 1) * sizeof(uint16_t));
        if (!row) {
            #pragma omp atomic write
            err = 1;
        } else {
            #pragma omp for schedule(static)
            for (int64_t n = 0; n < d_out; ++n) {
                weff_row(w_base, signs, alpha, per_row, n, d_in, row);
                for (int64_t m = 0; m < M; ++m) y[m * d_out + n] = dot_f64(x + m * d_in, row, d_in);
            }
            free(row);
        }
    }
    return err ? ORC_ERR_ARG : ORC_OK;
}

/* Selected outputs y[ms[i], ns[i]] only, for checks at full size. */
int orc_linear_sampled(const uint16_t* x, const uint16_t* w_base, const uint8_t* signs,
                       const float* alpha, int per_row, int64_t M, int64_t d_out, int64_t d_in,
                       const int64_t* ms, const int64_t* ns, int64_t count, double* out)
{
    if (!x || !w_base || !signs || !alpha || !ms || !ns || !out || d_in % 8 != 0) return ORC_ERR_ARG;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= d_out) return ORC_ERR_ARG;
    int err = 0;
    #pragma omp parallel
    {
        uint16_t* row = (uint16_t*)malloc((size_t)(d_in > 0 ? d_in : 1) * sizeof(uint16_t));
        if (!row) {
            #pragma omp atomic write
            err = 1;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < count; ++i) {
                weff_row(w_base, signs, alpha, per_row, ns[i], d_in, row);
                out[i] = dot_f64(x + ms[i] * d_in, row, d_in);
            }
            free(row);
        }
    }
    return err ? ORC_ERR_ARG : ORC_OK;
}

/*
 * Several variants over one shared base ("Serving architecture" diagram:
 * one HBM-resident base read by all, one (α, sign(Δ)) entry per variant in
 * the delta cache, the router picking the entry from the request's model).
 * Token m uses variant ids[m]: y[m] = x[m] · W_eff(ids[m])ᵀ.  A token whose id
 * is outside [0, G) gets a row of NaN.
 */
int orc_linear_grouped(const uint16_t* x, const int32_t* ids, const uint16_t* w_base,
                       const uint8_t* const* signs, const float* const* alpha, int per_row,
                       int32_t G, int64_t M, int64_t d_out, int64_t d_in, double* y)
{
    if (!x || !ids || !w_base || !signs || !alpha || !y || G <= 0 || M < 0 || d_out < 0 ||
        d_in < 0 || d_in % 8 != 0)
        return ORC_ERR_ARG;
    for (int32_t g = 0; g < G; ++g)
        if (!signs[g] || !alpha[g]) return ORC_ERR_ARG;
    int err = 0;
    #pragma omp parallel
    {
        uint16_t* row = (uint16_t*)malloc((size_t)(d_in > 0 ? d_in : 1) * sizeof(uint16_t));
        if (!row) {
            #pragma omp atomic write
            err = 1;
        } else {
            #pragma omp for schedule(static)
            for (int64_t n = 0; n < d_out; ++n) {
                for (int32_t g = 0; g < G; ++g) {
                    int used = 0;
                    for (int64_t m = 0; m < M && !used; ++m) used = (ids[m] == g);
                    if (!used) continue;
                    weff_row(w_base, signs[g], alpha[g], per_row, n, d_in, row);
                    for (int64_t m = 0; m < M; ++m)
                        if (ids[m] == g) y[m * d_out + n] = dot_f64(x + m * d_in, row, d_in);
                }
                for (int64_t m = 0; m < M; ++m)
                    if (ids[m] < 0 || ids[m] >= G) y[m * d_out + n] = NAN;
            }
            free(row);
        }
    }
    return err ? ORC_ERR_ARG : ORC_OK;
}

/* Grouped, selected outputs only. */
int orc_linear_grouped_sampled(const uint16_t* x, const int32_t* ids, const uint16_t* w_base,
                               const uint8_t* const* signs, const float* const* alpha,
                               int per_row, int32_t G, int64_t M, int64_t d_out, int64_t d_in,
                               const int64_t* ms, const int64_t* ns, int64_t count, double* out)
{
    if (!x || !ids || !w_base || !signs || !alpha || !ms || !ns || !out || G <= 0 ||
        d_in % 8 != 0)
        return ORC_ERR_ARG;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= d_out) return ORC_ERR_ARG;
    int err = 0;
    #pragma omp parallel
    {
        uint16_t* row = (uint16_t*)malloc((size_t)(d_in > 0 ? d_in : 1) * sizeof(uint16_t));
        if (!row) {
            #pragma omp atomic write
            err = 1;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < count; ++i) {
                int32_t g = ids[ms[i]];
                if (g < 0 || g >= G) { out[i] = NAN; continue; }
                weff_row(w_base, signs[g], alpha[g], per_row, ns[i], d_in, row);
                out[i] = dot_f64(x + ms[i] * d_in, row, d_in);
            }
            free(row);
        }
    }
    return err ? ORC_ERR_ARG : ORC_OK;
}
