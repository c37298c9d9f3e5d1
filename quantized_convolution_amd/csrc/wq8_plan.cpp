// Host plan: descriptor validation and the scaled Winograd transforms.
//
// Transforms (review page, "What carries the argument"; appendix 7.1 for the
// Vandermonde matrix of homogeneous points):
//   V_{a x b}[i][j] = f_i^j * g_i^(b-1-j), finite p -> (p, 1), infinity -> (1, 0)
//   B^T = S_B V_n^-T,  G = S_G V_{n x 3},  A^T = V_{n x m}^T S_A,  S_A = (S_B S_G)^-1
// Every entry is computed exactly as a rational with 128-bit numerator and
// denominator (points and scales are binary floating-point numbers, hence
// rationals) and rounded once to fp32, ties to even. An entry can sit exactly
// on an fp32 midpoint (e.g. s * 17/18 when s carries a factor 9), so only
// exact arithmetic decides such ties the same way every time. If a rational
// overflows 128 bits (extreme scales or points with long binary expansions)
// the plan falls back to Gauss-Jordan in long double, rounded once to fp32.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "wq8_internal.h"

namespace wq8 {

static thread_local char g_err[512];

wq8_status fail(wq8_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

void clear_error() { g_err[0] = 0; }

static const double kStd4[6] = {0.0, 1.0, -1.0, 2.0, -2.0, INFINITY};
static const double kStd6[8] = {0.0, 1.0, -1.0, 2.0, -2.0, 0.5, -0.5, INFINITY};

// Homogeneous Vandermonde row: entry j = f^j g^(cols-1-j).
static void vrow(double p, int cols, long double *row) {
    long double f = isinf(p) ? 1.0L : (long double)p;
    long double g = isinf(p) ? 0.0L : 1.0L;
    for (int j = 0; j < cols; ++j) {
        long double v = 1.0L;
        for (int e = 0; e < j; ++e) v *= f;
        for (int e = 0; e < cols - 1 - j; ++e) v *= g;
        row[j] = v;
    }
}

// In-place inverse of the n x n matrix a (row-major); false if singular.
static bool invert(int n, long double *a, long double *inv) {
    long double w[kMaxN][2 * kMaxN];
    long double amax = 0;
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) {
            w[i][j] = a[i * n + j];
            w[i][n + j] = (i == j) ? 1.0L : 0.0L;
            if (fabsl(w[i][j]) > amax) amax = fabsl(w[i][j]);
        }
    for (int col = 0; col < n; ++col) {
        int piv = col;
        for (int r = col + 1; r < n; ++r)
            if (fabsl(w[r][col]) > fabsl(w[piv][col])) piv = r;
        if (!(fabsl(w[piv][col]) > 1e-12L * amax)) return false;
        if (piv != col)
            for (int j = 0; j < 2 * n; ++j) {
                long double t = w[col][j];
                w[col][j] = w[piv][j];
                w[piv][j] = t;
            }
        long double p = w[col][col];
        for (int j = 0; j < 2 * n; ++j) w[col][j] /= p;
        for (int r = 0; r < n; ++r) {
            if (r == col || w[r][col] == 0) continue;
            long double f = w[r][col];
            for (int j = 0; j < 2 * n; ++j) w[r][j] -= f * w[col][j];
        }
    }
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) inv[i * n + j] = w[i][n + j];
    return true;
}

// ------------------------------------------------------- exact rationals
typedef __int128 i128;

struct Rat {
    i128 num = 0, den = 1;  // den > 0, gcd(num, den) = 1
};

static i128 iabs(i128 v) { return v < 0 ? -v : v; }
static i128 igcd(i128 a, i128 b) {
    a = iabs(a);
    b = iabs(b);
    while (b) {
        i128 t = a % b;
        a = b;
        b = t;
    }
    return a;
}

// All operations set *ok = false on overflow and return garbage.
static Rat rnorm(i128 n, i128 d, bool *ok) {
    Rat r;
    if (d == 0) {
        *ok = false;
        return r;
    }
    if (d < 0) {
        n = -n;
        d = -d;
    }
    i128 g = igcd(n, d);
    if (g == 0) g = 1;
    r.num = n / g;
    r.den = d / g;
    return r;
}
static i128 mulc(i128 a, i128 b, bool *ok) {
    i128 r;
    if (__builtin_mul_overflow(a, b, &r)) *ok = false;
    return r;
}
static Rat rmul(Rat a, Rat b, bool *ok) {
    i128 g1 = igcd(a.num, b.den), g2 = igcd(b.num, a.den);
    if (g1 == 0) g1 = 1;
    if (g2 == 0) g2 = 1;
    return rnorm(mulc(a.num / g1, b.num / g2, ok), mulc(a.den / g2, b.den / g1, ok), ok);
}
static Rat rinv(Rat a, bool *ok) { return rnorm(a.den, a.num, ok); }
static Rat rsub(Rat a, Rat b, bool *ok) {
    i128 g = igcd(a.den, b.den);
    i128 da = a.den / g, db = b.den / g;
    i128 n1 = mulc(a.num, db, ok), n2 = mulc(b.num, da, ok), n;
    if (__builtin_sub_overflow(n1, n2, &n)) *ok = false;
    return rnorm(n, mulc(a.den, db, ok), ok);
}
// Exact value of a finite double.
static Rat rfrom(double v, bool *ok) {
    if (v == 0.0) return Rat{};
    int e;
    double fr = frexp(v, &e);                       // v = fr * 2^e, 0.5 <= |fr| < 1
    i128 mant = (i128)(long long)ldexp(fr, 53);      // exact 53-bit integer
    e -= 53;
    if (e >= 0) {
        if (e > 70) {
            *ok = false;
            return Rat{};
        }
        return rnorm(mant << e, 1, ok);
    }
    if (-e > 120) {
        *ok = false;
        return Rat{};
    }
    return rnorm(mant, (i128)1 << (-e), ok);
}
static int bitlen(i128 v) {
    int b = 0;
    for (v = iabs(v); v; v >>= 1) ++b;
    return b;
}
// Nearest fp32 to an exact rational, ties to even.
static float rround(Rat q, bool *ok) {
    if (q.num == 0) return 0.0f;
    const bool neg = q.num < 0;
    const i128 a = iabs(q.num), d = q.den;
    // choose e with 2^23 <= a / (d 2^e) < 2^25, then fix to < 2^24
    int e = bitlen(a) - bitlen(d) - 24;
    i128 k, rem, div;
    for (int pass = 0; pass < 2; ++pass) {
        if (e >= 0) {
            if (e > 100 || bitlen(d) + e > 125) {
                *ok = false;
                return 0.0f;
            }
            div = d << e;
            k = a / div;
            rem = a % div;
        } else {
            if (-e > 100 || bitlen(a) - e > 125) {
                *ok = false;
                return 0.0f;
            }
            div = d;
            k = (a << (-e)) / d;
            rem = (a << (-e)) % d;
        }
        if (k < ((i128)1 << 24)) break;
        ++e;  // quotient had 25 bits
    }
    if (2 * rem > div || (2 * rem == div && (k & 1))) ++k;
    float r = ldexpf((float)(long long)k, e);
    if (!isfinite(r)) *ok = false;
    return neg ? -r : r;
}

// Exact homogeneous Vandermonde row.
static void vrow_exact(double p, int cols, Rat *row, bool *ok) {
    Rat f, g;
    if (isinf(p)) {
        f = rnorm(1, 1, ok);
        g = Rat{};
    } else {
        f = rfrom(p, ok);
        g = rnorm(1, 1, ok);
    }
    for (int j = 0; j < cols; ++j) {
        Rat v = rnorm(1, 1, ok);
        for (int e = 0; e < j; ++e) v = rmul(v, f, ok);
        for (int e = 0; e < cols - 1 - j; ++e) v = rmul(v, g, ok);
        row[j] = v;
    }
}

// Exact inverse by Gauss-Jordan; false if singular. *ok false on overflow.
static bool invert_exact(int n, const Rat *a, Rat *inv, bool *ok) {
    Rat w[kMaxN][2 * kMaxN];
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) {
            w[i][j] = a[i * n + j];
            w[i][n + j] = (i == j) ? rnorm(1, 1, ok) : Rat{};
        }
    for (int col = 0; col < n && *ok; ++col) {
        int piv = -1;
        for (int r = col; r < n; ++r)
            if (w[r][col].num != 0) {
                piv = r;
                break;
            }
        if (piv < 0) return false;
        if (piv != col)
            for (int j = 0; j < 2 * n; ++j) {
                Rat t = w[col][j];
                w[col][j] = w[piv][j];
                w[piv][j] = t;
            }
        Rat pinv = rinv(w[col][col], ok);
        for (int j = 0; j < 2 * n; ++j) w[col][j] = rmul(w[col][j], pinv, ok);
        for (int r = 0; r < n; ++r) {
            if (r == col || w[r][col].num == 0) continue;
            Rat f = w[r][col];
            for (int j = 0; j < 2 * n; ++j) w[r][j] = rsub(w[r][j], rmul(f, w[col][j], ok), ok);
        }
    }
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) inv[i * n + j] = w[i][n + j];
    return true;
}

// Exact construction; returns false (and leaves mt untouched) on overflow.
static bool mats_exact(int m, const double *pts, const float *sB, const float *sG, Mats *mt,
                       bool *singular) {
    const int n = m + 2;
    bool ok = true;
    Rat vn[kMaxN * kMaxN], vinv[kMaxN * kMaxN], vr[kMaxN * 3], vm[kMaxN * 6], rb[kMaxN], rg[kMaxN];
    for (int i = 0; i < n; ++i) {
        vrow_exact(pts[i], n, vn + i * n, &ok);
        vrow_exact(pts[i], 3, vr + i * 3, &ok);
        vrow_exact(pts[i], m, vm + i * m, &ok);
        rb[i] = rfrom(sB[i], &ok);
        rg[i] = rfrom(sG[i], &ok);
    }
    if (!ok) return false;
    if (!invert_exact(n, vn, vinv, &ok)) {
        *singular = true;
        return ok;
    }
    Mats out;
    memset(&out, 0, sizeof out);
    for (int i = 0; i < n; ++i) {
        for (int k = 0; k < n; ++k) out.Bt[i * n + k] = rround(rmul(rb[i], vinv[k * n + i], &ok), &ok);
        for (int k = 0; k < 3; ++k) out.G[i * 3 + k] = rround(rmul(rg[i], vr[i * 3 + k], &ok), &ok);
    }
    for (int k = 0; k < n; ++k) {
        Rat sa = rinv(rmul(rb[k], rg[k], &ok), &ok);
        for (int a = 0; a < m; ++a) out.At[a * n + k] = rround(rmul(vm[k * m + a], sa, &ok), &ok);
    }
    if (!ok) return false;
    *mt = out;
    return true;
}

static size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static wq8_status build(const wq8_desc *d, wq8_plan *p) {
    if (d->m != 4 && d->m != 6)
        return fail(WQ8_ERR_UNSUPPORTED, "m = %d: only F(4,3) and F(6,3) are built", d->m);
    const int m = d->m, n = m + 2;
    if (d->group != 16 && d->group != 32 && d->group != 64 && d->group != 128 && d->group != 256)
        return fail(WQ8_ERR_UNSUPPORTED, "group = %d: must be 16, 32, 64, 128 or 256", d->group);
    if (d->N < 1 || d->Cin < 1 || d->Cout < 1 || d->H < 1 || d->W < 1)
        return fail(WQ8_ERR_INVALID_ARG, "sizes must be positive (N=%d Cin=%d Cout=%d H=%d W=%d)",
                    d->N, d->Cin, d->Cout, d->H, d->W);
    if (d->Cin % d->group != 0)
        return fail(WQ8_ERR_INVALID_ARG, "Cin = %d is not a multiple of group = %d", d->Cin,
                    d->group);
    if (d->pad < 0 || d->pad > 2) return fail(WQ8_ERR_INVALID_ARG, "pad = %d: must be 0..2", d->pad);
    if ((d->x_dtype != WQ8_F32 && d->x_dtype != WQ8_BF16) ||
        (d->y_dtype != WQ8_F32 && d->y_dtype != WQ8_BF16))
        return fail(WQ8_ERR_INVALID_ARG, "unknown dtype");
    Geo &g = p->geo;
    g.m = m;
    g.n = n;
    g.G = d->group;
    g.ng = d->Cin / d->group;
    g.N = d->N;
    g.Cin = d->Cin;
    g.Cout = d->Cout;
    g.H = d->H;
    g.W = d->W;
    g.pad = d->pad;
    g.Ho = d->H + 2 * d->pad - 2;
    g.Wo = d->W + 2 * d->pad - 2;
    if (g.Ho < 1 || g.Wo < 1)
        return fail(WQ8_ERR_INVALID_ARG, "empty output: H=%d W=%d pad=%d", d->H, d->W, d->pad);
    g.tH = (g.Ho + m - 1) / m;
    g.tW = (g.Wo + m - 1) / m;
    g.T = (int64_t)g.N * g.tH * g.tW;
    // every buffer must be addressable with 64-bit offsets and the
    // per-tap planes with 32-bit element counts inside a kernel
    const int64_t n2 = (int64_t)n * n;
    const int64_t lim = (int64_t)1 << 31;
    // the kernels address x, y, Vq, sV, Uq, sU and M with 32-bit byte offsets
    if (n2 * g.T * d->Cin >= lim || n2 * g.T * d->Cout * 4 >= lim ||
        n2 * (int64_t)d->Cout * d->Cin >= lim ||
        (int64_t)d->N * d->Cin * d->H * d->W * 4 >= lim ||
        (int64_t)d->N * d->Cout * g.Ho * g.Wo * 4 >= lim)
        return fail(WQ8_ERR_UNSUPPORTED, "problem too large: an array would reach 2^31 bytes (32-bit buffer offsets)");
    p->xdt = d->x_dtype;
    p->ydt = d->y_dtype;

    // points and scales
    const double *pts = d->points ? d->points : (m == 4 ? kStd4 : kStd6);
    int ninf = 0;
    for (int i = 0; i < n; ++i) {
        double v = pts[i];
        if (isnan(v) || (isinf(v) && v < 0))
            return fail(WQ8_ERR_INVALID_ARG, "point %d is not a number or +infinity", i);
        ninf += isinf(v) ? 1 : 0;
        p->points[i] = v;
        float sb = d->s_B ? d->s_B[i] : 1.0f;
        float sg = d->s_G ? d->s_G[i] : 1.0f;
        if (!isfinite(sb) || !isfinite(sg) || sb == 0.0f || sg == 0.0f)
            return fail(WQ8_ERR_INVALID_ARG, "scale %d must be finite and non-zero", i);
        p->sB[i] = sb;
        p->sG[i] = sg;
    }
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j)
            if (pts[i] == pts[j]) return fail(WQ8_ERR_SINGULAR_POINTS, "points %d and %d coincide", i, j);
    if (ninf > 1) return fail(WQ8_ERR_SINGULAR_POINTS, "more than one point at infinity");

    Mats &mt = p->mats;
    bool singular = false;
    if (!mats_exact(m, pts, p->sB, p->sG, &mt, &singular)) {
        // rationals overflowed 128 bits: long double Gauss-Jordan instead
        long double vn[kMaxN * kMaxN], vinv[kMaxN * kMaxN], vr[kMaxN * 3], vm[kMaxN * 6];
        for (int i = 0; i < n; ++i) {
            vrow(pts[i], n, vn + i * n);
            vrow(pts[i], 3, vr + i * 3);
            vrow(pts[i], m, vm + i * m);
        }
        if (!invert(n, vn, vinv))
            return fail(WQ8_ERR_SINGULAR_POINTS, "Vandermonde matrix of the points is singular");
        memset(&mt, 0, sizeof mt);
        for (int i = 0; i < n; ++i) {
            const long double sb = p->sB[i], sg = p->sG[i];
            for (int k = 0; k < n; ++k) mt.Bt[i * n + k] = (float)(sb * vinv[k * n + i]);
            for (int k = 0; k < 3; ++k) mt.G[i * 3 + k] = (float)(sg * vr[i * 3 + k]);
        }
        for (int a = 0; a < m; ++a)
            for (int k = 0; k < n; ++k) {
                const long double sa = 1.0L / ((long double)p->sB[k] * (long double)p->sG[k]);
                mt.At[a * n + k] = (float)(vm[k * m + a] * sa);
            }
    } else if (singular) {
        return fail(WQ8_ERR_SINGULAR_POINTS, "Vandermonde matrix of the points is singular");
    }
    for (int i = 0; i < n * n; ++i)
        if (!isfinite(mt.Bt[i])) return fail(WQ8_ERR_INVALID_ARG, "B^T overflows fp32");
    for (int i = 0; i < m * n; ++i)
        if (!isfinite(mt.At[i])) return fail(WQ8_ERR_INVALID_ARG, "A^T overflows fp32");
    for (int i = 0; i < n * 3; ++i)
        if (!isfinite(mt.G[i])) return fail(WQ8_ERR_INVALID_ARG, "G overflows fp32");

    // power-of-two prescale of the output transform's Kronecker matrix
    // (A^T (x) A^T, formed on the GPU in fp16 parts): largest entry <= 2^14
    {
        float amax = 0.0f;
        for (int i = 0; i < m * n; ++i) amax = fmaxf(amax, fabsf(mt.At[i]));
        int e = 0;
        if (amax > 0.0f) {
            frexp((double)amax * (double)amax, &e);  // amax^2 < 2^e
            e -= 14;
        }
        mt.kscale = (float)ldexp(1.0, -e);
        mt.oscale = (float)ldexp(1.0, e);
        if (mt.kscale == 0.0f || !isfinite(mt.kscale) || !isfinite(mt.oscale))
            return fail(WQ8_ERR_UNSUPPORTED, "A^T entries span more than fp32 allows");
    }

    // may the kernels skip the structurally zero terms of the standard points?
    {
        uint64_t bt_nz = 0, at_nz = 0;
        for (int i = 0; i < n * n; ++i)
            if (mt.Bt[i] != 0.0f) bt_nz |= 1ull << i;
        for (int i = 0; i < m * n; ++i)
            if (mt.At[i] != 0.0f) at_nz |= 1ull << i;
        const uint64_t bt_pat = m == 4 ? kBtPattern4 : kBtPattern6;
        const uint64_t at_pat = m == 4 ? kAtPattern4 : kAtPattern6;
        g.bt_std = (bt_nz & ~bt_pat) == 0;
        g.at_std = (at_nz & ~at_pat) == 0;
    }

    // integer input stage: B^T codes and row scales (fp32 absmax quantizer)
    if (d->in_quant != WQ8_INQ_FP32 && d->in_quant != WQ8_INQ_INT_TENSOR &&
        d->in_quant != WQ8_INQ_INT_ROW)
        return fail(WQ8_ERR_INVALID_ARG, "unknown in_quant %d", (int)d->in_quant);
    g.in_quant = (int)d->in_quant;
    if (g.in_quant != WQ8_INQ_FP32) {
        const bool rows = g.in_quant == WQ8_INQ_INT_ROW;
        for (int r0 = 0; r0 < n; r0 += rows ? 1 : n) {
            const int len = rows ? n : n * n;
            float a = 0.0f;
            for (int i = 0; i < len; ++i) a = fmaxf(a, fabsf(mt.Bt[r0 * n + i]));
            float sc = 0.0f, inv = 0.0f;
            if (a != 0.0f) {
                inv = 127.0f / a;
                sc = a / 127.0f;
            }
            for (int i = 0; i < len; ++i) {
                const float r = rintf(mt.Bt[r0 * n + i] * inv);
                mt.Bq[r0 * n + i] = (int)fminf(fmaxf(r, -127.0f), 127.0f);
            }
            for (int i = 0; i < (rows ? 1 : n); ++i) mt.sqb[r0 + i] = sc;
        }
    }

    // workspace: Vq | sV | M, each 256-byte aligned
    p->off_vq = 0;
    p->off_sv = round_up((size_t)(n2 * g.T * g.Cin), 256);
    p->off_m = p->off_sv + round_up((size_t)(n2 * g.T * g.ng) * 4, 256);
    p->u_code_bytes = (size_t)(n2 * g.Cout * g.Cin);
    p->u_scale_bytes = (size_t)(n2 * g.Cout * g.ng) * 4;
    if (d->algo != WQ8_ALGO_AUTO && d->algo != WQ8_ALGO_STAGED && d->algo != WQ8_ALGO_FUSED)
        return fail(WQ8_ERR_INVALID_ARG, "unknown algo %d", (int)d->algo);
    if (d->y_group != WQ8_YGROUP_TILE && d->y_group != WQ8_YGROUP_ROW)
        return fail(WQ8_ERR_INVALID_ARG, "unknown y_group %d", (int)d->y_group);
    g.y_rows = d->y_group == WQ8_YGROUP_ROW;
    if (g.y_rows && d->algo == WQ8_ALGO_FUSED)
        return fail(WQ8_ERR_UNSUPPORTED, "per-row Y scales run the staged schedule only");
    if (g.y_rows) {
        p->fused = 0;
    } else if (d->algo == WQ8_ALGO_AUTO) {
        // the fused kernel re-reads the weights once per 16-tile block (from
        // L2 / Infinity Cache when they fit); the staged one writes and reads M.
        // Up to 2 MiB of weight codes the re-reads stay cheap (measured on
        // MI355X: fused is faster at 0.25 and 1 MiB of codes, staged from
        // 3.5 MiB on)
        const double reread = (double)p->u_code_bytes * (double)((g.T + 15) / 16);
        const double mbytes = 8.0 * (double)(n2 * g.T * g.Cout);
        p->fused = p->u_code_bytes <= ((size_t)2 << 20) || reread <= mbytes;
    } else {
        p->fused = d->algo == WQ8_ALGO_FUSED;
    }
    p->ws_bytes = p->fused ? p->off_m : p->off_m + (size_t)(n2 * g.T * g.Cout) * 4;
    // W8A8 direct convolution: workspace Xq | sX, weights Wq / sW
    {
        const size_t npx = (size_t)g.N * g.H * g.W;
        p->d_off_sx = round_up(npx * g.Cin, 256);
        p->d_ws_bytes = p->d_off_sx + round_up(npx * g.ng * 4, 256);
        p->d_w_code_bytes = (size_t)9 * g.Cout * g.Cin;
        p->d_w_scale_bytes = (size_t)9 * g.Cout * g.ng * 4;
    }
    // every output-channel block reads all activation codes of its tiles and
    // every tile block all weights of its channels: keep the larger operand
    // split across the XCDs' L2s
    p->geo.co_major = p->u_code_bytes > (size_t)(n2 * g.T * g.Cin);
    // Kernel shapes. Every shape performs the same operations per output in
    // the same order, so the results do not depend on them. 0 leaves the
    // choice to the launch, which weighs the block count against the
    // device's compute units; the descriptor may force one (tests, tuning).
    if (d->stage1_rows < 0 || d->stage1_rows > 2)
        return fail(WQ8_ERR_INVALID_ARG, "stage1_rows = %d: must be 0, 1 or 2", d->stage1_rows);
    if (d->stage1_rows == 2 && g.in_quant != WQ8_INQ_FP32)
        return fail(WQ8_ERR_UNSUPPORTED, "half-row windows need the fp32 input stage");
    p->geo.s1_rows = d->stage1_rows;
    if (d->fused_waves != 0 && d->fused_waves != 4 && d->fused_waves != 8 && d->fused_waves != 16)
        return fail(WQ8_ERR_INVALID_ARG, "fused_waves = %d: must be 0, 4, 8 or 16", d->fused_waves);
    if (d->fused_waves > 4 && m != 6)
        return fail(WQ8_ERR_UNSUPPORTED, "8- and 16-wave fused blocks are built for F(6,3) only");
    p->geo.fused_waves = d->fused_waves;
    if (d->fused_block < 0 || d->fused_block > 4)
        return fail(WQ8_ERR_INVALID_ARG, "fused_block = %d: must be 0..4", d->fused_block);
    if (d->fused_block > 1 && !(m == 6 && d->group <= 64))
        return fail(WQ8_ERR_UNSUPPORTED, "wide fused blocks are built for F(6,3) with G <= 64 only");
    // Geo: -1 chosen at launch; 0 16 x 16; 1 32 x 32; 2 32 tiles x 16; 3 16 x 32
    p->geo.fused_wide = d->fused_block - 1;
    if (d->stage2_rows != 0 && d->stage2_rows != 1 && d->stage2_rows != 4 && d->stage2_rows != 5 &&
        d->stage2_rows != 6 && d->stage2_rows != 8)
        return fail(WQ8_ERR_INVALID_ARG, "stage2_rows = %d: must be 0, 1, 4, 5, 6 or 8", d->stage2_rows);
    p->geo.s2_rows = d->stage2_rows;
    if (d->stage2_cols != 0 && d->stage2_cols != 1 && d->stage2_cols != 2)
        return fail(WQ8_ERR_INVALID_ARG, "stage2_cols = %d: must be 0, 1 or 2", d->stage2_cols);
    if (d->stage2_cols == 2 && (d->stage2_rows == 6 || d->stage2_rows == 8))
        return fail(WQ8_ERR_UNSUPPORTED, "two channel tiles per wave are built for stage2_rows 4 and 5 only");
    p->geo.s2_cols = d->stage2_cols;
    if (d->stage2_waves != 0 && d->stage2_waves != 2 && d->stage2_waves != 4)
        return fail(WQ8_ERR_INVALID_ARG, "stage2_waves = %d: must be 0, 2 or 4", d->stage2_waves);
    p->geo.s2_waves = d->stage2_waves;
    if (d->stage3_lanes < 0 || d->stage3_lanes > 2)
        return fail(WQ8_ERR_INVALID_ARG, "stage3_lanes = %d: must be 0, 1 or 2", d->stage3_lanes);
    p->geo.s3_lanes = d->stage3_lanes;
    return WQ8_OK;
}

}  // namespace wq8

extern "C" {

wq8_status wq8_plan_create(const wq8_desc *desc, wq8_plan **out) {
    wq8::clear_error();
    if (!desc || !out) return wq8::fail(WQ8_ERR_INVALID_ARG, "null descriptor or output pointer");
    *out = nullptr;
    wq8_plan *p = new (std::nothrow) wq8_plan;
    if (!p) return wq8::fail(WQ8_ERR_NO_MEMORY, "plan allocation failed");
    memset(p, 0, sizeof *p);
    wq8_status st = wq8::build(desc, p);
    if (st != WQ8_OK) {
        delete p;
        return st;
    }
    *out = p;
    return WQ8_OK;
}

void wq8_plan_destroy(wq8_plan *plan) { delete plan; }

wq8_status wq8_plan_query(const wq8_plan *p, size_t *ws, size_t *ucode, size_t *uscale,
                          int64_t *tiles, wq8_algo *algo) {
    wq8::clear_error();
    if (!p) return wq8::fail(WQ8_ERR_INVALID_ARG, "null plan");
    if (ws) *ws = p->ws_bytes;
    if (ucode) *ucode = p->u_code_bytes;
    if (uscale) *uscale = p->u_scale_bytes;
    if (tiles) *tiles = p->geo.T;
    if (algo) *algo = p->fused ? WQ8_ALGO_FUSED : WQ8_ALGO_STAGED;
    return WQ8_OK;
}

wq8_status wq8_plan_matrices(const wq8_plan *p, float *Bt, float *G, float *At) {
    wq8::clear_error();
    if (!p) return wq8::fail(WQ8_ERR_INVALID_ARG, "null plan");
    const int n = p->geo.n, m = p->geo.m;
    if (Bt) memcpy(Bt, p->mats.Bt, sizeof(float) * n * n);
    if (G) memcpy(G, p->mats.G, sizeof(float) * n * 3);
    if (At) memcpy(At, p->mats.At, sizeof(float) * m * n);
    return WQ8_OK;
}

wq8_status wq8_plan_bt_codes(const wq8_plan *p, int8_t *Bq, float *sq) {
    wq8::clear_error();
    if (!p) return wq8::fail(WQ8_ERR_INVALID_ARG, "null plan");
    if (p->geo.in_quant == WQ8_INQ_FP32)
        return wq8::fail(WQ8_ERR_INVALID_ARG, "the plan's input stage does not quantize B^T");
    const int n = p->geo.n;
    if (Bq)
        for (int i = 0; i < n * n; ++i) Bq[i] = (int8_t)p->mats.Bq[i];
    if (sq) memcpy(sq, p->mats.sqb, sizeof(float) * n);
    return WQ8_OK;
}

const char *wq8_status_string(wq8_status s) {
    switch (s) {
        case WQ8_OK: return "ok";
        case WQ8_ERR_INVALID_ARG: return "invalid argument";
        case WQ8_ERR_UNSUPPORTED: return "unsupported configuration";
        case WQ8_ERR_SINGULAR_POINTS: return "interpolation points are not distinct";
        case WQ8_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case WQ8_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
        case WQ8_ERR_HIP: return "HIP error";
        case WQ8_ERR_NO_MEMORY: return "out of host memory";
    }
    return "unknown status";
}

const char *wq8_last_error(void) { return wq8::g_err; }

}  // extern "C"
