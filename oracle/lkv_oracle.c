/*
 * lkv_oracle.c -- plain, slow, obviously-correct CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product library.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp
 * (x86-64 SSE arithmetic, default rounding mode, no flush-to-zero).
 * OpenMP only splits independent (sequence, head) units; every result is
 * the same for any thread count.
 *
 * Storage format (the "memory layout reorganised for the quantised format",
 * LeanKV page, implementation details).  Tokens are grouped in blocks of 64;
 * one chunk holds one block of one KV head, in six sections, each padded to
 * a multiple of 128 bytes:
 *   K codes   64 token rows, each the D channel codes as a kb-bit bitstream
 *   V codes   D channel rows, each the 64 slot codes as a vb-bit bitstream
 *   K scales  fp32 [D/g groups][64 slots]
 *   V scales  fp32 [D/g groups][64 slots]
 *   K zeros   uint8 [D/g groups][64 slots]
 *   V zeros   uint8 [D/g groups][64 slots]
 * A bitstream stores field i in bits [i*b, i*b+b), bit n of the stream being
 * bit n%8 of byte n/8 (the same as LSB-first packing into little-endian
 * 32-bit words).  For the fp16 format (kb = vb = 16) the fields are fp16 bit
 * patterns and the four metadata sections are empty.
 */
#include "lkv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BT ORC_BLOCK_TOKENS

static int64_t pad128(int64_t x) { return (x + 127) / 128 * 128; }

static int valid_bits(int b) { return b == 4 || b == 6; }

int orc_chunk_layout(int D, int g, int kb, int vb, int64_t off[7])
{
    if (D <= 0 || D % 16 != 0) return -1;
    int fp16 = (kb == 16 && vb == 16);
    if (!fp16 && !(valid_bits(kb) && valid_bits(vb))) return -1;
    if (!fp16 && (g <= 0 || D % g != 0)) return -1;
    int64_t ngroups = fp16 ? 0 : D / g;
    int64_t sz[6];
    sz[0] = (int64_t)BT * D * kb / 8;   /* K codes  */
    sz[1] = (int64_t)D * BT * vb / 8;   /* V codes  */
    sz[2] = ngroups * BT * 4;           /* K scales */
    sz[3] = ngroups * BT * 4;           /* V scales */
    sz[4] = ngroups * BT;               /* K zeros  */
    sz[5] = ngroups * BT;               /* V zeros  */
    int64_t at = 0;
    for (int i = 0; i < 6; i++) {
        off[i] = at;
        at += pad128(sz[i]);
    }
    off[6] = at;
    return 0;
}

/* ---------------------------------------------------------------- bits */

uint32_t orc_get_field(const uint8_t* stream, int64_t idx, int bits)
{
    uint32_t v = 0;
    for (int t = 0; t < bits; t++) {
        int64_t pos = idx * bits + t;
        v |= (uint32_t)((stream[pos >> 3] >> (pos & 7)) & 1u) << t;
    }
    return v;
}

void orc_put_field(uint8_t* stream, int64_t idx, int bits, uint32_t value)
{
    for (int t = 0; t < bits; t++) {
        int64_t pos = idx * bits + t;
        uint8_t m = (uint8_t)(1u << (pos & 7));
        if ((value >> t) & 1u) stream[pos >> 3] |= m;
        else stream[pos >> 3] &= (uint8_t)~m;
    }
}

/* ---------------------------------------------------------------- fp16 */

/* Round-to-nearest-even conversion written from the IEEE 754 binary16
 * definition: 1 sign, 5 exponent (bias 15), 10 fraction bits; subnormals
 * have spacing 2^-24; magnitudes that round past 65504 become infinity. */
uint16_t orc_f32_to_f16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t ex = (u >> 23) & 0xFFu, man = u & 0x7FFFFFu;
    if (ex == 0xFFu) return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
    uint64_t sig;
    int lsb_exp; /* |x| = sig * 2^lsb_exp */
    if (ex == 0) { sig = man; lsb_exp = -149; }
    else { sig = man | 0x800000u; lsb_exp = (int)ex - 150; }
    if (sig == 0) return sign;
    int top = 63 - __builtin_clzll(sig);
    int k = top + lsb_exp;            /* floor(log2|x|) */
    int ulp_exp = k - 10;             /* 11 significant bits */
    if (ulp_exp < -24) ulp_exp = -24; /* subnormal spacing */
    int shift = ulp_exp - lsb_exp;    /* >= 13 for every fp32 input */
    uint64_t r;
    if (shift >= 64) {
        r = 0;
    } else {
        uint64_t qv = sig >> shift;
        uint64_t rem = sig & ((1ull << shift) - 1);
        uint64_t half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (qv & 1))) qv++;
        r = qv;
    }
    if (r == 0) return sign;
    if (r >= 2048) { r >>= 1; ulp_exp++; }
    if (r < 1024) return (uint16_t)(sign | (uint16_t)r); /* subnormal */
    int e16 = ulp_exp + 25;
    if (e16 >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((e16 << 10) | (int)(r & 0x3FF)));
}

double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0) v = ldexp((double)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* --------------------------------------------------------- quantisation */

/* One group, fp32, in this order (asymmetric grouped quantisation, TurboQuant
 * page, core innovation; bit widths from the Super KV Compression page, first
 * layer):
 *   mn, mx     = exact minimum / maximum of the group
 *   constant   (mn == mx, value c): (s, z, q) = (c, 0, 1) if c > 0,
 *              (-c, 1, 0) if c < 0, (0, 0, 0) if c == 0, so (q - z) * s == c
 *   otherwise  lo = min(mn, 0), hi = max(mx, 0)   (range holds 0)
 *              s  = (hi - lo) / qmax               (correctly rounded)
 *              z  = clamp(rint(-lo / s), 0, qmax)
 *              q  = clamp(rint(x / s) + z, 0, qmax)
 * rint rounds half to even. */
void orc_quantize_group(const float* x, int n, int bits,
                        float* scale, uint8_t* zero, uint8_t* codes)
{
    const int qmax = (1 << bits) - 1;
    float mn = x[0], mx = x[0];
    for (int i = 1; i < n; i++) {
        if (x[i] < mn) mn = x[i];
        if (x[i] > mx) mx = x[i];
    }
    if (mn == mx) {
        float c = mn;
        float s;
        int z, q;
        if (c > 0.0f) { s = c; z = 0; q = 1; }
        else if (c < 0.0f) { s = -c; z = 1; q = 0; }
        else { s = 0.0f; z = 0; q = 0; }
        *scale = s;
        *zero = (uint8_t)z;
        for (int i = 0; i < n; i++) codes[i] = (uint8_t)q;
        return;
    }
    float lo = mn < 0.0f ? mn : 0.0f;
    float hi = mx > 0.0f ? mx : 0.0f;
    float r = hi - lo;
    float s = r / (float)qmax;
    float neg_lo = -lo;
    int z = (int)rintf(neg_lo / s);
    if (z < 0) z = 0;
    if (z > qmax) z = qmax;
    for (int i = 0; i < n; i++) {
        int q = (int)rintf(x[i] / s) + z;
        if (q < 0) q = 0;
        if (q > qmax) q = qmax;
        codes[i] = (uint8_t)q;
    }
    *scale = s;
    *zero = (uint8_t)z;
}

/* -------------------------------------------------------------- chunks */

typedef struct {
    int D, g, kb, vb, H, fp16, ngroups;
    int knorm;      /* direction-preserving K: factor section at off_kn */
    int64_t off_kn;
    int64_t off[7]; /* [6]: chunk bytes, the factor section included */
    int64_t krow; /* bytes per K token row */
    int64_t vrow; /* bytes per V channel row */
} fmt_t;

static int make_fmt(const orc_cache* c, fmt_t* f)
{
    if (orc_chunk_layout(c->head_dim, c->group_size, c->k_bits, c->v_bits, f->off) != 0)
        return -1;
    if (c->head_dim > 1024) return -1; /* bounds the per-row scratch arrays */
    if (c->num_kv_heads <= 0 || c->num_blocks <= 0 || !c->pool) return -1;
    f->D = c->head_dim;
    f->g = c->group_size;
    f->kb = c->k_bits;
    f->vb = c->v_bits;
    f->H = c->num_kv_heads;
    f->fp16 = (c->k_bits == 16);
    f->ngroups = f->fp16 ? 0 : c->head_dim / c->group_size;
    f->krow = (int64_t)f->D * f->kb / 8;
    f->vrow = (int64_t)BT * f->vb / 8;
    f->knorm = c->k_norm != 0;
    f->off_kn = f->off[6];
    if (f->knorm) {
        if (f->fp16) return -1;
        f->off[6] += BT * 4; /* one fp32 factor per slot (256 B, a multiple of 128) */
    }
    return 0;
}

static float get_knorm(const uint8_t* ch, const fmt_t* f, int slot)
{
    float r;
    memcpy(&r, ch + f->off_kn + (int64_t)slot * 4, 4);
    return r;
}

static uint8_t* chunk_ptr(const orc_cache* c, const fmt_t* f, int64_t blk, int kvh)
{
    return c->pool + (blk * f->H + kvh) * f->off[6];
}

static float get_scale(const uint8_t* ch, const fmt_t* f, int sec, int gi, int slot)
{
    float s;
    memcpy(&s, ch + f->off[sec] + ((int64_t)gi * BT + slot) * 4, 4);
    return s;
}

static void set_scale(uint8_t* ch, const fmt_t* f, int sec, int gi, int slot, float s)
{
    memcpy(ch + f->off[sec] + ((int64_t)gi * BT + slot) * 4, &s, 4);
}

static uint8_t get_zero(const uint8_t* ch, const fmt_t* f, int sec, int gi, int slot)
{
    return ch[f->off[sec] + (int64_t)gi * BT + slot];
}

static void set_zero(uint8_t* ch, const fmt_t* f, int sec, int gi, int slot, uint8_t z)
{
    ch[f->off[sec] + (int64_t)gi * BT + slot] = z;
}

/* K code of channel d of the token in `slot`, and V code of channel d. */
static uint32_t get_k(const uint8_t* ch, const fmt_t* f, int slot, int d)
{
    return orc_get_field(ch + f->off[0] + slot * f->krow, d, f->kb);
}
static uint32_t get_v(const uint8_t* ch, const fmt_t* f, int slot, int d)
{
    return orc_get_field(ch + f->off[1] + d * f->vrow, slot, f->vb);
}
static void put_k(uint8_t* ch, const fmt_t* f, int slot, int d, uint32_t v)
{
    orc_put_field(ch + f->off[0] + slot * f->krow, d, f->kb, v);
}
static void put_v(uint8_t* ch, const fmt_t* f, int slot, int d, uint32_t v)
{
    orc_put_field(ch + f->off[1] + d * f->vrow, slot, f->vb, v);
}

/* Quantise (or, for fp16, convert) one row of D values into a slot.
 * is_v selects the V sections. */
static void store_row(uint8_t* ch, const fmt_t* f, int slot, const float* x, int is_v)
{
    int bits = is_v ? f->vb : f->kb;
    if (f->fp16) {
        for (int d = 0; d < f->D; d++) {
            uint32_t h = orc_f32_to_f16(x[d]);
            if (is_v) put_v(ch, f, slot, d, h);
            else put_k(ch, f, slot, d, h);
        }
        return;
    }
    uint8_t codes[1024];
    for (int gi = 0; gi < f->ngroups; gi++) {
        float s;
        uint8_t z;
        orc_quantize_group(x + gi * f->g, f->g, bits, &s, &z, codes);
        for (int i = 0; i < f->g; i++) {
            int d = gi * f->g + i;
            if (is_v) put_v(ch, f, slot, d, codes[i]);
            else put_k(ch, f, slot, d, codes[i]);
        }
        set_scale(ch, f, is_v ? 3 : 2, gi, slot, s);
        set_zero(ch, f, is_v ? 5 : 4, gi, slot, z);
    }
    if (!is_v && f->knorm) {
        /* Direction-preserving K (norm-direction page, insight of the method):
         * the group codes carry the key's direction (group quantisation is
         * invariant to scaling the whole key); the factor r = |k| / |k_hat|
         * restores the norm, so that the key read back is r * k_hat, with
         * the direction of the codes and the norm of k.  Norms in fp64, r
         * rounded once to fp32; a zero k_hat takes r = 1. */
        double nx = 0.0, nk = 0.0;
        for (int d = 0; d < f->D; d++) {
            const int gi = d / f->g;
            const double kh = (double)((int)get_k(ch, f, slot, d) - (int)get_zero(ch, f, 4, gi, slot)) *
                              (double)get_scale(ch, f, 2, gi, slot);
            nx += (double)x[d] * (double)x[d];
            nk += kh * kh;
        }
        const float r = nk > 0.0 ? (float)sqrt(nx / nk) : 1.0f;
        memcpy(ch + f->off_kn + (int64_t)slot * 4, &r, 4);
    }
}

/* ------------------------------------------------------------- append */

int orc_append(const orc_cache* c, const float* k, const float* v,
               const int32_t* cu_new, const int32_t* start_pos,
               const int32_t* block_table, int32_t max_blocks, int32_t batch)
{
    fmt_t f;
    if (make_fmt(c, &f) != 0 || batch < 0 || max_blocks <= 0) return -1;
    /* validate every destination before writing anything */
    for (int b = 0; b < batch; b++) {
        int n = cu_new[b + 1] - cu_new[b];
        if (n < 0 || start_pos[b] < 0) return -1;
        if (n == 0) continue;
        int64_t last = (int64_t)start_pos[b] + n - 1;
        if (last / BT >= max_blocks) return -1;
        for (int64_t lb = start_pos[b] / BT; lb <= last / BT; lb++) {
            int32_t blk = block_table[(int64_t)b * max_blocks + lb];
            if (blk < 0 || blk >= c->num_blocks) return -1;
        }
    }
    /* (sequence, KV head) units write disjoint chunks when block tables do
     * not share blocks between sequences, so they run in parallel. */
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < batch; b++) {
        for (int kvh = 0; kvh < f.H; kvh++) {
            int n = cu_new[b + 1] - cu_new[b];
            for (int t = 0; t < n; t++) {
                int64_t pos = (int64_t)start_pos[b] + t;
                int32_t blk = block_table[(int64_t)b * max_blocks + pos / BT];
                int slot = (int)(pos % BT);
                uint8_t* ch = chunk_ptr(c, &f, blk, kvh);
                int64_t row = ((int64_t)(cu_new[b] + t) * f.H + kvh) * f.D;
                store_row(ch, &f, slot, k + row, 0);
                store_row(ch, &f, slot, v + row, 1);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------- decode */

/* Dequantised value of one cached element, exact in fp64: (q - z) * s, or
 * the fp16 value. */
static double deq_k(const uint8_t* ch, const fmt_t* f, int slot, int d)
{
    uint32_t code = get_k(ch, f, slot, d);
    if (f->fp16) return orc_f16_to_f64((uint16_t)code);
    int gi = d / f->g;
    const double kh = (double)((int)code - (int)get_zero(ch, f, 4, gi, slot)) * (double)get_scale(ch, f, 2, gi, slot);
    return f->knorm ? kh * (double)get_knorm(ch, f, slot) : kh;
}
static double deq_v(const uint8_t* ch, const fmt_t* f, int slot, int d)
{
    uint32_t code = get_v(ch, f, slot, d);
    if (f->fp16) return orc_f16_to_f64((uint16_t)code);
    int gi = d / f->g;
    return (double)((int)code - (int)get_zero(ch, f, 5, gi, slot)) * (double)get_scale(ch, f, 3, gi, slot);
}

/* Softmax attention of one query per head over every live token of every
 * segment, with the sparse-V skip of the Super KV Compression page, third
 * layer, read as follows.  Tokens are visited per split (split_tokens, a
 * multiple of 64, counted from the start of each segment) and, inside a
 * split, per 64-token block.  After a block's scores have been folded into
 * the split's running maximum m and running sum L of exp(s - m), a token j
 * of that block has its V term skipped for head h when
 *     exp(s_j - m) < tau_low * L.
 * Since the final weight of j is at most exp(s_j - m) / L, only tokens whose
 * true softmax weight is under tau_low are skipped.  Skipped tokens stay in
 * the softmax denominator; only their V contribution is dropped.
 *
 * Accumulated attention scores (the signal of the attention-aware tiers,
 * Super KV Compression page, second layer): when score_acc is given, the
 * softmax weight a_jh = exp(s_jh - M_h) / L_h of every live token j of
 * segment s, summed over the query heads h of the sequence, is added to
 * score_acc[s][b][j].  Skipped tokens keep their weight (they stay in the
 * softmax); the sum over heads runs in head order. */
static int decode_impl(const orc_cache* segs, const orc_view* views, int32_t nseg,
                       const float* q, int32_t batch, int32_t num_q_heads,
                       float sm_scale, float tau_low, int32_t split_tokens,
                       double* out, uint8_t* skip, double* score_acc, int32_t acc_stride,
                       const uint8_t* given, double band, uint8_t* ambiguous, double* margin)
{
    if (nseg < 1 || nseg > 8 || batch < 0 || num_q_heads <= 0) return -1;
    if (split_tokens < 0 || split_tokens % BT != 0) return -1;
    fmt_t f[8];
    for (int s = 0; s < nseg; s++) {
        if (make_fmt(&segs[s], &f[s]) != 0) return -1;
        if (f[s].D != f[0].D || f[s].H != f[0].H) return -1;
    }
    const int D = f[0].D, H = f[0].H;
    if (num_q_heads % H != 0) return -1;
    const int G = num_q_heads / H;
    int64_t max_tok = 0, total_cap = 0;
    for (int s = 0; s < nseg; s++) {
        int64_t cap = (int64_t)views[s].max_blocks * BT;
        if (cap > max_tok) max_tok = cap;
        total_cap += cap;
        for (int b = 0; b < batch; b++) {
            int32_t len = views[s].seq_lens[b];
            if (len < 0 || len > cap) return -1;
            for (int lb = 0; lb < (len + BT - 1) / BT; lb++) {
                int32_t blk = views[s].block_table[(int64_t)b * views[s].max_blocks + lb];
                if (blk < 0 || blk >= segs[s].num_blocks) return -1;
            }
        }
    }
    if (score_acc) {
        for (int s = 0; s < nseg; s++)
            for (int b = 0; b < batch; b++)
                if (views[s].seq_lens[b] > acc_stride) return -1;
    }
    /* the weights of every (b, h), summed over h after the parallel loop */
    double* wts = NULL;
    if (score_acc && batch > 0 && total_cap > 0) {
        wts = (double*)malloc(sizeof(double) * (size_t)batch * (size_t)num_q_heads * (size_t)total_cap);
        if (!wts) return -1;
    }
    int fail = 0;
#pragma omp parallel
    {
        double* sc = (double*)malloc(sizeof(double) * (size_t)(total_cap > 0 ? total_cap : 1));
        uint8_t* kept = (uint8_t*)malloc((size_t)(total_cap > 0 ? total_cap : 1));
        double* qd = (double*)malloc(sizeof(double) * (size_t)D);
        if (!sc || !kept || !qd) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for collapse(2) schedule(dynamic)
        for (int b = 0; b < batch; b++) {
            for (int h = 0; h < num_q_heads; h++) {
                if (fail) continue;
                const int kvh = h / G; /* consecutive query heads share a KV head */
                for (int d = 0; d < D; d++) qd[d] = (double)q[((int64_t)b * num_q_heads + h) * D + d];
                /* pass 1: scores, and the skip decision of each token */
                int64_t n = 0;
                for (int s = 0; s < nseg; s++) {
                    const int32_t len = views[s].seq_lens[b];
                    const int32_t split = split_tokens > 0 ? split_tokens : (len > 0 ? len : 1);
                    for (int32_t s0 = 0; s0 < len; s0 += split) {
                        const int32_t s1 = s0 + split < len ? s0 + split : len;
                        double m_run = -INFINITY, l_run = 0.0;
                        for (int32_t b0 = s0; b0 < s1; b0 += BT) {
                            const int32_t b1 = b0 + BT < s1 ? b0 + BT : s1;
                            const int32_t blk = views[s].block_table[(int64_t)b * views[s].max_blocks + b0 / BT];
                            const uint8_t* ch = chunk_ptr(&segs[s], &f[s], blk, kvh);
                            double bmax = -INFINITY;
                            for (int32_t j = b0; j < b1; j++) {
                                double acc = 0.0;
                                for (int d = 0; d < D; d++) acc += qd[d] * deq_k(ch, &f[s], j - b0, d);
                                sc[n + j] = (double)sm_scale * acc;
                                if (sc[n + j] > bmax) bmax = sc[n + j];
                            }
                            double m_new = m_run > bmax ? m_run : bmax;
                            double l_new = l_run * exp(m_run - m_new);
                            for (int32_t j = b0; j < b1; j++) l_new += exp(sc[n + j] - m_new);
                            m_run = m_new;
                            l_run = l_new;
                            for (int32_t j = b0; j < b1; j++) {
                                const double e = exp(sc[n + j] - m_run), t = (double)tau_low * l_run;
                                int sk = tau_low > 0.0f && e < t;
                                /* a margin within band * t of the bound: either
                                 * decision is correct; take the given one */
                                const int64_t at = (((int64_t)b * num_q_heads + h) * nseg + s) * max_tok + j;
                                if (margin && tau_low > 0.0f) margin[at] = (e - t) / t;
                                if (tau_low > 0.0f && fabs(e - t) <= band * t) {
                                    if (ambiguous) ambiguous[at] = 1;
                                    if (given) sk = given[at] != 0;
                                }
                                kept[n + j] = (uint8_t)!sk;
                            }
                        }
                    }
                    n += len;
                }
                /* pass 2: exact softmax over all live tokens, V of kept tokens */
                double M = -INFINITY;
                for (int64_t j = 0; j < n; j++)
                    if (sc[j] > M) M = sc[j];
                double L = 0.0;
                for (int64_t j = 0; j < n; j++) L += exp(sc[j] - M);
                double* o = out + ((int64_t)b * num_q_heads + h) * D;
                for (int d = 0; d < D; d++) o[d] = 0.0;
                int64_t base = 0;
                for (int s = 0; s < nseg; s++) {
                    const int32_t len = views[s].seq_lens[b];
                    for (int32_t j = 0; j < len; j++) {
                        if (skip) {
                            int64_t at = (((int64_t)b * num_q_heads + h) * nseg + s) * max_tok + j;
                            skip[at] = (uint8_t)!kept[base + j];
                        }
                        if (!kept[base + j]) continue;
                        const int32_t blk = views[s].block_table[(int64_t)b * views[s].max_blocks + j / BT];
                        const uint8_t* ch = chunk_ptr(&segs[s], &f[s], blk, kvh);
                        double p = exp(sc[base + j] - M);
                        for (int d = 0; d < D; d++) o[d] += p * deq_v(ch, &f[s], j % BT, d);
                    }
                    base += len;
                }
                if (n > 0)
                    for (int d = 0; d < D; d++) o[d] /= L;
                if (wts) {
                    double* w = wts + ((int64_t)b * num_q_heads + h) * total_cap;
                    for (int64_t j = 0; j < n; j++) w[j] = exp(sc[j] - M) / L;
                }
            }
        }
        free(sc);
        free(kept);
        free(qd);
    }
    if (wts && !fail) {
#pragma omp parallel for schedule(dynamic)
        for (int b = 0; b < batch; b++) {
            int64_t base = 0;
            for (int s = 0; s < nseg; s++) {
                const int32_t len = views[s].seq_lens[b];
                double* acc = score_acc + ((int64_t)s * batch + b) * acc_stride;
                for (int32_t j = 0; j < len; j++) {
                    double sum = 0.0;
                    for (int h = 0; h < num_q_heads; h++)
                        sum += wts[((int64_t)b * num_q_heads + h) * total_cap + base + j];
                    acc[j] += sum;
                }
                base += len;
            }
        }
    }
    free(wts);
    return fail ? -1 : 0;
}

int orc_decode(const orc_cache* segs, const orc_view* views, int32_t nseg,
               const float* q, int32_t batch, int32_t num_q_heads,
               float sm_scale, float tau_low, int32_t split_tokens,
               double* out, uint8_t* skip, double* score_acc, int32_t acc_stride)
{
    return decode_impl(segs, views, nseg, q, batch, num_q_heads, sm_scale, tau_low, split_tokens, out, skip,
                       score_acc, acc_stride, NULL, 0.0, NULL, NULL);
}

/* Several skip sets are correct.  The rule compares exp(s - m) with
 * tau_low * L, and an evaluation in finite precision (fp32 on the GPU) can
 * take either side when the two are closer than its rounding error.  A pair
 * (token, head) whose exact margin |exp(s - m) - tau_low * L| is at most
 * band * tau_low * L is therefore ambiguous: the decision given for it is
 * taken (given may be NULL: the exact decision stays), and it is flagged in
 * ambiguous.  Every other decision is the exact one.  A flipped decision
 * moves the output by at most that token's weight, which is below
 * tau_low * (1 + band), times max |v_hat|.  margin (may be NULL) receives
 * the relative margin (exp(s - m) - tau_low * L) / (tau_low * L) of every
 * live pair when tau_low > 0.  score_acc (may be NULL) accumulates the
 * softmax weights as orc_decode does: they do not depend on the skip. */
int orc_decode_resolved(const orc_cache* segs, const orc_view* views, int32_t nseg,
                        const float* q, int32_t batch, int32_t num_q_heads,
                        float sm_scale, float tau_low, int32_t split_tokens,
                        double* out, uint8_t* skip, const uint8_t* given, double band, uint8_t* ambiguous,
                        double* margin, double* score_acc, int32_t acc_stride)
{
    if (!(band >= 0.0)) return -1;
    return decode_impl(segs, views, nseg, q, batch, num_q_heads, sm_scale, tau_low, split_tokens, out, skip,
                       score_acc, acc_stride, given, band, ambiguous, margin);
}

/* --------------------------------------------------------- tier update */

/* Attention-aware tiers, Super KV Compression page, second layer: tokens
 * with score >= tau_high are HIGH and keep K6 and V6; tokens with
 * tau_low <= score < tau_high are MID, keep K6 and get V requantised to 4
 * bits from their dequantised 6-bit values; tokens with score < tau_low are
 * evicted.  Survivors are compacted in increasing token order. */
int orc_tier_update(const orc_cache* src, const orc_view* src_view,
                    const float* scores, int32_t scores_stride,
                    float tau_low, float tau_high,
                    const orc_cache* dst_h, const int32_t* h_block_table, int32_t h_max_blocks,
                    const orc_cache* dst_m, const int32_t* m_block_table, int32_t m_max_blocks,
                    int32_t* n_high, int32_t* n_mid, uint8_t* tiers, int32_t batch)
{
    fmt_t fs, fh, fm;
    if (make_fmt(src, &fs) || make_fmt(dst_h, &fh) || make_fmt(dst_m, &fm)) return -1;
    if (fs.fp16 || fs.vb != 6) return -1;
    if (fs.knorm || fh.knorm || fm.knorm) return -1; /* tiers hold the plain K codec */
    if (fh.D != fs.D || fh.g != fs.g || fh.H != fs.H || fh.kb != fs.kb || fh.vb != 6) return -1;
    if (fm.D != fs.D || fm.g != fs.g || fm.H != fs.H || fm.kb != fs.kb || fm.vb != 4) return -1;
    if (batch < 0 || scores_stride < 0) return -1;
    for (int b = 0; b < batch; b++) {
        int32_t len = src_view->seq_lens[b];
        if (len < 0 || len > scores_stride || len > (int64_t)src_view->max_blocks * BT) return -1;
        int32_t nh = 0, nm = 0;
        for (int32_t j = 0; j < len; j++) {
            float sc = scores[(int64_t)b * scores_stride + j];
            if (sc >= tau_high) nh++;
            else if (sc >= tau_low) nm++;
        }
        if (nh > (int64_t)h_max_blocks * BT || nm > (int64_t)m_max_blocks * BT) return -1;
        for (int lb = 0; lb < (nh + BT - 1) / BT; lb++) {
            int32_t blk = h_block_table[(int64_t)b * h_max_blocks + lb];
            if (blk < 0 || blk >= dst_h->num_blocks) return -1;
        }
        for (int lb = 0; lb < (nm + BT - 1) / BT; lb++) {
            int32_t blk = m_block_table[(int64_t)b * m_max_blocks + lb];
            if (blk < 0 || blk >= dst_m->num_blocks) return -1;
        }
        for (int lb = 0; lb < (len + BT - 1) / BT; lb++) {
            int32_t blk = src_view->block_table[(int64_t)b * src_view->max_blocks + lb];
            if (blk < 0 || blk >= src->num_blocks) return -1;
        }
    }
#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < batch; b++) {
        const int32_t len = src_view->seq_lens[b];
        int32_t nh = 0, nm = 0;
        for (int32_t j = 0; j < len; j++) {
            const float sc = scores[(int64_t)b * scores_stride + j];
            const int tier = sc >= tau_high ? 2 : (sc >= tau_low ? 1 : 0);
            tiers[(int64_t)b * scores_stride + j] = (uint8_t)tier;
            if (tier == 0) continue;
            const int32_t sblk = src_view->block_table[(int64_t)b * src_view->max_blocks + j / BT];
            const int sslot = j % BT;
            int32_t dpos = tier == 2 ? nh++ : nm++;
            const orc_cache* dc = tier == 2 ? dst_h : dst_m;
            const fmt_t* fd = tier == 2 ? &fh : &fm;
            const int32_t* dbt = tier == 2 ? h_block_table : m_block_table;
            const int32_t dmax = tier == 2 ? h_max_blocks : m_max_blocks;
            const int32_t dblk = dbt[(int64_t)b * dmax + dpos / BT];
            const int dslot = dpos % BT;
            for (int kvh = 0; kvh < fs.H; kvh++) {
                const uint8_t* sch = chunk_ptr(src, &fs, sblk, kvh);
                uint8_t* dch = chunk_ptr(dc, fd, dblk, kvh);
                /* K row, K scales and K zeros: copied bit for bit */
                for (int d = 0; d < fs.D; d++) put_k(dch, fd, dslot, d, get_k(sch, &fs, sslot, d));
                for (int gi = 0; gi < fs.ngroups; gi++) {
                    set_scale(dch, fd, 2, gi, dslot, get_scale(sch, &fs, 2, gi, sslot));
                    set_zero(dch, fd, 4, gi, dslot, get_zero(sch, &fs, 4, gi, sslot));
                }
                if (tier == 2) {
                    /* HIGH: V6 codes, scales and zeros copied bit for bit */
                    for (int d = 0; d < fs.D; d++) put_v(dch, fd, dslot, d, get_v(sch, &fs, sslot, d));
                    for (int gi = 0; gi < fs.ngroups; gi++) {
                        set_scale(dch, fd, 3, gi, dslot, get_scale(sch, &fs, 3, gi, sslot));
                        set_zero(dch, fd, 5, gi, dslot, get_zero(sch, &fs, 5, gi, sslot));
                    }
                } else {
                    /* MID: dequantise V6 in fp32 ((q - z) * s, one rounding),
                     * then quantise those values at 4 bits */
                    float row[1024];
                    for (int d = 0; d < fs.D; d++) {
                        int gi = d / fs.g;
                        float s6 = get_scale(sch, &fs, 3, gi, sslot);
                        int z6 = get_zero(sch, &fs, 5, gi, sslot);
                        row[d] = (float)((int)get_v(sch, &fs, sslot, d) - z6) * s6;
                    }
                    store_row(dch, fd, dslot, row, 1);
                }
            }
        }
        n_high[b] = nh;
        n_mid[b] = nm;
    }
    return 0;
}

/* One token of one KV head from a source chunk to a destination chunk: the
 * K row, K scales and K zeros bit for bit; the V row bit for bit when the
 * formats match, else (V6 -> V4) dequantised in fp32 and quantised at 4
 * bits, as the tier update does for MID tokens. */
static void move_token(const uint8_t* sch, const fmt_t* fs, int sslot, uint8_t* dch, const fmt_t* fd, int dslot)
{
    for (int d = 0; d < fs->D; d++) put_k(dch, fd, dslot, d, get_k(sch, fs, sslot, d));
    for (int gi = 0; gi < fs->ngroups; gi++) {
        set_scale(dch, fd, 2, gi, dslot, get_scale(sch, fs, 2, gi, sslot));
        set_zero(dch, fd, 4, gi, dslot, get_zero(sch, fs, 4, gi, sslot));
    }
    if (fs->vb == fd->vb) {
        for (int d = 0; d < fs->D; d++) put_v(dch, fd, dslot, d, get_v(sch, fs, sslot, d));
        for (int gi = 0; gi < fs->ngroups; gi++) {
            set_scale(dch, fd, 3, gi, dslot, get_scale(sch, fs, 3, gi, sslot));
            set_zero(dch, fd, 5, gi, dslot, get_zero(sch, fs, 5, gi, sslot));
        }
    } else {
        float row[1024];
        for (int d = 0; d < fs->D; d++) {
            int gi = d / fs->g;
            row[d] = (float)((int)get_v(sch, fs, sslot, d) - get_zero(sch, fs, 5, gi, sslot)) *
                     get_scale(sch, fs, 3, gi, sslot);
        }
        store_row(dch, fd, dslot, row, 1);
    }
}

static int blocks_valid(const orc_view* v, const orc_cache* c, int b, int32_t n)
{
    for (int lb = 0; lb < (n + BT - 1) / BT; lb++) {
        int32_t blk = v->block_table[(int64_t)b * v->max_blocks + lb];
        if (blk < 0 || blk >= c->num_blocks) return 0;
    }
    return 1;
}

/* Re-tiering of a tiered cache with fresh scores (the periodic form of the
 * attention-aware tiers, Super KV Compression page, second layer).  The
 * HIGH segment (K6V6) and the MID segment (K6V4) are rebuilt into new ones:
 *   HIGH token, score >= tau_high           stays HIGH (copied)
 *   HIGH token, tau_low <= score < tau_high demoted to MID (V requantised)
 *   MID token,  score >= tau_low            stays MID (copied; its 6-bit
 *                                           values are gone, so it is never
 *                                           promoted)
 *   any token,  score < tau_low             evicted
 * New HIGH: HIGH-kept tokens in order.  New MID: MID-kept tokens in order,
 * then demoted tokens in order.  h_tiers / m_tiers receive the new tier of
 * every token of each source (2, 1 or 0). */
int orc_retier(const orc_cache* h, const orc_view* h_view, const float* h_scores, int32_t h_stride,
               const orc_cache* m, const orc_view* m_view, const float* m_scores, int32_t m_stride,
               float tau_low, float tau_high,
               const orc_cache* dst_h, const int32_t* dh_bt, int32_t dh_max_blocks,
               const orc_cache* dst_m, const int32_t* dm_bt, int32_t dm_max_blocks,
               int32_t* n_high, int32_t* n_mid, uint8_t* h_tiers, uint8_t* m_tiers, int32_t batch)
{
    fmt_t fh, fm, fdh, fdm;
    if (make_fmt(h, &fh) || make_fmt(m, &fm) || make_fmt(dst_h, &fdh) || make_fmt(dst_m, &fdm)) return -1;
    if (fh.fp16 || fh.vb != 6 || fm.vb != 4 || fdh.vb != 6 || fdm.vb != 4) return -1;
    if (fh.knorm || fm.knorm || fdh.knorm || fdm.knorm) return -1; /* tiers hold the plain K codec */
    const fmt_t* all[3] = {&fm, &fdh, &fdm};
    for (int i = 0; i < 3; i++)
        if (all[i]->D != fh.D || all[i]->g != fh.g || all[i]->H != fh.H || all[i]->kb != fh.kb) return -1;
    if (batch < 0 || h_stride < 0 || m_stride < 0) return -1;
    for (int b = 0; b < batch; b++) {
        const int32_t lh = h_view->seq_lens[b], lm = m_view->seq_lens[b];
        if (lh < 0 || lh > h_stride || lh > (int64_t)h_view->max_blocks * BT) return -1;
        if (lm < 0 || lm > m_stride || lm > (int64_t)m_view->max_blocks * BT) return -1;
        int32_t nh = 0, nm = 0;
        for (int32_t j = 0; j < lh; j++) {
            const float sc = h_scores[(int64_t)b * h_stride + j];
            nh += sc >= tau_high;
            nm += sc >= tau_low && sc < tau_high;
        }
        for (int32_t j = 0; j < lm; j++) nm += m_scores[(int64_t)b * m_stride + j] >= tau_low;
        if (nh > (int64_t)dh_max_blocks * BT || nm > (int64_t)dm_max_blocks * BT) return -1;
        const orc_view dh_view = {dh_bt, NULL, dh_max_blocks}, dm_view = {dm_bt, NULL, dm_max_blocks};
        if (!blocks_valid(h_view, h, b, lh) || !blocks_valid(m_view, m, b, lm) ||
            !blocks_valid(&dh_view, dst_h, b, nh) || !blocks_valid(&dm_view, dst_m, b, nm))
            return -1;
    }
#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < batch; b++) {
        const int32_t lh = h_view->seq_lens[b], lm = m_view->seq_lens[b];
        int32_t nh = 0, nm = 0;
        /* MID-kept tokens first, then the demoted ones */
        for (int pass = 0; pass < 3; pass++) {
            const int from_m = pass == 0;
            const int32_t len = from_m ? lm : lh;
            for (int32_t j = 0; j < len; j++) {
                const float sc = from_m ? m_scores[(int64_t)b * m_stride + j] : h_scores[(int64_t)b * h_stride + j];
                const int tier = from_m ? (sc >= tau_low ? 1 : 0) : (sc >= tau_high ? 2 : (sc >= tau_low ? 1 : 0));
                if (pass == 0) m_tiers[(int64_t)b * m_stride + j] = (uint8_t)tier;
                if (pass == 1) h_tiers[(int64_t)b * h_stride + j] = (uint8_t)tier;
                /* pass 1 places demoted tokens, pass 2 HIGH-kept ones */
                const int place = pass == 0 ? tier == 1 : (pass == 1 ? tier == 1 : tier == 2);
                if (!place) continue;
                const orc_cache* sc_c = from_m ? m : h;
                const fmt_t* fs = from_m ? &fm : &fh;
                const orc_view* sv = from_m ? m_view : h_view;
                const int32_t sblk = sv->block_table[(int64_t)b * sv->max_blocks + j / BT];
                const int to_h = pass == 2;
                const int32_t dpos = to_h ? nh++ : nm++;
                const int32_t dblk = to_h ? dh_bt[(int64_t)b * dh_max_blocks + dpos / BT]
                                          : dm_bt[(int64_t)b * dm_max_blocks + dpos / BT];
                for (int kvh = 0; kvh < fh.H; kvh++)
                    move_token(chunk_ptr(sc_c, fs, sblk, kvh), fs, j % BT,
                               chunk_ptr(to_h ? dst_h : dst_m, to_h ? &fdh : &fdm, dblk, kvh), to_h ? &fdh : &fdm,
                               dpos % BT);
            }
        }
        n_high[b] = nh;
        n_mid[b] = nm;
    }
    return 0;
}

void orc_default_thresholds(int32_t n_tokens, float* tau_low, float* tau_high)
{
    const double eps4 = 1.0 / (2.0 * 15.0); /* half a 4-bit step, relative to the range */
    const double eps6 = 1.0 / (2.0 * 63.0); /* half a 6-bit step */
    const double n = n_tokens > 0 ? (double)n_tokens : 1.0;
    *tau_low = (float)(eps4 / n);
    *tau_high = (float)((eps4 / eps6) / n);
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
