/*
 * mxoracle.c -- plain, slow CPU oracle for MXFP4 block quantization and
 * MXFP4 attention (OCP / UOS scale rules, optional Pre-Normalization
 * Quantization).  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and
 * the CPU-baseline leg of the benchmark call it; the GPU library never does.
 * It shares no code, header, table or constant with the HIP path.
 *
 * Everything is computed in IEEE binary64.  Inputs arrive as their exact
 * stored values (fp32 or bf16 bit patterns) and are widened exactly.
 *
 * Sources (cited by page title and section):
 *  [MXA]  "MXAttention: Data-Free Optimal Scaling and Pre-Normalization
 *         Quantization for MXFP4 Attention", abstract: MXFP4 attention, the
 *         OCP baseline scale, Universal Optimal Scaling with boundary
 *         Qmax = 7.25, and PNQ (quantize the unnormalized softmax
 *         exponentials before the row-wise sum).
 *  [EFQ]  "EFQ-Softmax", abstract: low-bit attention runs QK^T and PV on
 *         FP4 engines; the quantized probability operand feeds both the
 *         P~V numerator and the P~1 denominator; the FlashAttention row-max
 *         update, historical rescaling, high-precision accumulation and
 *         final normalization are unchanged.
 *  [QE]   "Quantization Error" (Format / Analysis), section "Where the error
 *         comes from": one rounding step onto eight magnitudes, an exact
 *         power-of-two scale, order independence of blocks.
 *  [OCP-MX] the OCP Microscaling Formats v1.0 specification: E2M1 element
 *         magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, E8M0 scale 2^(X-127) with
 *         X in [0, 254] (255 = NaN), shared exponent floor(log2 amax) - 2.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - OCP rule: smallest e with amax < 8 * 2^e  (== floor(log2 amax) - 2).
 *  - UOS rule: smallest e with amax <= 7.25 * 2^e (boundary inclusive).
 *  - e is clamped to [-127, 127]; amax == 0 gives e = -127.
 *  - element rounding: nearest magnitude, ties to the even code, saturating
 *    at 6; sign kept as a separate bit (a negative value that rounds to zero
 *    gets code 0x8).
 *  - packing: element 2j in the low nibble of byte j.
 *  - attention: scale 1/sqrt(D) applied to the raw dot product of the
 *    dequantized operands; running max updated per KV tile of Bc keys in
 *    ascending order; P~ blocks are 32 keys aligned at key 0; in the OCP and
 *    UOS modes the row sum uses the unquantized p, in UOS+PNQ the quantized
 *    p~.  Query head h reads KV head h / (Hq / Hkv).  Causal: key j <= i.
 *  - UOS+EFQ mode ([EFQ] abstract: exponent-only block scale from the local
 *    maximum, scores mapped to a residual domain, nonnegative E2M1 codes by
 *    one affine rule; the same P~ in numerator and denominator).  The rule's
 *    constants are not on the pages; reading: in log2 units
 *    z = (s - m) * log2(e), e_b = the smallest exponent >= -127 with
 *    z_max - e_b < rho, r = z - e_b, code = clamp(rne(2 r + beta), 0, 7),
 *    p~ = E2M1(code) * 2^e_b.  "2 codes per binade" matches the E2M1 grid
 *    above 1; beta is the least-squares fit of the five rounding boundaries
 *    of codes 2..7 (log2 of the midpoints 1.25 .. 5); rho = (7.5 - beta)/2
 *    - 2^-10 keeps the block maximum below code 8.  Q, K, V use UOS.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_RULE_OCP 0
#define ORC_RULE_UOS 1

#define ORC_MODE_FP16 0
#define ORC_MODE_OCP 1
#define ORC_MODE_UOS 2
#define ORC_MODE_UOS_PNQ 3
#define ORC_MODE_UOS_EFQ 4

#define ORC_BLOCK 32

/* The eight E2M1 magnitudes, indexed by the 3-bit magnitude code [OCP-MX]. */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Exact widening of one stored input element. */
static double load_elem(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORC_F32)
        return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* 2^e exactly (e well inside binary64's normal range here). */
static double pow2i(int e) { return ldexp(1.0, e); }

/* EFQ affine-rule offset beta: least-squares fit of round(2 r + beta) to the
 * E2M1 rounding boundaries between codes c and c+1 (c = 2..6), which lie at
 * r = log2((mag[c] + mag[c+1]) / 2); the rule puts them at (c + 1/2 - beta)/2. */
double oracle_efq_beta(void)
{
    double sum = 0.0;
    for (int c = 2; c <= 6; ++c)
        sum += (double)c + 0.5 - 2.0 * log2(0.5 * (E2M1_MAG[c] + E2M1_MAG[c + 1]));
    return sum / 5.0;
}

/* Largest residual the block maximum may take: 2 r + beta stays below 7.5
 * (code 7 at most), with a 2^-10 margin. */
double oracle_efq_rho(void)
{
    return 0.5 * (7.5 - oracle_efq_beta()) - ldexp(1.0, -10);
}

/* EFQ block exponent: the smallest e in [-127, 127] with zmax - e < rho
 * (zmax = log2 of the block's largest unnormalized probability; -inf for a
 * block without a visible key gives -127). */
int oracle_efq_exponent(double zmax)
{
    const double rho = oracle_efq_rho();
    for (int e = -127; e < 127; ++e)
        if (zmax - (double)e < rho)
            return e;
    return 127;
}

/* EFQ code of one residual r = z - e_b: round half to even of 2 r + beta,
 * clamped to [0, 7]. */
int oracle_efq_code(double r)
{
    if (r == -INFINITY)
        return 0;
    double c = nearbyint(2.0 * r + oracle_efq_beta());
    if (c < 0.0)
        c = 0.0;
    if (c > 7.0)
        c = 7.0;
    return (int)c;
}

/* Scale exponent of one block, by its definition: the smallest e >= -127
 * whose scaled block maximum lies inside the rule's range.
 *  OCP : amax <  8    * 2^e   [OCP-MX shared exponent]
 *  UOS : amax <= 7.25 * 2^e   [MXA, Universal Optimal Scaling, Qmax = 7.25]
 * The search walks e upward from the E8M0 minimum; every step is exact. */
int oracle_scale_exponent(double amax, int rule)
{
    int e = -127;
    double bound = (rule == ORC_RULE_UOS ? 7.25 : 8.0) * pow2i(-127);
    for (;;) {
        int inside = (rule == ORC_RULE_UOS) ? (amax <= bound) : (amax < bound);
        if (inside || e == 127)
            return e;
        e += 1;
        bound *= 2.0;
    }
}

/* Round a non-negative scaled magnitude onto the E2M1 grid: values beyond
 * the grid first saturate to the largest magnitude, then the nearest grid
 * value is taken, ties to the even code [QE: rounding to one of eight
 * magnitudes].  With v clipped to [0, 6] every distance to an adjacent grid
 * point is exact in binary64 (Sterbenz), so ties are detected exactly. */
int oracle_round_e2m1(double v)
{
    if (v > E2M1_MAG[7])
        v = E2M1_MAG[7];
    int best = 0;
    double best_d = fabs(v - E2M1_MAG[0]);
    for (int c = 1; c < 8; ++c) {
        double d = fabs(v - E2M1_MAG[c]);
        if (d < best_d || (d == best_d && (c % 2 == 0) && (best % 2 != 0))) {
            best = c;
            best_d = d;
        }
    }
    return best;
}

/* Quantize one block of 32 exact values: returns the E8M0 byte, writes the
 * 32 4-bit codes (sign bit 3, magnitude bits 0..2). */
static uint8_t quantize_block(const double *x, int rule, uint8_t *code)
{
    double amax = 0.0;
    for (int i = 0; i < ORC_BLOCK; ++i)
        if (fabs(x[i]) > amax)
            amax = fabs(x[i]);
    int e = oracle_scale_exponent(amax, rule);
    double inv = pow2i(-e); /* exact: -e in [-127, 127] */
    for (int i = 0; i < ORC_BLOCK; ++i) {
        int mag = oracle_round_e2m1(fabs(x[i]) * inv);
        int sgn = signbit(x[i]) ? 1 : 0;
        code[i] = (uint8_t)((sgn << 3) | mag);
    }
    return (uint8_t)(e + 127);
}

/* Value of one code under one E8M0 byte. */
static double dequant_code(uint8_t code, uint8_t scale_byte)
{
    double mag = E2M1_MAG[code & 7];
    double v = ldexp(mag, (int)scale_byte - 127);
    return (code & 8) ? -v : v;
}

/* Blocks of 32 along the contiguous axis of a flat tensor of n elements
 * (n % 32 == 0).  codes: n/2 bytes (element 2j low nibble), scales: n/32. */
int oracle_quantize(const void *x, int dtype, int64_t n, int rule,
                    uint8_t *codes, uint8_t *scales)
{
    if (n % ORC_BLOCK != 0 || n < 0)
        return -1;
    int64_t nb = n / ORC_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        double blk[ORC_BLOCK];
        uint8_t code[ORC_BLOCK];
        for (int i = 0; i < ORC_BLOCK; ++i)
            blk[i] = load_elem(x, dtype, b * ORC_BLOCK + i);
        scales[b] = quantize_block(blk, rule, code);
        for (int i = 0; i < ORC_BLOCK / 2; ++i)
            codes[b * (ORC_BLOCK / 2) + i] =
                (uint8_t)(code[2 * i] | (code[2 * i + 1] << 4));
    }
    return 0;
}

/* Blocks of 32 along the ROW axis of a row-major [rows][cols] matrix, output
 * transposed: codes_t [cols][rows_pad/2], scales_t [cols][rows_pad/32] with
 * rows_pad = ceil(rows/32)*32; rows beyond `rows` are zero. */
int oracle_quantize_t(const void *x, int dtype, int64_t rows, int64_t cols,
                      int rule, uint8_t *codes_t, uint8_t *scales_t)
{
    if (rows < 0 || cols < 0)
        return -1;
    int64_t nbr = (rows + ORC_BLOCK - 1) / ORC_BLOCK;
    int64_t rows_pad = nbr * ORC_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
        for (int64_t rb = 0; rb < nbr; ++rb) {
            double blk[ORC_BLOCK];
            uint8_t code[ORC_BLOCK];
            for (int i = 0; i < ORC_BLOCK; ++i) {
                int64_t r = rb * ORC_BLOCK + i;
                blk[i] = (r < rows) ? load_elem(x, dtype, r * cols + c) : 0.0;
            }
            scales_t[c * nbr + rb] = quantize_block(blk, rule, code);
            for (int i = 0; i < ORC_BLOCK / 2; ++i)
                codes_t[c * (rows_pad / 2) + rb * (ORC_BLOCK / 2) + i] =
                    (uint8_t)(code[2 * i] | (code[2 * i + 1] << 4));
        }
    }
    return 0;
}

/* Dequantize n elements (n % 32 == 0) to binary64. */
int oracle_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t n,
                      double *y)
{
    if (n % ORC_BLOCK != 0 || n < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint8_t byte = codes[i / 2];
        uint8_t code = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        y[i] = dequant_code(code, scales[i / ORC_BLOCK]);
    }
    return 0;
}

/* Fake-quantize a vector of length len (len % 32 == 0) in place: values are
 * replaced by their dequantized MXFP4 image. */
static void fake_quant(double *x, int64_t len, int rule)
{
    uint8_t code[ORC_BLOCK];
    for (int64_t b = 0; b < len / ORC_BLOCK; ++b) {
        uint8_t s = quantize_block(x + b * ORC_BLOCK, rule, code);
        for (int i = 0; i < ORC_BLOCK; ++i)
            x[b * ORC_BLOCK + i] = dequant_code(code[i], s);
    }
}

/* At the last tile of a split, fold the split's state (m, l, acc) into the
 * merged state (M, Lm, accm); a split that saw no key (m = -inf) adds
 * nothing. */
static void merge_if_split_end(int64_t t, int64_t tiles_per_split, int64_t ntiles, int D,
                               const double *m, const double *l, const double *acc,
                               double *M, double *Lm, double *accm)
{
    if ((t + 1) % tiles_per_split != 0 && t + 1 != ntiles)
        return;
    if (*m == -INFINITY)
        return;
    const double Mn = *M > *m ? *M : *m;
    const double wa = (*M == -INFINITY) ? 0.0 : exp(*M - Mn);
    const double wb = exp(*m - Mn);
    for (int d = 0; d < D; ++d)
        accm[d] = accm[d] * wa + acc[d] * wb;
    *Lm = *Lm * wa + *l * wb;
    *M = Mn;
}

/*
 * Attention on a list of query rows.
 *
 * q [B,Hq,Sq,D], k and v [B,Hkv,Skv,D], row-major, dtype fp32 or bf16.
 * rows[r] = (b*Hq + h)*Sq + i.  mode: 0 FP16 (no quantization), 1 OCP,
 * 2 UOS, 3 UOS+PNQ.  bc: keys per KV tile (multiple of 32) -- the running
 * max is updated once per tile, which fixes the scale of every P~ block.
 *
 * Outputs (nullable except out):
 *   out      [nrows][D]    O rows
 *   l_out    [nrows]       final denominator
 *   m_out    [nrows]       final running max (score units)
 *   m_tiles  [nrows][ceil(Skv/bc)]  running max after each tile (-inf if the
 *                          tile had no valid key and no earlier one did)
 *   p_codes  [nrows][skv_pad/2], p_scales [nrows][skv_pad/32] -- the P~
 *                          codes and E8M0 bytes (quantized modes only),
 *                          skv_pad = ceil(Skv/32)*32, unvisited blocks zero.
 *
 * Causal: query i sees keys j <= i + (Skv - Sq) (queries aligned to the end
 * of the key sequence; Sq == Skv gives j <= i).  Sq <= Skv is required.
 *
 * split (oracle_attn_rows_split): keys per split, a multiple of bc, or 0 for
 * none.  The keys are cut into splits [s*split, (s+1)*split) from key 0; each
 * split runs the tile loop above on its own from m = -inf, so its P~ blocks
 * are scaled by the split's own running max, and the splits are then merged
 * in ascending order by the usual rescaling: with M the larger of the two
 * maxima, acc = acc*exp(m - M) + acc_s*exp(m_s - M), and likewise l.  A
 * split with no visible key contributes nothing.  With one split (or none)
 * this is the unsplit result exactly.
 */
int oracle_attn_rows_split(const void *q, const void *k, const void *v, int dtype,
                           int B, int Hq, int Hkv, int Sq, int Skv, int D,
                           int causal, int mode, int bc, int64_t split,
                           const int64_t *rows, int64_t nrows, double *out,
                           double *l_out, double *m_out, double *m_tiles,
                           uint8_t *p_codes, uint8_t *p_scales)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || D < 1)
        return -1;
    if (Hq % Hkv != 0 || D % ORC_BLOCK != 0 || bc < ORC_BLOCK ||
        bc % ORC_BLOCK != 0 || mode < 0 || mode > 4)
        return -1;
    if (causal && Sq > Skv)
        return -1;
    if (split < 0 || split % bc != 0)
        return -1;
    const int quantized = (mode != ORC_MODE_FP16);
    const int rule = (mode == ORC_MODE_OCP) ? ORC_RULE_OCP : ORC_RULE_UOS;
    const int efq = (mode == ORC_MODE_UOS_EFQ);
    const int pnq = (mode == ORC_MODE_UOS_PNQ) || efq;
    const int group = Hq / Hkv;
    const int64_t skv_pad = ((int64_t)Skv + ORC_BLOCK - 1) / ORC_BLOCK * ORC_BLOCK;
    const int64_t ntiles = ((int64_t)Skv + bc - 1) / bc;
    const int64_t tiles_per_split = (split > 0) ? split / bc : ntiles;
    const double inv_sqrt_d = 1.0 / sqrt((double)D);

    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= (int64_t)B * Hq * Sq)
            return -1;

    double *kt = (double *)malloc(sizeof(double) * (size_t)Skv * D);
    double *vt = (double *)malloc(sizeof(double) * (size_t)skv_pad * D);
    if (!kt || !vt) {
        free(kt);
        free(vt);
        return -2;
    }

    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < Hkv; ++g) {
            /* any requested row in this (b, kv head)? */
            int any = 0;
            for (int64_t r = 0; r < nrows && !any; ++r) {
                int64_t bh = rows[r] / Sq;
                if (bh / Hq == b && (bh % Hq) / group == g)
                    any = 1;
            }
            if (!any)
                continue;
            const int64_t kvbase = ((int64_t)b * Hkv + g) * Skv * D;

            /* K~: blocks of 32 along D, one key row at a time. */
#pragma omp parallel for schedule(static)
            for (int64_t j = 0; j < Skv; ++j) {
                for (int d = 0; d < D; ++d)
                    kt[j * D + d] = load_elem(k, dtype, kvbase + j * D + d);
                if (quantized)
                    fake_quant(kt + j * D, D, rule);
            }
            /* V~: blocks of 32 along keys, per channel, zero-padded. */
#pragma omp parallel for schedule(static)
            for (int d = 0; d < D; ++d) {
                double *col = (double *)malloc(sizeof(double) * (size_t)skv_pad);
                for (int64_t j = 0; j < skv_pad; ++j)
                    col[j] = (j < Skv) ? load_elem(v, dtype, kvbase + j * D + d) : 0.0;
                if (quantized)
                    fake_quant(col, skv_pad, rule);
                for (int64_t j = 0; j < skv_pad; ++j)
                    vt[j * D + d] = col[j];
                free(col);
            }

#pragma omp parallel for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t bh = rows[r] / Sq;
                int i = (int)(rows[r] % Sq);
                int h = (int)(bh % Hq);
                if (bh / Hq != b || h / group != g)
                    continue;

                double *qr = (double *)malloc(sizeof(double) * (size_t)D);
                double *acc = (double *)calloc((size_t)D, sizeof(double));
                double *s = (double *)malloc(sizeof(double) * (size_t)bc);
                double *p = (double *)malloc(sizeof(double) * (size_t)bc);
                double *pt = (double *)malloc(sizeof(double) * (size_t)bc);
                for (int d = 0; d < D; ++d)
                    qr[d] = load_elem(q, dtype, rows[r] * D + d);
                if (quantized)
                    fake_quant(qr, D, rule);

                /* last visible key of this query */
                const int64_t klim = causal ? (int64_t)i + (Skv - Sq) : (int64_t)Skv - 1;
                /* merged state of the finished splits */
                double M = -INFINITY, Lm = 0.0;
                double *accm = (double *)calloc((size_t)D, sizeof(double));
                double m = -INFINITY, l = 0.0;
                uint8_t *pc = p_codes ? p_codes + r * (skv_pad / 2) : NULL;
                uint8_t *ps = p_scales ? p_scales + r * (skv_pad / ORC_BLOCK) : NULL;
                if (pc)
                    memset(pc, 0, (size_t)(skv_pad / 2));
                if (ps)
                    memset(ps, 0, (size_t)(skv_pad / ORC_BLOCK));

                for (int64_t t = 0; t < ntiles; ++t) {
                    if (t % tiles_per_split == 0) {
                        /* a new split starts from scratch */
                        m = -INFINITY;
                        l = 0.0;
                        for (int d = 0; d < D; ++d)
                            acc[d] = 0.0;
                    }
                    int64_t t0 = t * bc;
                    int64_t nvalid = Skv - t0 < bc ? Skv - t0 : bc;
                    if (klim + 1 - t0 < nvalid)
                        nvalid = klim + 1 - t0; /* keys j <= klim only */
                    if (nvalid <= 0) {       /* nothing visible: state unchanged */
                        if (m_tiles)
                            m_tiles[r * ntiles + t] = m;
                        merge_if_split_end(t, tiles_per_split, ntiles, D, &m, &l, acc, &M, &Lm, accm);
                        continue;
                    }
                    /* scores */
                    double tmax = -INFINITY;
                    for (int64_t jj = 0; jj < nvalid; ++jj) {
                        double dot = 0.0;
                        const double *kr = kt + (t0 + jj) * D;
                        for (int d = 0; d < D; ++d)
                            dot += qr[d] * kr[d];
                        s[jj] = dot * inv_sqrt_d;
                        if (s[jj] > tmax)
                            tmax = s[jj];
                    }
                    /* running max and history rescale [EFQ] */
                    double mnew = m > tmax ? m : tmax;
                    double alpha = (m == -INFINITY) ? 0.0 : exp(m - mnew);
                    /* unnormalized exponentials; padded / masked keys are 0 */
                    int64_t tlen = (t0 + bc <= skv_pad) ? bc : skv_pad - t0;
                    for (int64_t jj = 0; jj < tlen; ++jj)
                        p[jj] = (jj < nvalid) ? exp(s[jj] - mnew) : 0.0;
                    /* P~ : blocks of 32 keys aligned at key 0 [MXA PNQ] */
                    for (int64_t jj = 0; jj < tlen; ++jj)
                        pt[jj] = p[jj];
                    if (quantized) {
                        for (int64_t b0 = 0; b0 < tlen; b0 += ORC_BLOCK) {
                            uint8_t code[ORC_BLOCK];
                            uint8_t sb;
                            if (efq) {
                                /* exp-free: codes from the log2 residuals */
                                double z[ORC_BLOCK], zmax = -INFINITY;
                                for (int ii = 0; ii < ORC_BLOCK; ++ii) {
                                    int64_t jj = b0 + ii;
                                    z[ii] = (jj < nvalid) ? (s[jj] - mnew) / log(2.0) : -INFINITY;
                                    if (z[ii] > zmax)
                                        zmax = z[ii];
                                }
                                int eb = oracle_efq_exponent(zmax);
                                for (int ii = 0; ii < ORC_BLOCK; ++ii)
                                    code[ii] = (uint8_t)oracle_efq_code(z[ii] - (double)eb);
                                sb = (uint8_t)(eb + 127);
                            } else {
                                sb = quantize_block(p + b0, rule, code);
                            }
                            for (int ii = 0; ii < ORC_BLOCK; ++ii)
                                pt[b0 + ii] = dequant_code(code[ii], sb);
                            if (pc && ps) {
                                int64_t kb = (t0 + b0) / ORC_BLOCK;
                                ps[kb] = sb;
                                for (int ii = 0; ii < ORC_BLOCK / 2; ++ii)
                                    pc[kb * (ORC_BLOCK / 2) + ii] =
                                        (uint8_t)(code[2 * ii] | (code[2 * ii + 1] << 4));
                            }
                        }
                    }
                    /* denominator: quantized p~ under PNQ, plain p otherwise */
                    double rowsum = 0.0;
                    for (int64_t jj = 0; jj < tlen; ++jj)
                        rowsum += pnq ? pt[jj] : p[jj];
                    l = alpha * l + rowsum;
                    /* numerator: p~ times V~ */
                    for (int d = 0; d < D; ++d)
                        acc[d] *= alpha;
                    for (int64_t jj = 0; jj < tlen; ++jj) {
                        if (pt[jj] == 0.0)
                            continue;
                        const double *vr = vt + (t0 + jj) * D;
                        for (int d = 0; d < D; ++d)
                            acc[d] += pt[jj] * vr[d];
                    }
                    m = mnew;
                    if (m_tiles)
                        m_tiles[r * ntiles + t] = m;
                    /* (merge below) */
                    merge_if_split_end(t, tiles_per_split, ntiles, D, &m, &l, acc, &M, &Lm, accm);
                }
                /* final normalization [EFQ] */
                for (int d = 0; d < D; ++d)
                    out[r * D + d] = accm[d] / Lm;
                if (l_out)
                    l_out[r] = Lm;
                if (m_out)
                    m_out[r] = M;
                free(qr);
                free(acc);
                free(accm);
                free(s);
                free(p);
                free(pt);
            }
        }
    }
    free(kt);
    free(vt);
    return 0;
}

/* Number of OpenMP threads the oracle's parallel loops use. */
#ifdef _OPENMP
#include <omp.h>
#endif
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int oracle_attn_rows(const void *q, const void *k, const void *v, int dtype,
                     int B, int Hq, int Hkv, int Sq, int Skv, int D,
                     int causal, int mode, int bc,
                     const int64_t *rows, int64_t nrows, double *out,
                     double *l_out, double *m_out, double *m_tiles,
                     uint8_t *p_codes, uint8_t *p_scales)
{
    return oracle_attn_rows_split(q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, bc, 0,
                                  rows, nrows, out, l_out, m_out, m_tiles, p_codes, p_scales);
}
