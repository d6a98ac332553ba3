/*
 * qtcq_oracle.c -- plain, slow, single-threaded CPU oracle for the bitshift-trellis
 * hot path (computed codes, Viterbi search, bitstream pack, window decode, BCJR).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code, header, table or constant
 * generator with the HIP library; the two only ever see the same seeded input arrays.
 *
 * Built with:  gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (x86-64 SSE arithmetic: every float operation below is one IEEE-754 binary32 or
 * binary64 operation rounded to nearest-even; no fused multiply-add anywhere).
 *
 * Sources, cited by page title and section:
 *  [QTIP]  "QTIP: Trellis-Coded Quantization Puts 2-Bit LLM Weights 10% Above the
 *          Rate-Distortion Bound, and a Monotone Codebook Loses to Scalar Rounding"
 *          (blog reimplementation of QTIP).  Sections "The trellis: a stateful
 *          codebook" (the decode and Viterbi listings), "The codebook is computed"
 *          (1MAD listing, 3INST prose), "Tail-biting is worth its complexity".
 *  [XOR]   "XOR-Trellis -- Trellis-coded quantization vs VQ codebooks -- What does it
 *          mean?" (explainer).  Sections "Directions, not an atlas" (16-bit state),
 *          "The sign at each junction has to be cheap" (3INST cost: an FP16 add),
 *          "Cliff edges: weighting errors instead of rotating them" (each step's
 *          squared error multiplied by a per-weight weight D).
 *  [BCJR]  "BCJR-QAT: A Differentiable Relaxation of Trellis-Coded Weight
 *          Quantization" (abstract): forward-backward sum-product at temperature,
 *          soft codeword = Boltzmann expectation over trellis paths.
 *
 * Readings where the pages are silent (each listed with its reason in the design
 * notes): the search runs in binary32 with separate sub, square, [weight-multiply] and
 * add, each rounded; ties go to the lowest predecessor index and the lowest final
 * state; the start state is free (plain trellis); the 3INST LCG is the 1MAD LCG,
 * its mask keeps the sign, 2 low exponent bits and 10 mantissa bits of each fp16 half,
 * the magic constant is the fp16 nearest 0.922, the halves are added in fp16 (RNE)
 * and the sum is divided by the printed raw sigma 1.244.  BCJR energy = the Viterbi
 * path cost (a sum), path weight exp(-E / tau), uniform start prior, binary64.
 * Tail-biting: the walk is cyclic (low L-k bits of the last state = high L-k bits of
 * the first) and needs k*T >= L; the stream holds each state's k high bits at bits
 * [t*k, t*k + k) and windows are read modulo k*T; the two-search encoder rotates by
 * floor(T/2) with s'[t] = s[(t + r) mod T], takes the overlap from the high L-k bits
 * of the rotated walk's state at original position 0, and pins the start to states
 * with those high bits and the end to states with those low bits; the exact solver's
 * ties go to the lowest overlap.
 *
 * PARITY UNPINNED: the LCG inside 3INST.  The page names no LCG for 3INST; every
 * other 3INST choice above is pinned by the printed raw sigma, the LCG choice is not
 * (sigma is insensitive to it).
 *
 * XOR-Trellis palette code [XOR "The sign at each junction has to be cheap"]: the
 * state's newest 2 bits are the branch and the L-2 bits above them the branch history;
 * four masked parities of the history pick a palette (first two) and a branch shuffle
 * (last two), the shuffle XORed into the branch to pick the entry; the values are the
 * four printed FP4 palettes, unscaled.  The masks are not printed: they are inputs.
 *
 * Return codes: 0 = ok, 1 = invalid argument, 2 = out of memory.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ENOMEM 2

enum { ORC_CODE_1MAD = 0, ORC_CODE_3INST = 1 };

/* ------------------------------------------------------------------------------ */
/* Computed codes  ([QTIP] "The codebook is computed")                              */
/* ------------------------------------------------------------------------------ */

/* The LCG step of 1MAD: multiply-add, kept modulo 2^32. */
static uint32_t lcg(uint32_t x) { return 34038481u * x + 76625530u; }

/* 1MAD: LCG, then the sum of the four bytes of the result (Irwin-Hall, n = 4), then
 * centre by 510 and divide by 147.8 in binary64, rounded once to binary32. */
float oracle_code_1mad(uint32_t x)
{
    uint32_t u = lcg(x);
    uint32_t s = (u & 255u) + ((u >> 8) & 255u) + ((u >> 16) & 255u) + ((u >> 24) & 255u);
    double c = ((double)s - 510.0) / 147.8;
    return (float)c;
}

/* IEEE binary16 bit pattern -> its exact value as a double. */
static double half_to_double(uint32_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Round a double to the nearest binary16 value (ties to even); finite range only. */
static double round_to_half(double x)
{
    if (x == 0.0 || !isfinite(x))
        return x;
    double ax = fabs(x);
    int e2;
    frexp(ax, &e2);              /* ax = m * 2^e2, m in [0.5, 1) */
    int q = e2 - 11;             /* spacing of binary16 values near ax is 2^(e2-11) */
    if (q < -24) q = -24;        /* subnormal spacing */
    double scaled = ldexp(ax, -q);     /* exact */
    double r = nearbyint(scaled);      /* default rounding mode: nearest, ties to even */
    double v = ldexp(r, q);
    if (v > 65504.0) v = INFINITY;
    return x < 0 ? -v : v;
}

/* 3INST before its scale: the LCG output, masked to the sign, the 2 low exponent bits
 * and the 10 mantissa bits of each 16-bit half, XORed into the fp16 bit pattern of the
 * magic constant on both halves, and the two fp16 halves added in fp16. */
double oracle_code_3inst_raw(uint32_t x)
{
    const uint32_t magic16 = 0x3B60u; /* binary16 nearest to 0.922 (= 0.921875) */
    uint32_t u = lcg(x);
    uint32_t v = (u & 0x8FFF8FFFu) ^ ((magic16 << 16) | magic16);
    double hi = half_to_double(v >> 16);
    double lo = half_to_double(v & 0xFFFFu);
    return round_to_half(hi + lo); /* hi + lo is exact in binary64 */
}

/* 3INST: the raw fp16 sum divided by the printed raw sigma (1.244) in binary64,
 * rounded once to binary32. */
float oracle_code_3inst(uint32_t x)
{
    double h = oracle_code_3inst_raw(x);
    return (float)(h / 1.244);
}

/* Fill C[0 .. 2^L) with the code value of every L-bit state. */
/* XOR-Trellis palette code [XOR "The sign at each junction has to be cheap"]: the four
 * FP4 palettes as printed, the parity of a masked history read bit by bit. */
static const double XOR_PALETTE[4][4] = {
    {-6.0, -1.5, 0.0, 2.0},
    {-4.0, -1.0, 0.5, 3.0},
    {-3.0, -0.5, 1.0, 4.0},
    {-2.0, 0.0, 1.5, 6.0},
};

static uint32_t parity_of(uint32_t v)
{
    uint32_t p = 0;
    while (v) {
        p ^= v & 1u;
        v >>= 1;
    }
    return p;
}

float oracle_code_xor(uint32_t x, const uint32_t* masks)
{
    uint32_t branch = x & 3u;          /* the newest 2 bits: this step's branch */
    uint32_t history = x >> 2;         /* the L-2 earlier branch bits */
    uint32_t palette = 2u * parity_of(history & masks[0]) + parity_of(history & masks[1]);
    uint32_t shuffle = 2u * parity_of(history & masks[2]) + parity_of(history & masks[3]);
    return (float)XOR_PALETTE[palette][branch ^ shuffle];
}

/* Table of the XOR code at L (2 <= L <= 16, masks below 2^(L-2)). */
int oracle_code_table_xor(int L, const uint32_t* masks, float* C)
{
    if (L < 2 || L > 16 || !C || !masks) return ORC_EINVAL;
    for (int i = 0; i < 4; ++i)
        if ((masks[i] >> (L - 2)) != 0) return ORC_EINVAL;
    uint32_t n = 1u << L;
    for (uint32_t j = 0; j < n; ++j)
        C[j] = oracle_code_xor(j, masks);
    return ORC_OK;
}

int oracle_code_table(int code, int L, float* C)
{
    if (L < 1 || L > 24 || !C) return ORC_EINVAL;
    if (code != ORC_CODE_1MAD && code != ORC_CODE_3INST) return ORC_EINVAL;
    uint32_t n = 1u << L;
    for (uint32_t j = 0; j < n; ++j)
        C[j] = code == ORC_CODE_1MAD ? oracle_code_1mad(j) : oracle_code_3inst(j);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* Viterbi on the bitshift trellis  ([QTIP] "The trellis: a stateful codebook")     */
/* ------------------------------------------------------------------------------ */

/* Squared error of reconstructing target s with value c, in binary32, optionally
 * multiplied by the per-weight error weight ([XOR] "Cliff edges ...").  Each of the
 * sub, square and multiply is one rounded binary32 operation. */
static float step_error(float c, float s, const float* w, int t)
{
    float d = c - s;
    float e = d * d;
    if (w) e = w[t] * e;
    return e;
}

static int check_trellis(int T, int L, int k)
{
    if (T < 1 || L < 1 || L > 20 || k < 1 || k > L) return 0;
    return 1;
}

/* Minimum-cost walk through the (L, k) bitshift trellis for targets s[0..T).
 * State j follows state i when the top L-k bits of j equal the bottom L-k bits of i,
 * so the predecessors of j are (j >> k) | (a << (L-k)) for the 2^k values of a.
 * cost_0(j) = err_0(j); cost_t(j) = min over predecessors i of cost_{t-1}(i), plus
 * err_t(j); the first (lowest) predecessor wins a tie, and the first (lowest) final
 * state wins a tie.  The walk is read back through the stored predecessors.
 * Outputs: st[0..T) the state sequence, *cost_out its (binary32) cost. */
int oracle_viterbi(const float* C, const float* s, const float* w, int T, int L, int k,
                   uint32_t* st, float* cost_out)
{
    if (!C || !s || !st || !check_trellis(T, L, k)) return ORC_EINVAL;
    const uint32_t N = 1u << L;
    const uint32_t K = 1u << k;
    float* cost = (float*)malloc(sizeof(float) * N);
    float* next = (float*)malloc(sizeof(float) * N);
    uint32_t* back = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)T * N);
    if (!cost || !next || !back) {
        free(cost); free(next); free(back);
        return ORC_ENOMEM;
    }

    for (uint32_t j = 0; j < N; ++j)
        cost[j] = step_error(C[j], s[0], w, 0);

    for (int t = 1; t < T; ++t) {
        for (uint32_t j = 0; j < N; ++j) {
            uint32_t best_i = j >> k;            /* a = 0 */
            float best = cost[best_i];
            for (uint32_t a = 1; a < K; ++a) {
                uint32_t i = (j >> k) | (a << (L - k));
                if (cost[i] < best) {            /* strict: the lowest index keeps ties */
                    best = cost[i];
                    best_i = i;
                }
            }
            back[(size_t)t * N + j] = best_i;
            next[j] = best + step_error(C[j], s[t], w, t);
        }
        float* tmp = cost; cost = next; next = tmp;
    }

    uint32_t jstar = 0;
    for (uint32_t j = 1; j < N; ++j)
        if (cost[j] < cost[jstar]) jstar = j;
    *cost_out = cost[jstar];

    st[T - 1] = jstar;
    for (int t = T - 1; t > 0; --t)
        st[t - 1] = back[(size_t)t * N + st[t]];

    free(cost); free(next); free(back);
    return ORC_OK;
}

/* Per-sequence MSE as the page defines it: the minimum path cost divided by T (in
 * binary32). */
static float mse_of(float cost, int T) { return cost / (float)T; }

/* Batch driver: B independent sequences, row-major s[B][T], w[B][T] (or NULL).
 * st[B][T], cost[B], mse[B] (cost and mse may be NULL). */
int oracle_viterbi_batch(const float* C, const float* s, const float* w, int64_t B, int T,
                         int L, int k, uint32_t* st, float* cost, float* mse)
{
    if (B < 0) return ORC_EINVAL;
    for (int64_t b = 0; b < B; ++b) {
        float c;
        int rc = oracle_viterbi(C, s + b * T, w ? w + b * T : NULL, T, L, k, st + b * T, &c);
        if (rc) return rc;
        if (cost) cost[b] = c;
        if (mse) mse[b] = mse_of(c, T);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* Bitstream: pack and window decode  ([QTIP] "The trellis: a stateful codebook",    */
/* "Tail-biting is worth its complexity" for the plain-trellis bit count)            */
/* ------------------------------------------------------------------------------ */

/* A plain trellis stream stores the start state (L bits) and then k new bits per
 * later weight. */
int64_t oracle_stream_bits(int L, int k, int T) { return (int64_t)L + (int64_t)(T - 1) * k; }
int64_t oracle_stream_words(int L, int k, int T) { return (oracle_stream_bits(L, k, T) + 31) / 32; }

/* Stream position p (0 = most significant bit of the stream) lives in word p / 32 at
 * bit 31 - p % 32. */
static void put_bit(uint32_t* words, int64_t p, uint32_t bit)
{
    if (bit) words[p / 32] |= 1u << (31 - (int)(p % 32));
}
static uint32_t get_bit(const uint32_t* words, int64_t p)
{
    return (words[p / 32] >> (31 - (int)(p % 32))) & 1u;
}

/* Pack one state sequence: the L bits of st[0] most significant first, then for each
 * t >= 1 the k low bits of st[t] (the bits that entered the window).  Pad bits = 0. */
int oracle_pack(const uint32_t* st, int T, int L, int k, uint32_t* words)
{
    if (!st || !words || !check_trellis(T, L, k)) return ORC_EINVAL;
    int64_t nw = oracle_stream_words(L, k, T);
    memset(words, 0, sizeof(uint32_t) * (size_t)nw);
    for (int b = 0; b < L; ++b)
        put_bit(words, b, (st[0] >> (L - 1 - b)) & 1u);
    for (int t = 1; t < T; ++t)
        for (int b = 0; b < k; ++b)
            put_bit(words, (int64_t)L + (int64_t)(t - 1) * k + b, (st[t] >> (k - 1 - b)) & 1u);
    return ORC_OK;
}

int oracle_pack_batch(const uint32_t* st, int64_t B, int T, int L, int k, uint32_t* words)
{
    int64_t nw = oracle_stream_words(L, k, T);
    for (int64_t b = 0; b < B; ++b) {
        int rc = oracle_pack(st + b * T, T, L, k, words + b * nw);
        if (rc) return rc;
    }
    return ORC_OK;
}

/* Window decode: weight t reads the L stream bits starting at position t*k (the
 * window the page shifts out of the big-integer stream), and its value is the code
 * of that window.  windows[] (may be NULL) receives the window integers. */
int oracle_decode(const uint32_t* words, int T, int L, int k, const float* C,
                  uint32_t* windows, float* recon)
{
    if (!words || !C || !check_trellis(T, L, k)) return ORC_EINVAL;
    for (int t = 0; t < T; ++t) {
        uint32_t win = 0;
        for (int b = 0; b < L; ++b)
            win = (win << 1) | get_bit(words, (int64_t)t * k + b);
        if (windows) windows[t] = win;
        if (recon) recon[t] = C[win];
    }
    return ORC_OK;
}

int oracle_decode_batch(const uint32_t* words, int64_t B, int T, int L, int k, const float* C,
                        uint32_t* windows, float* recon)
{
    int64_t nw = oracle_stream_words(L, k, T);
    for (int64_t b = 0; b < B; ++b) {
        int rc = oracle_decode(words + b * nw, T, L, k, C, windows ? windows + b * T : NULL,
                               recon ? recon + b * T : NULL);
        if (rc) return rc;
    }
    return ORC_OK;
}

/* Path cost of a reconstruction: the binary32 sum over t = 0, 1, ..., T-1 (in that
 * order) of the step errors.  Dividing by T gives the per-sequence MSE. */
float oracle_path_cost(const float* recon, const float* s, const float* w, int T)
{
    float acc = 0.0f;
    for (int t = 0; t < T; ++t)
        acc = acc + step_error(recon[t], s[t], w, t);
    return acc;
}

/* ------------------------------------------------------------------------------ */
/* BCJR soft relaxation, binary64  ([BCJR] abstract)                                */
/* ------------------------------------------------------------------------------ */

/* Energy of state j at step t: the same weighted squared error as the search, but
 * evaluated exactly in binary64 from the binary32 inputs. */
static double energy64(const float* C, const float* s, const float* w, int t, uint32_t j)
{
    double d = (double)C[j] - (double)s[t];
    double e = d * d;
    if (w) e *= (double)w[t];
    return e;
}

/* log(sum_i exp(x_i)) of n values, shifted by their maximum. */
static double logsumexp(const double* x, int n)
{
    double m = -INFINITY;
    for (int i = 0; i < n; ++i)
        if (x[i] > m) m = x[i];
    if (m == -INFINITY) return m;
    double acc = 0.0;
    for (int i = 0; i < n; ++i)
        acc += exp(x[i] - m);
    return m + log(acc);
}

/* Forward-backward over the plain bitshift trellis with a uniform start prior.
 * Path weight exp(-E/tau), E = sum_t energy_t(state_t).
 *   la_0(j) = -e_0(j)/tau;  la_t(j) = LSE_{i in pred(j)} la_{t-1}(i) - e_t(j)/tau
 *   lb_{T-1}(i) = 0;        lb_t(i) = LSE_{j in succ(i)} (lb_{t+1}(j) - e_{t+1}(j)/tau)
 *   log Z = LSE_j la_{T-1}(j);  gamma_t(j) = exp(la_t(j) + lb_t(j) - log Z)
 *   soft_t = sum_j gamma_t(j) C_j / sum_j gamma_t(j)
 * Successors of i are ((i << k) | b) mod 2^L for the 2^k values of b.
 * Outputs soft[0..T) and *logz (natural log). */
int oracle_bcjr(const float* C, const float* s, const float* w, int T, int L, int k,
                double tau, double* soft, double* logz)
{
    if (!C || !s || !soft || !check_trellis(T, L, k) || !(tau > 0.0) || !isfinite(tau))
        return ORC_EINVAL;
    const uint32_t N = 1u << L;
    const uint32_t K = 1u << k;
    double* la = (double*)malloc(sizeof(double) * (size_t)T * N);
    double* lb = (double*)malloc(sizeof(double) * N);
    double* lb_next = (double*)malloc(sizeof(double) * N);
    double* terms = (double*)malloc(sizeof(double) * (K > N ? K : N));
    if (!la || !lb || !lb_next || !terms) {
        free(la); free(lb); free(lb_next); free(terms);
        return ORC_ENOMEM;
    }

    for (uint32_t j = 0; j < N; ++j)
        la[j] = -energy64(C, s, w, 0, j) / tau;
    for (int t = 1; t < T; ++t) {
        const double* prev = la + (size_t)(t - 1) * N;
        double* cur = la + (size_t)t * N;
        for (uint32_t j = 0; j < N; ++j) {
            for (uint32_t a = 0; a < K; ++a)
                terms[a] = prev[(j >> k) | (a << (L - k))];
            cur[j] = logsumexp(terms, (int)K) - energy64(C, s, w, t, j) / tau;
        }
    }
    double lz = logsumexp(la + (size_t)(T - 1) * N, (int)N);
    if (logz) *logz = lz;

    for (uint32_t i = 0; i < N; ++i)
        lb[i] = 0.0;
    for (int t = T - 1; t >= 0; --t) {
        /* posterior at t */
        const double* cur = la + (size_t)t * N;
        double num = 0.0, den = 0.0;
        for (uint32_t j = 0; j < N; ++j) {
            double g = exp(cur[j] + lb[j] - lz);
            num += g * (double)C[j];
            den += g;
        }
        soft[t] = num / den;
        if (t == 0) break;
        /* lb_{t-1} from lb_t */
        for (uint32_t i = 0; i < N; ++i) {
            for (uint32_t b = 0; b < K; ++b) {
                uint32_t j = ((i << k) | b) & (N - 1);
                terms[b] = lb[j] - energy64(C, s, w, t, j) / tau;
            }
            lb_next[i] = logsumexp(terms, (int)K);
        }
        double* tmp = lb; lb = lb_next; lb_next = tmp;
    }

    free(la); free(lb); free(lb_next); free(terms);
    return ORC_OK;
}

int oracle_bcjr_batch(const float* C, const float* s, const float* w, int64_t B, int T, int L,
                      int k, double tau, double* soft, double* logz)
{
    for (int64_t b = 0; b < B; ++b) {
        int rc = oracle_bcjr(C, s + b * T, w ? w + b * T : NULL, T, L, k, tau, soft + b * T,
                             logz ? logz + b : NULL);
        if (rc) return rc;
    }
    return ORC_OK;
}

/* Min-sum forward-backward in binary64: best[t][j] = the least energy of any walk
 * that is in state j at step t (exact-arithmetic counterpart of the Viterbi values).
 * Used to find how far the best walk with a different value at step t lies above the
 * optimum, which bounds how fast BCJR approaches the hard code as tau -> 0. */
int oracle_minsum_marginals(const float* C, const float* s, const float* w, int T, int L, int k,
                            double* best)
{
    if (!C || !s || !best || !check_trellis(T, L, k)) return ORC_EINVAL;
    const uint32_t N = 1u << L;
    const uint32_t K = 1u << k;
    double* fa = (double*)malloc(sizeof(double) * (size_t)T * N);
    double* fb = (double*)malloc(sizeof(double) * N);
    double* fb_next = (double*)malloc(sizeof(double) * N);
    if (!fa || !fb || !fb_next) {
        free(fa); free(fb); free(fb_next);
        return ORC_ENOMEM;
    }
    for (uint32_t j = 0; j < N; ++j)
        fa[j] = energy64(C, s, w, 0, j);
    for (int t = 1; t < T; ++t) {
        const double* prev = fa + (size_t)(t - 1) * N;
        double* cur = fa + (size_t)t * N;
        for (uint32_t j = 0; j < N; ++j) {
            double m = INFINITY;
            for (uint32_t a = 0; a < K; ++a) {
                double v = prev[(j >> k) | (a << (L - k))];
                if (v < m) m = v;
            }
            cur[j] = m + energy64(C, s, w, t, j);
        }
    }
    for (uint32_t i = 0; i < N; ++i)
        fb[i] = 0.0;
    for (int t = T - 1; t >= 0; --t) {
        for (uint32_t j = 0; j < N; ++j)
            best[(size_t)t * N + j] = fa[(size_t)t * N + j] + fb[j];
        if (t == 0) break;
        for (uint32_t i = 0; i < N; ++i) {
            double m = INFINITY;
            for (uint32_t b = 0; b < K; ++b) {
                uint32_t j = ((i << k) | b) & (N - 1);
                double v = fb[j] + energy64(C, s, w, t, j);
                if (v < m) m = v;
            }
            fb_next[i] = m;
        }
        double* tmp = fb; fb = fb_next; fb_next = tmp;
    }
    free(fa); free(fb); free(fb_next);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* Brute force over every walk (tiny instances only)                                */
/* ------------------------------------------------------------------------------ */

/* Walk number n (0 <= n < 2^(L + k(T-1))) read as a stream of L + k(T-1) bits, most
 * significant first: its first L bits are the start state, then k bits per step. */
static void walk_states(uint64_t n, int T, int L, int k, uint32_t* st)
{
    int nbits = L + k * (T - 1);
    uint32_t mask = (1u << L) - 1u;
    st[0] = (uint32_t)(n >> (nbits - L)) & mask;
    for (int t = 1; t < T; ++t) {
        uint32_t branch = (uint32_t)(n >> (nbits - L - t * k)) & ((1u << k) - 1u);
        st[t] = ((st[t - 1] << k) | branch) & mask;
    }
}

/* Every walk's binary32 cost (sequential sum, same step error as the search).
 * Returns the minimum cost, the number of walks attaining it, and among those the walk
 * whose state sequence read from the last step backwards is smallest (st_T-1 first). */
int oracle_brute_viterbi(const float* C, const float* s, const float* w, int T, int L, int k,
                         float* best_cost, uint32_t* best_path, int64_t* n_optimal)
{
    if (!C || !s || !best_cost || !check_trellis(T, L, k)) return ORC_EINVAL;
    int nbits = L + k * (T - 1);
    if (nbits > 26) return ORC_EINVAL;
    uint64_t nwalks = 1ull << nbits;
    uint32_t* st = (uint32_t*)malloc(sizeof(uint32_t) * T);
    uint32_t* cand = (uint32_t*)malloc(sizeof(uint32_t) * T);
    if (!st || !cand) { free(st); free(cand); return ORC_ENOMEM; }
    float best = INFINITY;
    int64_t count = 0;
    for (uint64_t n = 0; n < nwalks; ++n) {
        walk_states(n, T, L, k, st);
        float acc = 0.0f;
        for (int t = 0; t < T; ++t)
            acc = acc + step_error(C[st[t]], s[t], w, t);
        int take = 0;
        if (acc < best) {
            best = acc;
            count = 1;
            take = 1;
        } else if (acc == best) {
            ++count;
            /* reverse-lexicographic comparison: last state first */
            for (int t = T - 1; t >= 0; --t) {
                if (st[t] != cand[t]) { take = st[t] < cand[t]; break; }
            }
        }
        if (take) memcpy(cand, st, sizeof(uint32_t) * T);
    }
    *best_cost = best;
    if (best_path) memcpy(best_path, cand, sizeof(uint32_t) * T);
    if (n_optimal) *n_optimal = count;
    free(st); free(cand);
    return ORC_OK;
}

/* Boltzmann expectation by explicit enumeration of every walk, binary64.
 * soft[t] = sum_walks p(walk) C[state_t]; *logz = log sum_walks exp(-E/tau). */
int oracle_brute_bcjr(const float* C, const float* s, const float* w, int T, int L, int k,
                      double tau, double* soft, double* logz)
{
    if (!C || !s || !soft || !check_trellis(T, L, k) || !(tau > 0.0)) return ORC_EINVAL;
    int nbits = L + k * (T - 1);
    if (nbits > 22) return ORC_EINVAL;
    uint64_t nwalks = 1ull << nbits;
    uint32_t* st = (uint32_t*)malloc(sizeof(uint32_t) * T);
    double* E = (double*)malloc(sizeof(double) * nwalks);
    if (!st || !E) { free(st); free(E); return ORC_ENOMEM; }
    double emin = INFINITY;
    for (uint64_t n = 0; n < nwalks; ++n) {
        walk_states(n, T, L, k, st);
        double e = 0.0;
        for (int t = 0; t < T; ++t)
            e += energy64(C, s, w, t, st[t]);
        E[n] = e;
        if (e < emin) emin = e;
    }
    double zsum = 0.0;
    for (int t = 0; t < T; ++t)
        soft[t] = 0.0;
    for (uint64_t n = 0; n < nwalks; ++n) {
        double p = exp(-(E[n] - emin) / tau);
        zsum += p;
        walk_states(n, T, L, k, st);
        for (int t = 0; t < T; ++t)
            soft[t] += p * (double)C[st[t]];
    }
    for (int t = 0; t < T; ++t)
        soft[t] /= zsum;
    if (logz) *logz = -emin / tau + log(zsum);
    free(st); free(E);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* Tail-biting trellis  ([QTIP] "Tail-biting is worth its complexity")               */
/* ------------------------------------------------------------------------------ */

/* A tail-biting walk is cyclic: the low L-k bits of the last state equal the high L-k
 * bits of the first, so the stream is exactly k*T bits and weight t's state is the
 * L-bit window starting at bit t*k read cyclically.  That needs k*T >= L (a stream at
 * least one window long). */
static int check_tailbiting(int T, int L, int k)
{
    return check_trellis(T, L, k) && (int64_t)k * T >= L;
}

int64_t oracle_tb_stream_bits(int L, int k, int T) { (void)L; return (int64_t)k * T; }
int64_t oracle_tb_stream_words(int L, int k, int T) { return (oracle_tb_stream_bits(L, k, T) + 31) / 32; }

/* Viterbi with both ends pinned to an overlap value o (an (L-k)-bit integer): the walk
 * must start in a state whose high L-k bits are o and end in a state whose low L-k
 * bits are o.  Exactly the plain search (same arithmetic, same tie rules) with the
 * forbidden start states given cost +infinity and the final minimum taken over the
 * allowed end states only (the lowest allowed state wins a tie). */
int oracle_viterbi_pinned(const float* C, const float* s, const float* w, int T, int L, int k,
                          uint32_t o, uint32_t* st, float* cost_out)
{
    if (!C || !s || !st || !check_tailbiting(T, L, k)) return ORC_EINVAL;
    const uint32_t N = 1u << L;
    const uint32_t K = 1u << k;
    const uint32_t low_mask = (1u << (L - k)) - 1u;
    if (o > low_mask) return ORC_EINVAL;
    float* cost = (float*)malloc(sizeof(float) * N);
    float* next = (float*)malloc(sizeof(float) * N);
    uint32_t* back = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)T * N);
    if (!cost || !next || !back) {
        free(cost); free(next); free(back);
        return ORC_ENOMEM;
    }

    for (uint32_t j = 0; j < N; ++j)
        cost[j] = ((j >> k) == o) ? step_error(C[j], s[0], w, 0) : INFINITY;

    for (int t = 1; t < T; ++t) {
        for (uint32_t j = 0; j < N; ++j) {
            uint32_t best_i = j >> k;
            float best = cost[best_i];
            for (uint32_t a = 1; a < K; ++a) {
                uint32_t i = (j >> k) | (a << (L - k));
                if (cost[i] < best) {
                    best = cost[i];
                    best_i = i;
                }
            }
            back[(size_t)t * N + j] = best_i;
            next[j] = best + step_error(C[j], s[t], w, t);
        }
        float* tmp = cost; cost = next; next = tmp;
    }

    /* allowed end states: j with (j & low_mask) == o, i.e. j = o + a * 2^(L-k) */
    uint32_t jstar = o;
    for (uint32_t a = 1; a < K; ++a) {
        uint32_t j = o | (a << (L - k));
        if (cost[j] < cost[jstar]) jstar = j;
    }
    *cost_out = cost[jstar];

    st[T - 1] = jstar;
    for (int t = T - 1; t > 0; --t)
        st[t - 1] = back[(size_t)t * N + st[t]];

    free(cost); free(next); free(back);
    return ORC_OK;
}

/* Exact tail-biting optimum: one pinned search per overlap value, 2^(L-k) of them; the
 * cheapest wins (the lowest overlap on a tie).  Practical for L <= 12. */
int oracle_tailbiting_exact(const float* C, const float* s, const float* w, int T, int L, int k,
                            uint32_t* st, float* cost_out)
{
    if (!C || !s || !st || !cost_out || !check_tailbiting(T, L, k)) return ORC_EINVAL;
    uint32_t* cand = (uint32_t*)malloc(sizeof(uint32_t) * T);
    if (!cand) return ORC_ENOMEM;
    float best = INFINITY;
    const uint32_t n_over = 1u << (L - k);
    for (uint32_t o = 0; o < n_over; ++o) {
        float c;
        int rc = oracle_viterbi_pinned(C, s, w, T, L, k, o, cand, &c);
        if (rc) { free(cand); return rc; }
        if (c < best) {
            best = c;
            memcpy(st, cand, sizeof(uint32_t) * T);
        }
    }
    *cost_out = best;
    free(cand);
    return ORC_OK;
}

/* Two-search tail-biting (the page's Algorithm 4 summary): rotate the sequence by
 * r = floor(T/2) so that its ends meet in the middle, run the free-start search on the
 * rotated sequence, take the overlap from the state the rotated walk assigns to the
 * original position 0 (its high L-k bits, which by the trellis rule also equal the
 * low L-k bits of the state before it, the original position T-1), then search the
 * original sequence with both ends pinned to that overlap.
 * Rotated sequence: s'[t] = s[(t + r) mod T] (weights likewise); original position 0
 * sits at rotated position (T - r) mod T.  *overlap_out (may be NULL) = the overlap. */
int oracle_tailbiting_alg4(const float* C, const float* s, const float* w, int T, int L, int k,
                           uint32_t* st, float* cost_out, uint32_t* overlap_out)
{
    if (!C || !s || !st || !cost_out || !check_tailbiting(T, L, k)) return ORC_EINVAL;
    const int r = T / 2;
    float* sr = (float*)malloc(sizeof(float) * T);
    float* wr = w ? (float*)malloc(sizeof(float) * T) : NULL;
    uint32_t* str = (uint32_t*)malloc(sizeof(uint32_t) * T);
    if (!sr || !str || (w && !wr)) { free(sr); free(wr); free(str); return ORC_ENOMEM; }
    for (int t = 0; t < T; ++t) {
        sr[t] = s[(t + r) % T];
        if (w) wr[t] = w[(t + r) % T];
    }
    float c1;
    int rc = oracle_viterbi(C, sr, wr, T, L, k, str, &c1);
    if (!rc) {
        const uint32_t o = str[(T - r) % T] >> k;
        if (overlap_out) *overlap_out = o;
        rc = oracle_viterbi_pinned(C, s, w, T, L, k, o, st, cost_out);
    }
    free(sr); free(wr); free(str);
    return rc;
}

/* Batch driver for the two-search encoder: st[B][T], cost[B], mse[B] (cost, mse may
 * be NULL). */
int oracle_tailbiting_alg4_batch(const float* C, const float* s, const float* w, int64_t B,
                                 int T, int L, int k, uint32_t* st, float* cost, float* mse)
{
    if (B < 0) return ORC_EINVAL;
    for (int64_t b = 0; b < B; ++b) {
        float c;
        int rc = oracle_tailbiting_alg4(C, s + b * T, w ? w + b * T : NULL, T, L, k,
                                        st + b * T, &c, NULL);
        if (rc) return rc;
        if (cost) cost[b] = c;
        if (mse) mse[b] = mse_of(c, T);
    }
    return ORC_OK;
}

/* Tail-biting pack: each state contributes its k high bits, state t at stream bits
 * [t*k, t*k + k) (MSB first); the window rule then reproduces every state, the ones
 * near the end wrapping round to the start of the stream.  Pad bits = 0. */
int oracle_tb_pack(const uint32_t* st, int T, int L, int k, uint32_t* words)
{
    if (!st || !words || !check_tailbiting(T, L, k)) return ORC_EINVAL;
    int64_t nw = oracle_tb_stream_words(L, k, T);
    memset(words, 0, sizeof(uint32_t) * (size_t)nw);
    for (int t = 0; t < T; ++t) {
        uint32_t top = st[t] >> (L - k);
        for (int b = 0; b < k; ++b)
            put_bit(words, (int64_t)t * k + b, (top >> (k - 1 - b)) & 1u);
    }
    return ORC_OK;
}

int oracle_tb_pack_batch(const uint32_t* st, int64_t B, int T, int L, int k, uint32_t* words)
{
    int64_t nw = oracle_tb_stream_words(L, k, T);
    for (int64_t b = 0; b < B; ++b) {
        int rc = oracle_tb_pack(st + b * T, T, L, k, words + b * nw);
        if (rc) return rc;
    }
    return ORC_OK;
}

/* Tail-biting window decode: weight t reads stream bits t*k, t*k + 1, ..., t*k + L - 1,
 * every position taken modulo the stream length k*T. */
int oracle_tb_decode(const uint32_t* words, int T, int L, int k, const float* C,
                     uint32_t* windows, float* recon)
{
    if (!words || !C || !check_tailbiting(T, L, k)) return ORC_EINVAL;
    const int64_t nbits = oracle_tb_stream_bits(L, k, T);
    for (int t = 0; t < T; ++t) {
        uint32_t win = 0;
        for (int b = 0; b < L; ++b)
            win = (win << 1) | get_bit(words, ((int64_t)t * k + b) % nbits);
        if (windows) windows[t] = win;
        if (recon) recon[t] = C[win];
    }
    return ORC_OK;
}

int oracle_tb_decode_batch(const uint32_t* words, int64_t B, int T, int L, int k, const float* C,
                           uint32_t* windows, float* recon)
{
    int64_t nw = oracle_tb_stream_words(L, k, T);
    for (int64_t b = 0; b < B; ++b) {
        int rc = oracle_tb_decode(words + b * nw, T, L, k, C, windows ? windows + b * T : NULL,
                                  recon ? recon + b * T : NULL);
        if (rc) return rc;
    }
    return ORC_OK;
}

/* Brute force over every tail-biting walk: all 2^(k*T) cyclic streams, each walk's
 * cost summed sequentially in binary32.  *best_cost = the minimum; *n_optimal = how
 * many walks attain it. */
int oracle_brute_tailbiting(const float* C, const float* s, const float* w, int T, int L, int k,
                            float* best_cost, int64_t* n_optimal)
{
    if (!C || !s || !best_cost || !check_tailbiting(T, L, k)) return ORC_EINVAL;
    const int nbits = k * T;
    if (nbits > 24) return ORC_EINVAL;
    const uint32_t mask = (1u << L) - 1u;
    float best = INFINITY;
    int64_t count = 0;
    for (uint64_t n = 0; n < (1ull << nbits); ++n) {
        float acc = 0.0f;
        for (int t = 0; t < T; ++t) {
            uint32_t win = 0;
            for (int b = 0; b < L; ++b) {
                int p = (t * k + b) % nbits;              /* stream bit p, MSB first */
                win = (win << 1) | (uint32_t)((n >> (nbits - 1 - p)) & 1u);
            }
            acc = acc + step_error(C[win & mask], s[t], w, t);
        }
        if (acc < best) { best = acc; count = 1; }
        else if (acc == best) ++count;
    }
    *best_cost = best;
    if (n_optimal) *n_optimal = count;
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* Gradient of the soft codeword  ([BCJR] abstract: the relaxation is exactly       */
/* differentiable)                                                                  */
/* ------------------------------------------------------------------------------ */

/* Vector-Jacobian product of the BCJR soft codeword with respect to the targets.
 * With p(walk) proportional to exp(-E/tau) and dE/ds_u = -2 w_u (C(state_u) - s_u),
 *     d soft_t / d s_u = (2 w_u / tau) Cov_p( C(state_t), C(state_u) ),
 * so for an upstream gradient g (g_t = dLoss/dsoft_t)
 *     grad_u = sum_t g_t d soft_t / d s_u = (2 w_u / tau) Cov_p( F, C(state_u) ),
 *     F = sum_t g_t C(state_t).
 * The covariance uses the Markov structure of p: given state_u = j the walk's past and
 * future are independent, so E[F | state_u = j] = Phi_u(j) + g_u C_j + Psi_u(j) with
 *     Phi_0(j) = 0,      Phi_t(j) = sum_{i in pred(j)} P(i | j) (Phi_{t-1}(i) + g_{t-1} C_i),
 *                        P(i | j) proportional to exp(la_{t-1}(i))
 *     Psi_{T-1}(i) = 0,  Psi_t(i) = sum_{x in succ(i)} P(x | i) (g_{t+1} C_x + Psi_{t+1}(x)),
 *                        P(x | i) proportional to exp(lb_{t+1}(x) - e_{t+1}(x)/tau)
 * (la, lb the forward and backward log messages of oracle_bcjr), and
 *     Cov_p(F, C_u) = sum_j gamma_u(j) (C_j - soft_u) (E[F | j] - E[F]) / sum_j gamma_u(j).
 * Binary64 throughout.  grad[0..T) out; soft (may be NULL) receives the soft codeword. */
int oracle_bcjr_vjp(const float* C, const float* s, const float* w, int T, int L, int k,
                    double tau, const double* g, double* grad, double* soft)
{
    if (!C || !s || !g || !grad || !check_trellis(T, L, k) || !(tau > 0.0) || !isfinite(tau))
        return ORC_EINVAL;
    const uint32_t N = 1u << L;
    const uint32_t K = 1u << k;
    double* la = (double*)malloc(sizeof(double) * (size_t)T * N);
    double* lb = (double*)malloc(sizeof(double) * (size_t)T * N);
    double* psi = (double*)malloc(sizeof(double) * (size_t)T * N);
    double* phi = (double*)malloc(sizeof(double) * N);
    double* phi_next = (double*)malloc(sizeof(double) * N);
    double* terms = (double*)malloc(sizeof(double) * K);
    if (!la || !lb || !psi || !phi || !phi_next || !terms) {
        free(la); free(lb); free(psi); free(phi); free(phi_next); free(terms);
        return ORC_ENOMEM;
    }

    /* forward and backward log messages, every step kept */
    for (uint32_t j = 0; j < N; ++j)
        la[j] = -energy64(C, s, w, 0, j) / tau;
    for (int t = 1; t < T; ++t) {
        const double* prev = la + (size_t)(t - 1) * N;
        double* cur = la + (size_t)t * N;
        for (uint32_t j = 0; j < N; ++j) {
            for (uint32_t a = 0; a < K; ++a)
                terms[a] = prev[(j >> k) | (a << (L - k))];
            cur[j] = logsumexp(terms, (int)K) - energy64(C, s, w, t, j) / tau;
        }
    }
    const double lz = logsumexp(la + (size_t)(T - 1) * N, (int)N);
    for (uint32_t i = 0; i < N; ++i)
        lb[(size_t)(T - 1) * N + i] = 0.0;
    for (int t = T - 1; t >= 1; --t) {
        for (uint32_t i = 0; i < N; ++i) {
            for (uint32_t b = 0; b < K; ++b) {
                uint32_t x = ((i << k) | b) & (N - 1);
                terms[b] = lb[(size_t)t * N + x] - energy64(C, s, w, t, x) / tau;
            }
            lb[(size_t)(t - 1) * N + i] = logsumexp(terms, (int)K);
        }
    }

    /* Psi backward, every step kept */
    for (uint32_t i = 0; i < N; ++i)
        psi[(size_t)(T - 1) * N + i] = 0.0;
    for (int t = T - 2; t >= 0; --t) {
        for (uint32_t i = 0; i < N; ++i) {
            for (uint32_t b = 0; b < K; ++b) {
                uint32_t x = ((i << k) | b) & (N - 1);
                terms[b] = lb[(size_t)(t + 1) * N + x] - energy64(C, s, w, t + 1, x) / tau;
            }
            double m = logsumexp(terms, (int)K);
            double acc = 0.0;
            for (uint32_t b = 0; b < K; ++b) {
                uint32_t x = ((i << k) | b) & (N - 1);
                double q = exp(terms[b] - m);
                acc += q * (g[t + 1] * (double)C[x] + psi[(size_t)(t + 1) * N + x]);
            }
            psi[(size_t)t * N + i] = acc;
        }
    }

    /* Phi forward, combined with Psi step by step */
    for (uint32_t j = 0; j < N; ++j)
        phi[j] = 0.0;
    for (int u = 0; u < T; ++u) {
        if (u > 0) {
            const double* prev = la + (size_t)(u - 1) * N;
            for (uint32_t j = 0; j < N; ++j) {
                for (uint32_t a = 0; a < K; ++a)
                    terms[a] = prev[(j >> k) | (a << (L - k))];
                double m = logsumexp(terms, (int)K);
                double acc = 0.0;
                for (uint32_t a = 0; a < K; ++a) {
                    uint32_t i = (j >> k) | (a << (L - k));
                    acc += exp(terms[a] - m) * (phi[i] + g[u - 1] * (double)C[i]);
                }
                phi_next[j] = acc;
            }
            double* tmp = phi; phi = phi_next; phi_next = tmp;
        }
        const double* cur = la + (size_t)u * N;
        const double* bk = lb + (size_t)u * N;
        const double* ps = psi + (size_t)u * N;
        double den = 0.0, num_c = 0.0, num_f = 0.0;
        for (uint32_t j = 0; j < N; ++j) {
            double gm = exp(cur[j] + bk[j] - lz);
            den += gm;
            num_c += gm * (double)C[j];
            num_f += gm * (phi[j] + g[u] * (double)C[j] + ps[j]);
        }
        const double su = num_c / den, fbar = num_f / den;
        double cov = 0.0;
        for (uint32_t j = 0; j < N; ++j) {
            double gm = exp(cur[j] + bk[j] - lz);
            double ef = phi[j] + g[u] * (double)C[j] + ps[j];
            cov += gm * ((double)C[j] - su) * (ef - fbar);
        }
        cov /= den;
        grad[u] = 2.0 * (w ? (double)w[u] : 1.0) / tau * cov;
        if (soft) soft[u] = su;
    }

    free(la); free(lb); free(psi); free(phi); free(phi_next); free(terms);
    return ORC_OK;
}

int oracle_bcjr_vjp_batch(const float* C, const float* s, const float* w, int64_t B, int T, int L,
                          int k, double tau, const double* g, double* grad, double* soft)
{
    for (int64_t b = 0; b < B; ++b) {
        int rc = oracle_bcjr_vjp(C, s + b * T, w ? w + b * T : NULL, T, L, k, tau, g + b * T,
                                 grad + b * T, soft ? soft + b * T : NULL);
        if (rc) return rc;
    }
    return ORC_OK;
}

/* The same vector-Jacobian product by explicit enumeration of every walk: the
 * Boltzmann probabilities, then Cov(F, C(state_u)) with both factors centred.
 * Binary64; L + k(T-1) <= 22. */
int oracle_brute_bcjr_vjp(const float* C, const float* s, const float* w, int T, int L, int k,
                          double tau, const double* g, double* grad)
{
    if (!C || !s || !g || !grad || !check_trellis(T, L, k) || !(tau > 0.0)) return ORC_EINVAL;
    int nbits = L + k * (T - 1);
    if (nbits > 22) return ORC_EINVAL;
    uint64_t nwalks = 1ull << nbits;
    uint32_t* st = (uint32_t*)malloc(sizeof(uint32_t) * T);
    double* E = (double*)malloc(sizeof(double) * nwalks);
    double* cbar = (double*)malloc(sizeof(double) * T);
    if (!st || !E || !cbar) { free(st); free(E); free(cbar); return ORC_ENOMEM; }
    double emin = INFINITY;
    for (uint64_t n = 0; n < nwalks; ++n) {
        walk_states(n, T, L, k, st);
        double e = 0.0;
        for (int t = 0; t < T; ++t)
            e += energy64(C, s, w, t, st[t]);
        E[n] = e;
        if (e < emin) emin = e;
    }
    double z = 0.0, fbar = 0.0;
    for (int t = 0; t < T; ++t)
        cbar[t] = 0.0;
    for (uint64_t n = 0; n < nwalks; ++n) {
        double p = exp(-(E[n] - emin) / tau);
        walk_states(n, T, L, k, st);
        double f = 0.0;
        for (int t = 0; t < T; ++t) {
            f += g[t] * (double)C[st[t]];
            cbar[t] += p * (double)C[st[t]];
        }
        fbar += p * f;
        z += p;
    }
    fbar /= z;
    for (int t = 0; t < T; ++t) {
        cbar[t] /= z;
        grad[t] = 0.0;
    }
    for (uint64_t n = 0; n < nwalks; ++n) {
        double p = exp(-(E[n] - emin) / tau) / z;
        walk_states(n, T, L, k, st);
        double f = 0.0;
        for (int t = 0; t < T; ++t)
            f += g[t] * (double)C[st[t]];
        for (int u = 0; u < T; ++u)
            grad[u] += p * (f - fbar) * ((double)C[st[u]] - cbar[u]);
    }
    for (int u = 0; u < T; ++u)
        grad[u] *= 2.0 * (w ? (double)w[u] : 1.0) / tau;
    free(st); free(E); free(cbar);
    return ORC_OK;
}
