/*
 * qtcq.h -- C ABI of the MI355X (gfx950) bitshift-trellis library: batched Viterbi
 * encoding of weight sequences with computed codes, parallel window decode, and the
 * BCJR soft relaxation.
 *
 * Sources, cited by page title and section:
 *  [QTIP] "QTIP: Trellis-Coded Quantization Puts 2-Bit LLM Weights 10% Above the
 *         Rate-Distortion Bound, and a Monotone Codebook Loses to Scalar Rounding"
 *         (blog) -- "The trellis: a stateful codebook" (bitshift trellis, window
 *         decode, Viterbi with shift-computed predecessors), "The codebook is
 *         computed" (1MAD, 3INST), "Tail-biting is worth its complexity" (a plain
 *         trellis stores its L-k start bits; the tail-biting trellis and its
 *         two-search encoder).
 *  [XOR]  "XOR-Trellis -- Trellis-coded quantization vs VQ codebooks -- What does it
 *         mean?" (explainer) -- "Cliff edges: weighting errors instead of rotating
 *         them" (per-weight error weights in the path cost), "The sign at each junction
 *         has to be cheap" (3INST ends with an FP16 add).
 *  [BCJR] "BCJR-QAT: A Differentiable Relaxation of Trellis-Coded Weight
 *         Quantization" (abstract) -- forward-backward at temperature, soft codeword =
 *         Boltzmann expectation over trellis paths.
 *
 * Conventions shared by every entry point
 *  - All data pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors),
 *    row-major and contiguous; [B][T] means sequence b's element t at b*T + t.
 *  - The caller owns every buffer.  The library allocates no device memory and keeps
 *    no mutable global state, with two exceptions: qtcq_decode_matvec_mfma_noalloc's
 *    per-device scratch array, and a per-device, once-only set-up of each matvec
 *    product's LDS-table kernels (their dynamic-LDS limit raised, their resident
 *    workgroups per compute unit read; thread-safe).  Calls on different streams may run
 *    concurrently as long as their output and workspace buffers do not overlap.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is
 *    enqueued on it and the call returns without synchronising; outputs are valid
 *    once the stream has reached that point.
 *  - Arguments are validated before anything is launched; a non-OK status means
 *    nothing was enqueued (except QTCQ_ERR_DEVICE, which reports a failed launch).
 *    No C++ exception crosses this ABI.
 *  - Supported on the GPU: k = 2, L in {6, 8, 10, 12, 14, 16}, 1 <= T <= 4096.
 *    Inputs must be finite and weights > 0; other inputs give unspecified (but
 *    memory-safe) results.
 *  - Results are bit-deterministic: the same inputs give the same bits on every run
 *    and for every batch split.
 *
 * Bitstream layout (plain, non-tail-biting trellis [QTIP]): a sequence's stream holds
 * nbits = L + k*(T-1) bits -- the L bits of the start state, then the k newest bits of
 * each later state -- most significant first.  Stream bit p is bit 31 - (p mod 32) of
 * 32-bit word p / 32; each sequence owns qtcq_bitstream_words(L, k, T) words and the
 * bits after nbits are zero.  Weight t reads the window of stream bits [t*k, t*k + L)
 * as an L-bit integer (its trellis state) and decodes to code(window).
 */
#ifndef QTCQ_H
#define QTCQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QTCQ_OK = 0,
    QTCQ_ERR_INVALID_ARG = 1, /* NULL required pointer, B < 0, T out of range, tau <= 0 */
    QTCQ_ERR_UNSUPPORTED = 2, /* (L, k) or code id not built for the GPU */
    QTCQ_ERR_WORKSPACE = 3,   /* workspace smaller than one sequence needs, or misaligned */
    QTCQ_ERR_DEVICE = 4       /* a kernel launch failed (hipGetLastError) */
} qtcq_status;

/* Codes: the value of an L-bit trellis state x.
 *  1MAD, 3INST [QTIP "The codebook is computed"] start from the LCG
 *         u = 34038481 * x + 76625530 (mod 2^32).
 *  1MAD : value = float( (S - 510) / 147.8 ) with S the sum of u's four bytes and the
 *         division done in binary64 (one rounding to binary32 at the end).
 *  3INST: v = (u & 0x8FFF8FFF) ^ 0x3B603B60 (sign, 2 low exponent bits and mantissa of
 *         each half XORed into fp16(0.922)); h = fp16 sum of the two halves (RNE);
 *         value = float( h / 1.244 ) in binary64 -- unit variance.
 *  XOR  : the XOR-Trellis palette code [XOR "The sign at each junction has to be
 *         cheap"].  The newest k = 2 bits of x are the branch b = x & 3, the L - 2 bits
 *         above them the history h = x >> 2.  Four masked parities p_i =
 *         parity(h & m_i) pick the palette P = 2 p_0 + p_1 and the shuffle
 *         S = 2 p_2 + p_3; value = palette[P][b XOR S] with the printed FP4 palettes
 *         [-6, -1.5, 0, 2], [-4, -1, 0.5, 3], [-3, -0.5, 1, 4], [-2, 0, 1.5, 6] (as they
 *         are; a per-group scale of the weights is the caller's).  The four successors of
 *         a state share its history's low bits, so they offer the four distinct entries
 *         of one palette.  The masks m_0..m_3 are not printed: they are the caller's, as
 *         (L - 2)-bit history masks (14 bits at L = 16).
 * A code is passed as a qtcq_code descriptor: the id in bits 0-7 and, for XOR, the four
 * masks in 14-bit fields at bits 8, 22, 36 and 50 (qtcq_xor_code builds it).  1MAD and
 * 3INST are their plain ids.  Entry points return QTCQ_ERR_UNSUPPORTED for an unknown id
 * (or parameter bits on 1MAD/3INST) and QTCQ_ERR_INVALID_ARG for XOR masks with bits at
 * or above L - 2. */
typedef uint64_t qtcq_code;
typedef enum { QTCQ_CODE_1MAD = 0, QTCQ_CODE_3INST = 1, QTCQ_CODE_XOR = 2 } qtcq_code_id;
#define QTCQ_CODE_INVALID ((qtcq_code)0xFF)

/* The XOR palette code with parity masks m0 (palette high bit), m1 (palette low bit),
 * m2 (shuffle high bit), m3 (shuffle low bit); QTCQ_CODE_INVALID if a mask exceeds
 * 14 bits. */
qtcq_code qtcq_xor_code(uint32_t m0, uint32_t m1, uint32_t m2, uint32_t m3);

/* Human-readable name of a status code (static string, never NULL); takes any int, and
 * values outside qtcq_status give "unknown status". */
const char* qtcq_status_string(int status);

/* Words per sequence of the bitstream: ceil((L + k*(T-1)) / 32).  17 at (16, 2, 256).
 * Returns -1 for arguments outside 1 <= k <= L <= 32, T >= 1. */
int64_t qtcq_bitstream_words(int L, int k, int T);

/* Workspace bytes qtcq_viterbi_encode needs to encode `B` sequences in one pass
 * (backpointers: 2 bits per trellis group per step, plus a final state and cost per
 * sequence).  Any smaller workspace that still holds one sequence works: the batch is
 * then encoded in chunks.  Returns 0 for unsupported arguments. */
size_t qtcq_encode_workspace_bytes(int64_t B, int T, int L, int k);

/* Workspace bytes qtcq_bcjr_soft needs to process `B` sequences in one pass (the
 * forward messages of every step).  Smaller workspaces are used in chunks as above.
 * Returns 0 for unsupported arguments. */
size_t qtcq_bcjr_workspace_bytes(int64_t B, int T, int L, int k);

/* Code value of every L-bit state [QTIP "The codebook is computed"], evaluated by the
 * decode kernels' device code (the search kernels evaluate the same values in another
 * exact form once per workgroup).  out: [2^L] float32 (device).  L in 1..24 (1MAD,
 * 3INST) or 2..16 (XOR). */
qtcq_status qtcq_code_table(qtcq_code code, int L, float* out, void* stream);

/* Viterbi encoding [QTIP "The trellis: a stateful codebook"; XOR "Cliff edges"].
 * For each sequence b, finds the walk st[0..T) through the bitshift trellis (state j
 * may follow state i iff the top L-k bits of j equal the bottom L-k bits of i) that
 * minimises the binary32 path cost
 *     cost = (((e_0 + e_1) + e_2) + ... + e_{T-1}),
 *     e_t  = fl( fl(code(st[t]) - seq[b][t])^2 )          (unweighted)
 *     e_t  = fl( err_w[b][t] * fl( fl(code(st[t]) - seq[b][t])^2 ) )   (weighted)
 * with every operation rounded separately (no fused multiply-add).  Ties go to the
 * lowest-numbered predecessor at each step and to the lowest-numbered final state.
 * The start state is free (stored in the stream).
 *   seq       [B][T] float32 targets (in)
 *   err_w     [B][T] float32 positive error weights (in), or NULL for unweighted
 *   B         number of sequences (>= 0; 0 is a no-op)
 *   code      qtcq_code (1MAD, 3INST or an XOR palette code)
 *   bits      [B][qtcq_bitstream_words(L,k,T)] uint32 (out) -- the layout above
 *   mse       [B] float32 (out) = cost / T, or NULL
 *   states    [B][T] uint32 (out) = st, or NULL
 *   workspace device scratch, 16-byte aligned, `workspace_bytes` long; its contents
 *             are overwritten and meaningless after the call.
 * Errors: QTCQ_ERR_INVALID_ARG, QTCQ_ERR_UNSUPPORTED, QTCQ_ERR_WORKSPACE (workspace
 * NULL, misaligned or below qtcq_encode_workspace_bytes(1, T, L, k)), QTCQ_ERR_DEVICE. */
qtcq_status qtcq_viterbi_encode(const float* seq, const float* err_w, int64_t B, int T, int L,
                                int k, qtcq_code code, uint32_t* bits, float* mse, uint32_t* states,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Window decode [QTIP "The trellis: a stateful codebook"]: recon[b][t] = code(window
 * of stream bits [t*k, t*k + L)) -- every weight independently.
 *   bits   [B][qtcq_bitstream_words(L,k,T)] uint32 (in)
 *   recon  [B][T] float32 (out), or NULL (then only mse is produced)
 *   seq    [B][T] float32 targets (in), required when mse != NULL
 *   err_w  [B][T] float32 weights (in) or NULL
 *   mse    [B] float32 (out) or NULL: the binary32 path cost of the reconstruction,
 *          summed in t order exactly as qtcq_viterbi_encode defines it, divided by T.
 *          Decoding an encoder's output with the same seq/err_w reproduces its mse
 *          bit for bit.
 * Errors: QTCQ_ERR_INVALID_ARG (also: mse requested without seq, or neither recon nor
 * mse requested), QTCQ_ERR_UNSUPPORTED, QTCQ_ERR_DEVICE. */
qtcq_status qtcq_decode(const uint32_t* bits, int64_t B, int T, int L, int k, qtcq_code code,
                        float* recon, const float* seq, const float* err_w, float* mse,
                        void* stream);

/* BCJR soft relaxation [BCJR abstract].  Each walk's energy is the search's path cost
 * in exact arithmetic, E = sum_t err_w[b][t] * (code(st[t]) - seq[b][t])^2 (err_w = 1 if
 * NULL; the binary32 search rounds each term, the relaxation does not), and its weight
 * exp(-E / temperature); the start state is uniform.  Outputs, per sequence:
 *   soft  [B][T] float32: soft[b][t] = E_Boltzmann[ code(st[t]) ], the posterior mean
 *         of the reconstructed value at step t (forward-backward in the log2 domain,
 *         messages combined in binary64, exponentials in binary32; within
 *         1e-5 * RMS_t(soft[b]) of the exact value at temperatures down to 0.01);
 *   log_z [B] float32 (or NULL): natural log of sum over walks of exp(-E / temperature).
 * temperature: finite, > 0.  As it tends to 0 soft tends to the Viterbi code.  The
 * forward messages are stashed in 32 bits -- fixed point (2^-21 log2 units) within 1024
 * log2 units of each step's maximum, binary32 of the distance below that -- so the soft
 * codeword is resolved while the messages stay within about 1e10 log2 units of their
 * step's maximum (energy / temperature up to ~7e9 per sequence: temperatures down to
 * 1e-9 on N(0,1) targets of 48 steps were tested); beyond that the far states' binary32
 * precision is coarser than a posterior's exponent range and soft is unspecified (it
 * comes out NaN), while log_z stays accurate -- the Viterbi code of qtcq_viterbi_encode
 * is the limit there.
 * workspace: 16-byte aligned, >= qtcq_bcjr_workspace_bytes(1, T, L, k); larger
 * workspaces let more sequences run per pass.
 * Errors: as qtcq_viterbi_encode. */
qtcq_status qtcq_bcjr_soft(const float* seq, const float* err_w, int64_t B, int T, int L, int k,
                           qtcq_code code, float temperature, float* soft, float* log_z,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---- Gradient of the soft codeword [BCJR abstract: the relaxation is exactly
 * differentiable] -------------------------------------------------------------------
 * With p(walk) ~ exp(-E / temperature) and E the energy of qtcq_bcjr_soft,
 *     d soft[b][t] / d seq[b][u] = (2 w_u / temperature) Cov_p( C(st[t]), C(st[u]) ),
 * (w_u = err_w[b][u], or 1), so for an upstream gradient g = dLoss/dsoft the
 * vector-Jacobian product is
 *     grad_seq[b][u] = (2 w_u / temperature) Cov_p( sum_t g[b][t] C(st[t]), C(st[u]) ),
 * computed by one more forward-backward pass with expectation messages (fp32
 * expectation messages centred on the soft codeword).  The result is within
 * 1e-5 * RMS_u(grad_seq[b]) + 2^-100 of the exact value (the absolute term covers
 * gradients carried by posterior weights near binary32's underflow range) at
 * temperatures from QTCQ_VJP_MIN_TEMPERATURE up (tested on N(0,1) targets, with and
 * without log-normal weights, all three codes, and on targets 4 + 3 N(0,1) far outside
 * the codebook's range; below 0.01 the message stashes are kept in fp64).  Below that
 * floor the call is refused (QTCQ_ERR_UNSUPPORTED): there the gradient collapses onto a
 * few near-ties while the fp32 expectation messages and exp2 weights keep a fixed
 * relative precision, and the bound no longer holds (1.7e-5 * RMS measured at L = 16,
 * temperature 1e-3).  The soft codeword itself (qtcq_bcjr_soft) has no such floor. */
#define QTCQ_VJP_MIN_TEMPERATURE 3e-3f

/* Workspace bytes qtcq_bcjr_vjp needs for `B` sequences in one pass (both message
 * directions of every step -- in 32 bits, fixed point near each step's maximum and
 * binary32 far below it, or in fp64 below temperature 0.01; the size covers both -- plus
 * the expectation messages of the forward direction).  Smaller workspaces that hold one
 * sequence are used in chunks.
 * Returns 0 for unsupported arguments. */
size_t qtcq_bcjr_vjp_workspace_bytes(int64_t B, int T, int L, int k);

/* Vector-Jacobian product of the BCJR soft codeword with respect to the targets.
 *   seq, err_w, B, T, L, k, code, temperature : as qtcq_bcjr_soft
 *   grad_soft [B][T] float32 (in): the upstream gradient g
 *   grad_seq  [B][T] float32 (out): the product above
 *   soft      [B][T] float32 (out) or NULL: the soft codeword, bit-identical to
 *             qtcq_bcjr_soft's
 *   log_z     [B] float32 (out) or NULL
 *   workspace: 16-byte aligned, >= qtcq_bcjr_vjp_workspace_bytes(1, T, L, k)
 * Errors: QTCQ_ERR_INVALID_ARG (also grad_soft or grad_seq NULL), QTCQ_ERR_UNSUPPORTED
 * (also a finite temperature below QTCQ_VJP_MIN_TEMPERATURE), QTCQ_ERR_WORKSPACE,
 * QTCQ_ERR_DEVICE. */
qtcq_status qtcq_bcjr_vjp(const float* seq, const float* err_w, int64_t B, int T, int L, int k,
                          qtcq_code code, float temperature, const float* grad_soft, float* grad_seq,
                          float* soft, float* log_z, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ---- Tail-biting trellis [QTIP "Tail-biting is worth its complexity"] ------------
 * A tail-biting walk is cyclic: the low L-k bits of its last state equal the high L-k
 * bits of its first, so the stream needs no start state and is exactly k*T bits.
 * Layout: state st[t] contributes its k high bits at stream bits [t*k, t*k + k), most
 * significant first, in the word layout above; weight t reads the window of stream
 * bits t*k, ..., t*k + L - 1 taken modulo k*T (the last L/k - 1 windows wrap round to
 * the start).  Requires k*T >= L (the stream is at least one window long). */

/* Words per sequence of a tail-biting stream: ceil(k*T / 32) -- 16 at (16, 2, 256),
 * word-aligned whenever k*T is a multiple of 32.  Returns -1 for arguments outside
 * 1 <= k <= L <= 32, T >= 1, k*T >= L. */
int64_t qtcq_tailbiting_words(int L, int k, int T);

/* Workspace bytes qtcq_tailbiting_encode needs for `B` sequences in one pass (the
 * encode layout plus one overlap word per sequence).  Smaller workspaces that hold one
 * sequence are used in chunks.  Returns 0 for unsupported arguments. */
size_t qtcq_tailbiting_workspace_bytes(int64_t B, int T, int L, int k);

/* Tail-biting encode with two searches per sequence (the page's summary of QTIP's
 * Algorithm 4): (1) the free-start Viterbi search of qtcq_viterbi_encode over the
 * targets rotated by r = floor(T/2), s'[t] = seq[b][(t + r) mod T] (weights likewise),
 * so that the sequence's two ends meet in the middle; (2) the overlap o = the high
 * L-k bits of the state that search assigns to original position 0; (3) the search
 * over the original targets with the start restricted to states whose high L-k bits
 * are o and the end to states whose low L-k bits are o (ties as in
 * qtcq_viterbi_encode: lowest predecessor, then lowest allowed final state).  The
 * result is a valid tail-biting walk, not always the cheapest one (the exact optimum
 * needs 2^(L-k) pinned searches).
 *   seq, err_w, B, T, L, k, code : as qtcq_viterbi_encode; k*T >= L
 *   bits   [B][qtcq_tailbiting_words(L,k,T)] uint32 (out), the tail-biting layout
 *   mse    [B] float32 (out) = the binary32 path cost of step (3) / T, or NULL
 *   states [B][T] uint32 (out), or NULL
 *   workspace: 16-byte aligned, >= qtcq_tailbiting_workspace_bytes(1, T, L, k)
 * Errors: QTCQ_ERR_INVALID_ARG (also k*T < L), QTCQ_ERR_UNSUPPORTED,
 * QTCQ_ERR_WORKSPACE, QTCQ_ERR_DEVICE. */
qtcq_status qtcq_tailbiting_encode(const float* seq, const float* err_w, int64_t B, int T, int L,
                                   int k, qtcq_code code, uint32_t* bits, float* mse, uint32_t* states,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Window decode of tail-biting streams (cyclic windows, layout above); arguments,
 * outputs and errors as qtcq_decode, with bits [B][qtcq_tailbiting_words(L,k,T)] and
 * k*T >= L.  Decoding qtcq_tailbiting_encode's output with the same seq/err_w
 * reproduces its mse bit for bit. */
qtcq_status qtcq_tailbiting_decode(const uint32_t* bits, int64_t B, int T, int L, int k, qtcq_code code,
                                   float* recon, const float* seq, const float* err_w, float* mse,
                                   void* stream);

/* ---- Decode -> matrix-vector product [QTIP "What it buys end to end": each 16x16 tile
 * of a weight matrix is one 256-weight sequence that decodes straight into the matrix
 * operand; batch-1 inference streams the 2-bit weights] ------------------------------
 * y[i][m] = sum_n W[m][n] x[i][n] for the M x N matrix W whose 16x16 tiles are the
 * sequences of `bits`, numbered row-major: sequence I*(N/16) + J is tile (I, J), and its
 * weight t = 16 r + c is W[16 I + r][16 J + c] (the window decode of qtcq_decode, or of
 * qtcq_tailbiting_decode when `tailbiting` != 0, at T = 256).
 *   bits  [(M/16)*(N/16)][W] uint32, W = qtcq_bitstream_words(L,k,256) (17 at L=16) or,
 *         tail-biting, qtcq_tailbiting_words(L,k,256) (16)
 *   M, N  multiples of 16, N <= 2^22 (N = 0 gives y = 0)
 *   x     [batch][N] float32, 16-byte aligned (may be NULL when N = 0);
 *         y [batch][M] float32 (out)
 *   batch 0..8 activation rows (0: nothing to do)
 * Arithmetic: fp32 FMA of each code value before its rescale (exact in fp32) with x,
 * partial sums added in a fixed order, then the code's rescale applied once per output
 * (bit-deterministic; a one-hot x returns a column of W exactly); error
 * <= (4 ceil(N/1024) + 22) * 2^-24 * sum_n |W[m][n] x[i][n]| to first order.  For the
 * XOR code, when each workgroup's share of the matrix is large enough (2^(L-9) tiles),
 * the codes are read from a 2^L-entry table in LDS: the same results bit for bit.
 * Errors: QTCQ_ERR_INVALID_ARG (M or N negative or not multiples of 16, NULL or
 * misaligned buffers), QTCQ_ERR_UNSUPPORTED ((L, k) or code, batch > 8, N > 2^22),
 * QTCQ_ERR_DEVICE. */
qtcq_status qtcq_decode_matvec(const uint32_t* bits, int M, int N, int L, int k, qtcq_code code,
                               int tailbiting, const float* x, int batch, float* y, void* stream);

/* The same product with the multiplications on the matrix cores [same passage].  The
 * code values before their rescale are exact in fp16; each batch row of x is cut into
 * blocks of 32 columns, each scaled by a power of two 2^s (its largest magnitude into
 * [2^14, 2^15)) and split into two fp16 parts, hi = rn16(x 2^s) and
 * lo = rn16(x 2^s - hi); fp16 MFMAs take W times both parts, and their results, scaled
 * back by 2^-s, are added in a fixed order and rescaled once (bit-deterministic; a
 * one-hot x returns a column of W exactly).  With K = ceil(ceil(N/32)/16) and allowing
 * each addition inside the matrix instruction one unit in the last place, the error is
 *   <= (84.5 + K) * 2^-24 * sum_n |W[m][n] x[i][n]| + 2^-39 * max_n |x[i][n]| * sum_n |W[m][n]|
 * to first order, without underflow (blocks of x whose largest magnitude is below
 * 2^-111 keep less precision).  A row of x holding inf or NaN gives non-finite outputs
 * in that row.
 * Arguments as qtcq_decode_matvec, except that batch may be 0..32 (each group of 8 rows
 * adds one matrix instruction per 16 output rows and 32 columns; the decode is shared),
 * plus
 *   workspace  device scratch, 16-byte aligned, >= qtcq_decode_matvec_mfma_workspace_bytes(N)
 *              (the split x and its block scales; contents on entry are ignored)
 * Two kernels are enqueued on `stream` (the split, then the product).  For the XOR
 * code, when each workgroup's share of the matrix is large enough to pay for it
 * (2^(L-9) tiles of 16x16), the product reads the codes
 * from a 2^L-entry table in LDS instead of computing them: the same results bit for bit.
 * Errors: as qtcq_decode_matvec (QTCQ_ERR_UNSUPPORTED for batch > 32), also
 * QTCQ_ERR_UNSUPPORTED for N > 2^22, and QTCQ_ERR_WORKSPACE (workspace NULL, misaligned
 * or too small). */
size_t qtcq_decode_matvec_mfma_workspace_bytes(int N);   /* 0 if N < 0, N % 16 != 0 or N > 2^22 */
qtcq_status qtcq_decode_matvec_mfma(const uint32_t* bits, int M, int N, int L, int k, qtcq_code code,
                                    int tailbiting, const float* x, int batch, float* y,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* The two halves of qtcq_decode_matvec_mfma, for several matrices that multiply the same
 * x (in inference, projections that share their input): the split once, then one product
 * per matrix [same passage].  qtcq_matvec_mfma_split_x writes the split of x ([batch][N],
 * as above) into `workspace`; qtcq_decode_matvec_mfma_presplit multiplies the matrix of
 * `bits` (M, L, k, code, tailbiting as above) by it and writes y [batch][M], reading
 * `split` only (it is the workspace of a split of the same N and batch, enqueued earlier
 * on this stream or otherwise ordered before it).  Results equal those of
 * qtcq_decode_matvec_mfma bit for bit.
 * Errors: as qtcq_decode_matvec_mfma; QTCQ_ERR_WORKSPACE for a workspace or split NULL,
 * misaligned or below qtcq_decode_matvec_mfma_workspace_bytes(N). */
qtcq_status qtcq_matvec_mfma_split_x(const float* x, int N, int batch, void* workspace,
                                     size_t workspace_bytes, void* stream);
qtcq_status qtcq_decode_matvec_mfma_presplit(const uint32_t* bits, int M, int N, int L, int k,
                                             qtcq_code code, int tailbiting, const void* split,
                                             size_t split_bytes, int batch, float* y,
                                             void* stream);

/* ---- Without allocation -------------------------------------------------------------
 * For callers that cannot allocate device memory or pass a workspace -- code under HIP
 * graph capture with a fixed memory plan, tight serving loops, harnesses that forbid
 * hipMalloc: qtcq_decode_matvec_mfma with the split x in a scratch array the library
 * holds on each GPU instead of a caller workspace.  Same arguments, kernels and results
 * (bit for bit) as qtcq_decode_matvec_mfma without the workspace; the caller still owns
 * x and y.  The call itself allocates nothing: the array is a static device array of
 * QTCQ_NOALLOC_SCRATCH_BYTES (8 MiB) that each GPU holds from the library's load until
 * the process ends; its address on a device is looked up once, on the first call made
 * with that device current.
 *  - Limit: the split of x must fit the array, which holds N up to 63,520 columns at any
 *    batch up to 32; larger N returns QTCQ_ERR_WORKSPACE before anything is launched.
 *  - Every call on one GPU shares that GPU's array and leaves its split there: calls
 *    that overlap on one GPU (different streams, or different host threads on one
 *    stream without ordering) race and give undefined results.  Order them, or use
 *    qtcq_decode_matvec_mfma with a workspace per stream.
 * Errors: as qtcq_decode_matvec_mfma (no workspace errors besides the limit), and
 * QTCQ_ERR_DEVICE if the array's address cannot be looked up. */
#define QTCQ_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
qtcq_status qtcq_decode_matvec_mfma_noalloc(const uint32_t* bits, int M, int N, int L, int k,
                                            qtcq_code code, int tailbiting, const float* x,
                                            int batch, float* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QTCQ_H */
