/*
 * orbq.h -- C ABI of the OrbitQuant quantized linear layer on AMD Instinct MI355X (gfx950).
 *
 * Pages cited: "OrbitQuant: Data-Agnostic Quantization for Image and Video Diffusion
 * Transformers" (summary page on picx.dev; cited as "OrbitQuant summary" with its section
 * titles), the TurboQuant slide deck ("TurboQuant: Online Vector Quantization with
 * Near-optimal Distortion Rate", docswell; cited by slide number "Page. N"), "Quantizing With
 * Randomized Hadamard Transforms" (gist.science; composed rotations and the flatness check),
 * the ai-papers.net OrbitQuant article (AdaLN kept at BF16 activations) and the ai-papers.net
 * article on Nunchaku / SVDQuant in Diffusers (GELU fused with the MLP; weight-only kernels).
 *
 * What the library computes (OrbitQuant summary, picx.dev, "Methodology"):
 *   offline  "Offline Weight Quantization": W' = W Pi^T, r'_i = ||w'_i||, codes of
 *            w'_i / r'_i under a Lloyd-Max codebook, r' stored in bf16.
 *   online   "Online Activation Quantization": x' = Pi x, s = ||x'||, codes of
 *            x' / (s + eps) under a Lloyd-Max codebook; the product with the folded
 *            weights needs no inverse rotation because Pi^T Pi = I.
 *   Pi       "Randomized Permuted Block-Hadamard (RPBH) Rotation":
 *            Pi = blkdiag(H_h D_1, ..., H_h D_{d/h}) P_pi.
 *   codebook "Theoretical Basis" item 2: Lloyd-Max centroids for the marginal f_d of a
 *            rotated unit vector (item 1); one codebook per (d, bits), shared by all
 *            layers and by weights and activations ("Data-Agnostic Codebook").
 *
 * Conventions fixed here where the pages are silent:
 *   - H_h is the Sylvester (natural order) Hadamard matrix scaled by 1/sqrt(h), so Pi is
 *     orthogonal.  (P_pi x)[j] = x[perm[j]]; signs[j] multiplies position j after the
 *     permutation.
 *   - Quantization is q(t) = argmin_k |t - c_k| over the ascending codebook, ties to the
 *     lower index k; t = x' / (s + eps) with the unrounded norm.
 *   - Code value (sign-magnitude): for N = 2^bits centroids, centroid k >= N/2 is stored
 *     as k - N/2 and centroid k < N/2 as N/2 + (N/2 - 1 - k): the top bit is the sign
 *     (1 = negative), the low bits rank |c_k| from the smallest magnitude up.
 *   - Packed rows: the d codes of a row in order, rows back to back, d*bits/8 bytes per
 *     row, least significant bits first:
 *        bits = 4: code j in byte j/2, bits 4*(j%2)..+3
 *        bits = 2: code j in byte j/4, bits 2*(j%4)..+1
 *        bits = 6: code j in the 3-byte little-endian group j/4, bits 6*(j%4)..+5
 *        bits = 3: code j in the 3-byte little-endian group j/8, bits 3*(j%8)..+2
 *   - The product decodes each centroid to bf16 (round to nearest even), multiplies in
 *     bf16 with fp32 accumulation, and scales by s_i (fp32) and r'_j (bf16) in fp32.
 *
 * Memory: every buffer is owned by the caller.  Pointers marked [device] are HIP device
 * pointers, [host] are host pointers.  The library allocates no device memory: the
 * workspaces of orbq_linear, orbq_linear_act and orbq_linear_a16 come from the caller.
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream) and
 * re-entrant (calls that share a workspace must not overlap); argument errors are
 * detected on the host before anything is launched and are returned synchronously.
 * Device faults surface at the caller's next synchronisation.  Device arrays (perm,
 * signs) are read, never validated, by the kernels: a perm entry outside [0, d) is
 * clamped into range (garbage in, garbage out, no out-of-bounds access).
 *
 * Supported shapes: block a power of two in [64, 4096] (composed passes: at most 1024); d a multiple
 * of block and at most 16384;
 * activation bits and weight bits each in {2, 3, 4, 6}, 3-bit codes in the product only with
 * 3-bit codes (W3A3; the OrbitQuant summary's 3-bit setting).  n or m equal to 0 is a no-op.
 * Alignment: bf16 matrices and code buffers 16-byte aligned with row pitches that
 * are multiples of 16 bytes; norm arrays 4-byte (fp32) or 2-byte (bf16) aligned;
 * Y 16-byte aligned with a row pitch that is a multiple of 16 bytes.
 */
#ifndef ORBQ_H
#define ORBQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ORBQ_OK = 0,
  ORBQ_ERR_INVALID_ARG = -1,  /* null pointer, bad size, ld < d, n/m/d negative        */
  ORBQ_ERR_UNSUPPORTED = -2,  /* block, bits or d outside the supported set            */
  ORBQ_ERR_ALIGNMENT = -3,    /* pointer or pitch not aligned as documented above      */
  ORBQ_ERR_WORKSPACE = -4,    /* workspace smaller than orbq_linear_workspace_bytes    */
  ORBQ_ERR_HIP = -5,          /* a HIP runtime call failed (launch, device query)      */
  ORBQ_ERR_CODEBOOK = -6      /* codebook not ascending, not antisymmetric, not finite */
} orbq_status;

typedef enum { ORBQ_F32 = 0, ORBQ_BF16 = 1 } orbq_dtype;

/* Activation applied to the product before it is stored (Nunchaku / SVDQuant in Diffusers,
 * ai-papers.net, section on quantizing one's own model: GELU fused with the MLP).  The
 * pages name GELU without a formula; both standard forms are offered:
 *   ORBQ_ACT_GELU_TANH  x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
 *   ORBQ_ACT_GELU_ERF   x Phi(x), Phi the standard normal CDF (Abramowitz & Stegun 7.1.26,
 *                       absolute error of Phi below 1e-7)
 * evaluated in fp32 on the scaled fp32 product, before rounding to the output type. */
typedef enum { ORBQ_ACT_NONE = 0, ORBQ_ACT_GELU_TANH = 1, ORBQ_ACT_GELU_ERF = 2 } orbq_activation;

/* RPBH rotation for one dimension d (OrbitQuant summary, "Randomized Permuted
 * Block-Hadamard (RPBH) Rotation"; fixed once per dimension).
 *   d      dimension, multiple of block
 *   block  Hadamard block size h, a power of two in [64, 4096] (the OrbitQuant summary's
 *          "RPBH Rotation" takes the largest power of two dividing d by default; the layers
 *          here use 128)
 *   perm   [device] int32[d], a permutation of 0..d-1: (P x)[j] = x[perm[j]]; NULL means the
 *          identity (the block randomized Hadamard transform without the permutation, the
 *          "Block-RHT" row of the OrbitQuant summary's "Rotation Ablation (Table 3)")
 *   signs  [device] int8[d], each +1 or -1, applied to position j after the permutation
 * Both arrays 16-byte aligned (ORBQ_ERR_ALIGNMENT otherwise); they must stay valid until the
 * calls that use them have completed on their stream.
 *   passes 0 or 1: one RPBH pass.  2 or 3: the composition Pi = Pi_passes ... Pi_1 of that
 *          many RPBH passes ("Quantizing With Randomized Hadamard Transforms", gist.science:
 *          composing two randomized Hadamard transforms gives Gaussian scalar marginals for
 *          any input, three bound the coordinates' conditional covariance), pass p (from 0)
 *          with its own permutation perm + p*d and signs signs + p*d, so both arrays then
 *          hold passes*d entries (perm NULL: every pass without permutation).  Weights folded
 *          with a composed rotation pair only with activations quantized with the same one.
 *          Other values: ORBQ_ERR_UNSUPPORTED. */
typedef struct {
  int32_t d;
  int32_t block;
  const int32_t* perm;
  const int8_t* signs;
  int32_t passes;
} orbq_rpbh;

/* Lloyd-Max codebook for (d, bits) ("Theoretical Basis" item 2).
 *   centroids  [host] float[2^bits], strictly ascending, exactly antisymmetric
 *              (c[N-1-k] == -c[k]), in units of the normalised coordinate t. */
typedef struct {
  int32_t d;
  int32_t bits;
  const float* centroids;
} orbq_codebook;

/* Offline, host only.  Lloyd-Max centroids of f_d(t) ~ (1 - t^2)^((d-3)/2) on [-1, 1]
 * ("Theoretical Basis" items 1-2; TurboQuant slides, docswell, "Page. 13"-"Page. 16"),
 * by Lloyd iteration with Gauss-Legendre cell integrals in float64, rounded to float32.
 * centroids_out [host] receives 2^bits floats.  bits in 1..8, d >= 3.
 * Returns ORBQ_OK or ORBQ_ERR_INVALID_ARG. */
int orbq_codebook_lloyd_max(int32_t d, int32_t bits, float* centroids_out);

/* Host only, O(d): checks that perm_host is a permutation of 0..d-1 (or NULL: identity),
 * signs_host holds only +1/-1, block is supported and divides d.  Use it on the host copies
 * before uploading. */
int orbq_rpbh_validate(int32_t d, int32_t block, const int32_t* perm_host, const int8_t* signs_host);

/* Host only: checks a codebook as every entry point does (see ORBQ_ERR_CODEBOOK). */
int orbq_codebook_validate(const orbq_codebook* cb);

/* Bytes of one packed code row: d*bits/8.  0 if d*bits is not a multiple of 8. */
size_t orbq_codes_row_bytes(int64_t d, int32_t bits);

/* Offline weight fold and quantize ("Offline Weight Quantization", steps 1-4).
 *   W          [device] bf16[m][ldw] (row-major; row i is w_i), ldw >= d
 *   rot, cb_w  rotation and weight codebook for dimension d (cb_w->d == d == rot->d)
 *   eps        added to the row norm before dividing (the page writes no eps for weights;
 *              1e-8 keeps zero rows finite)
 *   w_codes    [device] uint8[m][d*bits/8], packed codes of Q(w'_i / (r'_i + eps))
 *   w_norms    [device] bf16[m], r'_i = ||Pi w_i|| rounded to nearest even
 * The same kernel as orbq_rpbh_quantize, with bf16 norms. */
int orbq_fold_weights(const void* W, int64_t m, int64_t d, int64_t ldw, const orbq_rpbh* rot,
                      const orbq_codebook* cb_w, float eps, uint8_t* w_codes, void* w_norms,
                      void* stream);

/* Online activation quantization ("Online Activation Quantization", steps 1-3).
 *   X          [device] bf16[n][ldx], token rows, ldx >= d
 *   x_codes    [device] uint8[n][d*bits/8], packed codes of Q(x'_i / (s_i + eps))
 *   x_norms    [device] float[n], s_i = ||Pi x_i|| in fp32
 * One pass over X: permute, sign, block FWHT, norm, threshold, pack. */
int orbq_rpbh_quantize(const void* X, int64_t n, int64_t d, int64_t ldx, const orbq_rpbh* rot,
                       const orbq_codebook* cb_a, float eps, uint8_t* x_codes, float* x_norms,
                       void* stream);

/* Product in the rotated basis ("Online Activation Quantization", last paragraph: the
 * rotations cancel):  Y[i][j] = s_i * r'_j * sum_k bf16(C_a[a_ik]) * bf16(C_w[w_jk]).
 *   x_codes, x_norms   [device] as written by orbq_rpbh_quantize (n rows)
 *   w_codes, w_norms   [device] as written by orbq_fold_weights (m rows)
 *   Y                  [device] float or bf16 [n][ldy], ldy >= m
 * bf16 MFMA with fp32 accumulation; the epilogue scales in fp32 and rounds to y_type. */
int orbq_lut_gemm(const uint8_t* x_codes, const float* x_norms, const orbq_codebook* cb_a,
                  const uint8_t* w_codes, const void* w_norms, const orbq_codebook* cb_w,
                  int64_t n, int64_t m, int64_t d, void* Y, orbq_dtype y_type, int64_t ldy,
                  void* stream);

/* orbq_lut_gemm followed by an activation in its epilogue: Y[i][j] = act(s_i r'_j sum_k ...),
 * the MLP up-projection with its GELU fused.  Arguments and errors as orbq_lut_gemm; an
 * unknown `act` returns ORBQ_ERR_INVALID_ARG.  ORBQ_ACT_NONE gives orbq_lut_gemm's bits. */
int orbq_lut_gemm_act(const uint8_t* x_codes, const float* x_norms, const orbq_codebook* cb_a,
                      const uint8_t* w_codes, const void* w_norms, const orbq_codebook* cb_w,
                      int64_t n, int64_t m, int64_t d, orbq_activation act, void* Y,
                      orbq_dtype y_type, int64_t ldy, void* stream);

/* Workspace bytes orbq_linear needs for n tokens of dimension d at bits_a: packed codes
 * (rounded up to 256 bytes) followed by n fp32 norms.  For bits_a = 6 the space holds 2 d bytes
 * per token: with m >= 2048 output columns the layer keeps the codes' bf16 centroids instead of
 * the packed codes, which its product then stages without decoding (the output is the same
 * bit for bit; the codes' six-bit lookups cost more than the wider operand once every token row
 * is decoded for 8 or more column tiles). */
size_t orbq_linear_workspace_bytes(int64_t n, int64_t d, int32_t bits_a);

/* The online layer: orbq_rpbh_quantize into `workspace`, then orbq_lut_gemm, on one
 * stream.  Arguments as in those two calls; ws_bytes >= orbq_linear_workspace_bytes. */
int orbq_linear(const void* X, int64_t n, int64_t d, int64_t ldx, const orbq_rpbh* rot,
                const orbq_codebook* cb_a, float eps, const uint8_t* w_codes, const void* w_norms,
                const orbq_codebook* cb_w, int64_t m, void* workspace, size_t ws_bytes, void* Y,
                orbq_dtype y_type, int64_t ldy, void* stream);

/* orbq_linear with orbq_lut_gemm_act's activation in the product's epilogue. */
int orbq_linear_act(const void* X, int64_t n, int64_t d, int64_t ldx, const orbq_rpbh* rot,
                    const orbq_codebook* cb_a, float eps, const uint8_t* w_codes, const void* w_norms,
                    const orbq_codebook* cb_w, int64_t m, void* workspace, size_t ws_bytes,
                    orbq_activation act, void* Y, orbq_dtype y_type, int64_t ldy, void* stream);

/* orbq_linear_act for callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops, harnesses that forbid hipMalloc): the same kernels and the same outputs, bit
 * for bit, with the workspace taken from a device array inside the library instead of an
 * argument.  The call allocates nothing.
 *   Limit: orbq_linear_workspace_bytes(n, d, cb_a->bits) <= ORBQ_NOALLOC_SCRATCH_BYTES (16 MiB:
 *   the 4608 x 3072 layer needs 7.1 MB, the 9216 x 3072 one 14.2 MB); larger calls return
 *   ORBQ_ERR_WORKSPACE without launching.
 *   Each GPU holds one such array (16 MiB, from the library's first call on that device until
 *   the process ends), shared by every call on that GPU: calls on one GPU that overlap in time
 *   (on different streams, or from several host threads without ordering) race on it; calls
 *   ordered on one stream do not.  Every byte a call reads from it was written by the same call
 *   (rpbh_quantize writes the whole workspace before the product reads it).
 *   Other arguments, errors and layouts as in orbq_linear_act. */
#define ORBQ_NOALLOC_SCRATCH_BYTES (16u << 20)
int orbq_linear_noalloc(const void* X, int64_t n, int64_t d, int64_t ldx, const orbq_rpbh* rot,
                        const orbq_codebook* cb_a, float eps, const uint8_t* w_codes, const void* w_norms,
                        const orbq_codebook* cb_w, int64_t m, orbq_activation act, void* Y, orbq_dtype y_type,
                        int64_t ldy, void* stream);

/* Weight-only product with bf16 activations (W4A16 and, with 2- or 6-bit weight codes,
 * W2A16 / W6A16).  The OrbitQuant pages keep the AdaLN activations in BF16 (ai-papers.net
 * OrbitQuant article, section on AdaLN handling and compression) while the AdaLN modulation
 * weights go to 4 bits (OrbitQuant summary, "AdaLN Bit-Width Ablation (Figure 6)"); Nunchaku /
 * SVDQuant in Diffusers (ai-papers.net) names a weight-only 4-bit GEMM for such layers.  The weights are the usual
 * folded codes; the activations are rotated but not quantized:
 *   Y[i][j] = r'_j * sum_k bf16((Pi x_i)_k) * bf16(C_w[w_jk])
 * with Pi x_i computed in fp32 and rounded to bf16 (the matrix cores' input type), fp32
 * accumulation.  Built for few tokens (modulation vectors, small batches): the weight codes are
 * streamed once per 16 tokens, so the call is bound by the code bytes.
 *   X        [device] bf16[n][ldx], 16-byte aligned rows; d a multiple of 128
 *   rot      rotation the weights were folded with (any passes)
 *   w_codes, w_norms, cb_w, m   as for orbq_lut_gemm
 *   workspace [device] >= orbq_linear_a16_workspace_bytes(n, d, m), 256-byte aligned: the
 *            rotated tokens of a 16-token chunk (bf16) and their norms
 *   Y        [device] float or bf16 [n][ldy], ldy >= m
 * Errors as orbq_linear; d % 128 != 0 gives ORBQ_ERR_UNSUPPORTED. */
size_t orbq_linear_a16_workspace_bytes(int64_t n, int64_t d, int64_t m);
int orbq_linear_a16(const void* X, int64_t n, int64_t d, int64_t ldx, const orbq_rpbh* rot,
                    const uint8_t* w_codes, const void* w_norms, const orbq_codebook* cb_w, int64_t m,
                    void* workspace, size_t ws_bytes, void* Y, orbq_dtype y_type, int64_t ldy,
                    void* stream);

/* The adaptive check ("Quantizing With Randomized Hadamard Transforms", gist.science,
 * "Method": an O(d) look at the input's l3 norm, for scalar quantization, or its l_inf
 * norm, for vector quantization, decides whether 1, 2 or 3 composed transforms are needed).
 *   X       [device] bf16[n][ldx], 16-byte aligned, 16-byte pitch; d a multiple of 8
 *   rho3    [device] float[n], sqrt(d) ||x||_3^3 / ||x||_2^3 (1: constant row, sqrt(d): one-hot)
 *   rhoinf  [device] float[n], sqrt(d) ||x||_inf / ||x||_2 (same scale)
 * A zero row gives 0 for both.  fp32 sums (relative error ~1e-6).  One HBM pass over X. */
int orbq_rpbh_flatness(const void* X, int64_t n, int64_t d, int64_t ldx, float* rho3,
                       float* rhoinf, void* stream);

/* [host] Pass count for a row (or the largest statistics of a batch or a weight matrix) with
 * the given flatness.  The pages give the rule's inputs but no thresholds; this reading
 * compares against a Gaussian row (rho3 -> 2 sqrt(2/pi), rhoinf ~ sqrt(2 ln 2d)):
 *   scalar quantization (vector_quantization = 0): 1 if rho3 <= 2 * 2 sqrt(2/pi), else 2;
 *   vector quantization: 1 if rhoinf <= sqrt(2 ln 2d), 2 if <= 2 sqrt(2 ln 2d), else 3.
 * In the layer the rotation is fixed per dimension and shared with the folded weights, so the
 * count is a per-layer choice, not a per-token one.  Negative statistics or d < 2:
 * ORBQ_ERR_INVALID_ARG. */
int32_t orbq_rht_passes(float rho3, float rhoinf, int32_t d, int32_t vector_quantization);

/* Human-readable name of a status code, and the detail of the last error on this thread. */
const char* orbq_status_string(int status);
const char* orbq_last_error(void);

/* ---- test-only entry points (stable names, not part of the layer's contract) ---- */

/* x' = Pi x in fp32 [n][d] (the FWHT output scaled by 1/sqrt(block)) and s_i as
 * orbq_rpbh_quantize computes it: exposes the rotation alone for checking. */
int orbq_test_rotate(const void* X, int64_t n, int64_t d, int64_t ldx, const orbq_rpbh* rot,
                     float* x_rot, float* x_norms, void* stream);

/* Quantize `count` given fp32 values t (already normalised) with the decision the kernels
 * use; writes one sign-magnitude code per byte.  cb->d selects nothing here but is
 * validated like elsewhere. */
int orbq_test_quantize_t(const float* t, int64_t count, const orbq_codebook* cb, uint8_t* codes,
                         void* stream);

/* Sustained bf16 matrix-core rate: `workgroups` workgroups of 512 threads (two waves per SIMD,
 * as in orbq_lut_gemm) each run `iters` v_mfma_f32_32x32x16_bf16 steps into 9 accumulators per
 * wave, on register operands with pseudo-random bits (no memory or LDS traffic).  Time it on
 * `stream` to get the rate the matrix cores hold under load; *flops (host) receives the
 * floating-point operations of the call.  sink [device] receives workgroups * 512 floats
 * (4-byte aligned).  Errors: workgroups outside [1, 65536], iters not a positive multiple of 4
 * up to 2^24, or a NULL pointer give ORBQ_ERR_INVALID_ARG. */
int orbq_test_mfma_rate(int32_t workgroups, int32_t iters, float* sink, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ORBQ_H */
