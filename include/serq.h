/*
 * serq.h -- C ABI of libserq, the SERQ quantized linear layer for MI355X (gfx950).
 *
 * SERQ ("SERQ: Saliency-Aware Low-Rank Error Reconstruction for LLM
 * Quantization") computes a linear layer Y = X W (X: M x K tokens by input
 * channels, W: K x N) as a pure 4-bit GEMM plus one small residual product:
 *
 *     Y  ~  Q(X^) Q(W^)  +  X~_{s,q} Q(R)
 *
 * where, after calibration,
 *   X~ = X diag(s^-1), W~ = diag(s) W          static per-channel flattening
 *   W^ = P W~ = [W~_s; W~_r], X^ = X~ P^-1     rows in descending saliency
 *   R  = W~_s - Q(W~_s)                        r x N compensator of the r
 *                                              most salient rows
 * and X~_{s,q} is the first r columns of the quantized activations.
 * Sources: papernotes.org ICLR 2026 notes on SERQ, sections 核心 idea,
 * 方法详解 / 整体框架 and 关键设计 1-3; gist.science/de/paper/2603.08185,
 * "Technische Zusammenfassung" 2.A-2.C.
 *
 * Conventions for every call
 *   - Sizes are element counts. Matrices are row-major and contiguous.
 *   - 4-bit codes are packed two per byte: byte t of a row holds code 2t in
 *     bits 0-3 and code 2t+1 in bits 4-7, each a 4-bit two's complement
 *     value in [-8, 7]. int8 codes are plain signed bytes.
 *   - Quantizer (weights, R, activations): symmetric, one scale per group,
 *     scale = fl32(m / qmax), code = clamp(rne(fl32(v * fl32(qmax / m)))),
 *     m the group's absolute maximum, qmax 7 (int4) or 127 (int8), rne round
 *     half to even. A group whose fl32(qmax / m) overflows (an all-zero group
 *     in particular) gets scale 0 and zero codes.
 *   - The caller owns every input and output. The library creates no
 *     streams and allocates no memory; the only device memory it holds is
 *     scratch for two paths (serq_linear's K split, chunked activation
 *     quantization) in file-scope device arrays, described at those calls:
 *     calls that take them must not overlap on one device.
 *   - Argument errors are detected on the host and returned before anything
 *     is launched; the output buffers are then untouched.
 *   - Online calls only enqueue work on `stream` (a hipStream_t; NULL is the
 *     null stream) and return without synchronizing. A launch failure
 *     returns SERQ_EHIP.
 */
#ifndef SERQ_H_
#define SERQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SERQ_OK = 0,
  SERQ_EINVAL = -1,       /* bad size, NULL pointer, bad enum value           */
  SERQ_EALIGN = -2,       /* a device pointer is not 16-byte aligned          */
  SERQ_EUNSUPPORTED = -3, /* valid request the library does not implement    */
  SERQ_EHIP = -4          /* the HIP runtime reported an error at launch      */
} serq_status;

typedef enum { SERQ_F32 = 0, SERQ_BF16 = 1 } serq_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* serq_strerror(int status);

/* Version of the ABI described by this header (major * 100 + minor). */
int serq_abi_version(void);

/* Bytes per row of the packed Q(R) buffer for r salient rows: r codes
 * padded with zero codes to a multiple of 32 (16 bytes). */
#define SERQ_RQ_ROW_BYTES(r) ((((r) + 31) / 32) * 16)

/* SERQ_RQ_ROW_BYTES as a function (for bindings that cannot use macros);
 * returns -1 for r < 0. */
int serq_rq_row_bytes(int r);

/*
 * serq_calibrate -- offline, host memory, synchronous, deterministic.
 *
 * Follows the calibration phase of the pages (papernotes.org SERQ notes,
 * 方法详解 / 整体框架: calibration fixes the scale factors, the salient rows
 * and the permutation; 关键设计 1: SmoothQuant-style static per-channel s;
 * 关键设计 2: salient rows identified by their scale, rows permuted in
 * descending saliency, compensator R on the first r rows, R itself
 * quantized; 核心 idea: R = W~_s - Q(W~_s)).
 *
 *   W          K x N, dtype w_dtype (SERQ_F32 or SERQ_BF16), Y = X W.
 *   act_absmax K floats: max over the calibration tokens of |X[t, j]|.
 *   alpha      smoothing exponent in [0, 1]:
 *              s_j = fl32( max(a_j,1e-5)^alpha / max(w_j,1e-5)^(1-alpha) ),
 *              a_j = act_absmax[j], w_j = max_n |W[j, n]|, evaluated in
 *              double (for alpha = 0.5 exactly sqrt(a)/sqrt(w)).
 *   r          number of salient rows, 0 <= r <= K, r even.
 * Outputs (caller-allocated host buffers):
 *   perm       K int32: perm[i] = original channel placed at position i,
 *              descending s, equal s keep ascending channel order.
 *   s_hat_inv  K floats: fl32(1 / s[perm[i]]), the activation multiplier
 *              in saliency order.
 *   Wq         N x K/2 bytes: column n of Q(W^) as packed int4 along K
 *              (N-major), W^[i, n] = fl32(s[perm[i]] * W[perm[i], n]).
 *   sw         N floats: per-output-channel weight scale.
 *   Rq         N x SERQ_RQ_ROW_BYTES(r) bytes: column n of Q(R) packed
 *              along r, where R[i, n] = fl32(W^[i, n] - fl32(Wq[n, i] * sw[n])),
 *              i < r; each row is padded with zero codes to a multiple of 32
 *              codes (16 bytes), so rows stay 16-byte aligned.
 *              May be NULL when r == 0.
 *   sr         N floats: per-output-channel scale of R (all 0 when r == 0).
 *              May be NULL when r == 0.
 * Errors: SERQ_EINVAL for NULL inputs/outputs, K or N <= 0, odd K, odd r,
 * r outside [0, K], alpha outside [0, 1], unknown w_dtype.
 */
int serq_calibrate(const void* W, serq_dtype w_dtype, int K, int N,
                   const float* act_absmax, float alpha, int r,
                   int32_t* perm, float* s_hat_inv,
                   uint8_t* Wq, float* sw, uint8_t* Rq, float* sr);

/*
 * serq_calibrate_gptq -- offline, host memory, synchronous, deterministic.
 *
 * serq_calibrate with GPTQ codes for the weights (SERQ(GPTQ); the method
 * works with RTN and with GPTQ: gist.science/de/paper/2603.08185,
 * "Technische Zusammenfassung" 3; the pages' accuracy rows use it:
 * papernotes.org SERQ notes, 实验关键数据). GPTQ (Frantar et al., ICLR 2023)
 * quantizes the rows of W^ one at a time in the saliency order and moves
 * each row's error onto the rows not yet quantized, weighted by the upper
 * Cholesky factor U of H^-1, H = X^^T X^ over calibration inputs. Same
 * arguments and outputs as serq_calibrate, plus:
 *   X_cal      T x K calibration activations in the original channel order,
 *              dtype x_dtype (SERQ_F32 or SERQ_BF16); the Hessian is taken
 *              over the inputs the layer sees, x^ = fl32(X_cal[t, perm[i]] *
 *              s_hat_inv[i]), summed over t in order in double.
 *   T          calibration tokens, T > 0.
 *   damp       dampening: damp * mean(diag H) is added to the diagonal
 *              (0.01 in GPTQ); an all-zero H is replaced by the identity.
 * The r salient rows lead the order and their error is left to the
 * compensator, so their codes, R, Q(R) and every scale equal
 * serq_calibrate's; rows r..K-1 get GPTQ codes on the same per-column grid
 * (scale from the column maximum of W^, codes clamped to [-8, 7]). Every
 * step is one double operation in a fixed order, so the result does not
 * depend on the number of host threads. Cost ~ K^3 / 3 + K^2 (T + N) / 2
 * multiply-adds and 8 (3 K^2 + K N) bytes of host memory.
 * Errors: as serq_calibrate, plus SERQ_EINVAL for NULL X_cal, T <= 0, bad
 * x_dtype, damp negative or not finite, and for a Hessian that is not
 * positive definite (possible only with damp == 0; the outputs then hold
 * serq_calibrate's results).
 */
int serq_calibrate_gptq(const void* W, serq_dtype w_dtype, int K, int N,
                        const float* act_absmax, float alpha, int r,
                        const void* X_cal, serq_dtype x_dtype, int T, float damp,
                        int32_t* perm, float* s_hat_inv,
                        uint8_t* Wq, float* sw, uint8_t* Rq, float* sr);

/*
 * serq_permute_outputs -- offline, host memory, in place.
 *
 * Pushes the next layer's input order into this layer's output channels so
 * that its output already arrives in that order and no layer reorders at run
 * time (papernotes.org SERQ notes, 关键设计 3: the down projection's order P4
 * is propagated into the gate/up weight columns; gist.science/de
 * "Technische Zusammenfassung" 2.C).
 *
 *   perm_next  N int32, a permutation of 0..N-1: new output channel i is old
 *              channel perm_next[i].
 *   K, N, r    this layer's sizes, in serq_calibrate's order (K inputs, N
 *              outputs, r salient rows).
 *   Wq (N x K/2 bytes), sw (N), Rq (N x SERQ_RQ_ROW_BYTES(r)), sr (N) are
 *   reordered in place. Rq and sr may be NULL when r == 0.
 * Errors: SERQ_EINVAL for NULL pointers, bad sizes, or perm_next not a
 * permutation (detected before anything is modified).
 */
int serq_permute_outputs(const int32_t* perm_next, int K, int N, int r,
                         uint8_t* Wq, float* sw, uint8_t* Rq, float* sr);

/*
 * serq_quant_act -- online, device memory, asynchronous on `stream`.
 *
 * Per-token symmetric quantization of the flattened activations
 * (papernotes.org SERQ notes, 方法详解 / 整体框架: the main path runs on
 * Q(X^); output node "W4A4/W4A8"). X arrives already in saliency order
 * (关键设计 3), so no gather is done: x^[m, k] = fl32(X[m, k] * s_hat_inv[k]),
 * then one scale per row over all K columns.
 *
 *   X          M x K, dtype x_dtype (SERQ_F32 or SERQ_BF16), device.
 *   s_hat_inv  K floats, device (from serq_calibrate).
 *   a_bits     4 (W4A4) or 8 (W4A8).
 *   Xq         device, M x K/2 bytes (a_bits 4, packed) or M x K int8.
 *   sx         device, M floats: per-token scale.
 * Scratch: up to 64 rows with K > 8192 are cut into chunks over two
 * launches whose chunk maxima meet in a 32 KB device array the library holds
 * per device (no allocation call); such calls on one device must not overlap.
 * M == 0 is a no-op; X, Xq and sx may then be NULL. Errors: SERQ_EINVAL
 * (NULL pointer, M < 0, K <= 0, odd K, bad a_bits or dtype), SERQ_EALIGN
 * (pointer not 16-byte aligned), SERQ_EHIP.
 */
int serq_quant_act(const void* X, serq_dtype x_dtype, int M, int K,
                   const float* s_hat_inv, int a_bits,
                   void* Xq, float* sx, void* stream);

/*
 * serq_silu_mul_quant_act -- online, device memory, asynchronous on `stream`.
 *
 * The MLP step between gate/up and down, fused with down's activation
 * quantization: h = silu(g) * u elementwise, then exactly serq_quant_act on
 * h (per token: x^ = h * s_hat_inv, absmax, codes, sx). The gate and up
 * outputs arrive already in down's saliency order, the permutation having
 * been pushed into their output channels offline with serq_permute_outputs
 * (papernotes.org SERQ notes, 关键设计 3), so no gather is needed. The pages
 * do not spell out the nonlinearity; silu(g) = g / (1 + e^-g) as in the
 * LLaMA MLP, evaluated by a fixed fp32 recipe so results are reproducible
 * bit for bit: e = exp(-g) with the argument clamped to [-80, 80], by
 * Cody-Waite reduction (e^x = 2^n e^r, n = rne(x log2 e), ln 2 split in a
 * head c_hi = 22713 * 2^-15 of 15 significant bits, so n c_hi is exact for
 * |n| <= 116, and a tail; r by two fused multiply-adds) and the degree-7
 * Taylor polynomial of e^r (Horner, one fused multiply-add per degree); then
 * fl32(fl32(g / fl32(1 + e)) * u) with IEEE division and no other fused op.
 *
 *   G, U       device, row m of gate at G + m * ld, of up at U + m * ld, K
 *              elements each, of x_dtype (a gate/up output stored as one
 *              M x 2K buffer is G = Y, U = Y + K, ld = 2K).
 *   ld         row stride in elements, ld >= K. G and U need only be
 *              aligned to their element; rows that are all 16-byte aligned
 *              (and K % 8 == 0) take the vector path, others a scalar one
 *              with the same results.
 *   s_hat_inv  K floats, device (down's, from serq_calibrate).
 *   a_bits, Xq, sx as for serq_quant_act (so is the scratch rule, here for
 *              up to 64 rows with K > 4096, or 128 with K > 16384).
 * M == 0 is a no-op. Errors: SERQ_EINVAL (NULL pointer, M < 0, K <= 0, odd
 * K, ld < K, bad a_bits or dtype), SERQ_EALIGN (G or U not aligned to its
 * element, Xq or sx not 16-byte aligned), SERQ_EHIP. Subnormal inputs are
 * outside the contract.
 */
int serq_silu_mul_quant_act(const void* G, const void* U, int ld, serq_dtype x_dtype,
                            int M, int K, const float* s_hat_inv, int a_bits,
                            void* Xq, float* sx, void* stream);

/*
 * serq_linear -- online, device memory, asynchronous on `stream`.
 *
 * The SERQ linear: acc_main = Xq . Q(W^) over all K, acc_res = Xq[:, :r] . Q(R)
 * over the r salient channels, reusing the same activation codes (no second
 * quantization; papernotes.org SERQ notes, 关键设计 2: the residual is one
 * (tokens x r)(r x d) product on the salient activation channels, R is
 * quantized, no intermediate quantization), and
 *     Y[m, n] = sx[m] * (sw[n] * acc_main[m, n] + sr[n] * acc_res[m, n])
 * evaluated in fp32 and stored as y_dtype (bf16 with round to nearest even).
 * Integer accumulation is exact (int32) for every K the call accepts (the
 * matrix-core kernels serve K < 2^17, longer rows a plain kernel).
 *
 *   Xq, sx     from serq_quant_act with the same a_bits (device).
 *   Wq, sw     N x K/2 bytes and N floats (device).
 *   Rq, sr     N x SERQ_RQ_ROW_BYTES(r) bytes (the layout serq_calibrate
 *              writes, zero codes in the padding) and N floats (device);
 *              may be NULL when r == 0.
 *   M, K, N, r sizes; 0 <= r <= K, r even, K even. M == 0 is a no-op (the
 *              M-sized buffers Xq, sx, Y and the debug buffers may then be
 *              NULL; the weights are still validated).
 *   Y          device, M x N of y_dtype.
 *   acc_main_dbg, acc_res_dbg
 *              NULL on the hot path; when non-NULL, device M x N int32
 *              buffers that receive the exact integer accumulators (both
 *              must then be given).
 * No allocation, no synchronization: the call only enqueues kernels, so it
 * may be captured into a HIP graph, the first call on a device included.
 * Scratch: for 4..32 tokens whose activation rows exceed the kernel's LDS
 * budget (long K), the K range is split across workgroups whose int32
 * partial sums meet in file-scope device arrays of the library (16 MiB of
 * partial sums and 64 KiB of counters per device, held from the moment the
 * library's code is loaded on the device until the process ends). Sizes
 * whose split would need more take a kernel without a split, so no size is
 * refused for it. Calls that take the split path on one device share the
 * arrays, so they must not overlap in time (e.g. on two streams at once).
 * Errors: SERQ_EINVAL (NULL pointer, bad sizes, bad a_bits or dtype, only one
 * debug buffer), SERQ_EALIGN (pointer not 16-byte aligned), SERQ_EHIP.
 */
int serq_linear(const void* Xq, const float* sx, int a_bits,
                const uint8_t* Wq, const float* sw,
                const uint8_t* Rq, const float* sr,
                int M, int K, int N, int r,
                void* Y, serq_dtype y_dtype,
                int32_t* acc_main_dbg, int32_t* acc_res_dbg,
                void* stream);

/*
 * serq_linear_kernel_name -- which kernel serq_linear would launch for these
 * sizes (static string: "gemv", "decode16", "decode32_ksplit" (the K split
 * with scratch), "tile128x128", ..., "generic"), or NULL for invalid sizes.
 * Host only; launches nothing. For profiling and tests.
 */
const char* serq_linear_kernel_name(int M, int K, int N, int r, int a_bits);

/*
 * The same linear on gfx950's scaled FP6 matrix instruction (bf6 route).
 *
 * The pages run SERQ on integer or microscaling-FP4 matrix hardware alike
 * (gist.science/de/paper/2603.08185, "3. Wichtige Beiträge": the method is
 * compatible with INT4 and MXFP4 formats; "4. Ergebnisse", Performance &
 * Latenz: the fast path is the hardware FP4 product, the residual adding
 * about 1 %). CDNA4 has no int4 matrix instruction, but every int4 code in
 * [-8, 7] is exactly a bf6 (E3M2) value, and a product of two such codes
 * summed in fp32 stays an exact integer while |sum| <= 2^24, i.e. for K up to
 * 2^18. So this route computes bit for bit the accumulators of serq_linear
 * (W4A4 only) at the FP6 instruction rate, on operands re-encoded as bf6:
 *
 * bf6 tile layout of a matrix of `rows` x `k` int4 codes. Rows are padded
 * with zero codes to a multiple of 128 (Rp) and k to a multiple of 128 (Kp).
 * The buffer is a sequence of 3072-byte fragment blocks, block (kt, rb) at
 * byte ((kt * Rp / 32) + rb) * 3072 for k-tile kt (codes [128 kt, +128)) and
 * 32-row block rb; inside a block, step s (0, 1) at +1536 s and lane l
 * (0..63) at +24 l hold the 32 codes of row 32 rb + l % 32 at
 * k = 128 kt + 64 s + 32 (l / 32) + f, f = 0..31, each as the 6-bit E3M2
 * pattern (sign bit 5, exponent bits 4..2 with bias 3, mantissa bits 1..0)
 * in bits [6 f, 6 f + 6) of the 24 bytes read as one little-endian 192-bit
 * integer. Code -> pattern: 0 -> 0x00, 1 -> 0x0C, 2 -> 0x10, 3 -> 0x12,
 * 4 -> 0x14, 5 -> 0x15, 6 -> 0x16, 7 -> 0x17, and -v -> 0x20 | pattern(v),
 * -8 -> 0x38. Size: SERQ_BF6_BYTES(rows, k) bytes.
 */
#define SERQ_BF6_BYTES(rows, k) ((size_t)(((k) + 127) / 128) * (size_t)(((rows) + 127) / 128) * 12288u)

/* SERQ_BF6_BYTES as a function; returns -1 for rows < 0 or k < 0. */
int64_t serq_bf6_bytes(int rows, int k);

/*
 * serq_prepack_bf6 -- offline, host memory, synchronous.
 *
 * Re-encodes a packed int4 matrix (serq_calibrate's Q(W^) with k = K and
 * pitch = K/2, or Q(R) with k = r and pitch = SERQ_RQ_ROW_BYTES(r)) into the
 * bf6 tile layout, writing every byte of `out` (padding included).
 *   codes  rows x pitch bytes, canonical nibble order (host).
 *   rows, k, pitch  rows > 0, 0 < k <= 2 * pitch, k even.
 *   out    SERQ_BF6_BYTES(rows, k) bytes (host), caller-owned.
 * Errors: SERQ_EINVAL (NULL pointer, bad sizes).
 */
int serq_prepack_bf6(const uint8_t* codes, int rows, int k, int pitch, uint8_t* out);

/*
 * serq_act_bf6 -- online, device memory, asynchronous on `stream`.
 *
 * Re-encodes W4A4 activation codes (serq_quant_act's Xq, M x K/2 bytes) into
 * the bf6 tile layout, padding included, for serq_linear_bf6. The token
 * scales sx are used as they are.
 *   Xq   device, M x K/2 bytes, 16-byte aligned.
 *   M, K M >= 0 (0: no-op), K > 0 even, K <= 262144.
 *   X6   device, SERQ_BF6_BYTES(M, K) bytes, 16-byte aligned.
 * Errors: SERQ_EINVAL, SERQ_EALIGN, SERQ_EHIP.
 */
int serq_act_bf6(const void* Xq, int M, int K, void* X6, void* stream);

/*
 * serq_linear_bf6 -- online, device memory, asynchronous on `stream`.
 *
 * serq_linear (W4A4) on bf6 operands: the same acc_main, acc_res (exact
 * integers) and the same fp32 epilogue, so Y and the debug accumulators are
 * bit-identical to serq_linear's on the same codes.
 *   X6         SERQ_BF6_BYTES(M, K) bytes from serq_act_bf6 (device).
 *   sx         M floats from serq_quant_act (device).
 *   W6, sw     SERQ_BF6_BYTES(N, K) bytes from serq_prepack_bf6 of Q(W^),
 *              and N floats (device).
 *   R6, sr     SERQ_BF6_BYTES(N, r) bytes from serq_prepack_bf6 of Q(R),
 *              and N floats (device); may be NULL when r == 0.
 *   M, K, N, r M >= 0 (0: no-op), K > 0 even, K <= 262144, N > 0,
 *              0 <= r <= min(K, 256), r even.
 *   Y, y_dtype, acc_main_dbg, acc_res_dbg  as for serq_linear.
 * Uses no scratch memory. Errors: SERQ_EINVAL (NULL pointer, bad sizes or
 * dtype, only one debug buffer), SERQ_EALIGN (pointer not 16-byte aligned),
 * SERQ_EHIP.
 */
int serq_linear_bf6(const void* X6, const float* sx,
                    const uint8_t* W6, const float* sw,
                    const uint8_t* R6, const float* sr,
                    int M, int K, int N, int r,
                    void* Y, serq_dtype y_dtype,
                    int32_t* acc_main_dbg, int32_t* acc_res_dbg,
                    void* stream);

/*
 * serq_linear_bf6_kernel_name -- which tile serq_linear_bf6 launches for M
 * tokens, N outputs and r salient rows (static string "bf6_tile128x128" or
 * "bf6_tile256x256"), or NULL for M <= 0, N <= 0 or r < 0. Host only;
 * launches nothing. For profiling and tests.
 */
const char* serq_linear_bf6_kernel_name(int M, int N, int r);

/*
 * The MXFP4 variant of the layer.
 *
 * The pages run SERQ on MXFP4 as well as INT4 (gist.science/de/paper/
 * 2603.08185, "Technische Zusammenfassung" 3: compatible with INT4 and
 * MXFP4; 4, Performance & Latenz: measured on hardware FP4 products, the
 * residual adding about 1 %). The format is OCP Microscaling (MX): blocks of
 * 32 consecutive elements along K share an E8M0 exponent e (stored as the
 * byte e + 127; the scale is 2^e), e = floor(log2(max |v|)) - 2 clamped to
 * [-127, 127] (-127 for an all-zero block); each element is the FP4 E2M1
 * value (sign bit 3, exponent bits 2-1 with bias 1, mantissa bit 0:
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) nearest to v / 2^e, ties to the
 * even mantissa, saturated at 6; a value that rounds to zero is code 0.
 * Codes are packed two per byte, element 2t in the low nibble. In the layer
 * the blocks run along K: per output column of W^, per token row of the
 * activations, per output column of R over its r rows (K and r multiples of
 * 32). s, P and W^ are those of serq_calibrate; R = W~_s - Q(W~_s) with the
 * MX quantizer's own dequantized salient rows, in fp32; Q(R) in MXFP4. The
 * block exponents are the only scales:
 *   Y[m, n] = sum over blocks b of 2^(ex_mb + ew_nb) sum_{k in b} x_mk w_nk
 *           + sum over the first r/32 blocks of 2^(ex_mb + er_nb) sum x_mk rho_nk.
 */

/*
 * serq_calibrate_mx -- offline, host memory, synchronous, deterministic.
 * As serq_calibrate, with MXFP4 outputs:
 *   Wq   N x K/2 bytes: column n of Q(W^), FP4 codes along K.
 *   Wsc  N x K/32 bytes: E8M0 exponent bytes of those blocks.
 *   Rq   N x r/2 bytes, Rsc N x r/32 bytes: Q(R) likewise (NULL when r == 0).
 * Errors: SERQ_EINVAL for NULL pointers, K or N <= 0, K or r not a multiple
 * of 32, r outside [0, K], alpha outside [0, 1], unknown w_dtype.
 */
int serq_calibrate_mx(const void* W, serq_dtype w_dtype, int K, int N,
                      const float* act_absmax, float alpha, int r,
                      int32_t* perm, float* s_hat_inv,
                      uint8_t* Wq, uint8_t* Wsc, uint8_t* Rq, uint8_t* Rsc);

/*
 * serq_quant_act_mx -- online, device memory, asynchronous on `stream`.
 * x^ = fl32(X[m, k] * s_hat_inv[k]) (X already in saliency order), then
 * MXFP4 per token row in blocks of 32 along K.
 *   X      M x K, SERQ_F32 or SERQ_BF16; K a multiple of 32.
 *   Xq     M x K/2 bytes of FP4 codes; Xsc M x K/32 exponent bytes.
 * M == 0 is a no-op. Errors: SERQ_EINVAL (NULL pointer, M < 0, K not a
 * positive multiple of 32, bad dtype), SERQ_EALIGN (X, Xq or s_hat_inv not
 * 16-byte aligned), SERQ_EHIP. Uses no scratch memory.
 */
int serq_quant_act_mx(const void* X, serq_dtype x_dtype, int M, int K,
                      const float* s_hat_inv, uint8_t* Xq, uint8_t* Xsc, void* stream);

/*
 * serq_linear_mx -- online, device memory, asynchronous on `stream`.
 * Y = acc_main + acc_res (the formula above) on gfx950's scaled FP4 matrix
 * instructions, whose operands are these codes and exponent bytes as
 * stored; one token (two when N < 16384) takes a dot-product kernel instead
 * (each 32-element block summed exactly, then scaled and added). Either way
 * accumulation is fp32 with one rounding per block (rounded, unlike the
 * integer layer) plus a fixed-order sum of partial sums; Y is stored as
 * y_dtype (bf16 with round to nearest even).
 *   Xq, Xsc    from serq_quant_act_mx; Wq, Wsc, Rq, Rsc from
 *              serq_calibrate_mx (Rq, Rsc may be NULL when r == 0).
 *   M, K, N, r M >= 0 (0: no-op), K > 0 and 0 <= r <= K multiples of 32,
 *              N > 0.
 *   acc_main_dbg, acc_res_dbg  NULL, or both device M x N floats that
 *              receive the two fp32 accumulators.
 * Uses no scratch memory. Errors: SERQ_EINVAL, SERQ_EALIGN (Xq, Wq, Rq, Y or
 * the debug buffers not 16-byte aligned), SERQ_EHIP.
 */
int serq_linear_mx(const uint8_t* Xq, const uint8_t* Xsc,
                   const uint8_t* Wq, const uint8_t* Wsc,
                   const uint8_t* Rq, const uint8_t* Rsc,
                   int M, int K, int N, int r,
                   void* Y, serq_dtype y_dtype,
                   float* acc_main_dbg, float* acc_res_dbg,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SERQ_H_ */
