/*
 * gemv_nibble_unpack.h -- C ABI of the MI355X (gfx950) low-bit-weight matmul
 * library.
 *
 * The library computes the mixed-precision product stated on the BitBLAS
 * practical-guide page, section "What is BitBLAS":
 *
 *     C[M,N] = A[M,K] x W[N,K]^T          (layout "nt": both K-contiguous)
 *
 * with W stored as 4-bit codes, two per byte (INT4 quantization page, Part 1
 * step 1 "storage"), or as 2-bit ternary codes, four per byte (BitBLAS page,
 * data-type table row INT8 x INT2 and the BitNet-b1.58 case), and A either
 * INT8 with a per-token scale (INT4 page, Part 1 steps 2-4: INT32 accumulate,
 * then multiply by weight_scale * activation_scale) or fp16 (BitBLAS page,
 * table row FP16 x INT4 with the group scales and zeros of "Advanced
 * features 2").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers unless stated otherwise, owned by
 *   the caller, row-major and dense. fp16 data is passed as uint16_t holding
 *   IEEE binary16 bit patterns.
 * - Every call is asynchronous on `stream` (NULL = the default stream). The
 *   library never allocates device memory, never synchronises, and holds no
 *   state besides its code objects and the process-wide table of pinned plans
 *   (w4_plan_pin; empty until a caller pins one).
 * - Every call validates its arguments before touching the GPU and returns
 *   W4_OK (0) or a negative status; nothing is launched when it fails.
 *   W4_ERR_HIP means the launch itself failed (hipGetLastError).
 * - Large buffers (W, Wq, Wp, A, Aq, C, codes, workspace) must be 16-byte
 *   aligned; small vectors (scales, zeros, bias, a_scale, rowsum) need their
 *   natural alignment.
 * - Sizes: N >= 1, K >= 1, M >= 1 (M = 0 is accepted by the matmul entry
 *   points and returns W4_OK without a launch). K is limited to W4_MAX_K =
 *   131056 so that INT32 accumulators cannot overflow for ANY int8 activation
 *   and ANY stored weight code: the kernels sum products scaled by 16 (4-bit
 *   codes) or 64 (2-bit codes), whose magnitude is at most 16 * 128 * 8 =
 *   64 * 128 * 2 = 128 * 128 = 16384, and 16384 * 131056 < 2^31 <= 16384 *
 *   131072 (the next multiple of 16 would overflow when every activation is
 *   -128 and every code is -8, -2 or -128).
 */
#ifndef GEMV_NIBBLE_UNPACK_H
#define GEMV_NIBBLE_UNPACK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define W4_OK             0
#define W4_ERR_NULL      -1   /* a required pointer is NULL                   */
#define W4_ERR_SHAPE     -2   /* a size is out of range / breaks a multiple   */
#define W4_ERR_ALIGN     -3   /* a pointer is not aligned as required         */
#define W4_ERR_ARG       -4   /* an enumerated argument has an unknown value  */
#define W4_ERR_WORKSPACE -5   /* workspace NULL or smaller than required      */
#define W4_ERR_HIP       -6   /* the HIP runtime rejected the launch          */
#define W4_ERR_SCRATCH   -7   /* needs more than the static scratch holds     */

/* ---- enumerations -------------------------------------------------------- */
/* weight schemes for quantize_pack_w4 */
#define W4_SYM_PER_CHANNEL 0  /* INT4 in [-7,7], float32 scale per row n      */
#define W4_ASYM_GROUP      1  /* uINT4 in [0,15], fp16 scale + uint8 zero per
                                 row n and group of 128 consecutive k         */
/* matmul output types */
#define W4_OUT_F16 0
#define W4_OUT_F32 1
#define W4_OUT_I32 2          /* the raw INT32 accumulators (A8 paths only)  */
#define W4_OUT_I8  3          /* INT8 re-quantized by an output scale (w8a8) */
/* activation input types for quantize_a8 */
#define W4_IN_F16 0
#define W4_IN_F32 1
/* prepacked weight layouts (what the matmul kernels read) */
#define W4_LAYOUT_W4A8  0     /* INT4 codes for the INT8-activation kernels   */
#define W4_LAYOUT_W4A16 1     /* uINT4 codes + group scales/zeros, fp16 acts  */
#define W4_LAYOUT_W2A8  2     /* ternary 2-bit codes, INT8 activations        */
#define W4_LAYOUT_W8A8  3     /* INT8 codes, INT8 activations                 */

#define W4_OP_W4A8  0         /* w4a8_gemm and w4a8_gemm_fused_act            */
#define W4_OP_W4A16 1         /* w4a16_gemm                                   */
#define W4_OP_W2A8  2         /* w2a8_gemm and w2a8_gemm_fused_act            */
#define W4_OP_W2A16 3         /* w2a16_gemm                                   */
#define W4_OP_W8A8  4         /* w8a8_gemm                                    */
#define W4_OP_F8F8  5         /* f8f8_gemm                                    */

#define W4_GROUP_SIZE 128
#define W4_MAX_K 131056
#define W4_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)  /* w4a8_gemm_fused_act_noalloc */

/* Human-readable text for a status code (static string, never NULL). */
const char* w4_status_string(int status);

/* ---- offline weight preparation ------------------------------------------ */

/*
 * quantize_pack_w4 -- quantize float32 weights to 4-bit codes and pack them.
 *
 * W4_SYM_PER_CHANNEL (INT4 page, Part 1 step 1, with the INT4 range):
 *   s[n] = max_k |W[n,k]| / 7 (float32 division), q = clip(rint(W / s[n]),
 *   -7, 7) with round-half-to-even; s[n] == 0 gives q = 0.
 *   `scales` is float32[N]; `zeros` must be NULL; group_size must be -1.
 * W4_ASYM_GROUP (BitBLAS page, "Advanced features 2", zeros_mode original):
 *   per group g of 128 consecutive k: s = fp16((max - min) / 15), then with
 *   sf = float(s): z = clip(rint(-min / sf), 0, 15), q = clip(rint(W / sf) + z,
 *   0, 15); sf == 0 gives q = z = 0. Reconstruction is (q - z) * s.
 *   `scales` is fp16[N, K/128]; `zeros` is uint8[N, K/128]; group_size = 128;
 *   K must be a multiple of 128.
 * Packing (both): Wq[n, j] = (q[n,2j] & 15) | (q[n,2j+1] & 15) << 4, i.e.
 *   even k in the low nibble, signed codes as two's complement. Wq is
 *   uint8[N, K/2]; K must be even. W must be finite.
 */
int quantize_pack_w4(const float* W, int N, int K, int scheme, int group_size,
                     uint8_t* Wq, void* scales, uint8_t* zeros, hipStream_t stream);

/*
 * quantize_pack_w2 -- pack ternary codes four per byte (BitBLAS page,
 * data-type table row INT8 x INT2; BitNet-b1.58 case).
 *   Wq[n, j] = sum_i (codes[n,4j+i] & 3) << 2i (2-bit two's complement:
 *   1 -> 01, 0 -> 00, -1 -> 11). codes is int8[N,K] with values in [-2,1];
 *   Wq is uint8[N, K/4]; K must be a multiple of 4.
 */
int quantize_pack_w2(const int8_t* codes, int N, int K, uint8_t* Wq, hipStream_t stream);

/*
 * ternary_scale_f16 -- per-tensor scale of a ternary weight: fp16 of the mean
 * absolute value of the float32 source (summed in float64, rounded once to
 * fp16, half-to-even). Writes one fp16 value to the DEVICE pointer scale.
 * count >= 1.
 */
int ternary_scale_f16(const float* src, int64_t count, uint16_t* scale, hipStream_t stream);

/*
 * prepack_bytes -- size in bytes of the prepacked buffer for a layout, or 0 if
 * the arguments are invalid. The prepacked buffer is opaque: it holds the
 * codes in the order the kernels stream them (16 rows x 128 k per 1 KiB tile
 * for 4-bit codes, 16 rows x 256 k for 2-bit), padded with zero codes to whole
 * tiles, and for W4_LAYOUT_W4A16 also the group scales and zeros.
 * This is the offline "compressed format" of the BitBLAS page (performance
 * advice 2): the weight is transformed once so no work is spent at run time.
 */
size_t prepack_bytes(int layout, int N, int K);

/*
 * prepack_w -- canonical packed codes -> prepacked buffer Wp.
 *   W4_LAYOUT_W4A8 : Wq uint8[N,K/2] (signed INT4); scales, zeros unused
 *                    (pass NULL); K multiple of 16.
 *   W4_LAYOUT_W4A16: Wq uint8[N,K/2] (uINT4), scales fp16[N,K/128], zeros
 *                    uint8[N,K/128]; K multiple of 128.
 *   W4_LAYOUT_W2A8 : Wq uint8[N,K/4]; scales, zeros unused; K multiple of 16.
 *   W4_LAYOUT_W8A8 : Wq int8[N,K] (from quantize_pack_w8), tiles of 16 rows x
 *                    64 k, bytes in k order; scales, zeros unused.
 * Wp must hold prepack_bytes(layout, N, K) bytes.
 */
int prepack_w(int layout, const uint8_t* Wq, const void* scales, const uint8_t* zeros,
              int N, int K, uint8_t* Wp, hipStream_t stream);

/* unprepack_w -- exact inverse of prepack_w (for checking a layout). */
int unprepack_w(int layout, const uint8_t* Wp, int N, int K, uint8_t* Wq, void* scales,
                uint8_t* zeros, hipStream_t stream);

/* ---- per-call activation quantization ------------------------------------- */

/*
 * quantize_a8 -- per-token dynamic INT8 activations (INT4 page, Part 1 step 2):
 *   a_scale[m] = max_k |A[m,k]| / 127 (float32; fp16 input widened exactly),
 *   Aq = clip(rint(A / a_scale[m]), -127, 127) (half-to-even; a_scale == 0
 *   gives 0), rowsum[m] = sum_k Aq[m,k] (int32; pass NULL to skip).
 *   A is fp16 or float32 [M,K] per in_dtype; Aq is int8[M,K]; K multiple of 8.
 */
int quantize_a8(const void* A, int in_dtype, int M, int K, int8_t* Aq, float* a_scale,
                int32_t* rowsum, hipStream_t stream);

/* ---- the matmul ------------------------------------------------------------ */

/*
 * w4_workspace_bytes -- device workspace a matmul call needs (0 if none), for
 * the op that owns the layout (W4A8, W4A16, W2A8, W8A8); w2a16_gemm and
 * f8f8_gemm share a layout with another op and use w4_plan_workspace_bytes.
 * The workspace must be zero-filled once before its first use; every call
 * leaves the part it relies on zero again, so the same buffer can be reused
 * by later calls on the same stream, whatever their shapes and plans: its
 * first 16 KiB only ever hold split-K arrival counters (zero between calls),
 * and every byte past them is scratch that a call writes before it reads.
 * Calls that overlap in time must not share a workspace.
 */
size_t w4_workspace_bytes(int layout, int M, int N, int K);

/*
 * w4a8_gemm -- INT8 activations x symmetric INT4 weights (INT4 page, Part 1
 * steps 3-4):
 *   acc[m,n] = sum_k Aq[m,k] * q[n,k]  (exact INT32),
 *   W4_OUT_I32: C = acc (int32[M,N]);
 *   W4_OUT_F32: C = acc * w_scale[n] * a_scale[m] (float32[M,N]);
 *   W4_OUT_F16: C = fp16(acc * w_scale[n] * a_scale[m] + bias[n]) (fp16[M,N]).
 *   Aq int8[M,K]; a_scale float32[M]; Wp from prepack_w(W4_LAYOUT_W4A8);
 *   w_scale float32[N]; bias fp16[N] or NULL (ignored for W4_OUT_I32).
 *   K multiple of 16. Small M runs the decode GEMV kernel (or the skinny
 *   kernel, when the rows would be re-read too often), large M the LDS-tiled
 *   MFMA GEMM kernel; the plan table at the end of this header lists and pins
 *   the choices per shape.
 */
int w4a8_gemm(const int8_t* Aq, const float* a_scale, const uint8_t* Wp, const float* w_scale,
              const uint16_t* bias, void* C, int out_dtype, int M, int N, int K,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * w2a8_gemm -- INT8 activations x ternary 2-bit weights with one per-tensor
 * fp16 scale (device pointer w_scale16, e.g. from ternary_scale_f16). Same
 * outputs as w4a8_gemm with w_scale[n] replaced by the tensor scale. Wp from
 * prepack_w(W4_LAYOUT_W2A8). K multiple of 16.
 */
int w2a8_gemm(const int8_t* Aq, const float* a_scale, const uint8_t* Wp,
              const uint16_t* w_scale16, const uint16_t* bias, void* C, int out_dtype,
              int M, int N, int K, void* workspace, size_t workspace_bytes,
              hipStream_t stream);

/*
 * w4a16_gemm -- fp16 activations x group-128 uINT4 weights (BitBLAS page,
 * table row FP16 x INT4; "Advanced features 2"):
 *   C[m,n] = fp16( sum_g s[n,g] * sum_{k in g} A[m,k] * (q[n,k] - z[n,g])
 *                  + bias[n] ),
 *   accumulated in float32. A fp16[M,K]; Wp from prepack_w(W4_LAYOUT_W4A16)
 *   (it carries the scales and zeros); group_size must be 128; bias fp16[N]
 *   or NULL; C fp16[M,N]. K multiple of 128.
 */
int w4a16_gemm(const uint16_t* A, const uint8_t* Wp, int group_size, const uint16_t* bias,
               uint16_t* C, int M, int N, int K, void* workspace, size_t workspace_bytes,
               hipStream_t stream);

/*
 * w2a16_gemm -- fp16 activations x ternary 2-bit weights (BitBLAS page,
 * data-type table row FP16 x INT2, on the ternary weights of the BitNet-b1.58
 * case):
 *   C[m,n] = fp16( s * sum_k A[m,k] * c[n,k] + bias[n] ), float32 sums,
 *   A fp16[M,K]; Wp from prepack_w(W4_LAYOUT_W2A8) -- the same prepacked
 *   buffer w2a8_gemm reads; w_scale16 the per-tensor fp16 scale s (device
 *   pointer); bias fp16[N] or NULL; C fp16[M,N]. K multiple of 16. Runs
 *   the decode kernel over 16-row tiles, or the skinny kernel when many
 *   16-row tiles share few columns or the rows would be re-read too often.
 *   Its workspace size is w4_plan_workspace_bytes(W4_OP_W2A16, M, N, K) (its
 *   plan can differ from w2a8_gemm's on the same layout).
 */
int w2a16_gemm(const uint16_t* A, const uint8_t* Wp, const uint16_t* w_scale16,
               const uint16_t* bias, uint16_t* C, int M, int N, int K, void* workspace,
               size_t workspace_bytes, hipStream_t stream);

/*
 * quantize_pack_w8 -- symmetric per-output-channel INT8 weights (INT4 page,
 * Part 1 step 1 as printed there, with the INT8 range: scale = max|w| / 127,
 * code = round(w / scale) clipped to [-127, 127]; float32 division, round
 * half to even):
 *   W float32[N,K] -> Wq int8[N,K], scales float32[N]. K multiple of 16.
 *   Wq goes through prepack_w(W4_LAYOUT_W8A8).
 */
int quantize_pack_w8(const float* W, int N, int K, int8_t* Wq, float* scales,
                     hipStream_t stream);

/*
 * w8a8_gemm -- INT8 activations x INT8 weights (BitBLAS page, data-type table
 * row INT8 x INT8, INT32 accumulation, INT8 output; INT4 page, Part 1 step 3:
 * the INT32 result either dequantized or handed to a following quantized
 * layer):
 *   acc[m,n] = sum_k Aq[m,k] * q[n,k] (exact INT32; K <= W4_MAX_K keeps it
 *   in range), then as w4a8_gemm for W4_OUT_I32 / W4_OUT_F32 / W4_OUT_F16, and
 *   W4_OUT_I8: v = float32(float32(float32(acc) * w_scale[n]) * a_scale[m]),
 *   C = clip(rint(v / out_scale[0]), -127, 127) (int8[M,N]; float32 division,
 *   half to even; an out_scale of 0 gives 0), bias must be NULL.
 *   Wp from prepack_w(W4_LAYOUT_W8A8); out_scale a device float32[1] (may be
 *   NULL unless W4_OUT_I8). Every M runs the decode or skinny kernels.
 */
int w8a8_gemm(const int8_t* Aq, const float* a_scale, const uint8_t* Wp, const float* w_scale,
              const uint16_t* bias, const float* out_scale, void* C, int out_dtype, int M, int N,
              int K, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * quantize_f8 -- per-row FP8 E4M3 quantization (BitBLAS page, data-type
 * table row FP8_E4M3 x FP8_E4M3; the format is the OCP E4M3: bias 7, 3
 * mantissa bits, subnormals, largest magnitude 448, no infinities). For each
 * of `rows` rows of X [rows,K] (fp16 with in_dtype W4_IN_F16, float32 with
 * W4_IN_F32; device, 16-byte aligned): scale = max|x| / 448 (float32),
 * code = E4M3(x / scale) with a float32 division, rounded to nearest with
 * ties to the even code, sign kept, saturated at 448; a zero row gets scale
 * 0 and codes 0. Serves both operands: weights per output channel (then
 * prepack_w(W4_LAYOUT_W8A8, ...), the INT8 byte-tile layout) and activations
 * per token. Xq uint8 [rows,K] (16-byte aligned), scales float32 [rows].
 * K multiple of 16. W4_ERR_ARG for an unknown in_dtype.
 */
int quantize_f8(const void* X, int in_dtype, int rows, int K, uint8_t* Xq, float* scales,
                hipStream_t stream);

/*
 * f8f8_gemm -- FP8 x FP8 (BitBLAS page, data-type table row FP8_E4M3 x
 * FP8_E4M3: float32 accumulation, fp16 output):
 *   C[m,n] = out( a_scale[m] * w_scale[n] * sum_k a[m,k] * w[n,k] + bias[n] )
 * Aq uint8 [M,K] E4M3 codes and a_scale float32 [M] from quantize_f8; Wp
 * from prepack_w(W4_LAYOUT_W8A8) of E4M3 weight codes, w_scale float32 [N].
 * out_dtype W4_OUT_F16 (bias applied) or W4_OUT_F32 (bias ignored). K
 * multiple of 16. M <= 16 (and small grids) run the decode kernel; more rows
 * run the tiled GEMM (128 x 128 blocks on v_mfma_f32_16x16x128_f8f6f4, the
 * whole K per block) once it has at least 128 blocks, else the skinny kernel.
 * Workspace: w4_plan_workspace_bytes(W4_OP_F8F8, M, N, K). Errors as
 * w8a8_gemm.
 */
int f8f8_gemm(const uint8_t* Aq, const float* a_scale, const uint8_t* Wp, const float* w_scale,
              const uint16_t* bias, void* C, int out_dtype, int M, int N, int K, void* workspace,
              size_t workspace_bytes, hipStream_t stream);

/*
 * w4_fused_act_workspace_bytes -- device workspace w4a8_gemm_fused_act
 * (layout W4_LAYOUT_W4A8) or w2a8_gemm_fused_act (W4_LAYOUT_W2A8) needs, 0 if
 * none. Same zero-fill and sharing rules as w4_workspace_bytes; the buffer
 * must be 256-byte aligned.
 */
size_t w4_fused_act_workspace_bytes(int layout, int M, int N, int K);

/*
 * w4a8_gemm_fused_act -- quantize_a8 followed by w4a8_gemm in one call
 * (INT4 page, Part 1 steps 2-4: dynamic per-token INT8 activations, INT8 x
 * INT4 products summed in INT32, dequantization): the outputs are identical,
 * bit for bit, to those two calls. A holds fp16 (in_dtype W4_IN_F16) or
 * float32 (W4_IN_F32) rows [M,K], 16-byte aligned; the other arguments are
 * those of w4a8_gemm. Decode shapes whose rows fit the kernel's LDS staging
 * quantize in the matmul kernel's prologue (one launch, no int8 copy of A in
 * memory); other shapes quantize into the workspace first (two launches).
 * Errors as w4a8_gemm, plus W4_ERR_ARG for an unknown in_dtype.
 */
int w4a8_gemm_fused_act(const void* A, int in_dtype, const uint8_t* Wp, const float* w_scale,
                        const uint16_t* bias, void* C, int out_dtype, int M, int N, int K,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * w4a8_gemm_fused_act_noalloc -- w4a8_gemm_fused_act without a workspace,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Same
 * arguments (minus the workspace), same kernels, same outputs bit for bit.
 * The scratch the call needs (w4_fused_act_workspace_bytes(W4_LAYOUT_W4A8,
 * M, N, K): split-K counters and partial sums, and for shapes that quantize
 * in a separate launch the int8 rows and their scales) is a static device
 * array of W4_NOALLOC_SCRATCH_BYTES (32 MiB) inside the library; every GPU
 * the library runs on holds its own copy until the process ends. Nothing is
 * allocated, nothing freed. A shape that needs more scratch than that (e.g.
 * M * K above about 33.5 million with the two-launch form) returns
 * W4_ERR_SCRATCH before any GPU work. Every call on one GPU shares that
 * GPU's array and leaves its counter area zero; calls that overlap in time on
 * one GPU (several streams, or several threads) race on it and must not be
 * issued.
 */
int w4a8_gemm_fused_act_noalloc(const void* A, int in_dtype, const uint8_t* Wp,
                                const float* w_scale, const uint16_t* bias, void* C, int out_dtype,
                                int M, int N, int K, hipStream_t stream);

/*
 * w2a8_gemm_fused_act -- quantize_a8 followed by w2a8_gemm in one call, as
 * w4a8_gemm_fused_act with the ternary weights and per-tensor fp16 scale of
 * w2a8_gemm.
 */
int w2a8_gemm_fused_act(const void* A, int in_dtype, const uint8_t* Wp,
                        const uint16_t* w_scale16, const uint16_t* bias, void* C, int out_dtype,
                        int M, int N, int K, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* ---- plan table ---------------------------------------------------------
 * A shape-keyed table of launch plans, after the KoGPT FasterTransformer
 * page, section 2.3 (GEMM tuning per matrix shape, with its table of the best
 * algorithm and tile per (M, N, K), and the advice to re-tune per GPU).
 *
 * Every matmul call runs one of several plans that compute the same result:
 * the decode kernel or the skinny kernel, each at one of its k splits, or
 * (INT8 activations, M > 16) the tiled GEMM at one of its block shapes (the
 * ternary 128 x 128 block also at each of its k splits). Without a
 * pin the library picks one from the shape (built-in choice). A caller that
 * has timed the candidates (the Python package's tune module does) pins the
 * fastest per (op, M, N, K); every later call of that op and shape, on any
 * device and stream of the process, then uses it. Results do not depend on
 * the plan: INT32 accumulators and INT8 outputs are identical across plans;
 * floating-point outputs differ only by the order of the k-split reduction.
 *
 * The table is guarded by a mutex and may be changed from any thread. A pin
 * changes what w4_workspace_bytes and w4_fused_act_workspace_bytes return for
 * its shape: query them after pinning. A call whose workspace is too small for
 * the plan in force fails with W4_ERR_WORKSPACE, as usual.
 *
 * `op` is one of W4_OP_*; M >= 1, N and K as the op's matmul entry point
 * (K a multiple of 16, or of 128 for W4_OP_W4A16). Each of these calls returns
 * W4_ERR_ARG for an unknown op and W4_ERR_SHAPE for a size out of range.
 */

/* Number of candidate plans for the shape (>= 1), or a negative status. The
 * list and its order are fixed for a given (op, M, N, K) and library build. */
int w4_plan_count(int op, int M, int N, int K);

/* Writes the name of candidate `index` (NUL-terminated, at most len bytes,
 * host memory) to buf: "decode:ksplit=S", "decode:ksplit=S,waves=W" (W = 4 or
 * 16 waves per block instead of 8), "skinny", "skinny:ksplit=S",
 * "skinny:rows=32", "skinny:rows=32,ksplit=S", "gemm:RxC" or
 * "gemm:RxC,ksplit=S" (R rows x C columns per block, K split S ways).
 * W4_ERR_NULL for buf NULL; W4_ERR_ARG for an index out of range or a buffer
 * too small. */
int w4_plan_name(int op, int M, int N, int K, int index, char* buf, size_t len);

/* Pins candidate `index` for the shape; index -1 removes the shape's pin. */
int w4_plan_pin(int op, int M, int N, int K, int index);

/* Index of the candidate a call with this shape would run now (pinned or
 * built-in), or a negative status. */
int w4_plan_current(int op, int M, int N, int K);

/* Removes every pin. Always returns W4_OK. */
int w4_plan_reset(void);

/* Workspace bytes a call of `op` with this shape needs under the plan in
 * force now (0 if none, or if an argument is invalid). For the ops with a
 * layout of their own this equals w4_workspace_bytes of that layout;
 * W4_OP_W2A16 needs this query, since it shares the W2A8 layout but not the
 * W2A8 op's pin. */
size_t w4_plan_workspace_bytes(int op, int M, int N, int K);

/* ---- measurement aid -------------------------------------------------------
 * w4_read_probe -- read `bytes` of device memory at `buf` once with 16-byte
 * loads and do nothing else (`per` = 1, 2, 4 or 8 loads per lane, all issued
 * before any is used; 256 lanes per block; every wave instruction reads 1 KiB
 * contiguous). Not a step of the matmul: the INT4 page's T4 discussion names
 * memory bandwidth as what a weight-streaming GEMV is bound by, and this is
 * the plain streaming read that such a kernel of the same size is measured
 * against (the read rate the chip reaches for that transfer, launch and drain
 * included). `sink` is a device uint32[1024]; the kernel writes it only when
 * the XOR of a block's data equals a fixed constant, which keeps the loads
 * from being removed. bytes >= 16 and a multiple of 16; buf 16-byte aligned;
 * W4_ERR_ARG for another `per`.
 */
int w4_read_probe(const void* buf, size_t bytes, int per, uint32_t* sink, hipStream_t stream);

/* ---- decode-step graphs --------------------------------------------------
 * After the INT4 quantization page, Part 2 (steps 2-4): the kernel launches of
 * a decode step are captured once from a stream, instantiated, and launched
 * as one graph per step; before a launch the graph's kernel-node parameters
 * are updated so that the captured step reads and writes the current step's
 * buffers (the page's cudaGraphExecKernelNodeSetParams).
 *
 * w4_graph_begin starts capturing `stream` (a stream created by the caller;
 * thread-local capture mode). Matmul calls issued on it are recorded, not run
 * (their argument checks still run and can fail; a workspace must already be
 * allocated, since nothing may be allocated while capturing).
 * w4_graph_end ends the capture and instantiates it into *out (host handle,
 * owned by the caller until w4_graph_destroy).
 * w4_graph_update ends a capture begun again with w4_graph_begin, in which
 * the caller issued the same sequence of calls with other pointers, and gives
 * every kernel node of `graph` the parameters of the node at the same position
 * (in dependency order) of the new capture. All nodes must launch the same
 * kernels with the same grid, block and LDS size (same shapes and plans);
 * otherwise W4_ERR_ARG and the graph is left as it was. The new capture is
 * discarded either way.
 * w4_graph_launch launches the graph on `stream` (any stream of the device).
 * w4_graph_kernel_nodes returns the number of kernel nodes (>= 0).
 * w4_graph_destroy frees the graph (NULL is a no-op).
 * Errors: W4_ERR_NULL for a NULL handle, output pointer or (begin, end,
 * update) stream; W4_ERR_HIP when the runtime refuses a capture, instantiation
 * or update (the capture is then ended and discarded). A graph's launches on
 * one stream run in order; launching it on two streams at once races on its
 * buffers and workspaces like any other pair of calls.
 */
typedef struct w4_graph_s* w4_graph_t;
int w4_graph_begin(hipStream_t stream);
int w4_graph_end(hipStream_t stream, w4_graph_t* out);
int w4_graph_update(w4_graph_t graph, hipStream_t stream);
int w4_graph_launch(w4_graph_t graph, hipStream_t stream);
int w4_graph_kernel_nodes(w4_graph_t graph);
int w4_graph_destroy(w4_graph_t graph);

#ifdef __cplusplus
}
#endif

#endif /* GEMV_NIBBLE_UNPACK_H */
