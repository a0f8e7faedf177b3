/*
 * nvfp4.h - C ABI of the MI355X (gfx950) NVFP4 W4A4 linear-layer library.
 *
 * The library computes one NVFP4 W4A4 linear layer: activations are quantized
 * to NVFP4 on the fly and multiplied against pre-quantized, pre-swizzled NVFP4
 * weights with FP32 accumulation.  This is the operation the pages apply to
 * every linear layer of the hybrid Gated DeltaNet model ("Why Gated DeltaNet
 * Survives 4-Bit Quantization: NVFP4 W4A4 for the Recurrent Half of a Hybrid
 * 27B LLM", section "Performance and Efficiency Gains": weights and
 * activations in NVFP4 on all 496 linear layers) and to nGPT's dot products
 * ("Normalized Architectures are Natively 4-Bit", section "Approach").
 *
 * NVFP4 tensor (canonical layout, used for every input and output of this ABI
 * except the packed weight blob):
 *   - codes  : uint8 [rows][K/2]; byte j of a row holds element 2j in its low
 *              nibble and element 2j+1 in its high nibble; each nibble is an
 *              E2M1 code (bit 3 sign, bits 2..1 exponent with bias 1, bit 0
 *              mantissa; magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6).
 *   - scales : uint8 [rows][K/16]; one E4M3 ("FN": bias 7, max 448, no
 *              infinities) scale per 16 consecutive elements along K
 *              (blocks of 16: section "Why the 'Fragile' Recurrence is
 *              Actually Robust" of the Gated DeltaNet page).
 *   - g      : one FP32 per-tensor (per-module) global scale.
 *   value(row, k) = e2m1(code) * e4m3(scale[row][k/16]) * g.
 *
 * Conventions for every entry point:
 *   - All tensor arguments are device pointers to caller-owned memory.  The
 *     library never allocates or frees device memory and keeps no state
 *     between calls apart from a thread-local error message.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All device work is enqueued asynchronously on it; nothing synchronizes.
 *   - Arguments are validated on the host before any HIP call.  On error no
 *     work is enqueued, a status other than NVFP4_OK is returned and
 *     nvfp4_last_error() describes it.  No C++ exception crosses the ABI.
 *   - Input values must be finite.  NaN or infinity in an input is outside
 *     the contract (the outputs are then unspecified but no memory outside
 *     the given buffers is touched).
 *   - The functions are thread-safe; calls that share output buffers must be
 *     ordered by the caller.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 1

typedef enum nvfp4_status {
    NVFP4_OK = 0,
    NVFP4_ERR_INVALID_ARG = 1, /* null pointer or unknown enum value */
    NVFP4_ERR_SHAPE = 2,       /* negative size, K not a multiple of 16, leading dimension too small */
    NVFP4_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace_bytes query */
    NVFP4_ERR_UNSUPPORTED = 4, /* well-formed request outside what the kernels handle (documented per call) */
    NVFP4_ERR_NO_DEVICE = 5,   /* no gfx950 GPU is visible */
    NVFP4_ERR_HIP = 6,         /* a HIP runtime call failed; nvfp4_last_error() has its message */
    NVFP4_ERR_DESCRIPTOR = 7   /* weight descriptor has a wrong magic/version or inconsistent fields */
} nvfp4_status;

/* Element type of an unquantized input tensor. */
typedef enum nvfp4_in_dtype {
    NVFP4_IN_F32 = 0,
    NVFP4_IN_BF16 = 1
} nvfp4_in_dtype;

/* How the per-tensor global scale g is obtained. */
typedef enum nvfp4_g_mode {
    /* g = fl32(amax / 2688) from the tensor's largest magnitude (g = 1 for an
     * all-zero tensor, floored at 2^-100), written to *g.  2688 = 6 * 448 puts
     * the largest element of the tensor on code 6 of a block scaled by 448. */
    NVFP4_G_COMPUTE = 0,
    /* g is read from *g (finite, positive, normal FP32).  With g = 1 this is
     * NVFP4 without per-tensor scaling ("Normalized Architectures are
     * Natively 4-Bit", sections "Problem" and "Approach"); with a calibrated
     * value it is the per-module calibrated scale of the Gated DeltaNet page
     * ("Critical Lessons for Model Serving"). */
    NVFP4_G_GIVEN = 1
} nvfp4_g_mode;

/* Element type of the product's output Y. */
typedef enum nvfp4_out_dtype {
    NVFP4_OUT_F32 = 0,
    /* bf16, rounded to nearest (ties to even) from the FP32 value the F32
     * output would hold: half the bytes for a projection whose consumer reads
     * bf16 (the GDN recurrence after the fused input projection). */
    NVFP4_OUT_BF16 = 1
} nvfp4_out_dtype;

/* Library ABI version (NVFP4_ABI_VERSION of the build). */
int nvfp4_abi_version(void);

/* Message describing the last error returned on the calling thread ("" if none). */
const char* nvfp4_last_error(void);

/* NVFP4_OK if a gfx950 device is current, NVFP4_ERR_NO_DEVICE otherwise. */
nvfp4_status nvfp4_device_check(void);

/* ---------------------------------------------------------------------------
 * Quantize: unquantized [rows][K] tensor -> canonical NVFP4 (codes, scales, g).
 *
 * Per tensor: amax = max |x|, g as in nvfp4_g_mode, s_enc = fl32(1/g).
 * Per 16-element block along K: bamax = max |x|, S = E4M3 nearest to
 * fl32(fl32(bamax * s_enc) / 6) (ties to even, saturating at 448).
 * Per element: q = fl32(x * r) with r = fl32(s_enc / S) (r = 0 when S = 0),
 * code = sign(q) | E2M1 magnitude nearest to |q| (ties to even, saturating
 * at 6; the sign bit is kept when the magnitude rounds to 0).
 * All of it in IEEE FP32 with one rounding per operation, so codes and scales
 * are a deterministic function of the input.
 *
 * x        : device, rows x K elements of in_dtype, row r at x + r*ld_x elements
 * rows     : >= 0 (rows == 0 is an empty tensor: g = 1 in COMPUTE mode)
 * K        : > 0, multiple of 16
 * ld_x     : >= K
 * codes    : device, rows * K/2 bytes, written (dense, row stride K/2)
 * scales   : device, rows * K/16 bytes, written (dense, row stride K/16)
 * g        : device, one float; written in COMPUTE mode, read in GIVEN mode
 * workspace: device, >= nvfp4_quantize_workspace_bytes(rows, K) bytes
 *            (may be NULL when that is 0); contents need no initialisation.
 *            It holds the per-workgroup maxima of the call (tagged with the
 *            launch where the workgroups exchange them), so calls that may run
 *            concurrently must not share a workspace.
 * ------------------------------------------------------------------------- */
size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t K);
nvfp4_status nvfp4_quantize(const void* x, int in_dtype, int64_t rows, int64_t K, int64_t ld_x,
                            uint8_t* codes, uint8_t* scales, float* g, int g_mode,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Quantize along the other axis: unquantized [rows][cols] tensor x ->
 * canonical NVFP4 encoding of its transpose x^T ([cols][rows], blocks of 16
 * consecutive rows of x).
 *
 * End-to-end NVFP4 training ("Normalized Architectures are Natively 4-Bit",
 * abstract and section "Approach") also runs the backward products in NVFP4:
 * dX = dY * W contracts over W's rows and dW = dY^T * X over the token axis,
 * so W, dY and X each need the encoding of their transpose.  The result is
 * bit for bit nvfp4_quantize of x^T: same g (the amax does not depend on the
 * orientation), same block rule, same per-element rule.
 *
 * x        : device, rows x cols elements of in_dtype, row r at x + r*ld_x;
 *            aligned to the element size (rows that start on 16-byte
 *            boundaries are read with vector loads, others element by element)
 * rows     : >= 0, multiple of 16 (the blocked axis)
 * cols     : >= 0 (rows == 0 or cols == 0: empty; g = 1 in COMPUTE mode)
 * ld_x     : >= cols
 * codes    : device, 8-byte aligned, cols * rows/2 bytes, written ([cols][rows/2])
 * scales   : device, cols * rows/16 bytes, written ([cols][rows/16])
 * g        : device, one float; written in COMPUTE mode, read in GIVEN mode
 * workspace: device, >= nvfp4_quantize_workspace_bytes(rows, cols) bytes in
 *            COMPUTE mode (may be NULL in GIVEN mode); no initialisation needed
 * Errors: NVFP4_ERR_SHAPE for a bad rows/cols/ld_x, NVFP4_ERR_UNSUPPORTED for
 * misaligned pointers or strides, NVFP4_ERR_WORKSPACE for a short workspace;
 * nothing is launched then.
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_quantize_t(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                              uint8_t* codes, uint8_t* scales, float* g, int g_mode,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Both orientations from one read: nvfp4_quantize of x and nvfp4_quantize_t
 * of x with one g, bit for bit, reading x once (a training step needs dY
 * along N for dX = dY . W and along the tokens for dW = dY^T . X; the
 * "Normalized Architectures are Natively 4-Bit" page trains end to end in
 * NVFP4, abstract and section "Approach").
 *
 * x        : as for nvfp4_quantize_t (aligned to the element size)
 * rows,cols: >= 0, both multiples of 16
 * codes    : [rows][cols/2], 4-byte aligned; scales [rows][cols/16]
 * codes_t  : [cols][rows/2], 8-byte aligned; scales_t [cols][rows/16]
 * g, g_mode, workspace: as for nvfp4_quantize (nvfp4_quantize_workspace_bytes(rows, cols))
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_quantize_both(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                 uint8_t* codes, uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t,
                                 float* g, int g_mode, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Quantize behind a randomized Hadamard transform (RHT).
 *
 * Standard transformers trained in NVFP4 apply random Hadamard transforms
 * before quantization; nGPT trains without them ("Normalized Architectures
 * are Natively 4-Bit", sections "Problem" and "Approach").  Each 16-element
 * block along the quantization axis becomes v' = H16 . D . v / 4 (D negates
 * element i of every block when bit i of signs is set; H16 in natural order;
 * FP32 butterflies in the stage order h = 1, 2, 4, 8), and v' is quantized
 * exactly as nvfp4_quantize does, with g computed from the amax of the
 * transformed tensor in COMPUTE mode.  The transform is orthogonal, so the
 * product of two operands transformed with the same signs needs no change:
 * quantize both with the same mask and call nvfp4_gemm as usual.
 *
 * nvfp4_quantize_rht   : arguments of nvfp4_quantize, plus signs
 * nvfp4_quantize_t_rht : arguments of nvfp4_quantize_t, plus signs (blocks of
 *                        16 rows of x, for the backward products)
 * signs : 16-bit mask (the random draw is the caller's); larger values give
 *         NVFP4_ERR_INVALID_ARG.  Workspace sizes: nvfp4_quantize_workspace_bytes.
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_quantize_rht(const void* x, int in_dtype, int64_t rows, int64_t K, int64_t ld_x,
                                uint32_t signs, uint8_t* codes, uint8_t* scales, float* g, int g_mode,
                                void* workspace, size_t workspace_bytes, void* stream);
nvfp4_status nvfp4_quantize_t_rht(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                  uint32_t signs, uint8_t* codes, uint8_t* scales, float* g, int g_mode,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * FP8 KV cache: E4M3 bytes with one calibrated FP32 scale per tensor.
 *
 * The Gated DeltaNet page ("Why Gated DeltaNet Survives 4-Bit Quantization",
 * section "Critical Lessons for Model Serving") credits calibrated FP8 scales
 * on the KV cache with recovering most of the long-context loss.  Per tensor (a layer's
 * K or V cache, [rows][cols] = [tokens][heads * head_dim]): s given (a
 * calibrated value, s_mode NVFP4_G_GIVEN) or calibrated on the tensor itself
 * (NVFP4_G_COMPUTE: s = fl32(amax / 448), 1 for an all-zero tensor, floored at
 * 2^-100, written to *scale).  Per element: q = fl32(x * fl32(1/s)), byte =
 * sign of q (bit 7) | E4M3 "FN" magnitude nearest to |q| (bias 7, ties to the
 * even byte, saturating at 448; the sign is kept when the magnitude is 0);
 * a NaN gives 0x7F with its sign.  The dequantized value is e4m3(byte) * s.
 *
 * x        : device, rows x cols elements of in_dtype, row r at x + r*ld_x,
 *            aligned to the element size
 * rows,cols: >= 0 (either 0: empty; s = 1 in COMPUTE mode)
 * codes    : device, rows * cols bytes, written dense ([rows][cols])
 * scale    : device, one float; written in COMPUTE mode, read in GIVEN mode
 *            (finite and positive)
 * workspace: COMPUTE mode only, >= nvfp4_quantize_workspace_bytes(rows, cols)
 * Errors as for nvfp4_quantize; nothing is launched on an error.
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_kv_quantize_fp8(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                   uint8_t* codes, float* scale, int s_mode, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Packed weights.
 *
 * A projection is a stack of n_modules sub-modules (e.g. q,k,v,z,a,b of a
 * Gated DeltaNet input projection) sharing one input.  Each sub-module was
 * quantized on its own and keeps its own global scale g_w[s]: fused kernels
 * must not apply one module's scale to another (section "Critical Lessons for
 * Model Serving" of the Gated DeltaNet page).  Output column n of the fused
 * GEMM belongs to the module whose row range holds n and is scaled by that
 * module's g.
 *
 * The blob is opaque device memory holding a header, the codes and scales
 * rearranged into tiles that load straight into MFMA operand registers, and
 * one FP32 column scale per output row.  The descriptor is a host struct,
 * filled by nvfp4_pack_weights and passed by pointer to the GEMM; it holds the
 * device address of the blob, so the blob must outlive its use.
 * ------------------------------------------------------------------------- */
#define NVFP4_MAX_MODULES 16
#define NVFP4_WEIGHT_MAGIC 0x34504656u /* "VFP4" */
#define NVFP4_WEIGHT_VERSION 1u

typedef struct nvfp4_weight_desc {
    uint32_t magic;                  /* NVFP4_WEIGHT_MAGIC */
    uint32_t version;                /* NVFP4_WEIGHT_VERSION */
    int64_t n;                       /* total output features (sum of module rows) */
    int64_t k;                       /* input features */
    int64_t n_padded;                /* n rounded up to the packing tile (rows beyond n are zero) */
    int32_t n_modules;
    int32_t reserved;
    int64_t module_rows[NVFP4_MAX_MODULES];
    int64_t module_row_offset[NVFP4_MAX_MODULES];
    const void* blob;                /* device address of the packed blob */
    size_t blob_bytes;
    size_t codes_offset;             /* byte offsets of the three regions inside the blob */
    size_t scales_offset;
    size_t colscale_offset;
} nvfp4_weight_desc;

/* Bytes of the blob for the given module row counts and K (0 if the shape is
 * invalid: K not a multiple of 128, or the padded codes n_padded*K/2 above
 * 2 GiB, since the GEMM kernels address each operand with 32-bit offsets). */
size_t nvfp4_packed_weight_bytes(int n_modules, const int64_t* module_rows, int64_t K);

/*
 * Pack n_modules canonical NVFP4 tensors into one blob.
 *
 * n_modules   : 1..NVFP4_MAX_MODULES
 * module_rows : host array, module_rows[s] >= 1
 * K           : > 0, multiple of 128 (NVFP4_ERR_UNSUPPORTED otherwise)
 * codes       : host array of n_modules device pointers, codes[s] is [module_rows[s]][K/2]
 * scales      : host array of n_modules device pointers, scales[s] is [module_rows[s]][K/16]
 * g_w         : host array of n_modules device pointers to each module's FP32 global scale
 * blob        : device, blob_bytes >= nvfp4_packed_weight_bytes(...) (256-byte aligned)
 * desc_out    : host, filled on success
 */
nvfp4_status nvfp4_pack_weights(int n_modules, const int64_t* module_rows, int64_t K,
                                const uint8_t* const* codes, const uint8_t* const* scales,
                                const float* const* g_w, void* blob, size_t blob_bytes,
                                nvfp4_weight_desc* desc_out, void* stream);

/* Weight re-quantization for a training step ("Normalized Architectures are
 * Natively 4-Bit": nGPT trains end to end in NVFP4, abstract and section
 * "Approach"; the weight changes after every optimizer step).  One weight
 * W [n][k] (a single module, one g) is read once and written as both packed
 * operands: blob_fwd holds W quantized along k (for Y = X . W^T, as
 * nvfp4_pack_weights of nvfp4_quantize(W) would), blob_bwd holds W^T
 * quantized along n (for dX = dY . W, as nvfp4_pack_weights of
 * nvfp4_quantize_t(W) would); both bit for bit, including padding rows,
 * column scales and the header fields.
 *
 * w            : device, n x k elements of in_dtype, row r at w + r*ld_w,
 *                aligned to the element size
 * n, k         : positive multiples of 128 (each is the other blob's K)
 * g, g_mode    : as for nvfp4_quantize (one g for both blobs)
 * blob_fwd     : device, 256-byte aligned, >= nvfp4_packed_weight_bytes({n}, k)
 * blob_bwd     : device, 256-byte aligned, >= nvfp4_packed_weight_bytes({k}, n)
 * desc_fwd/bwd : host, filled in on success (blob pointers set)
 * workspace    : COMPUTE mode, >= nvfp4_quantize_workspace_bytes(n, k)
 * Errors: NVFP4_ERR_SHAPE for n or k not a positive multiple of 128 or too
 * large, NVFP4_ERR_WORKSPACE for short blobs or workspace, the rest as for
 * nvfp4_quantize; nothing is launched then. */
nvfp4_status nvfp4_pack_weights_train(const void* w, int in_dtype, int64_t n, int64_t k, int64_t ld_w, float* g,
                                      int g_mode, void* blob_fwd, size_t blob_fwd_bytes, nvfp4_weight_desc* desc_fwd,
                                      void* blob_bwd, size_t blob_bwd_bytes, nvfp4_weight_desc* desc_bwd,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Inverse of the packing, for checking and for saving weights: writes the
 * canonical codes [n][K/2], scales [n][K/16] and per-row column scale [n]
 * (the owning module's g) of all modules stacked in order.
 */
nvfp4_status nvfp4_unpack_weights(const nvfp4_weight_desc* w, uint8_t* codes, uint8_t* scales,
                                  float* colscale, void* stream);

/* ---------------------------------------------------------------------------
 * Block-scaled GEMM: Y[m][n] = sum_k xhat[m][k] * what[n][k], FP32 out.
 *
 * The product every linear layer runs with both operands in NVFP4 ("Why
 * Gated DeltaNet Survives 4-Bit Quantization", section "Performance and
 * Efficiency Gains": weights and activations in NVFP4 on all 496 linear
 * layers), the dot products of "Normalized Architectures are Natively 4-Bit"
 * (section "Approach"); blocks of 16 along K carry their own scales (the
 * Gated DeltaNet page, section "Why the 'Fragile' Recurrence is Actually
 * Robust") and a fused projection keeps each module's global scale (its
 * section "Critical Lessons for Model Serving").
 *
 * xhat = e2m1(a_code) * e4m3(a_scale) * g_x, what = e2m1(w_code) * e4m3(w_scale)
 * * g_w[module(n)].  The products of decoded codes and block scales are exact in
 * FP16 and are multiplied and summed on the matrix cores in FP32; the two
 * global scales are applied once per output as fl32(acc * fl32(g_x * g_w)).
 *
 * M        : >= 0 (M == 0 enqueues nothing); M*K/2 <= 2 GiB, else
 *            NVFP4_ERR_UNSUPPORTED (32-bit operand offsets)
 * a_codes  : device, canonical [M][K/2] codes of the activations (K = w->k)
 * a_scales : device, canonical [M][K/16]
 * g_x      : device, one float (the activations' global scale)
 * w        : host descriptor from nvfp4_pack_weights
 * y        : device, FP32, row m at y + m*ld_y; columns [0, w->n) are written
 * ld_y     : >= w->n
 * workspace: device, >= nvfp4_gemm_workspace_bytes(M, w) bytes, 256-byte aligned
 *            (may be NULL when that is 0, which it is for every shape of this
 *            version: the product keeps no state between workgroups).  For few
 *            tokens (1 <= M <= 16, K <= 8192) one workgroup takes each 32 rows
 *            of the weight (16 when K > 5120) over all of K and adds its
 *            wavefronts' partial sums per 16 rows in a fixed order, so results
 *            do not depend on scheduling.
 * ------------------------------------------------------------------------- */
size_t nvfp4_gemm_workspace_bytes(int64_t M, const nvfp4_weight_desc* w);
nvfp4_status nvfp4_gemm(int64_t M, const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                        const nvfp4_weight_desc* w, float* y, int64_t ld_y,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Linear layer: quantize the activations and multiply them by a packed weight
 * in one call (the W4A4 linear layer of the Gated DeltaNet page, section
 * "Performance and Efficiency Gains").  Same codes, scales, g and Y bits as
 * nvfp4_quantize followed by nvfp4_gemm on the same stream.
 *
 * For few tokens (1 <= M <= 16, K <= 8192) the whole call is one kernel.  On
 * each of the 8 XCDs, 8 encoder workgroups reduce max|x| over the tensor (an
 * eighth each, exchanged through that XCD's L2) and encode an eighth of the
 * blocks each, into a copy in the order the products read (in the workspace);
 * the product workgroups stream and decode their weight rows meanwhile, wait
 * for their own XCD's encoders and multiply, and each writes its share of the
 * 128-element k-steps of x_codes and x_scales from the operand it multiplied
 * (every output byte once).  A workgroup that runs on
 * another XCD than its index is meant for, or whose wait exceeds a bound,
 * encodes the activations itself (the same bytes), so no result depends on
 * placement or on another workgroup being resident; the environment variable
 * NVFP4_AMAX_POLLS overrides the bound (0 forces the local path, for tests).
 *
 * x, in_dtype, ld_x     : as for nvfp4_quantize, rows = M, K = w->k (M*K/2 <= 2 GiB)
 * x_codes, x_scales, g_x: the activations' NVFP4 encoding (outputs; g_x is an
 *                         input in NVFP4_G_GIVEN mode), as for nvfp4_quantize
 * w, y, ld_y            : as for nvfp4_gemm
 * workspace             : device, >= nvfp4_linear_workspace_bytes(M, in_dtype, w)
 *                         bytes (at most 2048 + 73728 + 4096), 256-byte aligned.
 *                         Its first 2048 bytes hold the few-token path's flags
 *                         (tagged with the launch, so no call needs them reset):
 *                         zero before the first use.  Then, for weights with
 *                         K <= 8192, K/128 * 1152 bytes (rounded up to 256) where
 *                         the few-token kernel's encoders leave a second copy of
 *                         the activation encoding in the order its products read
 *                         (per 128-element k-step the 16 token slots' code bytes,
 *                         then their scale bytes); then the amax partials of the
 *                         two-launch path.  Both need no initialisation.  The
 *                         sizes do not depend on M, so one workspace serves any
 *                         token count.  Calls that may run concurrently must not
 *                         share a workspace.
 * ------------------------------------------------------------------------- */
size_t nvfp4_linear_workspace_bytes(int64_t M, int in_dtype, const nvfp4_weight_desc* w);
nvfp4_status nvfp4_linear(const void* x, int in_dtype, int64_t M, int64_t ld_x, uint8_t* x_codes,
                          uint8_t* x_scales, float* g_x, int g_mode, const nvfp4_weight_desc* w, float* y,
                          int64_t ld_y, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * nvfp4_linear without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, results and bits as nvfp4_linear
 * otherwise.
 *
 * The workspace nvfp4_linear would take (the few-token kernel's flags and
 * activation copy, then the quantizer's amax partials) is a static 80 KiB device array inside
 * the library instead, which every shape fits (nvfp4_linear_workspace_bytes
 * never exceeds it; a larger request would give NVFP4_ERR_UNSUPPORTED).  Each
 * GPU holds its own copy until the process ends; the first call on a device
 * looks its address up and clears it with a small kernel on `stream`.  The
 * call itself allocates and frees nothing.
 *
 * Every call on one GPU shares that GPU's array: calls that may overlap on a
 * GPU (other streams, other host threads) race on it and must be ordered by
 * the caller.  Calls on one stream are ordered by the stream.
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_linear_noalloc(const void* x, int in_dtype, int64_t M, int64_t ld_x, uint8_t* x_codes,
                                  uint8_t* x_scales, float* g_x, int g_mode, const nvfp4_weight_desc* w, float* y,
                                  int64_t ld_y, void* stream);

/* ---------------------------------------------------------------------------
 * Gate epilogue of a fused Gated DeltaNet input projection (anthology-of-the-
 * sota record theory-128, Kozyrev and Maiboroda 2026, section "The account",
 * its paragraph on the gates' parameterization: the state decay is
 * exp(-exp(A) * softplus(a + b)) and the write strength a sigmoid).  The two small gate projections sit in
 * the same fused weight as q, k, v, z; the epilogue turns their output columns
 * into the gates as Y is written, so no second pass over Y is needed:
 *
 *   column a_col + h (0 <= h < n_a):  exp(-exp(a_log[h]) * softplus(y + dt_bias[h]))
 *   column b_col + h (0 <= h < n_b):  1 / (1 + exp(-y))
 *   every other column:               y unchanged (the same bits as without gates)
 *
 * y is the product's FP32 output (global scales applied); the gates are
 * evaluated in FP32 (softplus and the sigmoid in their overflow-free forms).
 * a_col, n_a, b_col, n_b: two disjoint column ranges inside [0, w->n), n >= 0
 * a_log, dt_bias        : device, n_a FP32 values each (may be NULL when n_a == 0)
 * ------------------------------------------------------------------------- */
typedef struct nvfp4_gdn_gates {
    int64_t a_col, n_a;
    int64_t b_col, n_b;
    const float* a_log;
    const float* dt_bias;
} nvfp4_gdn_gates;

/* nvfp4_gemm / nvfp4_linear with the gate epilogue; same arguments, workspace
 * sizes and behaviour otherwise.  NVFP4_ERR_INVALID_ARG for a NULL gates
 * pointer or missing parameters, NVFP4_ERR_SHAPE for ranges outside [0, w->n)
 * or overlapping. */
nvfp4_status nvfp4_gemm_gated(int64_t M, const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                              const nvfp4_weight_desc* w, const nvfp4_gdn_gates* gates, float* y, int64_t ld_y,
                              void* workspace, size_t workspace_bytes, void* stream);
nvfp4_status nvfp4_linear_gated(const void* x, int in_dtype, int64_t M, int64_t ld_x, uint8_t* x_codes,
                                uint8_t* x_scales, float* g_x, int g_mode, const nvfp4_weight_desc* w,
                                const nvfp4_gdn_gates* gates, float* y, int64_t ld_y, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Product with an output epilogue: the output type and, optionally, the GDN
 * gates (anthology-of-the-sota record theory-128, section "The account", the
 * paragraph on the gates' parameterization; the projection's output feeds
 * the recurrence).
 *
 * y_dtype : NVFP4_OUT_F32 or NVFP4_OUT_BF16 (else NVFP4_ERR_INVALID_ARG)
 * reserved: must be 0
 * gates   : NULL for none, else as for nvfp4_gemm_gated
 * y, ld_y : device, M rows of ld_y elements of y_dtype (4- or 2-byte aligned)
 * Everything else, workspace sizes included, as nvfp4_gemm / nvfp4_linear.
 * A bf16 element is the round-to-nearest-even of the FP32 element the same
 * call with NVFP4_OUT_F32 writes.
 * ------------------------------------------------------------------------- */
typedef struct nvfp4_epilogue {
    int32_t y_dtype;
    int32_t reserved;
    const nvfp4_gdn_gates* gates;
} nvfp4_epilogue;

nvfp4_status nvfp4_gemm_ex(int64_t M, const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                           const nvfp4_weight_desc* w, const nvfp4_epilogue* ep, void* y, int64_t ld_y,
                           void* workspace, size_t workspace_bytes, void* stream);
nvfp4_status nvfp4_linear_ex(const void* x, int in_dtype, int64_t M, int64_t ld_x, uint8_t* x_codes,
                             uint8_t* x_scales, float* g_x, int g_mode, const nvfp4_weight_desc* w,
                             const nvfp4_epilogue* ep, void* y, int64_t ld_y, void* workspace,
                             size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
